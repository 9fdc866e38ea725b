// The chunk plan of a prefill: every sequence is cut into chunks of at most
// `chunk` tokens, the chunks of one sequence consecutive in the table.  The
// running state of Mechanism step 3 ("Diving into MiniMax01 405B MoE",
// section "Hybrid Modeling") is a sum over past tokens, so each chunk can be
// walked from the state entering it.
//
// Plain C++ with no HIP dependency: plan_kernel (plan_scan_norm.hip) runs
// plan_sequences on the GPU with one 1024-thread workgroup, and a host build
// runs the same function with one thread per lane and a barrier for each
// workgroup barrier, to check its bounds on invalid inputs.  The includer
// defines LA_HD (__host__ __device__ for the GPU build).
#pragma once

#include <stdint.h>

#ifndef LA_HD
#define LA_HD
#endif

namespace la {

struct PlanHeader {
    int32_t n_chunks;  // chunks in the table (0 if cu_seqlens was invalid)
    int32_t error;     // 0 = ok, 1 = cu_seqlens inconsistent, 2 = table overflow,
                       // 3 = a cross-workgroup wait of an MFMA prefill timed out
    int32_t ticket;    // start-order ticket of the fused walk's workgroups
    int32_t wait_site; // error 3: which wait gave up first, where and who:
                       // 1 group sums, 4 norm factors (chunk, head)
    int32_t wait_chunk;
    int32_t wait_head;
    int32_t pad[10];
};
struct SegEntry {
    int32_t first;  // index of the sequence's first chunk
    int32_t count;  // number of chunks (0 for an empty sequence)
};
struct ChunkEntry {
    int64_t start;  // first token (packed index)
    int32_t len;    // tokens in the chunk, 1..chunk
    int32_t seg;    // owning sequence
};

// One workgroup of NT threads; Ctx gives the thread index (tid()), the
// workgroup barrier (sync()) and memory shared by the workgroup: scan[NT]
// (int64), and the flags *bad and *err (int32-like).
//
// Sequence s holds tokens [cu[s], cu[s+1]) (rows of `seqlen` tokens when cu
// is null).  Counts and offsets are 64-bit: with an invalid cu_seqlens (say,
// an uninitialised buffer) lengths swing by up to 2^32, and 32-bit sums of
// chunk counts could wrap to a negative first chunk.  A chunk record is only
// written inside [0, max_chunks), and an invalid plan (error 1 or 2) leaves
// every sequence with no chunk.  chunks may be null (counts only).
template <int NT, class Ctx>
LA_HD void plan_sequences(const Ctx& x, const int32_t* cu, int nseq, int64_t seqlen,
                          int64_t total, int chunk, int max_chunks, PlanHeader* hdr,
                          SegEntry* segs, ChunkEntry* chunks) {
    const int tid = x.tid();
    if (tid == 0) {
        hdr->ticket = 0;  // start-order ticket of the MFMA walk
        hdr->wait_site = hdr->wait_chunk = hdr->wait_head = 0;
        *x.bad = 0;
        if (cu != nullptr && (cu[0] != 0 || (int64_t)cu[nseq] != total)) *x.bad = 1;
    }
    x.sync();
    int64_t carry = 0;
    for (int base = 0; base < nseq; base += NT) {
        const int s = base + tid;
        int64_t start = 0, len = 0;
        if (s < nseq) {
            if (cu != nullptr) {
                start = cu[s];
                len = (int64_t)cu[s + 1] - start;
                if (len < 0) *x.bad = 1;
            } else {
                start = (int64_t)s * seqlen;
                len = seqlen;
            }
        }
        const int64_t cnt = len > 0 ? (len + chunk - 1) / chunk : 0;
        x.scan[tid] = cnt;
        x.sync();
        for (int off = 1; off < NT; off <<= 1) {  // inclusive Hillis-Steele
            const int64_t add = tid >= off ? x.scan[tid - off] : 0;
            x.sync();
            x.scan[tid] += add;
            x.sync();
        }
        const int64_t first = carry + x.scan[tid] - cnt;  // >= 0, nondecreasing in s
        if (s < nseq) {
            // values beyond 32 bits only occur with an invalid plan, whose
            // counts are reset to 0 below
            segs[s].first = (int32_t)(first < INT32_MAX ? first : INT32_MAX);
            segs[s].count = (int32_t)(cnt < INT32_MAX ? cnt : INT32_MAX);
            if (chunks != nullptr && first + cnt <= (int64_t)max_chunks) {
                for (int64_t c = 0; c < cnt; ++c) {
                    ChunkEntry e;
                    e.start = start + c * chunk;
                    const int64_t rem = len - c * chunk;
                    e.len = (int32_t)(rem < chunk ? rem : chunk);
                    e.seg = s;
                    chunks[first + c] = e;
                }
            }
        }
        carry += x.scan[NT - 1];
        x.sync();
    }
    if (tid == 0) {
        const int32_t err = *x.bad ? 1 : (chunks != nullptr && carry > (int64_t)max_chunks ? 2 : 0);
        *x.err = err;
        hdr->error = err;
        hdr->n_chunks = err ? 0 : (int32_t)carry;
    }
    x.sync();
    if (*x.err != 0)
        for (int s = tid; s < nseq; s += NT) segs[s].count = 0;
}

}  // namespace la
