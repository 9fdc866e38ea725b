// Chunk states of the Lightning Attention layer on bf16 MFMA for gfx950
// (head_dim 128, 64-token blocks, fp32 accumulation):
//   states[c][h][dk][dv] = sum over chunk c's tokens t of k~_t[dk] v~_t[dv],
// k~ = SiLU(k), v~ = SiLU(v) -- the running-state sum of Mechanism step 3 of
// "Diving into MiniMax01 405B MoE" (section "Hybrid Modeling") over one chunk.
// With the prefix scan over a sequence's chunks (plan_scan_norm.hip) it gives
// each sequence's final state without the walk (the state-only calls), and
// the state entering every chunk for the MFMA prefill, whose walk then
// starts every chunk at once.
#include "mfma_common.h"

namespace la {

namespace {

constexpr int ST_THREADS = 1024;  // 16 waves, all of which load, apply SiLU and multiply
constexpr int SPF = 4;           // blocks in flight per thread (register sets)

struct StateLds {
    __bf16 k[2][TILE];
    __bf16 v[2][TILE];
};

// The same kernel gives the backward's chunk sums of q~^T dy: its operands
// are any two bf16 activations, the first through SiLU when SA, the second
// when SB (k, v: both; q, dy: the first; operands a projection already
// activated: neither).
//
// One workgroup per (chunk, head), state written at states[c][h].  With
// skip_last, the last chunk of each sequence is left out (the prefill does
// not need its sum: its walk forms the final state).  Thread t loads row
// t / 16 of a block, features 8 (t % 16) .. + 7, applies SiLU and writes the
// swizzled bf16 tiles; wave w accumulates the state tile dk in
// [32 (w / 4), +32), dv in [32 (w % 4), +32).  Every wave takes part in the
// SiLU: it is a chain of dependent transcendental operations, and four waves
// per SIMD hide its latency better than two (8192 x 64 heads: 2-3 us less
// per prefill than 512 threads with two rows each).
// Uniform rows without a plan kernel: nseq rows of seqlen tokens cut into
// cps = ceil(seqlen / chunk) chunks each; the last `extra` workgroups of the
// grid write what the plan kernel would (tables and header; the state scan
// that follows clears the exchange words).
struct InlinePlan {
    int extra;  // 0: the plan kernel ran, read its tables
    int nseq, cps, chunk;
    int64_t seqlen;
    PlanHeader* hdr;
    SegEntry* segs;
    ChunkEntry* chunks;
    uint64_t* clear;
    int64_t clear_words;
};

__device__ __forceinline__ ChunkEntry uniform_chunk(const InlinePlan& ip, int c) {
    const int s = c / ip.cps, i = c - s * ip.cps;
    ChunkEntry ce;
    ce.start = (int64_t)s * ip.seqlen + (int64_t)i * ip.chunk;
    ce.len = (int)min((int64_t)ip.chunk, ip.seqlen - (int64_t)i * ip.chunk);
    ce.seg = s;
    return ce;
}

__device__ void write_plan(const InlinePlan& ip, int e, int tid) {
    const int64_t stride = (int64_t)ip.extra * ST_THREADS;
    const int64_t i0 = (int64_t)e * ST_THREADS + tid;
    for (int64_t i = i0; i < ip.clear_words; i += stride) ip.clear[i] = 0;
    const int64_t nch = (int64_t)ip.nseq * ip.cps;
    for (int64_t c = i0; c < nch; c += stride) ip.chunks[c] = uniform_chunk(ip, (int)c);
    for (int64_t s = i0; s < ip.nseq; s += stride)
        ip.segs[s] = SegEntry{(int32_t)(s * ip.cps), ip.cps};
    if (e == 0 && tid == 0) {
        ip.hdr->ticket = 0;
        ip.hdr->wait_site = ip.hdr->wait_chunk = ip.hdr->wait_head = 0;
        ip.hdr->error = 0;
        ip.hdr->n_chunks = (int32_t)nch;
    }
}

template <bool SA, bool SB>
__global__ __launch_bounds__(ST_THREADS) void chunk_state_mfma_kernel(
    const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const PlanHeader* __restrict__ hdr, const SegEntry* __restrict__ segs,
    const ChunkEntry* __restrict__ chunks, float* __restrict__ states, int H, SumSkip skip,
    const InlinePlan ip) {
    __shared__ __attribute__((aligned(16))) StateLds L;
    const int n_sum = (int)gridDim.x - ip.extra;
    if ((int)blockIdx.x >= n_sum) {
        write_plan(ip, (int)blockIdx.x - n_sum, threadIdx.x);
        return;
    }
    const int c = blockIdx.x / H, h = blockIdx.x - c * H;
    ChunkEntry ce;
    if (ip.extra > 0) {
        if (c >= ip.nseq * ip.cps) return;
        ce = uniform_chunk(ip, c);
        const int i = c - ce.seg * ip.cps;
        if ((skip == SumSkip::last && i == ip.cps - 1) || (skip == SumSkip::first && i == 0)) return;
    } else {
        if (c >= hdr->n_chunks) return;
        ce = chunks[c];
        if (skip != SumSkip::none) {
            const SegEntry se = segs[ce.seg];
            if (c == (skip == SumSkip::last ? se.first + se.count - 1 : se.first)) return;
        }
    }
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int HD = H * MD;
    const int len = ce.len;
    const int nblk = (len + MB - 1) / MB;
    const int64_t off0 = ce.start * (int64_t)HD + (int64_t)h * MD;
    const int cc = tid & 15, rg = tid >> 4;
    const int voff = (rg * HD + 8 * cc) * 2;
    // Block b is loaded into register set b % SPF, SPF blocks ahead.  Loads
    // are issued unconditionally (blocks past the chunk's end get an empty
    // range and return zeros): a conditional load would make the compiler
    // copy registers that still have a load in flight.
    bf16x8 tk[SPF], tv[SPF];
    // The blocks are visited last to first: a prefill's walk, which starts
    // with each chunk's first block, then finds the most recently read K and
    // V first (still in the caches).
    auto load_rows = [&](const __bf16* base, int i, bf16x8& t) {
        const int b = nblk - 1 - i;
        const int t0 = max(b, 0) * MB, n = b < 0 ? 0 : max(0, min(MB, len - t0));
        const __amdgpu_buffer_rsrc_t rs = tile_rsrc(base + off0 + (int64_t)t0 * HD, n, HD);
        t = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 0, 0));
    };
#pragma unroll
    for (int i = 0; i < SPF; ++i) {
        load_rows(k, i, tk[i]);
        load_rows(v, i, tv[i]);
        // keeps the compiler from issuing all sets' loads of one tensor first;
        // it still issues k1 k2 k3 before v1 v2 v3, so two steps of every
        // pass wait one set early (issuing the sets in order, which needs the
        // loads marked volatile, measured the same)
        __builtin_amdgcn_sched_barrier(0);
    }
    const int l32 = lane & 31, g = lane >> 5;
    const int n = w & 3, m = w >> 2;
    f32x16 acc = {};
    // One barrier per block with two LDS buffers: a wave writes buffer b & 1
    // only after passing block b - 1's barrier, which every wave reaches only
    // after its products of block b - 2 (the same buffer).  Passes of SPF
    // blocks run whole: blocks past the chunk's end hold zeros and add
    // nothing, and without a conditional exit inside the pass the compiler
    // keeps the later sets' loads in flight across the loop's back edge.
    for (int b0 = 0; b0 < nblk; b0 += SPF) {
#pragma unroll
        for (int i = 0; i < SPF; ++i) {
            const int b = b0 + i;
            __bf16* sK = L.k[b & 1];
            __bf16* sV = L.v[b & 1];
            *reinterpret_cast<bf16x8*>(sK + swz(rg, 8 * cc)) = act8<SA>(tk[i]);
            *reinterpret_cast<bf16x8*>(sV + swz(rg, 8 * cc)) = act8<SB>(tv[i]);
            load_rows(k, b + SPF, tk[i]);
            load_rows(v, b + SPF, tv[i]);
            __syncthreads();
            // all operands in flight before the products
            bf16x8 vb[MB / 16], ka[MB / 16];
#pragma unroll
            for (int s = 0; s < MB / 16; ++s) {
                vb[s] = ld_tr_operand(sV, 16 * s, 32 * n, lane);
                ka[s] = ld_tr_operand(sK, 16 * s, 32 * m, lane);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < MB / 16; ++s) acc = mfma32(ka[s], vb[s], acc);
        }
    }
    float* dst = states + ((int64_t)c * H + h) * MD * MD;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int dk = 32 * m + 8 * (r >> 2) + 4 * g + (r & 3);
        dst[dk * MD + 32 * n + l32] = acc[r];
    }
}

}  // namespace

bool state_mfma_supported(const PrefillArgs& a) { return a.bf16 && a.D == MD && a.block == MB; }

hipError_t launch_chunk_sums_mfma(const PrefillArgs& a, const void* x, const void* y, bool silu_x,
                                  bool silu_y, float* states, SumSkip skip, hipStream_t st) {
    if (a.max_chunks == 0) return hipSuccess;
    InlinePlan ip{};
    if (a.inline_plan) {
        ip.extra = 64;  // on the CUs the chunk sums leave idle
        ip.nseq = a.nseq;
        ip.chunk = a.chunk;
        ip.seqlen = a.seqlen;
        ip.cps = (int)((a.seqlen + a.chunk - 1) / a.chunk);
        ip.hdr = a.hdr;
        ip.segs = a.segs;
        ip.chunks = a.chunks;
        // the exchange words are cleared by the scan after this kernel
        // (stores here would compete with the sums' reads)
        ip.clear = nullptr;
        ip.clear_words = 0;
    }
    const dim3 grid((unsigned)((int64_t)a.max_chunks * a.H + ip.extra));
    auto* fn = silu_x ? (silu_y ? &chunk_state_mfma_kernel<true, true>
                                : &chunk_state_mfma_kernel<true, false>)
                      : (silu_y ? &chunk_state_mfma_kernel<false, true>
                                : &chunk_state_mfma_kernel<false, false>);
    hipLaunchKernelGGL(fn, grid, dim3(ST_THREADS), 0, st, (const __bf16*)x, (const __bf16*)y,
                       a.hdr, a.segs, a.chunks, states, a.H, skip, ip);
    return hipGetLastError();
}

hipError_t launch_chunk_state_mfma(const PrefillArgs& a, hipStream_t st) {
    return launch_chunk_sums_mfma(a, a.k, a.v, !a.preact, !a.preact, a.states,
                                  a.skip_last ? SumSkip::last : SumSkip::none, st);
}

}  // namespace la
