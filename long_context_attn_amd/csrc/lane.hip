// Lane-parallel bf16 MFMA prefill of the Lightning Attention layer for gfx950
// (head_dim 128, 64-token blocks, fp32 running state).
//
// Mechanism step 3 of "Diving into MiniMax01 405B MoE" (section "Hybrid
// Modeling") is a recurrence along each sequence; step 4 normalises every
// token over all heads.  Here one workgroup -- a lane -- owns one head h and
// one slice of 32 state columns, dv in [32 sl, 32 sl + 32), and walks every
// sequence's 64-token blocks in order, keeping its 128 x 32 slice S of the
// state in registers from block to block:
//   P^T  = K~_b Q~_b^T, masked to t' <= t            (all 128 features)
//   O^T  = S^T Q~_b^T + V~_b[:, slice]^T P^T         (32 x 64)
//   S   += K~_b^T V~_b[:, slice]                     (128 x 32)
// then writes out = y / sqrt(mean_{h,d} y^2 + eps) * w * sigmoid(gate) for its
// 32 columns.  No sequence is cut into chunks, so no chunk state is formed,
// handed over or re-read: each of Q, K, V and the gate is read once per
// lane.  The four lanes of a head share its Q and K; lanes are numbered so
// that they run on one XCD (workgroups go round-robin over the 8 XCDs), where
// three of the four reads of a Q or K block hit that XCD's L2.
//
// The lanes of all heads run concurrently (H * 4 <= CUs, one workgroup per
// CU) and advance in near lockstep: the RMSNorm of a block needs the sums of
// y^2 of every lane.  Those go through a three-level exchange of 8-byte
// words {float, tag = block + 1} in rings of XR slots per level:
//   * iteration j + 1 (after computing block j): every lane publishes its 64
//     per-token sums, part[j % XR][lane][t];
//   * iteration j + 1 + LAG1: the sub-reducer of each group of XG lanes
//     (rotating over the group's members) adds its group's words in lane
//     order, rsub[j % XR][group][t];
//   * iteration j + 1 + LAG1 + LAG2: lane j % NL adds the group sums in group
//     order, tot[j % XR][t];
//   * iteration j + 1 + LAG1 + LAG2 + LAG3: every lane reads tot and leaves
//     1 / sqrt(tot / (H * 128) + eps) in LDS; one iteration later its
//     producers write the block's outputs.
// Every wait is for words written at an earlier iteration, so no wait
// closes a cycle; the sums are formed in a fixed order, so results do not
// depend on timing.  A wait gives up after WAIT_POLLS polls (error 3 in the
// plan header) if not every lane could be resident.
//
// Waves (512 threads): 4-7 producers (16-byte loads two blocks ahead, SiLU
// in fp32, bf16 tiles in LDS, final stores); 0 the state wave (S, O, y, the
// state at sequence boundaries); 1-3 one score quadrant each, and the
// exchange (2: sub-reduction, 3: final reduction and the norm factors).
#include "mfma_common.h"

namespace la {

namespace {

constexpr int LT = 512;          // threads
constexpr int NSL = 4;           // state slices per head
constexpr int SW = MD / NSL;     // slice width (32 columns)
constexpr int LPP = MB + 8;      // pitch of the score tile
constexpr int LYP = SW + 8;      // pitch of the y slice tiles (rows 16-byte aligned)
constexpr int LAG1 = 2, LAG2 = 2, LAG3 = 2;
constexpr int LFIN = 2 + LAG1 + LAG2 + LAG3;  // iterations from staging a block to its stores
constexpr int LYR = LFIN - 1;    // y tiles in LDS
constexpr int XR = 16;           // exchange ring slots per level (power of two)
constexpr int XG = 16;           // lanes per sub-reduction group
constexpr int XGMAX = 16;        // groups at most (lanes <= 256)
static_assert(XR >= LFIN + LAG1 + 1 && XR >= LFIN + LAG2 + 1 && XR >= LFIN + LAG3 + 1,
              "a ring slot is rewritten only after every reader of its last block is done");
static_assert((XR & (XR - 1)) == 0, "XR is a power of two");

struct LaneLds {
    __bf16 q[2][TILE];           // Q~ (swizzled, all 128 features)
    __bf16 k[2][TILE];           // K~
    __bf16 v[2][TILE];           // V~, only this lane's 32 columns written
    __bf16 y[LYR][MB * LYP];     // y of the last blocks (bf16), until finalised
    __bf16 p[MB * LPP];          // masked scores P [t][t']
    float rn[2][MB];             // norm factors of the block finalised next
    float red[MB];               // this lane's sums of y^2 per token, block just computed
};

// Position in the sequence of blocks: block b of sequence s, which spans
// tokens [start, start + len).  s == nseq once past the last sequence (then
// the block has no rows).
struct Cursor {
    int s, b;
    int64_t start, len;
};

struct Seqs {
    const int32_t* cu;  // device cu_seqlens, or null for nseq rows of seqlen tokens
    int nseq;
    int64_t seqlen;
    __device__ __forceinline__ int64_t start(int s) const {
        return cu ? (int64_t)cu[s] : (int64_t)s * seqlen;
    }
    __device__ __forceinline__ int64_t len(int s) const {
        return cu ? (int64_t)cu[s + 1] - (int64_t)cu[s] : seqlen;
    }
    // from sequence s on, the first non-empty one
    __device__ __forceinline__ void seek(Cursor& c, int s) const {
        c.b = 0;
        c.start = 0;
        c.len = 0;
        for (c.s = s; c.s < nseq; ++c.s) {
            c.len = len(c.s);
            if (c.len > 0) {
                c.start = start(c.s);
                return;
            }
        }
        c.len = 0;
    }
    __device__ __forceinline__ void next(Cursor& c) const {
        if (c.s >= nseq) return;
        if ((int64_t)(c.b + 1) * MB < c.len) {
            ++c.b;
            return;
        }
        seek(c, c.s + 1);
    }
};
__device__ __forceinline__ int rows(const Cursor& c) {
    const int64_t r = c.len - (int64_t)c.b * MB;
    return r <= 0 ? 0 : (r < MB ? (int)r : MB);
}
__device__ __forceinline__ int64_t tok0(const Cursor& c) {
    return c.len > 0 ? c.start + (int64_t)c.b * MB : 0;
}
__device__ __forceinline__ bool last_block(const Cursor& c) {
    return (int64_t)(c.b + 1) * MB >= c.len;
}

// Buffer resource over the 32-column slices of rows 0 .. n-1 (rows HD
// elements apart); loads past the last row return zeros, stores are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slice_rsrc(const __bf16* base, int n, int HD) {
    const int bytes = n > 0 ? ((n - 1) * HD + SW) * 2 : 0;
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, bytes, 0x00020000);
}

// Exchange words of this kernel: the float in the low half, tag = block + 1
// in the high half (0 = cleared by the plan kernel).
__device__ __forceinline__ uint64_t put_tagged(uint64_t* p, float x, uint32_t tag) {
    const uint64_t word = ((uint64_t)tag << 32) | __float_as_uint(x);
    __hip_atomic_store(p, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return word;
}
__device__ __forceinline__ bool has_tag(uint64_t x, uint32_t tag) { return (uint32_t)(x >> 32) == tag; }

// One producer thread's share of a block: a quarter of the Q and K tiles'
// 16-byte pieces (rows 4 rg .. 4 rg + 3, features 8 cc ..) and one piece of
// the V slice (row vr, features 32 sl + 8 vc ..).
struct LTiles {
    Tile q, k;
    bf16x8 v;
};

__global__ __launch_bounds__(LT) void prefill_lane_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ gate, const __bf16* __restrict__ wgt, __bf16* __restrict__ out,
    PlanHeader* __restrict__ hdr, const int32_t* __restrict__ cu, int nseq, int64_t seqlen,
    const float* __restrict__ init_state, float* __restrict__ final_state,
    uint64_t* __restrict__ part, uint64_t* __restrict__ rsub, uint64_t* __restrict__ tot, int H,
    float eps) {
    __shared__ __attribute__((aligned(16))) LaneLds L;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int NL = H * NSL, NG = (NL + XG - 1) / XG;
    const int wg = blockIdx.x;
    // (head, slice) of this lane: the four slices of a head share wg % 8
    int h, sl;
    if ((H & 7) == 0) {
        const int j = wg >> 3;
        h = (j / NSL) * 8 + (wg & 7);
        sl = j % NSL;
    } else {
        h = wg / NSL;
        sl = wg % NSL;
    }
    if (hdr->error != 0) return;  // invalid cu_seqlens: nothing is written
    const int nb = hdr->n_chunks;  // blocks of all sequences (64-token plan)
    const Seqs sq{cu, nseq, seqlen};
    const int HD = H * MD;
    const int64_t DD = (int64_t)MD * MD;

    // empty sequences: final state = initial state (or zeros), this lane's slice
    if (final_state != nullptr) {
        for (int s0 = 0; s0 < nseq; s0 += LT) {
            const int s = s0 + tid;
            if (s < nseq && sq.len(s) == 0) {
                const int64_t base = ((int64_t)s * H + h) * DD + SW * sl;
                for (int r = 0; r < MD; ++r)
                    for (int c = 0; c < SW; c += 4) {
                        f32x4 x = {0.f, 0.f, 0.f, 0.f};
                        if (init_state) x = *reinterpret_cast<const f32x4*>(init_state + base + r * MD + c);
                        *reinterpret_cast<f32x4*>(final_state + base + r * MD + c) = x;
                    }
            }
        }
    }
    if (nb == 0) return;
    const int iters = nb + LFIN;

    if (w >= 4) {
        // ------------------------------------------------------ producers
        const int ptid = tid - 256;
        const int cc = ptid & 15, rg = ptid >> 4;  // Q, K tile pieces
        const int vr = ptid >> 2, vc = ptid & 3;   // slice pieces (V, gate, out)
        const int voff = (4 * rg * HD + 8 * cc) * 2, rstride = HD * 2;
        const int soff = (vr * HD + 8 * vc) * 2;
        const int hcol = h * MD, scol = h * MD + SW * sl;
        const bf16x8 wv = *reinterpret_cast<const bf16x8*>(wgt + scol + 8 * vc);
        // Two register sets: the tiles of block i are loaded into set i & 1
        // two iterations ahead, and so is the gate of the block that
        // iteration i finalises.  Loads are issued unconditionally (blocks
        // past the end get an empty range and return zeros).
        Cursor ld, gl, fz;
        sq.seek(ld, 0);
        gl = ld;
        fz = ld;
        auto load_q = [&](const Cursor& c, Tile& t) {
            load_tile(t, tile_rsrc(q + tok0(c) * HD + hcol, rows(c), HD), voff, rstride);
        };
        auto load_kv = [&](const Cursor& c, LTiles& t) {
            const int64_t o = tok0(c) * HD;
            load_tile(t.k, tile_rsrc(k + o + hcol, rows(c), HD), voff, rstride);
            t.v = __builtin_bit_cast(
                bf16x8, __builtin_amdgcn_raw_buffer_load_b128(slice_rsrc(v + o + scol, rows(c), HD),
                                                              soff, 0, 0));
        };
        LTiles t0, t1;
        bf16x8 g0, g1;
        load_q(ld, t0.q);
        load_kv(ld, t0);
        sq.next(ld);
        load_q(ld, t1.q);
        load_kv(ld, t1);
        sq.next(ld);
        // The output of block it - LFIN is computed in phase 1 (its y slot is
        // rewritten in phase 2) and stored at the end of phase 2, after the
        // loads of that iteration: a wait for a load then never covers a
        // store younger than two iterations.  The stored registers stay
        // allocated until barrier A of the next iteration.
        u32x4 od_prev = {0u, 0u, 0u, 0u};
        auto step = [&](int it, LTiles& t, bf16x8& tg) {
            const int buf = it & 1;
            // ---- phase 1: output of block it - LFIN, a gate load, stage Q~
            const bool fin = it >= LFIN;  // (it - LFIN < nb: the loop ends there)
            u32x4 od = {0u, 0u, 0u, 0u};
            if (fin) {
                const int jf = it - LFIN;
                const bf16x8 y = *reinterpret_cast<const bf16x8*>(L.y[jf % LYR] + vr * LYP + 8 * vc);
                const float rr = L.rn[jf & 1][vr];
                bf16x8 o;
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    o[u] = (__bf16)((float)y[u] * rr * (float)wv[u] * sigmoid_f((float)tg[u]));
                od = __builtin_bit_cast(u32x4, o);
            }
            {
                // gate of block it + 2 - LFIN, finalised in iteration it + 2
                const bool gv = it + 2 >= LFIN;
                const int n = gv ? rows(gl) : 0;
                tg = __builtin_bit_cast(
                    bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                slice_rsrc(gate + tok0(gl) * HD + scol, n, HD), soff, 0, 0));
                if (gv) sq.next(gl);
            }
            if (it < nb) {
                bf16x8 qs[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) qs[r] = silu8(t.q.r[r]);
                store_rows(qs, L.q[buf], cc, rg);
            }
            load_q(ld, t.q);  // block it + 2
            __syncthreads();  // A
            keep(od_prev);
            // ---- phase 2: stage K~ and the V~ slice; store the output
            if (it < nb) {
                bf16x8 ks[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) ks[r] = silu8(t.k.r[r]);
                store_rows(ks, L.k[buf], cc, rg);
                *reinterpret_cast<bf16x8*>(L.v[buf] + swz(vr, SW * sl + 8 * vc)) = silu8(t.v);
            }
            load_kv(ld, t);
            sq.next(ld);
            if (fin) {
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_raw_buffer_store_b128(
                    od, slice_rsrc(out + tok0(fz) * HD + scol, rows(fz), HD), soff, 0, 0);
                sq.next(fz);
            }
            od_prev = od;
            __syncthreads();  // B
        };
        for (int it = 0; it < iters; it += 2) {
            step(it, t0, g0);
            if (it + 1 < iters) step(it + 1, t1, g1);
        }
        return;
    }

    // ---------------------------------------------------------- consumers
    const int l32 = lane & 31, g = lane >> 5;
    if (w == 0) {
        // -------------------------------------------------- state wave
        // S, O, y and the per-token sums of y^2 (left in LDS for wave 1),
        // and the state at sequence boundaries.  It touches no exchange
        // word: its only waits are for the initial states it loads.
        const int dv = SW * sl + l32;  // state column of this lane
        // accumulator register r of tile m holds state entry
        // dk = 32 m + 8 (r / 4) + 4 g + r % 4, dv
        f32x16 S[4] = {};
        Cursor cs;
        sq.seek(cs, 0);
        for (int it = 0; it < iters; ++it) {
            const int jc = it - 1;  // block computed in this iteration
            const bool comp = jc >= 0 && jc < nb;
            const int buf = (it - 1) & 1;
            const __bf16* sQ = L.q[buf];
            const __bf16* sK = L.k[buf];
            const __bf16* sV = L.v[buf];
            // ---- phase 1: S^T Q~^T
            f32x16 O[2] = {};
            if (comp) {
                if (cs.b == 0) {
                    // first block of a sequence: its initial state (or zeros)
                    const __amdgpu_buffer_rsrc_t ir = __builtin_amdgcn_make_buffer_rsrc(
                        (void*)(init_state ? init_state + ((int64_t)cs.s * H + h) * DD : nullptr),
                        (short)0, init_state ? (int)(DD * 4) : 0, 0x00020000);
                    const int ioff = (4 * g * MD + dv) * 4;
#pragma unroll
                    for (int m = 0; m < 4; ++m)
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            S[m][r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                                ir, ioff, (32 * m + 8 * (r >> 2) + (r & 3)) * MD * 4, 0));
                }
                // Q~ operands first, all in flight at once (an MFMA chain that
                // waits for each operand load in turn exposes the LDS latency
                // at every step)
                bf16x8 qo[MD / 16][2];
#pragma unroll
                for (int s = 0; s < MD / 16; ++s)
#pragma unroll
                    for (int tb = 0; tb < 2; ++tb)
                        qo[s][tb] = ld_row_operand(sQ, 32 * tb + l32, 16 * s + 8 * g);
                __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the products
                // S^T as bf16 A operands: one exchange between the lane halves
                // turns dk = 16 s + 8 (j / 4) + 4 g + j % 4 into dk = 16 s + 8 g + j
#pragma unroll
                for (int s = 0; s < MD / 16; ++s) {
                    const int m = s >> 1, r0 = 8 * (s & 1);
                    unsigned p0 = pack_bf16(S[m][r0 + 0], S[m][r0 + 1]);
                    unsigned p1 = pack_bf16(S[m][r0 + 2], S[m][r0 + 3]);
                    unsigned p2 = pack_bf16(S[m][r0 + 4], S[m][r0 + 5]);
                    unsigned p3 = pack_bf16(S[m][r0 + 6], S[m][r0 + 7]);
                    const auto x02 = __builtin_amdgcn_permlane32_swap(p0, p2, false, false);
                    const auto x13 = __builtin_amdgcn_permlane32_swap(p1, p3, false, false);
                    const bf16x8 a =
                        __builtin_bit_cast(bf16x8, u32x4{x02[0], x13[0], x02[1], x13[1]});
#pragma unroll
                    for (int tb = 0; tb < 2; ++tb) O[tb] = mfma32(a, qo[s][tb], O[tb]);
                }
            }
            __syncthreads();  // A
            // ---- phase 2: V~^T P^T, state update, y and its sums
            if (comp) {
                // all operands of the phase are loaded before the products
                bf16x8 vop[MB / 16];  // V~^T operands, shared by both products
                bf16x8 pb[MB / 16][2];  // P^T operands (tile tb = 0 needs s < 2 only)
                bf16x8 ko[MB / 16][4];  // K~^T operands
#pragma unroll
                for (int s = 0; s < MB / 16; ++s) {
                    vop[s] = ld_tr_operand(sV, 16 * s, SW * sl, lane);
#pragma unroll
                    for (int tb = 0; tb < 2; ++tb)
                        if (tb == 1 || s < 2)
                            pb[s][tb] = *reinterpret_cast<const bf16x8*>(
                                L.p + (32 * tb + l32) * LPP + 16 * s + 8 * g);
                }
#pragma unroll
                for (int s = 0; s < MB / 16; ++s)
#pragma unroll
                    for (int m = 0; m < 4; ++m) ko[s][m] = ld_tr_operand(sK, 16 * s, 32 * m, lane);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                    for (int s = 0; s < MB / 16; ++s)
                        if (tb == 1 || s < 2)  // t < 32 sees only t' < 32
                            O[tb] = mfma32(vop[s], pb[s][tb], O[tb]);
#pragma unroll
                for (int s = 0; s < MB / 16; ++s)
#pragma unroll
                    for (int m = 0; m < 4; ++m) S[m] = mfma32(ko[s][m], vop[s], S[m]);
                if (final_state != nullptr && last_block(cs)) {
                    const __amdgpu_buffer_rsrc_t fr = __builtin_amdgcn_make_buffer_rsrc(
                        final_state + ((int64_t)cs.s * H + h) * DD, (short)0, (int)(DD * 4),
                        0x00020000);
                    const int ioff = (4 * g * MD + dv) * 4;
#pragma unroll
                    for (int m = 0; m < 4; ++m)
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            __builtin_amdgcn_raw_buffer_store_b32(
                                __float_as_uint(S[m][r]), fr, ioff,
                                (32 * m + 8 * (r >> 2) + (r & 3)) * MD * 4, 0);
                }
                // y staged as bf16; sum of y^2 over the slice for token t =
                // lane (tile tb = lane / 32 holds tokens 32 tb + lane % 32)
                __bf16* ys = L.y[jc % LYR];
                float ss[2];
#pragma unroll
                for (int tb = 0; tb < 2; ++tb) {
                    float a = 0.f;
#pragma unroll
                    for (int r = 0; r < 16; ++r) a += O[tb][r] * O[tb][r];
                    ss[tb] = a + __shfl_xor(a, 32);
                    const int t = 32 * tb + l32;
#pragma unroll
                    for (int qd = 0; qd < 4; ++qd) {
                        bf16x4 y;
#pragma unroll
                        for (int u = 0; u < 4; ++u) y[u] = (__bf16)O[tb][4 * qd + u];
                        *reinterpret_cast<bf16x4*>(ys + t * LYP + 8 * qd + 4 * g) = y;
                    }
                }
                L.red[lane] = g ? ss[1] : ss[0];
            }
            __syncthreads();  // B
            if (comp) sq.next(cs);
        }
        return;
    }

    // ------------------------------------------------ waves 1-3
    // Score quadrant t' in [32 qa, +32), t in [32 qb, +32) (the quadrant
    // t' > t is never needed); wave 1 publishes the lane's sums; wave 2
    // sub-reduces; wave 3 forms totals and the norm factors.  Exchange loads
    // are issued one iteration before they are consumed, and before the
    // wave's own store of that iteration, so a wait for them never waits
    // for a store to reach memory.
    const int qa = w == 3 ? 1 : 0, qb = w >= 2 ? 1 : 0;
    const float inv_hd = 1.0f / (float)HD;
    const int grp = wg / XG, m0 = grp * XG, nm = min(XG, NL - m0);
    auto sub_reducer = [&](int j) { return j >= 0 && j < nb && wg == m0 + j % nm; };
    auto final_reducer = [&](int j) { return j >= 0 && j < nb && wg == j % NL; };
    auto valid = [&](int j) { return j >= 0 && j < nb; };
    auto load_words = [&](uint64_t* base, bool on, int n, uint64_t (&x)[XG]) {
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            (void*)base, (short)0, on ? n * MB * 8 : 0, 0x00020000);
#pragma unroll
        for (int i = 0; i < XG; ++i)
            x[i] = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(
                                                    r, (i * MB + lane) * 8, 0, SC1));
    };
    // words not yet written when first loaded are polled one by one
    auto complete = [&](uint64_t* base, int n, uint32_t tag, uint64_t (&x)[XG], int site, int j) {
        float a = 0.f;
#pragma unroll
        for (int i = 0; i < XG; ++i) {
            if (i < n) {
                int polls = 0;
                while (!has_tag(x[i], tag) && poll_again(polls, hdr, site, j, wg))
                    x[i] = get_word(base + i * MB + lane);
                a += word_value(x[i]);
            }
        }
        return a;
    };
    auto load_one = [&](uint64_t* base, bool on) {
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            (void*)base, (short)0, on ? MB * 8 : 0, 0x00020000);
        return __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(r, lane * 8, 0, SC1));
    };
    uint64_t xs[XG];  // wave 2: the group's words; wave 3: the group sums
    uint64_t xf = 0;  // wave 3: the total
    uint64_t held = 0;  // this wave's last stored exchange word, kept live
    for (int it = 0; it < iters; ++it) {
        const int jc = it - 1;
        const bool comp = jc >= 0 && jc < nb;
        const int buf = (it - 1) & 1;
        const __bf16* sQ = L.q[buf];
        const __bf16* sK = L.k[buf];
        // ---- phase 1: scores
        if (comp) {
            bf16x8 ka[MD / 16], qb8[MD / 16];  // operands loaded before the products
#pragma unroll
            for (int s = 0; s < MD / 16; ++s) {
                ka[s] = ld_row_operand(sK, 32 * qa + l32, 16 * s + 8 * g);
                qb8[s] = ld_row_operand(sQ, 32 * qb + l32, 16 * s + 8 * g);
            }
            __builtin_amdgcn_sched_barrier(0);
            f32x16 pacc = {};
#pragma unroll
            for (int s = 0; s < MD / 16; ++s) pacc = mfma32(ka[s], qb8[s], pacc);
            const int t = 32 * qb + l32;
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
                const int tp0 = 32 * qa + 8 * qd + 4 * g;
                bf16x4 o;
#pragma unroll
                for (int u = 0; u < 4; ++u) o[u] = (__bf16)(tp0 + u <= t ? pacc[4 * qd + u] : 0.f);
                *reinterpret_cast<bf16x4*>(L.p + t * LPP + tp0) = o;
            }
        }
        __syncthreads();  // A
        keep(held);
        // ---- phase 2: exchange
        if (w == 2) {
            // sub-reduction of block j1 (its words were loaded last iteration)
            const int j1 = jc - LAG1;
            uint64_t* src = part + ((int64_t)(j1 & (XR - 1)) * NL + m0) * MB;
            float a = 0.f;
            const bool on = sub_reducer(j1);
            if (on) a = complete(src, nm, (uint32_t)j1 + 1, xs, 1, j1);
            const int jn = j1 + 1;
            load_words(part + ((int64_t)(jn & (XR - 1)) * NL + m0) * MB, sub_reducer(jn), nm, xs);
            if (on)
                held = put_tagged(rsub + ((int64_t)(j1 & (XR - 1)) * NG + grp) * MB + lane, a,
                                  (uint32_t)j1 + 1);
        } else if (w == 3) {
            // total of block j2, then the norm factors of block jx
            const int j2 = jc - LAG1 - LAG2, jx = j2 - LAG3;
            uint64_t* src = rsub + (int64_t)(j2 & (XR - 1)) * NG * MB;
            float a = 0.f;
            const bool on = final_reducer(j2);
            if (on) a = complete(src, NG, (uint32_t)j2 + 1, xs, 2, j2);
            if (valid(jx)) {
                uint64_t* fs = tot + (jx & (XR - 1)) * MB + lane;
                int polls = 0;
                while (!has_tag(xf, (uint32_t)jx + 1) && poll_again(polls, hdr, 4, jx, wg))
                    xf = get_word(fs);
                L.rn[jx & 1][lane] = __builtin_amdgcn_rsqf(word_value(xf) * inv_hd + eps);
            }
            const int j2n = j2 + 1, jxn = jx + 1;
            load_words(rsub + (int64_t)(j2n & (XR - 1)) * NG * MB, final_reducer(j2n), NG, xs);
            xf = load_one(tot + (jxn & (XR - 1)) * MB, valid(jxn));
            if (on) held = put_tagged(tot + (j2 & (XR - 1)) * MB + lane, a, (uint32_t)j2 + 1);
        }
        __syncthreads();  // B
        // ---- after phase 2 (wave 1): publish block jc's sums
        if (w == 1 && comp)
            held = put_tagged(part + ((int64_t)(jc & (XR - 1)) * NL + wg) * MB + lane, L.red[lane],
                              (uint32_t)jc + 1);
    }
}

}  // namespace

int lane_max_lanes() { return XG * XGMAX; }

int lane_ring_slots() { return XR; }
int lane_group_size() { return XG; }
int lane_slices() { return NSL; }

hipError_t launch_prefill_lane(const PrefillArgs& a, hipStream_t st) {
    const dim3 grid((unsigned)(a.H * NSL));
    hipLaunchKernelGGL(prefill_lane_kernel, grid, dim3(LT), 0, st, (const __bf16*)a.q,
                       (const __bf16*)a.k, (const __bf16*)a.v, (const __bf16*)a.g,
                       (const __bf16*)a.w, (__bf16*)a.out, a.hdr, a.cu, a.nseq, a.seqlen,
                       a.init_state, a.final_state, a.part, a.rsub, a.tot, a.H, a.eps);
    return hipGetLastError();
}

}  // namespace la
