// Backward pass of the Lightning Attention layer on bf16 MFMA for gfx950
// (head_dim 128, 64-token blocks, fp32 accumulation and running state).
//
// The gradients are the ones backward.hip states (chain rule through
// Mechanism steps 4, 3, 2 of "Diving into MiniMax01 405B MoE", section
// "Hybrid Modeling", in reverse).  y, dq~, dk~ and dv~ are each one
// linear-attention walk over the chunks,
//   Y_t = X_t R + sum_{u in window(t), same chunk} (X_t . K_u) V_u,
// run here by bwd_walk_mfma_kernel with the products of the forward walk
// (mfma.hip): per 64-token block, with R the D x D fp32 state before the block,
//   P^T = K_b X_b^T (masked),  O^T = R^T X_b^T + V_b^T P^T,  R += K_b^T V_b.
// Causal walks take u <= t and the blocks first to last; anti-causal walks
// u >= t and the blocks last to first.  Each operand is read from the
// activations with SiLU applied on the way into LDS, or as it is (dy), so
// q~, k~, v~ are never written out.  The walks are independent per (chunk,
// head): no cross-workgroup wait.
//   y   = causal(SiLU q, SiLU k, SiLU v; S_entry)      -> bf16
//   dq  = causal(dy, SiLU v, SiLU k; S_entry^T)        * SiLU'(q)
//   dk  = anti-causal(SiLU v, dy, SiLU q; G_exit^T)    * SiLU'(k)
//   dv  = anti-causal(SiLU k, SiLU q, dy; G_exit)      * SiLU'(v)
// S_entry and G_exit come from chunk sums on MFMA (state_mfma.hip) and the
// forward and reverse scans.  y and dq run as separate walks; dk and dv run
// together in bwd_dkdv_mfma_kernel, which stages the four operands once for
// both.  (y cannot share a walk with dq: dy needs the RMSNorm of y over all
// heads first, which the forward walk finishes only several blocks later.)
#include "mfma_common.h"

namespace la {

namespace {

constexpr int BW_THREADS = 512;  // 4 consumer + 4 producer waves
constexpr int BPP = MB + 8;      // pitch of the score tile

struct BwdLds {
    __bf16 x[2][TILE];  // X (the walk's queries)
    __bf16 k[2][TILE];  // K
    __bf16 v[2][TILE];  // V
    __bf16 p[MB * BPP]; // masked scores P^T [t][t']
};

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void keep2(u32x2 x) { asm volatile("" ::"v"(x)); }

__device__ __forceinline__ float silu_grad_f(float x) {
    const float s = sigmoid_f(x);
    return s * (1.0f + x * (1.0f - s));
}

// Buffer resource over the fp32 rows 0 .. n-1 of one head (rows HD floats
// apart); stores past the last row are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t f32_rsrc(const float* base, int n, int HD) {
    const int bytes = __builtin_amdgcn_readfirstlane(n > 0 ? ((n - 1) * HD + MD) * 4 : 0);
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, bytes, 0x00020000);
}

// Geometry of one walk: the chunk's rows of one head, visited first to last
// (causal) or last to first (anti-causal, REV).
template <bool REV>
struct WalkGeom {
    int64_t off0;  // element offset of the chunk's first token in this head
    int len, nblk, HD;
    // the i-th block visited, and its rows (0 outside the chunk)
    __device__ int blk_of(int i) const { return REV ? nblk - 1 - i : i; }
    __device__ int rows(int blk) const {
        return (blk < 0 || blk >= nblk) ? 0 : min(MB, len - blk * MB);
    }
};

// Producer waves (thread ptid in 0 .. 255): stage NT tiles of each block,
// SiLU applied to tile j when bit j of ACT is set, into LDS buffer
// (iteration % 2) at dst[j] + buffer * TILE, two blocks ahead in registers.
// The first NA tiles are written before the iteration's first barrier, the
// rest before its second; every tile of block `it` is in place at the end of
// iteration it, and the consumers read it in iteration it + 1.  Loads are
// issued unconditionally (blocks outside the chunk get an empty range and
// return zeros).
template <bool REV, int NT, int NA, unsigned ACT>
__device__ __forceinline__ void walk_producer(const WalkGeom<REV>& G, const __bf16* const (&src)[NT],
                                              __bf16* const (&dst)[NT], int ptid) {
    const int cc = ptid & 15, rg = ptid >> 4;
    const int voff = (4 * rg * G.HD + 8 * cc) * 2, rstride = G.HD * 2;
    auto load = [&](int i, int j, Tile& t) {
        const int blk = G.blk_of(i);
        load_tile(t, tile_rsrc(src[j] + G.off0 + (int64_t)max(blk, 0) * MB * G.HD, G.rows(blk), G.HD),
                  voff, rstride);
    };
    Tile t0[NT], t1[NT];
    auto put = [&](int it, int j, Tile& t) {
        if (it >= 0 && it < G.nblk) {
            bf16x8 xs[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) xs[r] = ((ACT >> j) & 1) ? silu8(t.r[r]) : t.r[r];
            store_rows(xs, dst[j] + (it & 1) * TILE, cc, rg);
        }
    };
    // Steps -2 and -1 only issue the loads of blocks 0 and 1: with every load
    // issued inside the loop, no load is pending when it is entered (one that
    // is makes the compiler wait for all loads at the top of every pass).
    auto step = [&](int it, Tile (&t)[NT]) {
#pragma unroll
        for (int j = 0; j < NA; ++j) put(it, j, t[j]);
#pragma unroll
        for (int j = 0; j < NA; ++j) load(it + 2, j, t[j]);
        if (it >= 0) __syncthreads();  // A
#pragma unroll
        for (int j = NA; j < NT; ++j) put(it, j, t[j]);
#pragma unroll
        for (int j = NA; j < NT; ++j) load(it + 2, j, t[j]);
        if (it >= 0) __syncthreads();  // B
    };
    const int iters = G.nblk + 1;
    for (int it = -2; it < iters; it += 2) {
        step(it, t0);
        if (it + 1 < iters) step(it + 1, t1);
    }
}

// Consumer waves (wave w in 0 .. 3 of the group): wave w holds columns
// [32 w, +32) of R and of the outputs, as in the forward walk, and stores its
// outputs straight from the accumulators.  The tiles of buffer b sit at
// sX + b * TILE (and likewise sK, sV); sP is this walk's score tile.  entry
// is the (chunk, head)'s D x D state, read transposed when TRS.  EPI = 0: Y
// to yout (fp32), 1: gout = Y * SiLU'(raw) (bf16), 2: gout = Y (bf16).
// LEAN fits the wave in 168 registers (three waves per SIMD): the operands
// of R^T X^T, of the scores and of the state update are read in halves and
// quarters, and the lane's LDS addresses are formed anew in every iteration
// instead of being held in registers for the whole walk.
template <bool REV, bool TRS, int EPI, bool LEAN>
__device__ __forceinline__ void walk_consumer(const WalkGeom<REV>& G, const __bf16* sX0,
                                              const __bf16* sK0, const __bf16* sV0, __bf16* sP,
                                              int w, int lane0, const float* entry, float* yout,
                                              const __bf16* raw, __bf16* gout) {
    const int64_t DD = (int64_t)MD * MD;
    const int HD = G.HD;
    const int iters = G.nblk + 1;
    // accumulator register r of tile m holds R[dk][dv], dk = 32 m + 8 (r / 4)
    // + 4 g + r % 4, dv = 32 w + l32
    f32x16 S[4] = {};
    // score quadrant t' in [32 qa, +32), t in [32 qb, +32); the one outside
    // the window (t' > t causal, t' < t anti-causal) is never formed
    const int qa = w >> 1, qb = w & 1;
    const bool scores = REV ? !(qa == 0 && qb == 1) : !(qa == 1 && qb == 0);
    // stored outputs, kept live until the next barrier
    u32x4 od[2][4];      // fp32 (EPI 0)
    u32x2 ob[2][4];      // bf16 (EPI 1, 2)
    for (int it = 0; it < iters; ++it) {
        int lane = lane0;
        if (LEAN) {
            lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
            asm volatile("" : "+v"(lane));
        }
        const int l32 = lane & 31, g = lane >> 5;
        const int dv = 32 * w + l32;
        const int jc = it - 1;  // visit index of the block computed in this iteration
        const bool comp = jc >= 0 && jc < G.nblk;
        const int buf = (it - 1) & 1;
        const __bf16* sX = sX0 + buf * TILE;
        const __bf16* sK = sK0 + buf * TILE;
        const __bf16* sV = sV0 + buf * TILE;
        f32x16 O[2];
        // R^T X^T into O (R as it stands before this block's update)
        auto state_term = [&]() {
            O[0] = f32x16{};
            O[1] = f32x16{};
            constexpr int XS = LEAN ? 2 : MD / 32;  // X operands read at once
            bf16x8 xo[XS][2];
#pragma unroll
            for (int s = 0; s < MD / 16; ++s) {
                if (s % XS == 0) {
#pragma unroll
                    for (int i = 0; i < XS; ++i)
#pragma unroll
                        for (int tb = 0; tb < 2; ++tb)
                            xo[i][tb] = ld_row_operand(sX, 32 * tb + l32, 16 * (s + i) + 8 * g);
                    __builtin_amdgcn_sched_barrier(0);
                }
                // R^T as bf16 A operands (one exchange between the lane halves
                // matches the k order of the X row read)
                const int m = s >> 1, r0 = 8 * (s & 1);
                unsigned p0 = pack_bf16(S[m][r0 + 0], S[m][r0 + 1]);
                unsigned p1 = pack_bf16(S[m][r0 + 2], S[m][r0 + 3]);
                unsigned p2 = pack_bf16(S[m][r0 + 4], S[m][r0 + 5]);
                unsigned p3 = pack_bf16(S[m][r0 + 6], S[m][r0 + 7]);
                const auto x02 = __builtin_amdgcn_permlane32_swap(p0, p2, false, false);
                const auto x13 = __builtin_amdgcn_permlane32_swap(p1, p3, false, false);
                const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{x02[0], x13[0], x02[1], x13[1]});
#pragma unroll
                for (int tb = 0; tb < 2; ++tb) O[tb] = mfma32(a, xo[s % XS][tb], O[tb]);
            }
        };
        const int blk = G.blk_of(jc), n = G.rows(blk);
        const int64_t tbase = G.off0 + (int64_t)max(blk, 0) * MB * HD;
        // output positions: token t = 32 tb + l32, dims 32 w + 8 q + 4 g .. + 3
        const int ooff = l32 * HD + 32 * w + 4 * g;
        // the raw inputs of the SiLU' factor: loaded at the start of the
        // iteration, so that both phases cover their latency (LEAN: after the
        // products with the scores, where fewer registers are in use)
        bf16x4 rw[2][4];
        auto load_raw = [&]() {
            const __amdgpu_buffer_rsrc_t rr = tile_rsrc(raw + tbase, n, HD);
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    rw[tb][q] = __builtin_bit_cast(
                        bf16x4, __builtin_amdgcn_raw_buffer_load_b64(
                                    rr, (ooff + 32 * tb * HD + 8 * q) * 2, 0, 0));
        };
        // ---- phase 1: R^T X^T and the scores
        if (comp) {
            if (EPI == 1 && !LEAN) load_raw();
            state_term();
            if (scores) {
                constexpr int SH = LEAN ? MD / 32 : MD / 16;  // operands read at once
                f32x16 pacc = {};
#pragma unroll
                for (int s0 = 0; s0 < MD / 16; s0 += SH) {
                    bf16x8 kr[SH], xr[SH];
#pragma unroll
                    for (int s = 0; s < SH; ++s) {
                        kr[s] = ld_row_operand(sK, 32 * qa + l32, 16 * (s0 + s) + 8 * g);
                        xr[s] = ld_row_operand(sX, 32 * qb + l32, 16 * (s0 + s) + 8 * g);
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int s = 0; s < SH; ++s) pacc = mfma32(kr[s], xr[s], pacc);
                }
                const int t = 32 * qb + l32;
#pragma unroll
                for (int qd = 0; qd < 4; ++qd) {
                    const int tp0 = 32 * qa + 8 * qd + 4 * g;
                    bf16x4 o;
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const bool in = REV ? tp0 + u >= t : tp0 + u <= t;
                        o[u] = (__bf16)(in ? pacc[4 * qd + u] : 0.f);
                    }
                    *reinterpret_cast<bf16x4*>(sP + t * BPP + tp0) = o;
                }
            }
        }
        __syncthreads();  // A
        // ---- phase 2, iteration 0: the state entering the chunk
        if (it == 0) {
            const __amdgpu_buffer_rsrc_t er =
                __builtin_amdgcn_make_buffer_rsrc((void*)entry, (short)0, (int)(DD * 4), 0x00020000);
            const int ioff = TRS ? (dv * MD + 4 * g) * 4 : (4 * g * MD + dv) * 4;
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int e = 32 * m + 8 * (r >> 2) + (r & 3);
                    S[m][r] = __uint_as_float(
                        __builtin_amdgcn_raw_buffer_load_b32(er, ioff, TRS ? e * 4 : e * MD * 4, 0));
                }
        }
        // ---- phase 2: V^T P^T into O, the state update, the outputs
        if (comp) {
            bf16x8 vop[MB / 16];
            bf16x8 pb[MB / 16][2];
            // P^T operand of token slice s for output tile tb (the slice that
            // lies outside the window is never read)
            auto used = [](int s, int tb) { return REV ? (tb == 0 || s >= 2) : (tb == 1 || s < 2); };
            auto load_p = [&](int s, int tb) {
                pb[s][tb] = *reinterpret_cast<const bf16x8*>(sP + (32 * tb + l32) * BPP + 16 * s + 8 * g);
            };
            // K operands of the state update, KS token slices of 16 at a time
            // (LEAN: read after the products with the scores)
            constexpr int KS = LEAN ? 1 : 2;
            bf16x8 ko[KS][4];
#pragma unroll
            for (int s = 0; s < MB / 16; ++s) {
                vop[s] = ld_tr_operand(sV, 16 * s, 32 * w, lane);
#pragma unroll
                for (int tb = 0; tb < 2; ++tb)
                    if (used(s, tb)) load_p(s, tb);
            }
            if (!LEAN) {
#pragma unroll
                for (int s = 0; s < KS; ++s)
#pragma unroll
                    for (int m = 0; m < 4; ++m) ko[s][m] = ld_tr_operand(sK, 16 * s, 32 * m, lane);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                for (int s = 0; s < MB / 16; ++s)
                    if (used(s, tb)) O[tb] = mfma32(vop[s], pb[s][tb], O[tb]);
            if (EPI == 1 && LEAN) load_raw();
#pragma unroll
            for (int s0 = 0; s0 < MB / 16; s0 += KS) {
                if (LEAN || s0 > 0) {
#pragma unroll
                    for (int s = 0; s < KS; ++s)
#pragma unroll
                        for (int m = 0; m < 4; ++m)
                            ko[s][m] = ld_tr_operand(sK, 16 * (s0 + s), 32 * m, lane);
                    __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int s = 0; s < KS; ++s)
#pragma unroll
                    for (int m = 0; m < 4; ++m) S[m] = mfma32(ko[s][m], vop[s0 + s], S[m]);
            }
            // outputs (rows past the block's end are dropped by the range)
            if (EPI == 0) {
                const __amdgpu_buffer_rsrc_t ro = f32_rsrc(yout + tbase, n, HD);
#pragma unroll
                for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        od[tb][q] = u32x4{__float_as_uint(O[tb][4 * q]), __float_as_uint(O[tb][4 * q + 1]),
                                          __float_as_uint(O[tb][4 * q + 2]),
                                          __float_as_uint(O[tb][4 * q + 3])};
                        __builtin_amdgcn_raw_buffer_store_b128(od[tb][q], ro,
                                                               (ooff + 32 * tb * HD + 8 * q) * 4, 0, 0);
                    }
            } else {
                const __amdgpu_buffer_rsrc_t ro = tile_rsrc(gout + tbase, n, HD);
#pragma unroll
                for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        bf16x4 o;
#pragma unroll
                        for (int u = 0; u < 4; ++u)
                            o[u] = (__bf16)(EPI == 1 ? O[tb][4 * q + u] * silu_grad_f((float)rw[tb][q][u])
                                                     : O[tb][4 * q + u]);
                        ob[tb][q] = __builtin_bit_cast(u32x2, o);
                        __builtin_amdgcn_raw_buffer_store_b64(ob[tb][q], ro,
                                                              (ooff + 32 * tb * HD + 8 * q) * 2, 0, 0);
                    }
            }
        }
        __syncthreads();  // B
        if (comp) {
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (EPI == 0) keep(od[tb][q]);
                    else keep2(ob[tb][q]);
                }
        }
    }
}

// One walk per (chunk, head).  SX, SK, SV: SiLU on X, K, V; REV: anti-causal;
// TRS: the state is read transposed; EPI as for walk_consumer.  Waves 4-7
// stage X and K, then V (two blocks ahead, two LDS buffers); waves 0-3
// compute.
template <bool SX, bool SK, bool SV, bool REV, bool TRS, int EPI>
__global__ __launch_bounds__(BW_THREADS) void bwd_walk_mfma_kernel(
    const __bf16* __restrict__ X, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const PlanHeader* __restrict__ hdr, const ChunkEntry* __restrict__ chunks,
    const float* __restrict__ entry, float* __restrict__ yout, const __bf16* __restrict__ raw,
    __bf16* __restrict__ gout, int H) {
    __shared__ __attribute__((aligned(16))) BwdLds L;
    const int c = blockIdx.x / H, h = blockIdx.x - (blockIdx.x / H) * H;
    if (c >= hdr->n_chunks) return;
    const ChunkEntry ce = chunks[c];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int HD = H * MD;
    const WalkGeom<REV> G{ce.start * (int64_t)HD + (int64_t)h * MD, ce.len, (ce.len + MB - 1) / MB, HD};
    if (w >= 4) {
        const __bf16* const src[3] = {X, K, V};
        __bf16* const dst[3] = {L.x[0], L.k[0], L.v[0]};
        walk_producer<REV, 3, 2, (SX ? 1u : 0u) | (SK ? 2u : 0u) | (SV ? 4u : 0u)>(G, src, dst,
                                                                                  tid - 256);
        return;
    }
    walk_consumer<REV, TRS, EPI, false>(G, L.x[0], L.k[0], L.v[0], L.p, w, lane,
                                 entry + ((int64_t)c * H + h) * MD * MD, yout, raw, gout);
}

// dk~ and dv~ in one workgroup per (chunk, head): both are anti-causal walks
// from G_exit over the same four operands (q~, k~, v~ and dy), so one set of
// producer waves stages each of them once per block for both.
//   waves 0-3:   dv walk, X = k~, K = q~, V = dy, state G_exit
//   waves 4-7:   dk walk, X = v~, K = dy, V = q~, state G_exit^T
//   waves 8-11:  stage k~, q~ (SiLU applied on the way in), then v~ (SiLU)
//                and dy
struct DkdvLds {
    __bf16 q[2][TILE];
    __bf16 k[2][TILE];
    __bf16 v[2][TILE];
    __bf16 d[2][TILE];
    __bf16 p[2][MB * BPP];  // each walk's masked scores
};
constexpr int DKDV_THREADS = 768;

__global__ __launch_bounds__(DKDV_THREADS) void bwd_dkdv_mfma_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ dy, const PlanHeader* __restrict__ hdr,
    const ChunkEntry* __restrict__ chunks, const float* __restrict__ gstates,
    __bf16* __restrict__ dk, __bf16* __restrict__ dv, int H) {
    __shared__ __attribute__((aligned(16))) DkdvLds L;
    const int c = blockIdx.x / H, h = blockIdx.x - (blockIdx.x / H) * H;
    if (c >= hdr->n_chunks) return;
    const ChunkEntry ce = chunks[c];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int HD = H * MD;
    const WalkGeom<true> G{ce.start * (int64_t)HD + (int64_t)h * MD, ce.len, (ce.len + MB - 1) / MB, HD};
    const float* entry = gstates + ((int64_t)c * H + h) * MD * MD;
    if (w >= 8) {
        // The producer shares its SIMD with a dk~ and a dv~ consumer; issuing
        // its loads and SiLU ahead of theirs keeps the tiles coming (8192 x 64
        // heads: backward 796 -> 777 us, identical gradients).
        __builtin_amdgcn_s_setprio(1);
        const __bf16* const src[4] = {k, q, v, dy};
        __bf16* const dst[4] = {L.k[0], L.q[0], L.v[0], L.d[0]};
        walk_producer<true, 4, 2, 7u>(G, src, dst, tid - 512);
    } else if (w >= 4) {
        walk_consumer<true, true, 1, true>(G, L.v[0], L.d[0], L.q[0], L.p[1], w - 4, lane, entry, nullptr,
                                     k, dk);
    } else {
        walk_consumer<true, false, 1, true>(G, L.k[0], L.q[0], L.d[0], L.p[0], w, lane, entry, nullptr,
                                      v, dv);
    }
}

template <bool SX, bool SK, bool SV, bool REV, bool TRS, int EPI>
hipError_t walk(const BackwardArgs& a, const void* x, const void* k, const void* v,
                const float* entry, float* yout, const void* raw, void* gout) {
    const dim3 grid((unsigned)((int64_t)a.p.max_chunks * a.p.H));
    hipLaunchKernelGGL((bwd_walk_mfma_kernel<SX, SK, SV, REV, TRS, EPI>), grid, dim3(BW_THREADS), 0,
                       a.stream, (const __bf16*)x, (const __bf16*)k, (const __bf16*)v, a.p.hdr,
                       a.p.chunks, entry, yout, (const __bf16*)raw, (__bf16*)gout, a.p.H);
    return hipGetLastError();
}

}  // namespace

bool backward_mfma_supported(const PrefillArgs& a) { return a.bf16 && a.D == MD; }

hipError_t launch_backward_walk_y(const BackwardArgs& a) {
    // Y in bf16 (the forward rounds it to bf16 before its norm as well)
    return walk<true, true, true, false, false, 2>(a, a.p.q, a.p.k, a.p.v, a.p.states, nullptr,
                                                   nullptr, a.y);
}

hipError_t launch_backward_walks_grad(const BackwardArgs& a) {
    hipError_t e = walk<false, true, true, false, true, 1>(a, a.dy, a.p.v, a.p.k, a.p.states,
                                                          nullptr, a.p.q, a.dq);
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)((int64_t)a.p.max_chunks * a.p.H));
    hipLaunchKernelGGL(bwd_dkdv_mfma_kernel, grid, dim3(DKDV_THREADS), 0, a.stream,
                       (const __bf16*)a.p.q, (const __bf16*)a.p.k, (const __bf16*)a.p.v,
                       (const __bf16*)a.dy, a.p.hdr, a.p.chunks, a.gstates, (__bf16*)a.dk,
                       (__bf16*)a.dv, a.p.H);
    return hipGetLastError();
}

}  // namespace la
