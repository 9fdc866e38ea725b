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
//   y   = causal(SiLU q, SiLU k, SiLU v; S_entry)      -> fp32
//   dq  = causal(dy, SiLU v, SiLU k; S_entry^T)        * SiLU'(q)
//   dk  = anti-causal(SiLU v, dy, SiLU q; G_exit^T)    * SiLU'(k)
//   dv  = anti-causal(SiLU k, SiLU q, dy; G_exit)      * SiLU'(v)
// S_entry and G_exit come from chunk sums on MFMA (state_mfma.hip) and the
// forward and reverse scans.
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

template <bool ON>
__device__ __forceinline__ bf16x8 act(bf16x8 x) {
    if constexpr (ON) return silu8(x);
    else return x;
}

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

// One walk per (chunk, head).  SX, SK, SV: SiLU on X, K, V; REV: anti-causal;
// TRS: the state is read transposed; EPI = 0: Y to yout (fp32), 1: gout =
// Y * SiLU'(raw) (bf16), 2: gout = Y (bf16).  Waves 4-7 stage the tiles (two blocks ahead, two
// LDS buffers), waves 0-3 hold 32 columns of R each and compute, as in the
// forward walk; the consumers store their outputs straight from the
// accumulators.
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
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int HD = H * MD;
    const int64_t DD = (int64_t)MD * MD;
    const int64_t off0 = ce.start * (int64_t)HD + (int64_t)h * MD;
    const int nblk = (ce.len + MB - 1) / MB;
    const int iters = nblk + 1;
    // the i-th block visited, and its rows (0 outside the chunk)
    auto blk_of = [&](int i) { return REV ? nblk - 1 - i : i; };
    auto rows = [&](int blk) { return (blk < 0 || blk >= nblk) ? 0 : min(MB, ce.len - blk * MB); };

    if (w >= 4) {
        // ------------------------------------------------------ producers
        const int ptid = tid - 256;
        const int cc = ptid & 15, rg = ptid >> 4;
        const int voff = (4 * rg * HD + 8 * cc) * 2, rstride = HD * 2;
        // loads are issued unconditionally (blocks outside the chunk get an
        // empty range and return zeros)
        auto load = [&](const __bf16* base, int i, Tile& t) {
            const int blk = blk_of(i);
            load_tile(t, tile_rsrc(base + off0 + (int64_t)max(blk, 0) * MB * HD, rows(blk), HD),
                      voff, rstride);
        };
        Tile x0, k0, v0, x1, k1, v1;
        load(X, 0, x0);
        load(K, 0, k0);
        load(V, 0, v0);
        load(X, 1, x1);
        load(K, 1, k1);
        load(V, 1, v1);
        auto step = [&](int it, Tile& tx, Tile& tk, Tile& tv) {
            const int buf = it & 1;
            if (it < nblk) {
                bf16x8 xs[4], ks[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    xs[r] = act<SX>(tx.r[r]);
                    ks[r] = act<SK>(tk.r[r]);
                }
                store_rows(xs, L.x[buf], cc, rg);
                store_rows(ks, L.k[buf], cc, rg);
            }
            load(X, it + 2, tx);
            load(K, it + 2, tk);
            __syncthreads();  // A
            if (it < nblk) {
                bf16x8 vs[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) vs[r] = act<SV>(tv.r[r]);
                store_rows(vs, L.v[buf], cc, rg);
            }
            load(V, it + 2, tv);
            __syncthreads();  // B
        };
        for (int it = 0; it < iters; it += 2) {
            step(it, x0, k0, v0);
            if (it + 1 < iters) step(it + 1, x1, k1, v1);
        }
        return;
    }

    // ---------------------------------------------------------- consumers
    const int l32 = lane & 31, g = lane >> 5;
    // accumulator register r of tile m holds R[dk][dv], dk = 32 m + 8 (r / 4)
    // + 4 g + r % 4, dv = 32 w + l32
    const int dv = 32 * w + l32;
    f32x16 S[4] = {};
    // score quadrant t' in [32 qa, +32), t in [32 qb, +32); the one outside
    // the window (t' > t causal, t' < t anti-causal) is never formed
    const int qa = w >> 1, qb = w & 1;
    const bool scores = REV ? !(qa == 0 && qb == 1) : !(qa == 1 && qb == 0);
    // stored outputs, kept live until the next barrier
    u32x4 od[2][4];      // fp32 (EPI 0)
    u32x2 ob[2][4];      // bf16 (EPI 1)
    for (int it = 0; it < iters; ++it) {
        const int jc = it - 1;  // visit index of the block computed in this iteration
        const bool comp = jc >= 0 && jc < nblk;
        const int buf = (it - 1) & 1;
        const __bf16* sX = L.x[buf];
        const __bf16* sK = L.k[buf];
        const __bf16* sV = L.v[buf];
        // ---- phase 1: R^T X^T into O, and the scores
        f32x16 O[2] = {};
        if (comp) {
            bf16x8 xo[MD / 32][2];
#pragma unroll
            for (int s = 0; s < MD / 16; ++s) {
                if (s % (MD / 32) == 0) {
#pragma unroll
                    for (int i = 0; i < MD / 32; ++i)
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
                for (int tb = 0; tb < 2; ++tb) O[tb] = mfma32(a, xo[s % (MD / 32)][tb], O[tb]);
            }
            if (scores) {
                bf16x8 kr[MD / 16], xr[MD / 16];
#pragma unroll
                for (int s = 0; s < MD / 16; ++s) {
                    kr[s] = ld_row_operand(sK, 32 * qa + l32, 16 * s + 8 * g);
                    xr[s] = ld_row_operand(sX, 32 * qb + l32, 16 * s + 8 * g);
                }
                __builtin_amdgcn_sched_barrier(0);
                f32x16 pacc = {};
#pragma unroll
                for (int s = 0; s < MD / 16; ++s) pacc = mfma32(kr[s], xr[s], pacc);
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
                    *reinterpret_cast<bf16x4*>(L.p + t * BPP + tp0) = o;
                }
            }
        }
        __syncthreads();  // A
        // ---- phase 2, iteration 0: the state entering the chunk
        if (it == 0) {
            const __amdgpu_buffer_rsrc_t er = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(entry + ((int64_t)c * H + h) * DD), (short)0, (int)(DD * 4), 0x00020000);
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
            const int blk = blk_of(jc), n = rows(blk);
            const int64_t tbase = off0 + (int64_t)blk * MB * HD;
            // output positions: token t = 32 tb + l32, dims 32 w + 8 q + 4 g .. + 3
            const int ooff = l32 * HD + 32 * w + 4 * g;
            bf16x4 rw[2][4];
            if (EPI == 1) {
                // the raw inputs of the SiLU' factor, loaded ahead of the products
                // (EPI 2 stores Y in bf16 with no factor)
                const __amdgpu_buffer_rsrc_t rr = tile_rsrc(raw + tbase, n, HD);
#pragma unroll
                for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        rw[tb][q] = __builtin_bit_cast(
                            bf16x4, __builtin_amdgcn_raw_buffer_load_b64(
                                        rr, (ooff + 32 * tb * HD + 8 * q) * 2, 0, 0));
            }
            bf16x8 vop[MB / 16];
            bf16x8 pb[MB / 16][2];
            bf16x8 ko[2][4];
#pragma unroll
            for (int s = 0; s < MB / 16; ++s) {
                vop[s] = ld_tr_operand(sV, 16 * s, 32 * w, lane);
#pragma unroll
                for (int tb = 0; tb < 2; ++tb)
                    if (REV ? (tb == 0 || s >= 2) : (tb == 1 || s < 2))
                        pb[s][tb] = *reinterpret_cast<const bf16x8*>(L.p + (32 * tb + l32) * BPP +
                                                                     16 * s + 8 * g);
            }
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int m = 0; m < 4; ++m) ko[s][m] = ld_tr_operand(sK, 16 * s, 32 * m, lane);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                for (int s = 0; s < MB / 16; ++s)
                    if (REV ? (tb == 0 || s >= 2) : (tb == 1 || s < 2))
                        O[tb] = mfma32(vop[s], pb[s][tb], O[tb]);
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int m = 0; m < 4; ++m) S[m] = mfma32(ko[s][m], vop[s], S[m]);
#pragma unroll
            for (int s = 2; s < MB / 16; ++s)
#pragma unroll
                for (int m = 0; m < 4; ++m) ko[s - 2][m] = ld_tr_operand(sK, 16 * s, 32 * m, lane);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 2; s < MB / 16; ++s)
#pragma unroll
                for (int m = 0; m < 4; ++m) S[m] = mfma32(ko[s - 2][m], vop[s], S[m]);
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
    if (e == hipSuccess)
        e = walk<true, false, true, true, true, 1>(a, a.p.v, a.dy, a.p.q, a.gstates, nullptr,
                                                   a.p.k, a.dk);
    if (e == hipSuccess)
        e = walk<true, true, false, true, false, 1>(a, a.p.k, a.p.q, a.dy, a.gstates, nullptr,
                                                    a.p.v, a.dv);
    return e;
}

}  // namespace la
