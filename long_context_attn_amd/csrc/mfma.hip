// bf16 MFMA kernels of the Lightning Attention layer for gfx950
// (head_dim 128, block 64 tokens, fp32 accumulation).
//
// Mechanism step 3 of "Diving into MiniMax01 405B MoE" (section "Hybrid
// Modeling"), Y = Q (K^T V) read causally, is computed per block b of 64
// tokens of a chunk, with S the fp32 state entering the block:
//   P^T  = K~_b Q~_b^T, masked to t' <= t          (intra-block scores)
//   O^T  = V~_b^T P^T + S^T Q~_b^T                  (intra + inter, transposed)
//   S   += K~_b^T V~_b                              (state update)
// Every product is a v_mfma_f32_32x32x16_bf16 (A: 32x16, B: 16x32, C: 32x32
// fp32).  Lane layouts (checked on the hardware): A row = lane % 32 with k =
// 8 (lane / 32) + j; B column = lane % 32, same k; C column = lane % 32, row =
// 8 (r / 4) + 4 (lane / 32) + r % 4 for accumulator r.
//
// A workgroup of 4 waves owns one (chunk, head).  Wave w keeps state columns
// dv in [32w, 32w+32) for all 128 key rows in four C tiles (64 fp32 registers
// per lane), so the state never leaves registers during the walk and the
// inter-block product reads it straight from the accumulators: transposed,
// S^T is an A operand whose rows are the lane's own column dv, and the k
// permutation of the C layout is matched in the Q~ operand.
//
// The block's q/k/v tiles (64 x 128 bf16) are loaded with 16-byte accesses
// (16 lanes per 256-byte token row), the loads of block b+1 are issued before
// block b is computed, SiLU is applied in fp32 and the results are stored to
// LDS as bf16 in the layouts the MFMA operands read: Q~ and K~ token-major,
// K~^T and V~^T feature-major.
#include "la_internal.h"

namespace la {

constexpr int MD = 128;        // head_dim
constexpr int MB = 64;         // block tokens
constexpr int MTHREADS = 256;  // 4 waves
constexpr int QP = MD + 8;     // pitch (elements) of token-major tiles
constexpr int TP = MB + 8;     // pitch (elements) of feature-major tiles

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 silu8(bf16x8 x) {
    bf16x8 o;
#pragma unroll
    for (int u = 0; u < 8; ++u) o[u] = (__bf16)silu_f((float)x[u]);
    return o;
}

// Loads of one 64 x 128 tile: thread (cc = tid % 16, rg = tid / 16) owns
// rows 4 rg .. 4 rg + 3, features 8 cc .. 8 cc + 7.  Rows >= n are zero.
struct Tile {
    bf16x8 r[4];
};

__device__ __forceinline__ void load_tile(Tile& t, const __bf16* __restrict__ base, int64_t HD,
                                          int n, int cc, int rg) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int row = 4 * rg + r;
        if (row < n)
            t.r[r] = *reinterpret_cast<const bf16x8*>(base + (int64_t)row * HD + 8 * cc);
        else
            t.r[r] = bf16x8{};
    }
}

// SiLU the tile and store it feature-major: dst[(8 cc + e) * TP + 4 rg + r].
__device__ __forceinline__ void store_transposed(const bf16x8 (&s)[4], __bf16* dst, int cc,
                                                 int rg) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        bf16x4 col = {s[0][e], s[1][e], s[2][e], s[3][e]};
        *reinterpret_cast<bf16x4*>(dst + (8 * cc + e) * TP + 4 * rg) = col;
    }
}

// ------------------------------------------------------------ chunk state
// states[c][h][dk][dv] = sum over the chunk's tokens of k~_dk v~_dv.
__global__ __launch_bounds__(MTHREADS) void chunk_state_mfma_kernel(
    const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const PlanHeader* __restrict__ hdr, const ChunkEntry* __restrict__ chunks,
    float* __restrict__ states, int H) {
    __shared__ __attribute__((aligned(16))) __bf16 sKT[MD * TP];
    __shared__ __attribute__((aligned(16))) __bf16 sVT[MD * TP];
    const int c = blockIdx.x / H, h = blockIdx.x - (blockIdx.x / H) * H;
    if (c >= hdr->n_chunks) return;
    const ChunkEntry ce = chunks[c];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int cc = tid & 15, rg = tid >> 4;
    const int l32 = lane & 31, g = lane >> 5;
    const int64_t HD = (int64_t)H * MD;
    const __bf16* kb = k + ce.start * HD + (int64_t)h * MD;
    const __bf16* vb = v + ce.start * HD + (int64_t)h * MD;
    f32x16 acc[4] = {};
    Tile tk, tv;
    load_tile(tk, kb, HD, min(MB, ce.len), cc, rg);
    load_tile(tv, vb, HD, min(MB, ce.len), cc, rg);
    for (int t0 = 0; t0 < ce.len; t0 += MB) {
        bf16x8 ks[4], vs[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            ks[r] = silu8(tk.r[r]);
            vs[r] = silu8(tv.r[r]);
        }
        if (t0 + MB < ce.len) {  // prefetch the next block
            const int n1 = min(MB, ce.len - t0 - MB);
            load_tile(tk, kb + (int64_t)(t0 + MB) * HD, HD, n1, cc, rg);
            load_tile(tv, vb + (int64_t)(t0 + MB) * HD, HD, n1, cc, rg);
        }
        store_transposed(ks, sKT, cc, rg);
        store_transposed(vs, sVT, cc, rg);
        __syncthreads();
#pragma unroll
        for (int s = 0; s < MB / 16; ++s) {
            const bf16x8 b = *reinterpret_cast<const bf16x8*>(sVT + (32 * w + l32) * TP + 16 * s + 8 * g);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(sKT + (32 * m + l32) * TP + 16 * s + 8 * g);
                acc[m] = mfma32(a, b, acc[m]);
            }
        }
        __syncthreads();
    }
    float* dst = states + ((int64_t)c * H + h) * MD * MD;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int dk = 32 * m + 8 * (r >> 2) + 4 * g + (r & 3);
            dst[dk * MD + 32 * w + l32] = acc[m][r];
        }
}

// ------------------------------------------------------------- chunk walk
// 8 waves: waves 0-3 are consumers (MFMA, state in registers), waves 4-7 are
// producers (global loads, SiLU, LDS tiles of the next block, Y stores), so
// the vector-ALU SiLU work of block b+1 overlaps the matrix work of block b.
// LDS tiles are double-buffered; each block costs two workgroup barriers.
constexpr int WTHREADS = 512;

struct WalkLds {
    __bf16 q[2][MB * QP];   // Q~ [t][d]
    __bf16 k[2][MB * QP];   // K~ [t][d]; after the scores, Y [t][dv] (bf16)
    __bf16 kt[2][MD * TP];  // K~^T [d][t]
    __bf16 vt[2][MD * TP];  // V~^T [d][t]
    __bf16 p[MB * TP];      // masked scores P [t][t']
};

// producer: loads of one 64 x 128 tile at 32-bit offsets from a uniform base
__device__ __forceinline__ void load_tile32(Tile& t, const __bf16* __restrict__ base, int HD,
                                            int n, int cc, int rg) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int row = 4 * rg + r;
        t.r[r] = row < n ? *reinterpret_cast<const bf16x8*>(base + (row * HD + 8 * cc))
                         : bf16x8{};
    }
}

__global__ __launch_bounds__(WTHREADS) void walk_mfma_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    __bf16* __restrict__ out, const PlanHeader* __restrict__ hdr,
    const ChunkEntry* __restrict__ chunks, const float* __restrict__ states, int H) {
    __shared__ __attribute__((aligned(16))) WalkLds L;
    const int c = blockIdx.x / H, h = blockIdx.x - (blockIdx.x / H) * H;
    if (c >= hdr->n_chunks) return;
    const ChunkEntry ce = chunks[c];
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int HD = H * MD;
    const int64_t off0 = ce.start * (int64_t)HD + (int64_t)h * MD;
    const int nblk = (ce.len + MB - 1) / MB;

    if (w >= 4) {
        // ------------------------------------------------------ producers
        const int ptid = tid - 256;
        const int cc = ptid & 15, rg = ptid >> 4;
        Tile tq, tk, tv;
        load_tile32(tq, q + off0, HD, min(MB, ce.len), cc, rg);
        load_tile32(tk, k + off0, HD, min(MB, ce.len), cc, rg);
        load_tile32(tv, v + off0, HD, min(MB, ce.len), cc, rg);
        // block b is produced into buffer b & 1 during iteration b - 1
        for (int b = 0; b <= nblk; ++b) {
            const int buf = b & 1;
            bf16x8 ks[4];
            // Y of block b - 2 (staged by the consumers in k[buf] during iteration
            // b - 1) leaves before this thread overwrites the same LDS words
            if (b >= 2) {
                const int t0y = (b - 2) * MB;
                const int ny = min(MB, ce.len - t0y);
                __bf16* ob = out + off0 + (int64_t)t0y * HD;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 4 * rg + r;
                    if (row < ny)
                        *reinterpret_cast<bf16x8*>(ob + (row * HD + 8 * cc)) =
                            *reinterpret_cast<const bf16x8*>(L.k[buf] + row * QP + 8 * cc);
                }
            }
            if (b < nblk) {
                bf16x8 qs[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    qs[r] = silu8(tq.r[r]);
                    ks[r] = silu8(tk.r[r]);
                }
                if (b + 1 < nblk) {
                    const int t1 = (b + 1) * MB;
                    const int n1 = min(MB, ce.len - t1);
                    const int64_t o1 = off0 + (int64_t)t1 * HD;
                    load_tile32(tq, q + o1, HD, n1, cc, rg);
                    load_tile32(tk, k + o1, HD, n1, cc, rg);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    *reinterpret_cast<bf16x8*>(L.q[buf] + (4 * rg + r) * QP + 8 * cc) = qs[r];
                    *reinterpret_cast<bf16x8*>(L.k[buf] + (4 * rg + r) * QP + 8 * cc) = ks[r];
                }
            }
            __syncthreads();  // A
            if (b < nblk) {
                bf16x8 vs[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) vs[r] = silu8(tv.r[r]);
                if (b + 1 < nblk) {
                    const int t1 = (b + 1) * MB;
                    load_tile32(tv, v + off0 + (int64_t)t1 * HD, HD, min(MB, ce.len - t1), cc, rg);
                }
                store_transposed(ks, L.kt[buf], cc, rg);
                store_transposed(vs, L.vt[buf], cc, rg);
            }
            __syncthreads();  // B
        }
        // the last block's Y, staged in k[(nblk - 1) & 1] during the final iteration
        __syncthreads();  // C: the consumers' final staging is complete
        {
            const int b = nblk - 1;
            const int t0y = b * MB;
            const int ny = min(MB, ce.len - t0y);
            __bf16* ob = out + off0 + (int64_t)t0y * HD;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 4 * rg + r;
                if (row < ny)
                    *reinterpret_cast<bf16x8*>(ob + (row * HD + 8 * cc)) =
                        *reinterpret_cast<const bf16x8*>(L.k[b & 1] + row * QP + 8 * cc);
            }
        }
        return;
    }

    // ---------------------------------------------------------- consumers
    const int l32 = lane & 31, g = lane >> 5;
    f32x16 S[4];
    {
        const float* src = states + ((int64_t)c * H + h) * MD * MD;
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int dk = 32 * m + 8 * (r >> 2) + 4 * g + (r & 3);
                S[m][r] = src[dk * MD + 32 * w + l32];
            }
    }
    const int qa = w >> 1, qb = w & 1;  // score quadrant: t' in [32 qa, +32), t in [32 qb, +32)
    // iteration b consumes buffer (b - 1) & 1 holding block b - 1
    for (int b = 0; b <= nblk; ++b) {
        const int buf = (b - 1) & 1;
        if (b >= 1) {
            const __bf16* sQ = L.q[buf];
            const __bf16* sK = L.k[buf];
            f32x16 pacc = {};
            if (!(qa == 1 && qb == 0)) {
#pragma unroll
                for (int s = 0; s < MD / 16; ++s) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8*>(sK + (32 * qa + l32) * QP + 16 * s + 8 * g);
                    const bf16x8 bb = *reinterpret_cast<const bf16x8*>(sQ + (32 * qb + l32) * QP + 16 * s + 8 * g);
                    pacc = mfma32(a, bb, pacc);
                }
            }
            const int t = 32 * qb + l32;
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
                const int tp0 = 32 * qa + 8 * qd + 4 * g;
                bf16x4 o;
#pragma unroll
                for (int u = 0; u < 4; ++u) o[u] = (__bf16)(tp0 + u <= t ? pacc[4 * qd + u] : 0.f);
                *reinterpret_cast<bf16x4*>(L.p + t * TP + tp0) = o;
            }
        }
        __syncthreads();  // A
        if (b >= 1) {
            const __bf16* sQ = L.q[buf];
            const __bf16* sKT = L.kt[buf];
            const __bf16* sVT = L.vt[buf];
            f32x16 O[2] = {};
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
                for (int s = 0; s < MB / 16; ++s) {
                    if (tb == 0 && s >= 2) continue;
                    const bf16x8 a = *reinterpret_cast<const bf16x8*>(sVT + (32 * w + l32) * TP + 16 * s + 8 * g);
                    const bf16x8 bb = *reinterpret_cast<const bf16x8*>(L.p + (32 * tb + l32) * TP + 16 * s + 8 * g);
                    O[tb] = mfma32(a, bb, O[tb]);
                }
#pragma unroll
                for (int s = 0; s < MD / 16; ++s) {
                    const int m = s >> 1, r0 = 8 * (s & 1);
                    bf16x8 a;
#pragma unroll
                    for (int j = 0; j < 8; ++j) a[j] = (__bf16)S[m][r0 + j];
                    const __bf16* qrow = sQ + (32 * tb + l32) * QP + 16 * s + 4 * g;
                    const bf16x4 b0 = *reinterpret_cast<const bf16x4*>(qrow);
                    const bf16x4 b1 = *reinterpret_cast<const bf16x4*>(qrow + 8);
                    const bf16x8 bb = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
                    O[tb] = mfma32(a, bb, O[tb]);
                }
            }
#pragma unroll
            for (int s = 0; s < MB / 16; ++s) {
                const bf16x8 bb = *reinterpret_cast<const bf16x8*>(sVT + (32 * w + l32) * TP + 16 * s + 8 * g);
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8*>(sKT + (32 * m + l32) * TP + 16 * s + 8 * g);
                    S[m] = mfma32(a, bb, S[m]);
                }
            }
            // stage Y token-major in k[buf]: every consumer wave finished its scores before A
            __bf16* sY = L.k[buf];
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
                const int t = 32 * tb + l32;
#pragma unroll
                for (int qd = 0; qd < 4; ++qd) {
                    bf16x4 o;
#pragma unroll
                    for (int u = 0; u < 4; ++u) o[u] = (__bf16)O[tb][4 * qd + u];
                    *reinterpret_cast<bf16x4*>(sY + t * QP + 32 * w + 8 * qd + 4 * g) = o;
                }
            }
        }
        __syncthreads();  // B
    }
    __syncthreads();  // C
}

bool mfma_supported(const PrefillArgs& a) { return a.bf16 && a.D == MD && a.block == MB; }

hipError_t launch_chunk_state_mfma(const PrefillArgs& a, hipStream_t st) {
    if (a.max_chunks == 0) return hipSuccess;
    const dim3 grid((unsigned)((int64_t)a.max_chunks * a.H));
    hipLaunchKernelGGL(chunk_state_mfma_kernel, grid, dim3(MTHREADS), 0, st, (const __bf16*)a.k,
                       (const __bf16*)a.v, a.hdr, a.chunks, a.states, a.H);
    return hipGetLastError();
}

hipError_t launch_walk_mfma(const PrefillArgs& a, hipStream_t st) {
    if (a.max_chunks == 0) return hipSuccess;
    const dim3 grid((unsigned)((int64_t)a.max_chunks * a.H));
    hipLaunchKernelGGL(walk_mfma_kernel, grid, dim3(WTHREADS), 0, st, (const __bf16*)a.q,
                       (const __bf16*)a.k, (const __bf16*)a.v, (__bf16*)a.out, a.hdr, a.chunks,
                       a.states, a.H);
    return hipGetLastError();
}

}  // namespace la
