// bf16 MFMA kernels of the Lightning Attention layer for gfx950
// (head_dim 128, block 64 tokens, fp32 accumulation).
//
// Mechanism step 3 of "Diving into MiniMax01 405B MoE" (section "Hybrid
// Modeling"), Y = Q (K^T V) read causally, is computed per block b of 64
// tokens of a chunk, with S the fp32 state entering the block:
//   P^T  = K~_b Q~_b^T, masked to t' <= t          (intra-block scores)
//   O^T  = V~_b^T P^T + S^T Q~_b^T                  (intra + inter, transposed)
//   S   += K~_b^T V~_b                              (state update)
// and step 4, out = y / sqrt(mean_{h,d} y^2 + eps) * w * sigmoid(gate), is
// applied in the same kernel.  Every product is a v_mfma_f32_32x32x16_bf16
// (A: 32x16, B: 16x32, C: 32x32 fp32).  Lane layouts (checked on the
// hardware): A row = lane % 32 with k = 8 (lane / 32) + j; B column =
// lane % 32, same k; C column = lane % 32, row = 8 (r / 4) + 4 (lane / 32) +
// r % 4 for accumulator r.
//
// Both kernels run 8 waves per workgroup: waves 4-7 are producers (16-byte
// global loads of the next block, SiLU in fp32, bf16 tiles in the layouts
// the MFMA operands read, coalesced stores), waves 0-3 are consumers (the
// matrix products).  Each SIMD hosts one wave of each kind, so the vector-ALU
// SiLU work overlaps the matrix work, and LDS tiles are double-buffered.
//
// Consumer wave w owns state columns dv in [32w, 32w+32) for all 128 key rows
// in four C tiles (64 fp32 registers per lane): the state never leaves
// registers during a walk, and the inter-block product reads it straight from
// the accumulators -- transposed, S^T is an A operand whose rows are the
// lane's own column dv, and the k permutation of the C layout is matched in
// the Q~ operand.
#include "la_internal.h"

namespace la {

constexpr int MD = 128;        // head_dim
constexpr int MB = 64;         // block tokens
constexpr int NTHREADS = 512;  // 4 consumer + 4 producer waves
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

// One 64 x 128 tile as loaded by a producer thread (cc = ptid % 16,
// rg = ptid / 16): rows 4 rg .. 4 rg + 3, features 8 cc .. 8 cc + 7.
struct Tile {
    bf16x8 r[4];
};

// 32-bit offsets from a uniform base; rows >= n read as zero.
__device__ __forceinline__ void load_tile(Tile& t, const __bf16* __restrict__ base, int HD, int n,
                                          int cc, int rg) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int row = 4 * rg + r;
        t.r[r] = row < n ? *reinterpret_cast<const bf16x8*>(base + (row * HD + 8 * cc))
                         : bf16x8{};
    }
}

// store a SiLU'd tile feature-major: dst[(8 cc + e) * TP + 4 rg + r]
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
// Chunks are visited in descending order so that the walk, which visits
// them in ascending order right after, finds the most recently read K and V
// still in the memory-side cache.
struct StateLds {
    __bf16 kt[2][MD * TP];
    __bf16 vt[2][MD * TP];
};

__global__ __launch_bounds__(NTHREADS) void chunk_state_mfma_kernel(
    const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const PlanHeader* __restrict__ hdr, const ChunkEntry* __restrict__ chunks,
    float* __restrict__ states, int H) {
    __shared__ __attribute__((aligned(16))) StateLds L;
    const int nch = hdr->n_chunks;
    const int cr = blockIdx.x / H, h = blockIdx.x - (blockIdx.x / H) * H;
    if (cr >= nch) return;
    const int c = nch - 1 - cr;
    const ChunkEntry ce = chunks[c];
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int HD = H * MD;
    const int64_t off0 = ce.start * (int64_t)HD + (int64_t)h * MD;
    const int nblk = (ce.len + MB - 1) / MB;

    if (w >= 4) {
        const int ptid = tid - 256;
        const int cc = ptid & 15, rg = ptid >> 4;
        Tile tk, tv;
        load_tile(tk, k + off0, HD, min(MB, ce.len), cc, rg);
        load_tile(tv, v + off0, HD, min(MB, ce.len), cc, rg);
        for (int b = 0; b <= nblk; ++b) {  // block b goes to buffer b & 1
            if (b < nblk) {
                bf16x8 ks[4], vs[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    ks[r] = silu8(tk.r[r]);
                    vs[r] = silu8(tv.r[r]);
                }
                if (b + 1 < nblk) {
                    const int t1 = (b + 1) * MB;
                    const int n1 = min(MB, ce.len - t1);
                    load_tile(tk, k + off0 + (int64_t)t1 * HD, HD, n1, cc, rg);
                    load_tile(tv, v + off0 + (int64_t)t1 * HD, HD, n1, cc, rg);
                }
                store_transposed(ks, L.kt[b & 1], cc, rg);
                store_transposed(vs, L.vt[b & 1], cc, rg);
            }
            __syncthreads();
        }
        return;
    }
    const int l32 = lane & 31, g = lane >> 5;
    f32x16 acc[4] = {};
    for (int b = 0; b <= nblk; ++b) {  // consumes block b - 1
        if (b >= 1) {
            const __bf16* sKT = L.kt[(b - 1) & 1];
            const __bf16* sVT = L.vt[(b - 1) & 1];
#pragma unroll
            for (int s = 0; s < MB / 16; ++s) {
                const bf16x8 bb = *reinterpret_cast<const bf16x8*>(sVT + (32 * w + l32) * TP + 16 * s + 8 * g);
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8*>(sKT + (32 * m + l32) * TP + 16 * s + 8 * g);
                    acc[m] = mfma32(a, bb, acc[m]);
                }
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

// --------------------------------------------- cross-workgroup exchange
// Agent-scope relaxed atomics compile to sc1 (coherent) loads and stores on
// gfx950, so values published this way are seen by workgroups on every XCD
// once the stores have completed; drain() waits for that before a counter or
// flag is raised, and keeps the compiler from moving memory accesses across.
__device__ __forceinline__ void put_agent(float* p, float x) {
    __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float get_agent(float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int get_agent_i(int* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void drain() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Bound on the polls of one cross-head wait (each poll is a coherent load,
// about a microsecond): a wait never legitimately lasts longer than one chunk
// walk, so reaching it means the workgroups of a chunk could not all run.
// The kernel then records error 3 in the plan header, every later wait gives
// up at once, and the launch finishes (with an unspecified output).
constexpr int WAIT_POLLS = 1 << 20;

// --------------------------------------------- fused chunk walk + RMSNorm
// Workgroups take (chunk, head) items in start order from a ticket, head
// fastest, so all heads of a chunk are started before any head of the next
// chunk: the per-block cross-head waits below only ever wait on workgroups
// that have started (or on earlier chunks that can always finish).
//
// Per 64-token block j of chunk c (slot = c * slots_per_chunk + j):
//   * iteration j + 1: the consumers compute y (fp32), reduce sum_dv y^2 per
//     token across the four waves and publish it as part[slot][h][t], then
//     count themselves in arrivals[slot]; the head that arrives last sums the
//     H partial sums in head order (deterministic), writes rnorm[slot][t] and
//     raises ready[slot].  y is staged in LDS as bf16;
//   * iteration j + 2: the producers store that y to its place in `out`;
//   * iteration j + LAG: the same producer threads wait for ready[slot],
//     re-read their own y from `out` (still in L2 or the memory-side cache),
//     and overwrite it with y * rnorm * w * sigmoid(gate).
// LAG iterations of slack hide the cross-XCD round trips of the exchange.
constexpr int LAG = 4;

struct WalkLds {
    __bf16 q[2][MB * QP];   // Q~ [t][d]
    __bf16 k[2][MB * QP];   // K~ [t][d]; once the scores are done, y [t][dv]
    __bf16 kt[2][MD * TP];  // K~^T [d][t]
    __bf16 vt[2][MD * TP];  // V~^T [d][t]
    __bf16 p[MB * TP];      // masked scores P [t][t']
    float red[4][MB];       // per-wave sums of y^2 per token
    float rn[2][MB];        // norm factors of the block the producers finalise next
    int item;
};

__global__ __launch_bounds__(NTHREADS) void walk_norm_mfma_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ gate, const __bf16* __restrict__ wgt, __bf16* __restrict__ out,
    PlanHeader* __restrict__ hdr, const ChunkEntry* __restrict__ chunks,
    const float* __restrict__ states, float* __restrict__ part, float* __restrict__ rnorm,
    int32_t* __restrict__ arrivals, int32_t* __restrict__ ready, int H, int slots_per_chunk,
    float eps) {
    __shared__ __attribute__((aligned(16))) WalkLds L;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    if (tid == 0) L.item = atomicAdd(&hdr->ticket, 1);
    __syncthreads();
    const int item = L.item;
    const int c = item / H, h = item - (item / H) * H;
    if (c >= hdr->n_chunks) return;
    const ChunkEntry ce = chunks[c];
    const int HD = H * MD;
    const int64_t off0 = ce.start * (int64_t)HD + (int64_t)h * MD;
    const int nblk = (ce.len + MB - 1) / MB;
    const int slot0 = c * slots_per_chunk;
    const int iters = nblk + LAG;

    if (w >= 4) {
        // ------------------------------------------------------ producers
        const int ptid = tid - 256;
        const int cc = ptid & 15, rg = ptid >> 4;
        const bf16x8 wv = *reinterpret_cast<const bf16x8*>(wgt + h * MD + 8 * cc);
        Tile tq, tk, tv;
        load_tile(tq, q + off0, HD, min(MB, ce.len), cc, rg);
        load_tile(tk, k + off0, HD, min(MB, ce.len), cc, rg);
        load_tile(tv, v + off0, HD, min(MB, ce.len), cc, rg);
        for (int b = 0; b < iters; ++b) {
            const int buf = b & 1;
            bf16x8 ks[4];
            // ---- phase 1: y of block b - 2 to `out`; q, k of block b to LDS
            if (b >= 2 && b - 2 < nblk) {  // staged in k[buf] by the consumers in iteration b - 1
                const int t0 = (b - 2) * MB;
                const int n = min(MB, ce.len - t0);
                __bf16* ob = out + off0 + (int64_t)t0 * HD;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 4 * rg + r;
                    if (row < n)
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
                    load_tile(tq, q + off0 + (int64_t)t1 * HD, HD, n1, cc, rg);
                    load_tile(tk, k + off0 + (int64_t)t1 * HD, HD, n1, cc, rg);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    *reinterpret_cast<bf16x8*>(L.q[buf] + (4 * rg + r) * QP + 8 * cc) = qs[r];
                    *reinterpret_cast<bf16x8*>(L.k[buf] + (4 * rg + r) * QP + 8 * cc) = ks[r];
                }
            }
            __syncthreads();  // A
            // ---- phase 2: v of block b to LDS; loads for the block finalised below
            const int jf = b - LAG;
            const bool fin = jf >= 0 && jf < nblk;
            Tile ty, tg;
            int nf = 0;
            if (fin) {
                const int t0 = jf * MB;
                nf = min(MB, ce.len - t0);
                load_tile(ty, out + off0 + (int64_t)t0 * HD, HD, nf, cc, rg);
                load_tile(tg, gate + off0 + (int64_t)t0 * HD, HD, nf, cc, rg);
            }
            if (b < nblk) {
                bf16x8 vs[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) vs[r] = silu8(tv.r[r]);
                if (b + 1 < nblk) {
                    const int t1 = (b + 1) * MB;
                    load_tile(tv, v + off0 + (int64_t)t1 * HD, HD, min(MB, ce.len - t1), cc, rg);
                }
                store_transposed(ks, L.kt[buf], cc, rg);
                store_transposed(vs, L.vt[buf], cc, rg);
            }
            __syncthreads();  // B
            // ---- phase 3: finalise block jf = b - LAG with the norm factors that
            // consumer wave 2 left in rn[jf & 1] before barrier A of this iteration
            if (fin) {
                __bf16* ob = out + off0 + (int64_t)jf * MB * HD;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 4 * rg + r;
                    if (row < nf) {
                        const float rr = L.rn[jf & 1][row];
                        bf16x8 o;
#pragma unroll
                        for (int u = 0; u < 8; ++u)
                            o[u] = (__bf16)((float)ty.r[r][u] * rr * (float)wv[u] *
                                            sigmoid_f((float)tg.r[r][u]));
                        *reinterpret_cast<bf16x8*>(ob + (row * HD + 8 * cc)) = o;
                    }
                }
            }
        }
        return;
    }

    // ---------------------------------------------------------- consumers
    const int l32 = lane & 31, g = lane >> 5;
    const float inv_hd = 1.0f / (float)HD;
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
    for (int b = 0; b < iters; ++b) {
        const int jc = b - 1;  // block computed in this iteration
        const bool comp = jc >= 0 && jc < nblk;
        const int buf = jc & 1;
        // ---- phase 1: scores of block jc
        if (comp) {
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
        // ---- phase 2: y of block jc (intra + inter), state update, staging
        if (comp) {
            const __bf16* sQ = L.q[buf];
            const __bf16* sKT = L.kt[buf];
            const __bf16* sVT = L.vt[buf];
            f32x16 O[2] = {};
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
                for (int s = 0; s < MB / 16; ++s) {
                    if (tb == 0 && s >= 2) continue;  // t < 32 sees only t' < 32
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
            // per-token sum of y^2 over this wave's 32 columns, and y (bf16) staged
            // token-major in k[buf], which no wave reads after the scores
            __bf16* sY = L.k[buf];
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
                float ss = 0.f;
#pragma unroll
                for (int r = 0; r < 16; ++r) ss += O[tb][r] * O[tb][r];
                ss += __shfl_xor(ss, 32);
                if (g == 0) L.red[w][32 * tb + l32] = ss;
                const int t = 32 * tb + l32;
#pragma unroll
                for (int qd = 0; qd < 4; ++qd) {
                    bf16x4 y;
#pragma unroll
                    for (int u = 0; u < 4; ++u) y[u] = (__bf16)O[tb][4 * qd + u];
                    *reinterpret_cast<bf16x4*>(sY + t * QP + 32 * w + 8 * qd + 4 * g) = y;
                }
            }
        }
        __syncthreads();  // B
        // ---- phase 3 (wave 2, whose score quadrant is empty, so it has slack):
        // publish block jc's sums of squares, then fetch the norm factors of
        // block jn for the producers' next iteration.  No other wave touches
        // coherent memory, so no wave with loads in flight waits on it.
        if (w == 2) {
            if (comp) {
                const int slot = slot0 + jc;
                const float mine = L.red[0][lane] + L.red[1][lane] + L.red[2][lane] + L.red[3][lane];
                put_agent(part + ((int64_t)slot * H + h) * MB + lane, mine);
                drain();
                int prev = 0;
                if (lane == 0) prev = atomicAdd(&arrivals[slot], 1);
                prev = __shfl(prev, 0);
                if (prev == H - 1) {  // last head of this block: reduce over heads in order
                    // loads are issued in batches so that each batch costs one round trip
                    constexpr int BATCH = 32;
                    float tot = 0.f;
                    for (int h0 = 0; h0 < H; h0 += BATCH) {
                        float vals[BATCH];
#pragma unroll
                        for (int i = 0; i < BATCH; ++i)
                            vals[i] = h0 + i < H
                                          ? get_agent(part + ((int64_t)slot * H + h0 + i) * MB + lane)
                                          : 0.f;
#pragma unroll
                        for (int i = 0; i < BATCH; ++i) tot += vals[i];
                    }
                    put_agent(rnorm + (int64_t)slot * MB + lane,
                              __builtin_amdgcn_rsqf(tot * inv_hd + eps));
                    drain();
                    if (lane == 0)
                        __hip_atomic_store(&ready[slot], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
            const int jn = b + 1 - LAG;
            if (jn >= 0 && jn < nblk) {
                const int slot = slot0 + jn;
                if (lane == 0) {
                    int polls = 0;
                    while (get_agent_i(&ready[slot]) == 0) {
                        __builtin_amdgcn_s_sleep(1);
                        ++polls;
                        if ((polls & 255) == 0 && get_agent_i(&hdr->error) == 3) break;
                        if (polls >= WAIT_POLLS) {
                            __hip_atomic_store(&hdr->error, 3, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
                            break;
                        }
                    }
                }
                __builtin_amdgcn_wave_barrier();
                drain();
                L.rn[jn & 1][lane] = get_agent(rnorm + (int64_t)slot * MB + lane);
            }
        }
    }
}

bool mfma_supported(const PrefillArgs& a) { return a.bf16 && a.D == MD && a.block == MB; }

hipError_t launch_chunk_state_mfma(const PrefillArgs& a, hipStream_t st) {
    if (a.max_chunks == 0) return hipSuccess;
    const dim3 grid((unsigned)((int64_t)a.max_chunks * a.H));
    hipLaunchKernelGGL(chunk_state_mfma_kernel, grid, dim3(NTHREADS), 0, st, (const __bf16*)a.k,
                       (const __bf16*)a.v, a.hdr, a.chunks, a.states, a.H);
    return hipGetLastError();
}

hipError_t launch_walk_mfma(const PrefillArgs& a, hipStream_t st) {
    if (a.max_chunks == 0) return hipSuccess;
    const dim3 grid((unsigned)((int64_t)a.max_chunks * a.H));
    hipLaunchKernelGGL(walk_norm_mfma_kernel, grid, dim3(NTHREADS), 0, st, (const __bf16*)a.q,
                       (const __bf16*)a.k, (const __bf16*)a.v, (const __bf16*)a.g,
                       (const __bf16*)a.w, (__bf16*)a.out, a.hdr, a.chunks, a.states, a.part,
                       a.rnorm, a.arrivals, a.ready, a.H, a.chunk / MB, a.eps);
    return hipGetLastError();
}

}  // namespace la
