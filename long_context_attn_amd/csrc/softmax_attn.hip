// The hybrid's softmax attention layer on gfx950: one softmax layer after
// every seven Lightning layers ("Diving into MiniMax01 405B MoE", section
// "Hybrid Modeling", 1/8 Softmax Attention; the model card, "2. Model
// Architecture", Positional Encoding: rotary embedding on half of the head
// dimension with base frequency 10,000,000).
//
//   q^, k^ = rope(q), rope(k)   (pairs (2i, 2i+1) of the first rope_dim features
//                                turned by pos * base^(-2i / rope_dim); pos
//                                counts from 0 in every sequence)
//   out_t  = sum_{u <= t} softmax_u(scale <q^_t, k^_u>) v_u   (causal, per sequence)
//
// Two kernels:
//  - rope_kernel: rotates k once into a bf16 copy in the workspace
//    (HBM-bound; the angles are reduced in fp64, so positions up to 2^31 keep
//    full fp32 accuracy); q is rotated the same way as the attention kernel
//    loads it (once per query tile);
//  - softmax_fwd_kernel: flash-style causal attention on bf16 MFMA.  A
//    workgroup of four waves takes a 128-query tile of one head (32 queries per
//    wave) and walks the key blocks from its sequence's start to the tile's
//    end, 64 keys at a time, K and V double-buffered in LDS.  Each wave
//    computes the scores transposed, S^T = K Q^T (v_mfma_f32_32x32x16_bf16, Q
//    held in registers as the B operand), so that every lane owns one query:
//    the running maximum, the rescale of the output and the row sum stay in
//    the lane, with one exchange between the lane halves per block.  The
//    probabilities become the B operand of O^T += V^T P^T through one
//    permlane32 swap; V^T comes from the transposing LDS read.  Softmax runs
//    in base 2 with scale * log2(e) folded into the logits.
#include <hip/hip_runtime.h>

#include <cmath>
#include <type_traits>

#include "la_internal.h"
#include "mfma_common.h"

namespace la {

namespace {

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ rope
constexpr int ROPE_THREADS = 256;
constexpr int ROPE_TOKENS = 8;   // tokens per workgroup
constexpr int ROPE_BATCH = 8;    // loads in flight per thread
constexpr int ROPE_MAX_PAIRS = 64;

// the rotation frequencies theta_p = base^(-2p / rope_dim), passed by value
struct RopeTheta {
    double t[ROPE_MAX_PAIRS];
};
RopeTheta rope_theta(const SoftmaxArgs& a) {
    RopeTheta th{};
    for (int p = 0; p < a.rope_dim / 2 && p < ROPE_MAX_PAIRS; ++p)
        th.t[p] = std::pow(a.rope_base, -2.0 * p / a.rope_dim);
    return th;
}

// Rotation of one feature pair p (< rope_dim / 2) at position pos: the angle
// pos * theta_p (theta_p = base^(-2p / rope_dim), computed on the host in
// fp64) is formed and reduced to [-pi, pi] in fp64, then its cosine and sine
// are taken in fp32.
__device__ __forceinline__ float2 rope_cs(int64_t pos, double theta) {
    const double two_pi = 6.283185307179586476925286766559;
    const double inv_two_pi = 0.15915494309189533576888376337251;
    double a = (double)pos * theta;
    a -= two_pi * rint(a * inv_two_pi);
    float sn, cn;
    sincosf((float)a, &sn, &cn);
    return make_float2(cn, sn);
}

// K's rotation (the attention kernel turns Q itself as it loads it).
// Workgroup (tile c, group j): the ROPE_TOKENS tokens from ROPE_TOKENS * j
// on of tile c.  Each
// token's cos / sin table is built once in LDS and serves all of its heads.
__global__ __launch_bounds__(ROPE_THREADS) void rope_kernel(
    const __bf16* __restrict__ k, __bf16* __restrict__ kr, const PlanHeader* __restrict__ hdr,
    const SegEntry* __restrict__ segs, const ChunkEntry* __restrict__ tiles, int H, int rope_dim,
    const RopeTheta th) {
    __shared__ float2 cs[ROPE_TOKENS][ROPE_MAX_PAIRS];
    constexpr int GROUPS = SOFTMAX_TILE / ROPE_TOKENS;
    const int c = blockIdx.x / GROUPS, grp = blockIdx.x - c * GROUPS;
    if (c >= hdr->n_chunks) return;
    const ChunkEntry ce = tiles[c];
    const int t0 = grp * ROPE_TOKENS;
    const int nt = min(ROPE_TOKENS, ce.len - t0);
    if (nt <= 0) return;
    const int64_t first = ce.start + t0;                      // packed index of the first token
    const int64_t pos0 = first - tiles[segs[ce.seg].first].start;  // its position in the sequence
    const int npairs = rope_dim / 2;
    for (int i = threadIdx.x; i < ROPE_TOKENS * npairs; i += ROPE_THREADS) {
        const int t = i / npairs, p = i - t * npairs;
        cs[t][p] = rope_cs(pos0 + t, th.t[p]);
    }
    __syncthreads();
    const int HD = H * MD;
    const int per_token = HD / 8;  // 16-byte pieces of one token
    const int64_t n = (int64_t)nt * per_token;
    // ROPE_BATCH pieces per thread are loaded before any is rotated and stored
    for (int64_t e0 = threadIdx.x; e0 < n; e0 += (int64_t)ROPE_BATCH * ROPE_THREADS) {
        bf16x8 x[ROPE_BATCH];
#pragma unroll
        for (int j = 0; j < ROPE_BATCH; ++j) {
            const int64_t e = e0 + (int64_t)j * ROPE_THREADS;
            if (e < n) x[j] = *reinterpret_cast<const bf16x8*>(k + first * HD + e * 8);
        }
#pragma unroll
        for (int j = 0; j < ROPE_BATCH; ++j) {
            const int64_t e = e0 + (int64_t)j * ROPE_THREADS;
            if (e >= n) break;
            const int t = (int)(e / per_token);
            const int piece = (int)(e - (int64_t)t * per_token);
            const int f = (piece % (MD / 8)) * 8;  // first feature of the piece within its head
            if (f < rope_dim) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float2 r = cs[t][f / 2 + u];
                    const float a = (float)x[j][2 * u], b = (float)x[j][2 * u + 1];
                    x[j][2 * u] = (__bf16)(a * r.x - b * r.y);
                    x[j][2 * u + 1] = (__bf16)(a * r.y + b * r.x);
                }
            }
            *reinterpret_cast<bf16x8*>(kr + first * HD + e * 8) = x[j];
        }
    }
}

// --------------------------------------------------------- attention
// One 32-query sub-tile per wave, four waves: two waves share each SIMD and
// overlap one's MFMA work with the other's VALU work.  Two sub-tiles per wave
// (half the LDS reads per FLOP, one wave per SIMD) measured 2300 against
// 1234 us at 8192 x 64 heads.
constexpr int FA_QT = 1;  // 32-query sub-tiles per wave
constexpr int FA_NW = 4;  // waves per workgroup

struct FaLds {
    __bf16 k[2][TILE];
    __bf16 v[2][TILE];
};

// max / sum of a lane's value and the one of its partner in the other half
// of the wave (the lanes that hold the same query)
__device__ __forceinline__ float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// QT: 32-query sub-tiles per wave; NW: waves per workgroup (QT * NW * 32 =
// 128 queries per tile).  Each K or V operand read from LDS feeds QT
// products, so QT = 2 halves the LDS reads per FLOP, at twice the registers
// (one wave per SIMD instead of two).
template <int QT, int NW>
__global__ __launch_bounds__(64 * NW, 2) void softmax_fwd_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    __bf16* __restrict__ out, const PlanHeader* __restrict__ hdr,
    const SegEntry* __restrict__ segs, const ChunkEntry* __restrict__ tiles, int H, float sl2,
    int rope_dim, const RopeTheta th) {
    static_assert(QT * NW * 32 == SOFTMAX_TILE, "a workgroup covers one query tile");
    __shared__ __attribute__((aligned(16))) FaLds L;
    const int ntile = hdr->n_chunks;
    // Workgroups are dealt to the eight XCDs in turn; when the heads divide
    // evenly, every XCD keeps its own eighth of the heads, so that the K and V
    // of a head are re-read from one L2.  Tiles go from the last (the longest
    // key range) to the first.
    int h, j;
    if ((H & 7) == 0) {
        const int x = blockIdx.x & 7, i = blockIdx.x >> 3, hpx = H >> 3;
        h = x * hpx + i % hpx;
        j = i / hpx;
    } else {
        h = blockIdx.x % H;
        j = blockIdx.x / H;
    }
    if (j >= ntile) return;
    const ChunkEntry ce = tiles[ntile - 1 - j];
    const int64_t s0 = tiles[segs[ce.seg].first].start;  // the sequence's first token
    const int64_t qstart = ce.start;
    const int qlen = ce.len;
    const int HD = H * MD;
    const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, in a scalar register
    const int64_t qend = qstart + qlen;
    const int nkb = (int)((qend - s0 + MB - 1) / MB);

    // this wave's queries: sub-tile qt holds queries q0w + 32 qt + l32; Q^T
    // operands with features 16 s + 8 g .. + 7
    const int64_t q0w = qstart + 32 * QT * w;
    const int qrows = max(0, min(32 * QT, qlen - 32 * QT * w));
    bf16x8 qb[QT][MD / 16];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        const int rows = max(0, min(32, qrows - 32 * qt));
        const __amdgpu_buffer_rsrc_t rs =
            tile_rsrc(q + (q0w + 32 * qt) * HD + (int64_t)h * MD, rows, HD);
        const int voff = (l32 * HD + 8 * g) * 2;
#pragma unroll
        for (int s = 0; s < MD / 16; ++s)
            qb[qt][s] = __builtin_bit_cast(
                bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 32 * s, 0));
        // rotate the first rope_dim features at the query's position (as
        // rope_kernel does for K)
        const int64_t pos = q0w + 32 * qt + l32 - s0;
#pragma unroll
        for (int s = 0; s < MD / 16; ++s) {
            const int f0 = 16 * s + 8 * g;
            if (f0 < rope_dim) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float2 r = rope_cs(pos, th.t[f0 / 2 + u]);
                    const float a = (float)qb[qt][s][2 * u], b = (float)qb[qt][s][2 * u + 1];
                    qb[qt][s][2 * u] = (__bf16)(a * r.x - b * r.y);
                    qb[qt][s][2 * u + 1] = (__bf16)(a * r.y + b * r.x);
                }
            }
        }
    }

    // K / V tiles go from HBM straight into LDS (buffer loads with the LDS
    // as destination, no registers): wave w stages rows 64 / NW * w .. of a
    // 64-key tile with 1 KiB loads, lane l of each filling physical 16-byte
    // chunk l % 16 of row 4 i + l / 16 with the logical chunk that the swizzle
    // puts there.  Rows past a ragged end repeat the last key: their scores
    // are always masked, so they only need to be finite.
    // K runs one block ahead of V: while the exponentials of block b run on
    // the VALU, the scores of block b + 1 run on the matrix cores.  In
    // iteration b the LDS holds K(b + 1) and V(b), and the loads of K(b + 2)
    // and V(b + 1) fill the buffers that K(b) and V(b - 1) left before the
    // last barrier; each wave waits for its own loads before the next barrier.
    constexpr int RPW = MB / NW;  // rows staged per wave
    auto stage = [&](const __bf16* base, int b, __bf16* dst) {
        const int64_t kb0 = s0 + (int64_t)b * MB;
        const int n = (int)min((int64_t)MB, qend - kb0);
        const __amdgpu_buffer_rsrc_t rs = tile_rsrc(base + kb0 * HD + (int64_t)h * MD, n, HD);
#pragma unroll
        for (int i = 0; i < RPW / 4; ++i) {
            const int row0 = RPW * w + 4 * i;
            const int row = row0 + (lane >> 4);
            const int f = ((row & 3) << 2) | ((row >> 2) & 3);
            const int vo = (min(row, n - 1) * HD + 8 * ((lane & 15) ^ f)) * 2;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs, (__attribute__((address_space(3))) void*)(dst + row0 * MD), 16, vo, 0, 0, 0);
        }
    };
    // vmcnt(0) with the other counters left alone: this wave's tile loads done
    auto loads_done = [] { __builtin_amdgcn_s_waitcnt(0x0F70); };
    // the last key block this wave's queries reach (-1: no queries)
    const int last_w = qrows > 0 ? (int)((q0w + qrows - 1 - s0) / MB) : -1;
    stage(k, 0, L.k[0]);
    stage(v, 0, L.v[0]);
    if (nkb > 1) stage(k, 1, L.k[1]);
    loads_done();
    __syncthreads();

    f32x16 O[QT][MD / 32] = {};
    float mrun[QT], lsum[QT];  // running maximum (raw score units) and sum
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        mrun[qt] = -INFINITY;
        lsum[qt] = 0.f;
    }
    // The running maximum only moves when a score exceeds it by more than
    // 8 / sl2, so that probabilities stay below 2^8 and the rescale of the
    // output is rare.
    const float tau = 8.f / sl2;
    auto scores = [&](const __bf16* sK, f32x16 (&S)[QT][2]) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) S[qt][0] = S[qt][1] = f32x16{};
#pragma unroll
        for (int s = 0; s < MD / 16; ++s)
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const bf16x8 ko = ld_row_operand(sK, 32 * m + l32, 16 * s + 8 * g);
#pragma unroll
                for (int qt = 0; qt < QT; ++qt) S[qt][m] = mfma32(ko, qb[qt][s], S[qt][m]);
            }
    };
    f32x16 Sa[QT][2], Sb[QT][2];
    if (last_w >= 0) scores(L.k[0], Sa);
    // iteration 0 loads K(2) into the buffer these scores read: every wave
    // must be done with it first
    __syncthreads();
    // iteration b (P = b % 2): softmax and O += P V for block b (scores in
    // Sc), scores of block b + 1 into Sn
    auto step = [&](auto par, int b, f32x16 (&Sc)[QT][2], f32x16 (&Sn)[QT][2]) {
        constexpr int P = decltype(par)::value;
        if (b + 2 < nkb) stage(k, b + 2, L.k[P]);
        if (b + 1 < nkb) stage(v, b + 1, L.v[1 - P]);
        if (b <= last_w) {
            const int64_t kb0 = s0 + (int64_t)b * MB;
            float msc[QT];
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) {
                const int64_t qabs = q0w + 32 * qt + l32;  // this lane's query
                if (kb0 + MB - 1 > q0w + 32 * qt) {  // reaches the diagonal: mask keys after the query
                    const int qrel = (int)max((int64_t)-1, min((int64_t)MB, qabs - kb0));
#pragma unroll
                    for (int m = 0; m < 2; ++m)
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            if (32 * m + 8 * (r >> 2) + 4 * g + (r & 3) > qrel)
                                Sc[qt][m][r] = -INFINITY;
                }
                float bm = -INFINITY;
#pragma unroll
                for (int m = 0; m < 2; ++m)
#pragma unroll
                    for (int r = 0; r < 16; ++r) bm = fmaxf(bm, Sc[qt][m][r]);
                bm = pair_max(bm);
                const bool up = bm > mrun[qt] + tau;
                if (__builtin_amdgcn_ballot_w64(up) != 0) {
                    const float mnew = up ? bm : mrun[qt];
                    const float alpha = __builtin_amdgcn_exp2f((mrun[qt] - mnew) * sl2);
                    mrun[qt] = mnew;
                    lsum[qt] *= alpha;
#pragma unroll
                    for (int n = 0; n < MD / 32; ++n)
#pragma unroll
                        for (int r = 0; r < 16; ++r) O[qt][n][r] *= alpha;
                }
                msc[qt] = mrun[qt] * sl2;
            }
            // Block b + 1's scores on the matrix cores with block b's
            // exponentials in between: step st issues the products of
            // features 16 st .. 16 st + 15 (K operands read two steps ahead)
            // and four of each sub-tile's 32 exponentials; every two steps
            // complete eight per sub-tile, and they become one P^T operand
            // (accumulator registers r0 .. r0 + 7 of tile m hold keys
            // 16 t + 8 (j / 4) + 4 g + j % 4; one swap between the lane
            // halves makes them keys 16 t + 8 g + j).  The fences keep this
            // order.  A wave past its last block computes scores from
            // whatever the buffer holds and never uses them.
            const __bf16* sK = L.k[1 - P];
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) Sn[qt][0] = Sn[qt][1] = f32x16{};
            // The two waves on a SIMD come from different workgroups and run
            // out of step; raising this wave's issue priority while it
            // interleaves its score products with the exponentials, and
            // dropping it for the P.V products, lets the SIMD favour the phase
            // that feeds both units (8192 x 64 heads: 1131 -> 1088 us per
            // call, identical outputs; priorities 1 to 3 measure alike).
            __builtin_amdgcn_s_setprio(1);
            bf16x8 ka[3][2];  // K operands, read two steps ahead
            ka[0][0] = ld_row_operand(sK, l32, 8 * g);
            ka[0][1] = ld_row_operand(sK, 32 + l32, 8 * g);
            ka[1][0] = ld_row_operand(sK, l32, 16 + 8 * g);
            ka[1][1] = ld_row_operand(sK, 32 + l32, 16 + 8 * g);
            float ps[QT], pv8[QT][8];
            bf16x8 pb[QT][MB / 16];
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) ps[qt] = 0.f;
#pragma unroll
            for (int st = 0; st < MD / 16; ++st) {
                if (st + 2 < MD / 16) {
                    ka[(st + 2) % 3][0] = ld_row_operand(sK, l32, 16 * (st + 2) + 8 * g);
                    ka[(st + 2) % 3][1] = ld_row_operand(sK, 32 + l32, 16 * (st + 2) + 8 * g);
                }
#pragma unroll
                for (int qt = 0; qt < QT; ++qt) {
                    Sn[qt][0] = mfma32(ka[st % 3][0], qb[qt][st], Sn[qt][0]);
                    Sn[qt][1] = mfma32(ka[st % 3][1], qb[qt][st], Sn[qt][1]);
                }
                const int t = st >> 1, m = t >> 1, r0 = 8 * (t & 1) + 4 * (st & 1);
#pragma unroll
                for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const float e =
                            __builtin_amdgcn_exp2f(__builtin_fmaf(Sc[qt][m][r0 + u], sl2, -msc[qt]));
                        pv8[qt][4 * (st & 1) + u] = e;
                        ps[qt] += e;
                    }
                    if (st & 1) {
                        const unsigned p0 = pack_bf16(pv8[qt][0], pv8[qt][1]);
                        const unsigned p1 = pack_bf16(pv8[qt][2], pv8[qt][3]);
                        const unsigned p2 = pack_bf16(pv8[qt][4], pv8[qt][5]);
                        const unsigned p3 = pack_bf16(pv8[qt][6], pv8[qt][7]);
                        const auto x02 = __builtin_amdgcn_permlane32_swap(p0, p2, false, false);
                        const auto x13 = __builtin_amdgcn_permlane32_swap(p1, p3, false, false);
                        pb[qt][t] = __builtin_bit_cast(bf16x8, u32x4{x02[0], x13[0], x02[1], x13[1]});
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) lsum[qt] += ps[qt];
            __builtin_amdgcn_s_setprio(0);
            // O^T += V^T P^T, V operands read three products ahead (LDS latency
            // is what the products wait on here)
            const __bf16* sV = L.v[P];
            constexpr int VA = 4, NPV = (MB / 16) * (MD / 32);
            bf16x8 va[VA];
#pragma unroll
            for (int i = 0; i < VA - 1; ++i) va[i] = ld_tr_operand(sV, 16 * (i >> 2), 32 * (i & 3), lane);
#pragma unroll
            for (int i = 0; i < NPV; ++i) {
                const int t = i >> 2, n = i & 3;
                if (i + VA - 1 < NPV)
                    va[(i + VA - 1) % VA] =
                        ld_tr_operand(sV, 16 * ((i + VA - 1) >> 2), 32 * ((i + VA - 1) & 3), lane);
#pragma unroll
                for (int qt = 0; qt < QT; ++qt) O[qt][n] = mfma32(va[i % VA], pb[qt][t], O[qt][n]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        loads_done();
        __syncthreads();
    };
    for (int b = 0; b < nkb; b += 2) {
        step(std::integral_constant<int, 0>{}, b, Sa, Sb);
        if (b + 1 < nkb) step(std::integral_constant<int, 1>{}, b + 1, Sb, Sa);
    }

    // out = O / sum, lane = query l32 of each sub-tile, features 32 n + 8 jj + 4 g .. + 3
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        const int rows = max(0, min(32, qrows - 32 * qt));
        if (rows > 0) {
            const float inv = 1.f / pair_sum(lsum[qt]);
            const __amdgpu_buffer_rsrc_t ro =
                tile_rsrc(out + (q0w + 32 * qt) * HD + (int64_t)h * MD, rows, HD);
            const int ovoff = (l32 * HD + 4 * g) * 2;
#pragma unroll
            for (int n = 0; n < MD / 32; ++n)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const unsigned lo =
                        pack_bf16(O[qt][n][4 * jj + 0] * inv, O[qt][n][4 * jj + 1] * inv);
                    const unsigned hi =
                        pack_bf16(O[qt][n][4 * jj + 2] * inv, O[qt][n][4 * jj + 3] * inv);
                    __builtin_amdgcn_raw_buffer_store_b64(u32x2{lo, hi}, ro, ovoff,
                                                          (32 * n + 8 * jj) * 2, 0);
                }
        }
    }
}

// ----------------------------------------------------------------- decode
// One decode step against a KV cache (bound by HBM: the cached keys and
// values are read once).  The cache is head-major, [S][H][max_len][128], so
// the keys of one (sequence, head) are one contiguous stream.  Step 1: per sequence, rotate the new key at
// position len and store it with the value at slot len; rotate the query
// (kept in fp32).  Step 2: one 256-thread workgroup per (sequence, head,
// 768-key range): 16 threads per key (8 features each), 16 keys at a time,
// each thread keeping a running maximum, sum and 8 output features over the
// keys it saw; the 16 key slots are merged in LDS into one partial.  Step 3:
// the partials of a (sequence, head) are merged and normalised.
#ifndef LA_SM_DEC_THREADS
#define LA_SM_DEC_THREADS 256
#endif
#ifndef LA_SM_DEC_UNROLL
#define LA_SM_DEC_UNROLL 4
#endif
constexpr int DEC_THREADS = LA_SM_DEC_THREADS;
constexpr int DEC_KEYS = DEC_THREADS / 16;  // keys per pass
constexpr int DEC_UNROLL = LA_SM_DEC_UNROLL;  // passes whose loads are in flight together
static_assert(DEC_THREADS >= MD && DEC_THREADS % 64 == 0, "the merge uses one thread per feature");

__global__ __launch_bounds__(DEC_THREADS) void softmax_append_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    __bf16* __restrict__ kc, __bf16* __restrict__ vc, const int32_t* __restrict__ len,
    float* __restrict__ qr, int32_t* __restrict__ status, int max_len, int H, int rope_dim,
    const RopeTheta th) {
    const int s = blockIdx.x;
    const int L = len[s];
    const bool bad = L < 0 || L >= max_len;
    if (threadIdx.x == 0) status[s] = bad ? 1 : 0;  // written on every call: nothing to clear
    if (bad) return;
    const int HD = H * MD;
    const int64_t src = (int64_t)s * HD;
    for (int e = threadIdx.x * 2; e < HD; e += DEC_THREADS * 2) {
        const int h = e / MD, f = e - h * MD;  // head, feature within it (even)
        const int64_t dst = (((int64_t)s * H + h) * max_len + L) * MD + f;
        float q0 = (float)q[src + e], q1 = (float)q[src + e + 1];
        float k0 = (float)k[src + e], k1 = (float)k[src + e + 1];
        if (f < rope_dim) {
            const float2 r = rope_cs(L, th.t[f / 2]);
            const float a = q0, b = q1;
            q0 = a * r.x - b * r.y;
            q1 = a * r.y + b * r.x;
            const float c = k0, d = k1;
            k0 = c * r.x - d * r.y;
            k1 = c * r.y + d * r.x;
        }
        qr[src + e] = q0;
        qr[src + e + 1] = q1;
        kc[dst] = (__bf16)k0;
        kc[dst + 1] = (__bf16)k1;
        vc[dst] = v[src + e];
        vc[dst + 1] = v[src + e + 1];
    }
}

__global__ __launch_bounds__(DEC_THREADS) void softmax_split_kernel(
    const float* __restrict__ qr, const __bf16* __restrict__ kc, const __bf16* __restrict__ vc,
    const int32_t* __restrict__ len, float* __restrict__ part, int max_len, int H, int nsplit,
    float sl2) {
    __shared__ float sm[DEC_KEYS], sl[DEC_KEYS];
    __shared__ float so[DEC_KEYS][MD + 4];
    const int sp = blockIdx.x % nsplit;
    const int sh = blockIdx.x / nsplit;  // sequence * H + head
    const int s = sh / H, h = sh - s * H;
    const int L = len[s];
    float* pp = part + (int64_t)blockIdx.x * (2 + MD);
    const int j0 = sp * SOFTMAX_DEC_SPLIT;
    const int nk = (L < 0 || L >= max_len) ? 0 : min(SOFTMAX_DEC_SPLIT, L + 1 - j0);
    const int t = threadIdx.x, slot = t >> 4, c = t & 15;
    if (nk <= 0) {  // no keys in this range
        if (t == 0) {
            pp[0] = -INFINITY;
            pp[1] = 0.f;
        }
        return;
    }
    float qv[8];
    {
        const float* qs = qr + (int64_t)sh * MD + 8 * c;
#pragma unroll
        for (int u = 0; u < 8; ++u) qv[u] = qs[u] * sl2;  // logits in base 2
    }
    const int64_t base = ((int64_t)sh * max_len + j0) * MD + 8 * c;
    float m = -INFINITY, l = 0.f, o[8] = {};
    for (int j = slot; j < nk; j += DEC_KEYS * DEC_UNROLL) {
        bf16x8 kk[DEC_UNROLL], vv[DEC_UNROLL];
#pragma unroll
        for (int u = 0; u < DEC_UNROLL; ++u) {
            const int jj = min(j + u * DEC_KEYS, nk - 1);
            kk[u] = __builtin_nontemporal_load(
                reinterpret_cast<const bf16x8*>(kc + base + (int64_t)jj * MD));
            vv[u] = __builtin_nontemporal_load(
                reinterpret_cast<const bf16x8*>(vc + base + (int64_t)jj * MD));
        }
#pragma unroll
        for (int u = 0; u < DEC_UNROLL; ++u) {
            float d = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) d += qv[e] * (float)kk[u][e];
            // sum over the 16 threads of the key
            d += __shfl_xor(d, 1, 16);
            d += __shfl_xor(d, 2, 16);
            d += __shfl_xor(d, 4, 16);
            d += __shfl_xor(d, 8, 16);
            if (j + u * DEC_KEYS < nk) {
                const float mn = fmaxf(m, d);
                const float al = __builtin_amdgcn_exp2f(m - mn);
                const float p = __builtin_amdgcn_exp2f(d - mn);
                l = l * al + p;
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] = o[e] * al + p * (float)vv[u][e];
                m = mn;
            }
        }
    }
    // merge the 16 key slots
    if (c == 0) {
        sm[slot] = m;
        sl[slot] = l;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) so[slot][8 * c + e] = o[e];
    __syncthreads();
    if (t < MD) {
        float M = -INFINITY;
        for (int i = 0; i < DEC_KEYS; ++i) M = fmaxf(M, sm[i]);
        float lt = 0.f, ot = 0.f;
        for (int i = 0; i < DEC_KEYS; ++i) {
            if (sm[i] == -INFINITY) continue;  // a slot that saw no key
            const float w = __builtin_amdgcn_exp2f(sm[i] - M);
            lt += sl[i] * w;
            ot += so[i][t] * w;
        }
        pp[2 + t] = ot;
        if (t == 0) {
            pp[0] = M;
            pp[1] = lt;
        }
    }
}

__global__ __launch_bounds__(MD) void softmax_combine_kernel(const float* __restrict__ part,
                                                             __bf16* __restrict__ out,
                                                             const int32_t* __restrict__ len,
                                                             int max_len, int H, int nsplit) {
    const int sh = blockIdx.x, s = sh / H, t = threadIdx.x;
    const int L = len[s];
    if (L < 0 || L >= max_len) return;  // reported by the append step; out left as it was
    const float* pp = part + (int64_t)sh * nsplit * (2 + MD);
    // only the ranges that hold some of the L + 1 keys (the others hold none)
    const int nused = min(nsplit, L / SOFTMAX_DEC_SPLIT + 1);
    float M = -INFINITY;
#pragma unroll 8
    for (int i = 0; i < nused; ++i) M = fmaxf(M, pp[i * (2 + MD)]);
    float lt = 0.f, ot = 0.f;
#pragma unroll 8
    for (int i = 0; i < nused; ++i) {
        const float mi = pp[i * (2 + MD)];
        if (mi == -INFINITY) continue;
        const float w = __builtin_amdgcn_exp2f(mi - M);
        lt += pp[i * (2 + MD) + 1] * w;
        ot += pp[i * (2 + MD) + 2 + t] * w;
    }
    out[(int64_t)sh * MD + t] = (__bf16)(ot / lt);
}

}  // namespace

hipError_t launch_softmax_decode(const SoftmaxDecodeArgs& a, hipStream_t st) {
    if (a.nseq == 0) return hipSuccess;
    SoftmaxArgs ra{};
    ra.rope_dim = a.rope_dim;
    ra.rope_base = a.rope_base;
    hipLaunchKernelGGL(softmax_append_kernel, dim3((unsigned)a.nseq), dim3(DEC_THREADS), 0, st,
                       (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v,
                       (__bf16*)a.k_cache, (__bf16*)a.v_cache, a.len, a.qr, a.status, a.max_len,
                       a.H, a.rope_dim, rope_theta(ra));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t blocks = (int64_t)a.nseq * a.H * a.nsplit;
    hipLaunchKernelGGL(softmax_split_kernel, dim3((unsigned)blocks), dim3(DEC_THREADS), 0, st,
                       a.qr, (const __bf16*)a.k_cache, (const __bf16*)a.v_cache, a.len, a.part,
                       a.max_len, a.H, a.nsplit, a.scale * 1.4426950408889634f);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(softmax_combine_kernel, dim3((unsigned)(a.nseq * a.H)), dim3(MD), 0, st,
                       a.part, (__bf16*)a.out, a.len, a.max_len, a.H, a.nsplit);
    return hipGetLastError();
}

hipError_t launch_softmax_rope(const SoftmaxArgs& a, hipStream_t st) {
    if (a.max_tiles == 0) return hipSuccess;
    const dim3 grid((unsigned)((int64_t)a.max_tiles * (SOFTMAX_TILE / ROPE_TOKENS)));
    hipLaunchKernelGGL(rope_kernel, grid, dim3(ROPE_THREADS), 0, st, (const __bf16*)a.k, a.kr,
                       a.hdr, a.segs, a.tiles, a.H, a.rope_dim, rope_theta(a));
    return hipGetLastError();
}

hipError_t launch_softmax_fwd(const SoftmaxArgs& a, hipStream_t st) {
    if (a.max_tiles == 0) return hipSuccess;
    const dim3 grid((unsigned)((int64_t)a.max_tiles * a.H));
    const __bf16* kk = a.rope_dim > 0 ? a.kr : (const __bf16*)a.k;
    hipLaunchKernelGGL((softmax_fwd_kernel<FA_QT, FA_NW>), grid, dim3(64 * FA_NW), 0, st,
                       (const __bf16*)a.q, kk,
                       (const __bf16*)a.v, (__bf16*)a.out, a.hdr, a.segs, a.tiles, a.H,
                       a.scale * 1.4426950408889634f, a.rope_dim, rope_theta(a));
    return hipGetLastError();
}

}  // namespace la
