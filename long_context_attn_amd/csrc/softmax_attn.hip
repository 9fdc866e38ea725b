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
//  - rope_kernel: rotates q and k once into bf16 copies in the workspace
//    (HBM-bound; the angles are reduced in fp64, so positions up to 2^31 keep
//    full fp32 accuracy);
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

#include "la_internal.h"
#include "mfma_common.h"

namespace la {

namespace {

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ rope
constexpr int ROPE_THREADS = 256;
constexpr int ROPE_TOKENS = 16;  // tokens per workgroup
constexpr int ROPE_MAX_PAIRS = 64;

// Workgroup (tile c, group j): tokens 16 j .. 16 j + 15 of tile c.  Each
// token's cos / sin table is built once in LDS and serves all of its heads.
__global__ __launch_bounds__(ROPE_THREADS) void rope_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, __bf16* __restrict__ qr,
    __bf16* __restrict__ kr, const PlanHeader* __restrict__ hdr, const SegEntry* __restrict__ segs,
    const ChunkEntry* __restrict__ tiles, int H, int rope_dim, double log2_base) {
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
    const double two_pi = 6.283185307179586476925286766559;
    for (int i = threadIdx.x; i < ROPE_TOKENS * npairs; i += ROPE_THREADS) {
        const int t = i / npairs, p = i - t * npairs;
        // theta_p = base^(-2p / rope_dim); angle reduced to [-pi, pi] in fp64
        const double theta = exp2(-(2.0 * p / rope_dim) * log2_base);
        double a = (double)(pos0 + t) * theta;
        a -= two_pi * rint(a / two_pi);
        float sn, cn;
        sincosf((float)a, &sn, &cn);
        cs[t][p] = make_float2(cn, sn);
    }
    __syncthreads();
    const int HD = H * MD;
    const int per_token = HD / 8;  // 16-byte pieces of one token
    const int64_t n = (int64_t)nt * per_token;
    for (int64_t i = threadIdx.x; i < 2 * n; i += ROPE_THREADS) {
        const bool isk = i >= n;
        const int64_t e = isk ? i - n : i;
        const int t = (int)(e / per_token);
        const int piece = (int)(e - (int64_t)t * per_token);
        const int f = (piece % (MD / 8)) * 8;  // first feature of the piece within its head
        const int64_t off = (first + t) * HD + (int64_t)piece * 8;
        bf16x8 x = *reinterpret_cast<const bf16x8*>((isk ? k : q) + off);
        if (f < rope_dim) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float2 r = cs[t][f / 2 + u];
                const float a = (float)x[2 * u], b = (float)x[2 * u + 1];
                x[2 * u] = (__bf16)(a * r.x - b * r.y);
                x[2 * u + 1] = (__bf16)(a * r.y + b * r.x);
            }
        }
        *reinterpret_cast<bf16x8*>((isk ? kr : qr) + off) = x;
    }
}

// --------------------------------------------------------- attention
constexpr int FA_THREADS = 256;  // four waves, 32 queries each

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

__global__ __launch_bounds__(FA_THREADS, 2) void softmax_fwd_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    __bf16* __restrict__ out, const PlanHeader* __restrict__ hdr,
    const SegEntry* __restrict__ segs, const ChunkEntry* __restrict__ tiles, int H, float sl2) {
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
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
    const int64_t qend = qstart + qlen;
    const int nkb = (int)((qend - s0 + MB - 1) / MB);

    // this wave's queries: Q^T operands, lane = query l32, features 16 s + 8 g .. + 7
    const int64_t q0w = qstart + 32 * w;
    const int qrows = max(0, min(32, qlen - 32 * w));
    bf16x8 qb[MD / 16];
    {
        const __amdgpu_buffer_rsrc_t rs = tile_rsrc(q + q0w * HD + (int64_t)h * MD, qrows, HD);
        const int voff = (l32 * HD + 8 * g) * 2;
#pragma unroll
        for (int s = 0; s < MD / 16; ++s)
            qb[s] = __builtin_bit_cast(bf16x8,
                                       __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 32 * s, 0));
    }

    // K / V tiles: thread loads rows 4 rg .. 4 rg + 3, features 8 cc .. + 7
    const int cc = tid & 15, rg = tid >> 4;
    const int voff = (4 * rg * HD + 8 * cc) * 2, rstride = HD * 2;
    auto load_kv = [&](int b, Tile& tk, Tile& tv) {
        const int64_t kb0 = s0 + (int64_t)min(b, nkb - 1) * MB;
        const int n = b < nkb ? (int)min((int64_t)MB, qend - kb0) : 0;
        const int64_t off = kb0 * HD + (int64_t)h * MD;
        load_tile(tk, tile_rsrc(k + off, n, HD), voff, rstride);
        load_tile(tv, tile_rsrc(v + off, n, HD), voff, rstride);
    };
    Tile tk, tv;
    load_kv(0, tk, tv);
    store_rows(tk.r, L.k[0], cc, rg);
    store_rows(tv.r, L.v[0], cc, rg);
    load_kv(1, tk, tv);
    __syncthreads();

    f32x16 O[MD / 32] = {};
    float mrun = -INFINITY, lsum = 0.f;
    const int64_t qabs = q0w + l32;  // this lane's query
    for (int b = 0; b < nkb; ++b) {
        const __bf16* sK = L.k[b & 1];
        const __bf16* sV = L.v[b & 1];
        const int64_t kb0 = s0 + (int64_t)b * MB;
        // a wave whose queries all precede the block has nothing to add
        if (qrows > 0 && q0w + qrows - 1 >= kb0) {
            f32x16 S[2] = {};
#pragma unroll
            for (int s = 0; s < MD / 16; ++s)
#pragma unroll
                for (int m = 0; m < 2; ++m)
                    S[m] = mfma32(ld_row_operand(sK, 32 * m + l32, 16 * s + 8 * g), qb[s], S[m]);
            // logits in base 2; keys after the query masked out
            const bool diag = kb0 + MB - 1 > q0w;
            float bm = -INFINITY;
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float x = S[m][r] * sl2;
                    if (diag && kb0 + 32 * m + 8 * (r >> 2) + 4 * g + (r & 3) > qabs) x = -INFINITY;
                    S[m][r] = x;
                    bm = fmaxf(bm, x);
                }
            const float mnew = fmaxf(mrun, pair_max(bm));
            const float alpha = __builtin_amdgcn_exp2f(mrun - mnew);
            mrun = mnew;
            float ps = 0.f;
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = __builtin_amdgcn_exp2f(S[m][r] - mnew);
                    S[m][r] = p;
                    ps += p;
                }
            lsum = lsum * alpha + ps;
#pragma unroll
            for (int n = 0; n < MD / 32; ++n)
#pragma unroll
                for (int r = 0; r < 16; ++r) O[n][r] *= alpha;
            // O^T += V^T P^T, 16 keys at a time: accumulator registers
            // r0 .. r0 + 7 of tile m hold keys 16 s + 8 (j / 4) + 4 g + j % 4;
            // one swap between the lane halves makes them keys 16 s + 8 g + j
#pragma unroll
            for (int s = 0; s < MB / 16; ++s) {
                const int m = s >> 1, r0 = 8 * (s & 1);
                const unsigned p0 = pack_bf16(S[m][r0 + 0], S[m][r0 + 1]);
                const unsigned p1 = pack_bf16(S[m][r0 + 2], S[m][r0 + 3]);
                const unsigned p2 = pack_bf16(S[m][r0 + 4], S[m][r0 + 5]);
                const unsigned p3 = pack_bf16(S[m][r0 + 6], S[m][r0 + 7]);
                const auto x02 = __builtin_amdgcn_permlane32_swap(p0, p2, false, false);
                const auto x13 = __builtin_amdgcn_permlane32_swap(p1, p3, false, false);
                const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{x02[0], x13[0], x02[1], x13[1]});
#pragma unroll
                for (int n = 0; n < MD / 32; ++n)
                    O[n] = mfma32(ld_tr_operand(sV, 16 * s, 32 * n, lane), pb, O[n]);
            }
        }
        // stage block b + 1 (loaded during block b - 1) and fetch block b + 2;
        // every wave finished block b - 1, which used the same buffers, before
        // the last barrier
        if (b + 1 < nkb) {
            store_rows(tk.r, L.k[(b + 1) & 1], cc, rg);
            store_rows(tv.r, L.v[(b + 1) & 1], cc, rg);
        }
        load_kv(b + 2, tk, tv);
        __syncthreads();
    }

    // out = O / sum, lane = query l32, features 32 n + 8 jj + 4 g .. + 3
    if (qrows > 0) {
        const float inv = 1.f / pair_sum(lsum);
        const __amdgpu_buffer_rsrc_t ro = tile_rsrc(out + q0w * HD + (int64_t)h * MD, qrows, HD);
        const int ovoff = (l32 * HD + 4 * g) * 2;
#pragma unroll
        for (int n = 0; n < MD / 32; ++n)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const unsigned lo = pack_bf16(O[n][4 * jj + 0] * inv, O[n][4 * jj + 1] * inv);
                const unsigned hi = pack_bf16(O[n][4 * jj + 2] * inv, O[n][4 * jj + 3] * inv);
                __builtin_amdgcn_raw_buffer_store_b64(u32x2{lo, hi}, ro, ovoff,
                                                      (32 * n + 8 * jj) * 2, 0);
            }
    }
}

}  // namespace

hipError_t launch_softmax_rope(const SoftmaxArgs& a, hipStream_t st) {
    if (a.max_tiles == 0) return hipSuccess;
    const dim3 grid((unsigned)((int64_t)a.max_tiles * (SOFTMAX_TILE / ROPE_TOKENS)));
    hipLaunchKernelGGL(rope_kernel, grid, dim3(ROPE_THREADS), 0, st, (const __bf16*)a.q,
                       (const __bf16*)a.k, a.qr, a.kr, a.hdr, a.segs, a.tiles, a.H, a.rope_dim,
                       log2(a.rope_base));
    return hipGetLastError();
}

hipError_t launch_softmax_fwd(const SoftmaxArgs& a, hipStream_t st) {
    if (a.max_tiles == 0) return hipSuccess;
    const dim3 grid((unsigned)((int64_t)a.max_tiles * a.H));
    const __bf16* qq = a.rope_dim > 0 ? a.qr : (const __bf16*)a.q;
    const __bf16* kk = a.rope_dim > 0 ? a.kr : (const __bf16*)a.k;
    hipLaunchKernelGGL(softmax_fwd_kernel, grid, dim3(FA_THREADS), 0, st, qq, kk,
                       (const __bf16*)a.v, (__bf16*)a.out, a.hdr, a.segs, a.tiles, a.H,
                       a.scale * 1.4426950408889634f);
    return hipGetLastError();
}

}  // namespace la
