// Single-token decode step of the Lightning Attention layer.
//
// With Mechanism step 3 of "Diving into MiniMax01 405B MoE" (section "Hybrid
// Modeling") read causally, the layer keeps one D x D state per head and a
// new token costs O(d^2): S += k~^T v~, then y = q~ S (the token sees itself),
// then step 4's RMSNorm over the token's H*D values times sigmoid(gate).
//
// The step is bound by HBM: the fp32 state (64 KiB per head at D = 128) is
// read and written once.  Kernel 1 streams the state of one (sequence, head)
// at a time per workgroup with 16-byte accesses, each thread keeping many
// loads in flight, and leaves y and the head's sum of squares in the
// workspace; kernel 2 applies the norm and gate per sequence.
#include "la_internal.h"

namespace la {

constexpr int DEC_THREADS = 1024;

template <class TT, int D>
__global__ __launch_bounds__(DEC_THREADS) void decode_state_kernel(
    const TT* __restrict__ q, const TT* __restrict__ k, const TT* __restrict__ v,
    float* __restrict__ state, float* __restrict__ ybuf, float* __restrict__ ssbuf,
    int64_t pairs) {
    constexpr int TPR = D / 4;               // threads per state row (4 columns each)
    constexpr int NRG = DEC_THREADS / TPR;   // row groups
    constexpr int RPT = (D + NRG - 1) / NRG; // rows per thread
    __shared__ float qs[D], ks[D], vs[D];
    __shared__ f32x4 red[NRG][TPR];
    __shared__ float wsum[DEC_THREADS / 64];
    const int tid = threadIdx.x;
    const int cq = tid % TPR, rg = tid / TPR;
    const int j0 = cq * 4;
    // a fixed set of workgroups (one per CU) walks over the (sequence, head)
    // pairs: long-lived workgroups keep the memory pipeline fuller than one
    // short workgroup per pair
    for (int64_t pair = blockIdx.x; pair < pairs; pair += gridDim.x) {  // sequence * H + head
        f32x4* S = reinterpret_cast<f32x4*>(state + pair * D * D);
        f32x4 rows[RPT];
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int i = rg + m * NRG;
            if (i < D) rows[m] = __builtin_nontemporal_load(&S[i * TPR + cq]);
        }
        if (tid < D) {
            const int64_t idx = pair * D + tid;
            qs[tid] = silu_f(to_f32(q[idx]));
            ks[tid] = silu_f(to_f32(k[idx]));
            vs[tid] = silu_f(to_f32(v[idx]));
        }
        __syncthreads();
        const f32x4 vj = {vs[j0], vs[j0 + 1], vs[j0 + 2], vs[j0 + 3]};
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int i = rg + m * NRG;
            if (i < D) {
                const f32x4 s = rows[m] + ks[i] * vj;
                __builtin_nontemporal_store(s, &S[i * TPR + cq]);
                y += qs[i] * s;
            }
        }
        red[rg][cq] = y;
        __syncthreads();
        float sq = 0.f;
        if (tid < D) {
            float yj = 0.f;
            for (int r = 0; r < NRG; ++r) yj += red[r][tid / 4][tid % 4];
            ybuf[pair * D + tid] = yj;
            sq = yj * yj;
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) sq += __shfl_xor(sq, off);
        if ((tid & 63) == 0) wsum[tid >> 6] = sq;
        __syncthreads();
        if (tid == 0) {
            float t = 0.f;
            for (int i = 0; i < DEC_THREADS / 64; ++i) t += wsum[i];
            ssbuf[pair] = t;
        }
        // qs/ks/vs, red and wsum are rewritten for the next pair
        __syncthreads();
    }
}

template <class TT>
__global__ __launch_bounds__(DEC_THREADS) void decode_norm_kernel(
    const TT* __restrict__ g, const TT* __restrict__ w, TT* __restrict__ out,
    const float* __restrict__ ybuf, const float* __restrict__ ssbuf, int H, int HD, float eps) {
    __shared__ float wsum[DEC_THREADS / 64];
    const int64_t s = blockIdx.x;
    float ss = 0.f;
    for (int h = threadIdx.x; h < H; h += DEC_THREADS) ss += ssbuf[s * H + h];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
    if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
    for (int i = 0; i < DEC_THREADS / 64; ++i) tot += wsum[i];
    const float r = 1.0f / __builtin_sqrtf(tot / (float)HD + eps);
    for (int e = threadIdx.x; e < HD; e += DEC_THREADS) {
        const int64_t idx = s * HD + e;
        out[idx] = from_f32<TT>(ybuf[idx] * r * to_f32(w[e]) * sigmoid_f(to_f32(g[idx])));
    }
}

// Workgroups of the state kernel: one per CU, each looping over pairs
// (measured on MI355X: 1024-thread workgroups, one per CU, stream the state
// faster than more or smaller workgroups).
static int cu_count() {
    static int cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

template <class TT, int D>
static hipError_t decode_state_d(const DecodeArgs& a, hipStream_t st) {
    const int64_t pairs = (int64_t)a.nseq * a.H;
    const int64_t ncu = cu_count();
    const unsigned grid = (unsigned)(pairs < ncu ? pairs : ncu);
    hipLaunchKernelGGL((decode_state_kernel<TT, D>), dim3(grid), dim3(DEC_THREADS), 0, st,
                       (const TT*)a.q, (const TT*)a.k, (const TT*)a.v, a.state, a.ybuf, a.ssbuf,
                       pairs);
    return hipGetLastError();
}

template <class TT>
static hipError_t decode_state_t(const DecodeArgs& a, hipStream_t st) {
    switch (a.D) {
        case 16: return decode_state_d<TT, 16>(a, st);
        case 32: return decode_state_d<TT, 32>(a, st);
        case 64: return decode_state_d<TT, 64>(a, st);
        case 128: return decode_state_d<TT, 128>(a, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_decode_state(const DecodeArgs& a, hipStream_t st) {
    if (a.nseq == 0) return hipSuccess;
    return a.bf16 ? decode_state_t<__bf16>(a, st) : decode_state_t<float>(a, st);
}

hipError_t launch_decode_norm(const DecodeArgs& a, hipStream_t st) {
    if (a.nseq == 0) return hipSuccess;
    if (a.bf16)
        hipLaunchKernelGGL((decode_norm_kernel<__bf16>), dim3((unsigned)a.nseq), dim3(DEC_THREADS),
                           0, st, (const __bf16*)a.g, (const __bf16*)a.w, (__bf16*)a.out, a.ybuf,
                           a.ssbuf, a.H, a.H * a.D, a.eps);
    else
        hipLaunchKernelGGL((decode_norm_kernel<float>), dim3((unsigned)a.nseq), dim3(DEC_THREADS),
                           0, st, (const float*)a.g, (const float*)a.w, (float*)a.out, a.ybuf,
                           a.ssbuf, a.H, a.H * a.D, a.eps);
    return hipGetLastError();
}

}  // namespace la
