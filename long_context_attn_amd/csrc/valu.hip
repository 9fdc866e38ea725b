// Portable fp32 vector-ALU kernels of the Lightning Attention layer: any
// supported head_dim / block, fp32 or bf16 storage.  They are the exact-
// arithmetic path for fp32 inputs (every product and sum in fp32).
//
// Mechanism step 3 of "Diving into MiniMax01 405B MoE" (section "Hybrid
// Modeling"), Y = Q (K^T V), is evaluated blockwise inside a chunk:
//   Y_b = (Q~_b K~_b^T (.) M) V~_b + Q~_b S,   S <- S + K~_b^T V~_b,
// M lower triangular with the diagonal (causal, the token sees itself).
//
// One workgroup of D threads per (chunk, head); thread j owns column j of the
// D x D fp32 state (D registers).
#include "la_internal.h"

namespace la {

constexpr int STATE_TILE = 16;  // tokens staged per step of the chunk-state kernel

// Per-chunk state sum K~_c^T V~_c into states[c][h].
template <class TT, int D>
__global__ __launch_bounds__(D) void chunk_state_valu_kernel(
    const TT* __restrict__ k, const TT* __restrict__ v, const PlanHeader* __restrict__ hdr,
    const ChunkEntry* __restrict__ chunks, float* __restrict__ states, int H) {
    __shared__ float ks[STATE_TILE][D];
    __shared__ float vs[STATE_TILE][D];
    const int c = blockIdx.x / H, h = blockIdx.x - (blockIdx.x / H) * H;
    if (c >= hdr->n_chunks) return;
    const ChunkEntry ce = chunks[c];
    const int j = threadIdx.x;
    const int64_t HD = (int64_t)H * D;
    float acc[D];
#pragma unroll
    for (int i = 0; i < D; ++i) acc[i] = 0.f;
    for (int t0 = 0; t0 < ce.len; t0 += STATE_TILE) {
        const int n = min(STATE_TILE, ce.len - t0);
        for (int a = 0; a < STATE_TILE; ++a) {
            const int64_t idx = (ce.start + t0 + a) * HD + (int64_t)h * D + j;
            ks[a][j] = a < n ? silu_f(to_f32(k[idx])) : 0.f;
            vs[a][j] = a < n ? silu_f(to_f32(v[idx])) : 0.f;
        }
        __syncthreads();
        for (int a = 0; a < n; ++a) {
            const float vj = vs[a][j];
#pragma unroll
            for (int i = 0; i < D; ++i) acc[i] += ks[a][i] * vj;
        }
        __syncthreads();
    }
    float* dst = states + ((int64_t)c * H + h) * D * D;
#pragma unroll
    for (int i = 0; i < D; ++i) dst[i * D + j] = acc[i];
}

// Chunk walk: starts from the state entering the chunk (states[c][h] after
// the scan) and writes the raw attention output y of every token to `out`.
template <class TT, int D, int BK>
__global__ __launch_bounds__(D) void walk_valu_kernel(
    const TT* __restrict__ q, const TT* __restrict__ k, const TT* __restrict__ v,
    TT* __restrict__ out, const PlanHeader* __restrict__ hdr,
    const ChunkEntry* __restrict__ chunks, const float* __restrict__ states, int H) {
    extern __shared__ float lds[];
    float* qs = lds;              // [BK][D]
    float* ks = qs + BK * D;      // [BK][D]
    float* vs = ks + BK * D;      // [BK][D]
    float* sc = vs + BK * D;      // [BK][BK] scores q~_a . k~_b
    const int c = blockIdx.x / H, h = blockIdx.x - (blockIdx.x / H) * H;
    if (c >= hdr->n_chunks) return;
    const ChunkEntry ce = chunks[c];
    const int j = threadIdx.x;
    const int64_t HD = (int64_t)H * D;
    float S[D];
    const float* src = states + ((int64_t)c * H + h) * D * D;
#pragma unroll
    for (int i = 0; i < D; ++i) S[i] = src[i * D + j];
    for (int t0 = 0; t0 < ce.len; t0 += BK) {
        const int n = min(BK, ce.len - t0);
        for (int a = 0; a < BK; ++a) {
            const int64_t idx = (ce.start + t0 + a) * HD + (int64_t)h * D + j;
            const bool ok = a < n;
            qs[a * D + j] = ok ? silu_f(to_f32(q[idx])) : 0.f;
            ks[a * D + j] = ok ? silu_f(to_f32(k[idx])) : 0.f;
            vs[a * D + j] = ok ? silu_f(to_f32(v[idx])) : 0.f;
        }
        __syncthreads();
        // intra-block scores for b <= a (masked entries are never read)
        for (int p = j; p < BK * BK; p += D) {
            const int a = p / BK, b = p - (p / BK) * BK;
            float s = 0.f;
            if (b <= a && a < n) {
                for (int i = 0; i < D; ++i) s += qs[a * D + i] * ks[b * D + i];
            }
            sc[p] = s;
        }
        __syncthreads();
        for (int a = 0; a < n; ++a) {
            float y = 0.f;
#pragma unroll
            for (int i = 0; i < D; ++i) y += qs[a * D + i] * S[i];  // inter-block
            for (int b = 0; b <= a; ++b) y += sc[a * BK + b] * vs[b * D + j];  // intra-block
            out[(ce.start + t0 + a) * HD + (int64_t)h * D + j] = from_f32<TT>(y);
        }
        // state update after the block's outputs used the state before it
        for (int a = 0; a < n; ++a) {
            const float vj = vs[a * D + j];
#pragma unroll
            for (int i = 0; i < D; ++i) S[i] += ks[a * D + i] * vj;
        }
        __syncthreads();
    }
}

template <class TT, int D>
static hipError_t chunk_state_d(const PrefillArgs& a, hipStream_t st) {
    const dim3 grid((unsigned)((int64_t)a.max_chunks * a.H));
    hipLaunchKernelGGL((chunk_state_valu_kernel<TT, D>), grid, dim3(D), 0, st, (const TT*)a.k,
                       (const TT*)a.v, a.hdr, a.chunks, a.states, a.H);
    return hipGetLastError();
}

template <class TT>
static hipError_t chunk_state_t(const PrefillArgs& a, hipStream_t st) {
    switch (a.D) {
        case 16: return chunk_state_d<TT, 16>(a, st);
        case 32: return chunk_state_d<TT, 32>(a, st);
        case 64: return chunk_state_d<TT, 64>(a, st);
        case 128: return chunk_state_d<TT, 128>(a, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_chunk_state_valu(const PrefillArgs& a, hipStream_t st) {
    if (a.max_chunks == 0) return hipSuccess;
    return a.bf16 ? chunk_state_t<__bf16>(a, st) : chunk_state_t<float>(a, st);
}

template <class TT, int D, int BK>
static hipError_t walk_db(const PrefillArgs& a, hipStream_t st) {
    const dim3 grid((unsigned)((int64_t)a.max_chunks * a.H));
    const size_t lds = sizeof(float) * (3 * BK * D + BK * BK);
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute(
            reinterpret_cast<const void*>(&walk_valu_kernel<TT, D, BK>),
            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((walk_valu_kernel<TT, D, BK>), grid, dim3(D), lds, st, (const TT*)a.q,
                       (const TT*)a.k, (const TT*)a.v, (TT*)a.out, a.hdr, a.chunks, a.states,
                       a.H);
    return hipGetLastError();
}

template <class TT, int D>
static hipError_t walk_d(const PrefillArgs& a, hipStream_t st) {
    switch (a.block) {
        case 16: return walk_db<TT, D, 16>(a, st);
        case 32: return walk_db<TT, D, 32>(a, st);
        case 64: return walk_db<TT, D, 64>(a, st);
    }
    return hipErrorInvalidValue;
}

template <class TT>
static hipError_t walk_t(const PrefillArgs& a, hipStream_t st) {
    switch (a.D) {
        case 16: return walk_d<TT, 16>(a, st);
        case 32: return walk_d<TT, 32>(a, st);
        case 64: return walk_d<TT, 64>(a, st);
        case 128: return walk_d<TT, 128>(a, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_walk_valu(const PrefillArgs& a, hipStream_t st) {
    if (a.max_chunks == 0) return hipSuccess;
    return a.bf16 ? walk_t<__bf16>(a, st) : walk_t<float>(a, st);
}

}  // namespace la
