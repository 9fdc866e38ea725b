// Chunk plan, per-sequence state scan and the RMSNorm * sigmoid(gate)
// epilogue of the Lightning Attention layer.
//
// The running state of Mechanism step 3 ("Diving into MiniMax01 405B MoE",
// section "Hybrid Modeling") is a sum over past tokens, so a sequence can be
// cut into chunks: the state entering chunk c is the exclusive prefix sum of
// the per-chunk sums K~_c^T V~_c (plus the initial state).  The epilogue is
// Mechanism step 4, RMSNorm over all heads*head_dim values of a token.
#include "la_internal.h"

namespace la {

// ------------------------------------------------------------------- plan
// Workgroup 0 (1024 threads): chunk counts per sequence, exclusive scan,
// then each thread writes the chunk records of its sequences (none when
// `chunks` is null: only the count is wanted).  The other
// workgroups zero the words the MFMA prefills expect cleared on every call
// (chunk-state flags and RMSNorm exchange words).
constexpr int PLAN_THREADS = 1024;
constexpr int CLEAR_BLOCKS = 256;

// the workgroup as plan_sequences sees it
struct PlanDevCtx {
    int64_t* scan;
    int32_t* bad;
    int32_t* err;
    __device__ int tid() const { return threadIdx.x; }
    __device__ void sync() const { __syncthreads(); }
};

__global__ __launch_bounds__(PLAN_THREADS) void plan_kernel(
    const int32_t* __restrict__ cu, int nseq, int64_t seqlen, int64_t total, int chunk,
    int max_chunks, PlanHeader* __restrict__ hdr, SegEntry* __restrict__ segs,
    ChunkEntry* __restrict__ chunks, uint64_t* __restrict__ clear, int64_t clear_words) {
    if (blockIdx.x > 0) {
        const int64_t stride = (int64_t)(gridDim.x - 1) * PLAN_THREADS;
        for (int64_t i = (int64_t)(blockIdx.x - 1) * PLAN_THREADS + threadIdx.x; i < clear_words;
             i += stride)
            clear[i] = 0;
        return;
    }
    __shared__ int64_t scan[PLAN_THREADS];
    __shared__ int32_t bad, err;
    plan_sequences<PLAN_THREADS>(PlanDevCtx{scan, &bad, &err}, cu, nseq, seqlen, total, chunk,
                                 max_chunks, hdr, segs, chunks);
}

hipError_t launch_plan(const PrefillArgs& a, hipStream_t st) {
    int64_t blocks = (a.clear_words + PLAN_THREADS - 1) / PLAN_THREADS;
    if (blocks > CLEAR_BLOCKS) blocks = CLEAR_BLOCKS;
    hipLaunchKernelGGL(plan_kernel, dim3((unsigned)(1 + blocks)), dim3(PLAN_THREADS), 0, st, a.cu,
                       a.nseq, a.seqlen, a.total, a.chunk, a.max_chunks, a.hdr, a.segs, a.chunks,
                       a.clear, a.clear_words);
    return hipGetLastError();
}

// ------------------------------------------------------------- state scan
// One thread per 4 state entries of one (sequence, head): walks the
// sequence's chunks in order, replacing each chunk sum by the state that
// enters the chunk, and stores the state after the last chunk.  With
// skip_last the last chunk of a sequence has no sum (only its entering
// state is written, and no final state).  For uniform rows on the MFMA path
// the scan also zeroes the walk's exchange words (`clear`): done here, after
// the chunk sums, the 5.6 MB of stores at 8192 x 64 heads no longer compete
// with the chunk sums' reads (3-4 us less per prefill).
constexpr int SCAN_THREADS = 256;

__global__ __launch_bounds__(SCAN_THREADS) void state_scan_kernel(
    float* __restrict__ states, const SegEntry* __restrict__ segs, const float* init,
    float* fin, int H, int DD, int tiles, bool skip_last, uint64_t* __restrict__ clear,
    int64_t clear_words) {
    {
        const int64_t stride = (int64_t)gridDim.x * SCAN_THREADS;
        for (int64_t i = (int64_t)blockIdx.x * SCAN_THREADS + threadIdx.x; i < clear_words;
             i += stride)
            clear[i] = 0;
    }
    const int pair = blockIdx.x / tiles;  // sequence * H + head
    const int tile = blockIdx.x - pair * tiles;
    const int e = (tile * SCAN_THREADS + threadIdx.x) * 4;
    if (e >= DD) return;
    const int s = pair / H, h = pair - s * H;
    f32x4 run = {0.f, 0.f, 0.f, 0.f};
    if (init != nullptr) run = *reinterpret_cast<const f32x4*>(init + (int64_t)pair * DD + e);
    const SegEntry se = segs[s];
    const int end = se.first + se.count;
    for (int c = se.first; c < end; ++c) {
        f32x4* p = reinterpret_cast<f32x4*>(states + ((int64_t)c * H + h) * DD + e);
        if (skip_last && c == end - 1) {
            *p = run;
            break;
        }
        const f32x4 sum = *p;
        *p = run;
        run += sum;
    }
    if (fin != nullptr && !skip_last) *reinterpret_cast<f32x4*>(fin + (int64_t)pair * DD + e) = run;
}

hipError_t launch_state_scan(const PrefillArgs& a, hipStream_t st) {
    const int DD = a.D * a.D;
    const int tiles = (DD / 4 + SCAN_THREADS - 1) / SCAN_THREADS;
    const int64_t grid = (int64_t)a.nseq * a.H * tiles;
    if (grid == 0) return hipSuccess;
    // uniform rows on the MFMA path: the chunk-sum kernel wrote the plan but
    // left the exchange words to this kernel
    const bool clr = a.inline_plan && a.clear != nullptr;
    hipLaunchKernelGGL(state_scan_kernel, dim3((unsigned)grid), dim3(SCAN_THREADS), 0, st,
                       a.states, a.segs, a.init_state, a.final_state, a.H, DD, tiles,
                       a.skip_last, clr ? a.clear : nullptr, clr ? a.clear_words : (int64_t)0);
    return hipGetLastError();
}

// ------------------------------------------------------ norm * gate epilogue
// One workgroup per token.  `out` holds the raw attention output y of the
// token on entry; it is overwritten with y * r * w * sigmoid(g), r =
// 1/sqrt(mean(y^2) + eps) over the token's H*D values.
constexpr int NORM_THREADS = 256;

__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int i = 0; i < NORM_THREADS / 64; ++i) tot += red[i];
    return tot;
}

// any dtype and H*D: one element per thread per step, y re-read from `out`
template <class TT>
__global__ __launch_bounds__(NORM_THREADS) void norm_gate_kernel(
    TT* __restrict__ out, const TT* __restrict__ g, const TT* __restrict__ w, int HD, float eps) {
    __shared__ float red[NORM_THREADS / 64];
    const int64_t base = (int64_t)blockIdx.x * HD;
    TT* y = out + base;
    const TT* gt = g + base;
    float ss = 0.f;
    for (int e = threadIdx.x; e < HD; e += NORM_THREADS) {
        const float t = to_f32(y[e]);
        ss += t * t;
    }
    const float r = 1.0f / __builtin_sqrtf(block_sum(ss, red) / (float)HD + eps);
    for (int e = threadIdx.x; e < HD; e += NORM_THREADS)
        y[e] = from_f32<TT>(to_f32(y[e]) * r * to_f32(w[e]) * sigmoid_f(to_f32(gt[e])));
}

// bf16 with H*D a multiple of 8 * NORM_THREADS and at most NV such vectors
// per thread: y stays in registers between the reduction and the epilogue.
template <int NV>
__global__ __launch_bounds__(NORM_THREADS) void norm_gate_bf16_kernel(
    __bf16* __restrict__ out, const __bf16* __restrict__ g, const __bf16* __restrict__ w, int HD,
    float eps) {
    __shared__ float red[NORM_THREADS / 64];
    const int64_t base = (int64_t)blockIdx.x * HD;
    bf16x8* y = reinterpret_cast<bf16x8*>(out + base);
    const bf16x8* gt = reinterpret_cast<const bf16x8*>(g + base);
    const bf16x8* wv = reinterpret_cast<const bf16x8*>(w);
    const int nvec = HD / (8 * NORM_THREADS);
    bf16x8 yv[NV], gv[NV];
    float ss = 0.f;
#pragma unroll
    for (int r = 0; r < NV; ++r) {
        if (r < nvec) {
            yv[r] = y[r * NORM_THREADS + threadIdx.x];
            gv[r] = gt[r * NORM_THREADS + threadIdx.x];
#pragma unroll
            for (int u = 0; u < 8; ++u) ss += (float)yv[r][u] * (float)yv[r][u];
        }
    }
    const float rr = 1.0f / __builtin_sqrtf(block_sum(ss, red) / (float)HD + eps);
#pragma unroll
    for (int r = 0; r < NV; ++r) {
        if (r < nvec) {
            const bf16x8 ww = wv[r * NORM_THREADS + threadIdx.x];
            bf16x8 o;
#pragma unroll
            for (int u = 0; u < 8; ++u)
                o[u] = (__bf16)((float)yv[r][u] * rr * (float)ww[u] * sigmoid_f((float)gv[r][u]));
            y[r * NORM_THREADS + threadIdx.x] = o;
        }
    }
}

hipError_t launch_norm_gate(const PrefillArgs& a, hipStream_t st) {
    const int HD = a.H * a.D;
    if (a.total == 0) return hipSuccess;
    const dim3 grid((unsigned)a.total);
    if (a.bf16 && HD % (8 * NORM_THREADS) == 0 && HD <= 4 * 8 * NORM_THREADS) {
        hipLaunchKernelGGL((norm_gate_bf16_kernel<4>), grid, dim3(NORM_THREADS), 0, st,
                           (__bf16*)a.out, (const __bf16*)a.g, (const __bf16*)a.w, HD, a.eps);
    } else if (a.bf16) {
        hipLaunchKernelGGL((norm_gate_kernel<__bf16>), grid, dim3(NORM_THREADS), 0, st,
                           (__bf16*)a.out, (const __bf16*)a.g, (const __bf16*)a.w, HD, a.eps);
    } else {
        hipLaunchKernelGGL((norm_gate_kernel<float>), grid, dim3(NORM_THREADS), 0, st,
                           (float*)a.out, (const float*)a.g, (const float*)a.w, HD, a.eps);
    }
    return hipGetLastError();
}

}  // namespace la
