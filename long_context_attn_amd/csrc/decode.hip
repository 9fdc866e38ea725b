// Single-token decode step of the Lightning Attention layer.
//
// With Mechanism step 3 of "Diving into MiniMax01 405B MoE" (section "Hybrid
// Modeling") read causally, the layer keeps one D x D state per head and a
// new token costs O(d^2): S += k~^T v~, then y = q~ S (the token sees itself),
// then step 4's RMSNorm over the token's H*D values times sigmoid(gate).
//
// The step is bound by HBM: the fp32 state (64 KiB per head at D = 128) is
// read and written once, with 16-byte accesses and every thread keeping
// several loads in flight.  With at least as many sequences as CUs, one
// workgroup per sequence streams its heads' states one after another, keeps
// y in LDS and applies the norm and gate itself; otherwise long-lived
// workgroups (one per CU) loop over (sequence, head) pairs, leave y and the
// per-head sums of squares in the workspace, and a second kernel applies the
// norm and gate per sequence.
#include <atomic>
#include <mutex>

#include "la_internal.h"

namespace la {

constexpr int DEC_THREADS = 1024;
#ifndef LA_DEC_ROT
#define LA_DEC_ROT 1
#endif

// One (sequence, head) pair: S += k~^T v~ in place, y = q~ S.  Leaves y[j] in
// ysum[j] and returns sum_j y_j^2 in every thread of the workgroup.
template <class TT, int D>
__device__ __forceinline__ float decode_pair(const TT* __restrict__ q, const TT* __restrict__ k,
                                             const TT* __restrict__ v, float* __restrict__ state,
                                             int64_t pair, float* __restrict__ ysum) {
    constexpr int TPR = D / 4;               // threads per state row (4 columns each)
    constexpr int NRG = DEC_THREADS / TPR;   // row groups
    constexpr int RPT = (D + NRG - 1) / NRG; // rows per thread
    __shared__ float qs[D], ks[D], vs[D];
    __shared__ f32x4 red[NRG][TPR];
    __shared__ float wsum[DEC_THREADS / 64];
    const int tid = threadIdx.x;
    const int cq = tid % TPR, rg = tid / TPR;
    const int j0 = cq * 4;
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
        ysum[tid] = yj;
        sq = yj * yj;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) sq += __shfl_xor(sq, off);
    if ((tid & 63) == 0) wsum[tid >> 6] = sq;
    __syncthreads();
    float t = 0.f;
    for (int i = 0; i < DEC_THREADS / 64; ++i) t += wsum[i];
    // qs/ks/vs, red and wsum are rewritten by the next pair
    __syncthreads();
    return t;
}

// A fixed set of workgroups (one per CU) walks over the (sequence, head)
// pairs: long-lived workgroups keep the memory pipeline fuller than one short
// workgroup per pair.  y and the per-head sums of squares go to the workspace
// for the norm kernel.
template <class TT, int D>
__global__ __launch_bounds__(DEC_THREADS) void decode_state_kernel(
    const TT* __restrict__ q, const TT* __restrict__ k, const TT* __restrict__ v,
    float* __restrict__ state, float* __restrict__ ybuf, float* __restrict__ ssbuf,
    int64_t pairs) {
    for (int64_t pair = blockIdx.x; pair < pairs; pair += gridDim.x) {  // sequence * H + head
        const float t = decode_pair<TT, D>(q, k, v, state, pair, ybuf + pair * D);
        if (threadIdx.x == 0) ssbuf[pair] = t;
    }
}

// One workgroup per sequence: all H heads in turn, their y kept in LDS, then
// the norm and the gate (used when there are at least as many sequences as
// CUs, so that whole sequences still fill the chip).  The heads are
// software-pipelined with one barrier each: step h issues the loads of head
// h + 1's state into the other register set and applies SiLU to its q, k, v,
// passes the barrier, finishes head h - 1's y (its per-wave partial sums,
// left in LDS by step h - 1), then updates head h's state and forms its
// partial y.  So a head's state loads are in flight while the previous head
// is processed.
template <class TT, int D>
__global__ __launch_bounds__(DEC_THREADS) void decode_seq_kernel(
    const TT* __restrict__ q, const TT* __restrict__ k, const TT* __restrict__ v,
    const TT* __restrict__ g, const TT* __restrict__ w, TT* __restrict__ out,
    float* __restrict__ state, int H, float eps) {
    constexpr int TPR = D / 4;               // threads per state row (4 columns each)
    constexpr int NRG = DEC_THREADS / TPR;   // row groups
    constexpr int RPT = (D + NRG - 1) / NRG; // rows per thread
    constexpr int YW = (D + 63) / 64;        // waves that finish a head's y
    constexpr int NW = DEC_THREADS / 64;     // waves
    extern __shared__ float ys[];            // [H * D] y of this token, then [H][YW] sums of y^2
    __shared__ float qkv[3][3][D];           // SiLU(q), SiLU(k), SiLU(v) of three heads (ring)
    __shared__ f32x4 red[2][NW][TPR];        // partial y of two heads, per wave
    const int64_t s = blockIdx.x;
    const int HD = H * D;
    float* ss = ys + HD;
    const int tid = threadIdx.x;
    const int cq = tid % TPR, rg = tid / TPR, j0 = cq * 4;
    const int64_t DD = (int64_t)D * D;
    // The heads are visited in an order rotated by the sequence: step i takes
    // head (i + rot) mod H.  All workgroups run in step, so without the
    // rotation every one of them would stream the state of the same head,
    // addresses a multiple of H * 64 KiB apart.  y and the sums of squares are
    // kept per head and summed in head order, so the output does not depend
    // on the rotation.
    const int rot = (int)((s * LA_DEC_ROT) % H);
    auto head = [&](int i) { return i + rot < H ? i + rot : i + rot - H; };
    // rows of step i's head with the non-temporal hint; a step past the last
    // gets an empty range (its loads return zeros and touch no memory)
    auto load_rows = [&](int i, f32x4 (&r)[RPT]) {
        const bool in = i < H;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(state + (s * H + (in ? head(i) : 0)) * DD), (short)0,
            __builtin_amdgcn_readfirstlane(in ? (int)(DD * 4) : 0), 0x00020000);
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int i = min(rg + m * NRG, D - 1);
            r[m] = __builtin_bit_cast(
                f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (i * TPR + cq) * 16, 0, 2));
        }
    };
    auto silu_qkv = [&](int i) {
        if (i < H && tid < D) {
            const int64_t idx = (s * H + head(i)) * D + tid;
            qkv[i % 3][0][tid] = silu_f(to_f32(q[idx]));
            qkv[i % 3][1][tid] = silu_f(to_f32(k[idx]));
            qkv[i % 3][2][tid] = silu_f(to_f32(v[idx]));
        }
    };
    // y of step i's head (sum over the row groups, in order) and its sum of
    // squares per wave
    auto finish = [&](int i) {
        const int hh = head(i);
        float sq = 0.f;
        if (tid < D) {
            float yj = 0.f;
            for (int r = 0; r < NW; ++r) yj += red[i & 1][r][tid / 4][tid % 4];
            ys[hh * D + tid] = yj;
            sq = yj * yj;
        }
        if (tid < 64 * YW) {
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) sq += __shfl_xor(sq, off);
            if ((tid & 63) == 0) ss[hh * YW + (tid >> 6)] = sq;
        }
    };
    f32x4 R0[RPT], R1[RPT], st[RPT];
    auto step = [&](int h, f32x4 (&cur)[RPT], f32x4 (&nxt)[RPT]) {
        load_rows(h + 1, nxt);
        silu_qkv(h + 1);
        __syncthreads();
        // the stored state of step h - 1 is no longer read by its stores
#pragma unroll
        for (int m = 0; m < RPT; ++m) asm volatile("" ::"v"(st[m]));
        if (h >= 1) finish(h - 1);
        const float* qs = qkv[h % 3][0];
        const float* ks = qkv[h % 3][1];
        const float* vs = qkv[h % 3][2];
        const f32x4 vj = {vs[j0], vs[j0 + 1], vs[j0 + 2], vs[j0 + 3]};
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
        f32x4* S = reinterpret_cast<f32x4*>(state + (s * H + head(h)) * DD);
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int i = rg + m * NRG;
            if (i < D) {
                st[m] = cur[m] + ks[i] * vj;
                __builtin_nontemporal_store(st[m], &S[i * TPR + cq]);
                y += qs[i] * st[m];
            }
        }
        // the row groups of a wave summed across its lanes, one partial per wave
#pragma unroll
        for (int off = TPR; off < 64; off *= 2)
#pragma unroll
            for (int u = 0; u < 4; ++u) y[u] += __shfl_xor(y[u], off);
        if ((tid & 63) < TPR) red[h & 1][tid >> 6][cq] = y;
    };
#pragma unroll
    for (int m = 0; m < RPT; ++m) st[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    load_rows(0, R0);
    silu_qkv(0);
    for (int h = 0; h < H; h += 2) {
        step(h, R0, R1);
        if (h + 1 < H) step(h + 1, R1, R0);
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < RPT; ++m) asm volatile("" ::"v"(st[m]));
    finish(H - 1);
    __syncthreads();
    float tot = 0.f;
    for (int h = 0; h < H; ++h)
        for (int i = 0; i < YW; ++i) tot += ss[h * YW + i];  // head order
    const float r = 1.0f / __builtin_sqrtf(tot / (float)HD + eps);
    for (int e = tid; e < HD; e += DEC_THREADS) {
        const int64_t idx = s * HD + e;
        out[idx] = from_f32<TT>(ys[e] * r * to_f32(w[e]) * sigmoid_f(to_f32(g[idx])));
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
int device_cu_count() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// The per-sequence kernel keeps a token's H * D values of y (and 2 H sums) in
// dynamic LDS, next to about 21 KiB of static LDS (two heads' per-wave partial
// y and three heads' q, k, v): 40 KiB of dynamic LDS keeps the total within
// the 64 KiB a launch gets without opting in to more.
constexpr size_t DEC_SEQ_LDS_MAX = 40 * 1024;

bool decode_fused(const DecodeArgs& a) {
    return a.nseq >= device_cu_count() &&
           sizeof(float) * ((size_t)a.H * a.D + 2 * (size_t)a.H) <= DEC_SEQ_LDS_MAX;
}

bool decode_uses_workspace(int nseq, int H, int D) {
    DecodeArgs a{};
    a.nseq = nseq;
    a.H = H;
    a.D = D;
    return !decode_fused(a);
}

// ------------------------------------------ fixed scratch (no allocation)
// The scratch of the two-kernel decode (y [S][H*D] fp32, then the per-head
// sums of squares [S][H], at the offsets of the caller's workspace) for the
// entry point that allocates nothing.  Each GPU holds its own copy from the
// library's load until the process ends.  The host never uses the array's
// name as an address: its device address is looked up once per device with
// hipGetSymbolAddress and kept.  Every call on a GPU shares the array (calls
// that overlap on one GPU race); nothing in it needs clearing, since the
// state kernel writes every value the norm kernel reads.
constexpr size_t DEC_SCRATCH_BYTES = (size_t(4) << 20) + (size_t(64) << 10);
static __device__ __align__(256) unsigned char scratch[DEC_SCRATCH_BYTES];

size_t decode_scratch_bytes() { return DEC_SCRATCH_BYTES; }

hipError_t decode_scratch(void** out) {
    constexpr int MAXDEV = 64;
    static std::atomic<void*> ptrs[MAXDEV];
    static std::mutex mu;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAXDEV) return hipErrorInvalidDevice;
    void* p = ptrs[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(mu);
        p = ptrs[dev].load(std::memory_order_acquire);
        if (p == nullptr) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (p == nullptr) return hipErrorInvalidSymbol;
            ptrs[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

template <class TT, int D>
static hipError_t decode_state_d(const DecodeArgs& a, hipStream_t st) {
    if (decode_fused(a)) {
        const size_t lds = sizeof(float) * ((size_t)a.H * D + 2 * (size_t)a.H);
        hipLaunchKernelGGL((decode_seq_kernel<TT, D>), dim3((unsigned)a.nseq), dim3(DEC_THREADS),
                           lds, st, (const TT*)a.q, (const TT*)a.k, (const TT*)a.v,
                           (const TT*)a.g, (const TT*)a.w, (TT*)a.out, a.state, a.H, a.eps);
        return hipGetLastError();
    }
    const int64_t pairs = (int64_t)a.nseq * a.H;
    const int64_t ncu = device_cu_count();
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
    if (a.nseq == 0 || decode_fused(a)) return hipSuccess;
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
