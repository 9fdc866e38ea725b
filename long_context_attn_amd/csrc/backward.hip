// Backward pass of the Lightning Attention layer: the portable fp32 vector-ALU
// kernels (any supported head_dim / block, fp32 or bf16 storage), the norm
// backward and scans shared with the bf16 MFMA path (backward_mfma.hip), and
// the launch sequence of both.
//
// The forward is Mechanism steps 2-4 of "Diving into MiniMax01 405B MoE"
// (section "Hybrid Modeling"): q~, k~, v~ = SiLU(q, k, v), S_t = S0 +
// sum_{u<=t} k~_u^T v~_u, y_t = q~_t S_t, out = y r w sigmoid(g) with
// r = (mean_{h,d} y^2 + eps)^-1/2.  Given dout (and optionally dS_final, the
// gradient reaching the final state), the chain rule in reverse gives:
//   norm:  a = dout w sigmoid(g), yhat = y r:  dy = r (a - yhat <a, yhat> / HD),
//          dgate = dout yhat w sigmoid'(g),  dw = sum_t dout yhat sigmoid(g);
//   state: dS_t = dS_final + sum_{u>=t} q~_u^T dy_u  (the gradient w.r.t. S_t),
//          dq~_t = dy_t S_t^T,  dk~_t = v~_t dS_t^T,  dv~_t = k~_t dS_t,
//          dS0 = dS at the first token;
//   input: dq = dq~ SiLU'(q), and likewise for k and v.
// Each of y, dq~, dk~ and dv~ is one linear-attention walk over the chunks,
//   Y_t = X_t R + sum_{u in window(t), same chunk} (X_t . K_u) V_u,
// causal (u <= t, R = the state entering the chunk from the left) or
// anti-causal (u >= t, R = the state entering from the right):
//   y   = causal(q~, k~, v~, S_entry)          dq~ = causal(dy, v~, k~, S_entry^T)
//   dk~ = anti-causal(v~, dy, q~, G_exit^T)    dv~ = anti-causal(k~, q~, dy, G_exit)
// with S_entry from the forward prefix of the chunk sums sum k~^T v~ and
// G_exit = dS_final + the suffix of the chunk sums sum q~^T dy.
#include "la_internal.h"

namespace la {

namespace {

constexpr int EW_THREADS = 256;  // elementwise and norm kernels
constexpr int NB_TOKENS = 8;     // tokens per workgroup of the norm backward, at least
constexpr int64_t NB_GROUPS = 2048;  // norm backward workgroups (dw partial rows), at most

__device__ __forceinline__ float silu_grad_f(float x) {
    const float s = sigmoid_f(x);
    return s * (1.0f + x * (1.0f - s));
}

// q~, k~, v~ = SiLU(q, k, v) in fp32
template <class TT>
__global__ __launch_bounds__(EW_THREADS) void silu3_kernel(const TT* __restrict__ q,
                                                           const TT* __restrict__ k,
                                                           const TT* __restrict__ v,
                                                           float* __restrict__ qs,
                                                           float* __restrict__ ks,
                                                           float* __restrict__ vs, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * EW_THREADS + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * EW_THREADS) {
        qs[i] = silu_f(to_f32(q[i]));
        ks[i] = silu_f(to_f32(k[i]));
        vs[i] = silu_f(to_f32(v[i]));
    }
}

// states[c][h][i][j] = sum over chunk c's tokens u of X_u[i] Y_u[j]
template <int D>
__global__ __launch_bounds__(D) void chunk_sum_kernel(const float* __restrict__ X,
                                                      const float* __restrict__ Y,
                                                      const PlanHeader* __restrict__ hdr,
                                                      const ChunkEntry* __restrict__ chunks,
                                                      float* __restrict__ states, int H) {
    constexpr int TILE = 16;
    __shared__ float xs[TILE][D];
    __shared__ float ys[TILE][D];
    const int c = blockIdx.x / H, h = blockIdx.x - (blockIdx.x / H) * H;
    if (c >= hdr->n_chunks) return;
    const ChunkEntry ce = chunks[c];
    const int j = threadIdx.x;
    const int64_t HD = (int64_t)H * D;
    float acc[D];
#pragma unroll
    for (int i = 0; i < D; ++i) acc[i] = 0.f;
    for (int t0 = 0; t0 < ce.len; t0 += TILE) {
        const int n = min(TILE, ce.len - t0);
        for (int a = 0; a < TILE; ++a) {
            const int64_t idx = (ce.start + t0 + a) * HD + (int64_t)h * D + j;
            xs[a][j] = a < n ? X[idx] : 0.f;
            ys[a][j] = a < n ? Y[idx] : 0.f;
        }
        __syncthreads();
        for (int a = 0; a < n; ++a) {
            const float yj = ys[a][j];
#pragma unroll
            for (int i = 0; i < D; ++i) acc[i] += xs[a][i] * yj;
        }
        __syncthreads();
    }
    float* dst = states + ((int64_t)c * H + h) * D * D;
#pragma unroll
    for (int i = 0; i < D; ++i) dst[i * D + j] = acc[i];
}

// Reverse exclusive scan per (sequence, head): each chunk sum B_c is replaced
// by G_exit(c) = dS_final + sum_{c' > c} B_c'; dS0 = dS_final + sum_c B_c.
// Without d_init the first chunk's sum is not read (it may not have been
// formed).
constexpr int RSCAN_THREADS = 256;
__global__ __launch_bounds__(RSCAN_THREADS) void reverse_scan_kernel(
    float* __restrict__ states, const SegEntry* __restrict__ segs, const float* d_final,
    float* d_init, int H, int DD, int tiles) {
    const int pair = blockIdx.x / tiles;
    const int tile = blockIdx.x - pair * tiles;
    const int e = (tile * RSCAN_THREADS + threadIdx.x) * 4;
    if (e >= DD) return;
    const int s = pair / H, h = pair - s * H;
    f32x4 run = {0.f, 0.f, 0.f, 0.f};
    if (d_final != nullptr) run = *reinterpret_cast<const f32x4*>(d_final + (int64_t)pair * DD + e);
    const SegEntry se = segs[s];
    for (int c = se.first + se.count - 1; c >= se.first; --c) {
        f32x4* p = reinterpret_cast<f32x4*>(states + ((int64_t)c * H + h) * DD + e);
        if (c == se.first && d_init == nullptr) {
            *p = run;
            break;
        }
        const f32x4 sum = *p;
        *p = run;
        run += sum;
    }
    if (d_init != nullptr) *reinterpret_cast<f32x4*>(d_init + (int64_t)pair * DD + e) = run;
}

// One linear-attention walk per (chunk, head), a workgroup of D threads;
// thread j owns column j of the D x D fp32 running state R (D registers).
// REV: anti-causal (blocks last to first, u >= t); TRS: R starts as the
// transpose of the chunk's state.  EPI = 0: Y to yout (fp32); EPI = 1:
// gout = Y * SiLU'(raw) in TT.
template <class TT, int D, int BK, bool REV, bool TRS, int EPI>
__global__ __launch_bounds__(D) void lin_walk_kernel(
    const float* __restrict__ Xm, const float* __restrict__ Km, const float* __restrict__ Vm,
    const PlanHeader* __restrict__ hdr, const ChunkEntry* __restrict__ chunks,
    const float* __restrict__ states, float* __restrict__ yout, const TT* __restrict__ raw,
    TT* __restrict__ gout, int H) {
    extern __shared__ float lds[];
    float* xs = lds;              // [BK][D]
    float* ks = xs + BK * D;      // [BK][D]
    float* vs = ks + BK * D;      // [BK][D]
    float* sc = vs + BK * D;      // [BK][BK] scores X_a . K_b
    const int c = blockIdx.x / H, h = blockIdx.x - (blockIdx.x / H) * H;
    if (c >= hdr->n_chunks) return;
    const ChunkEntry ce = chunks[c];
    const int j = threadIdx.x;
    const int64_t HD = (int64_t)H * D;
    float R[D];
    const float* src = states + ((int64_t)c * H + h) * D * D;
#pragma unroll
    for (int i = 0; i < D; ++i) R[i] = TRS ? src[j * D + i] : src[i * D + j];
    const int nblk = (ce.len + BK - 1) / BK;
    for (int bi = 0; bi < nblk; ++bi) {
        const int t0 = (REV ? nblk - 1 - bi : bi) * BK;
        const int n = min(BK, ce.len - t0);
        for (int a = 0; a < BK; ++a) {
            const int64_t idx = (ce.start + t0 + a) * HD + (int64_t)h * D + j;
            const bool ok = a < n;
            xs[a * D + j] = ok ? Xm[idx] : 0.f;
            ks[a * D + j] = ok ? Km[idx] : 0.f;
            vs[a * D + j] = ok ? Vm[idx] : 0.f;
        }
        __syncthreads();
        // scores inside the window (entries outside it are never read)
        for (int p = j; p < BK * BK; p += D) {
            const int a = p / BK, b = p - (p / BK) * BK;
            float s = 0.f;
            if ((REV ? b >= a : b <= a) && a < n && b < n) {
                for (int i = 0; i < D; ++i) s += xs[a * D + i] * ks[b * D + i];
            }
            sc[p] = s;
        }
        __syncthreads();
        for (int a = 0; a < n; ++a) {
            float y = 0.f;
#pragma unroll
            for (int i = 0; i < D; ++i) y += xs[a * D + i] * R[i];  // the state entering the block
            if (REV) {
                for (int b = a; b < n; ++b) y += sc[a * BK + b] * vs[b * D + j];
            } else {
                for (int b = 0; b <= a; ++b) y += sc[a * BK + b] * vs[b * D + j];
            }
            const int64_t idx = (ce.start + t0 + a) * HD + (int64_t)h * D + j;
            if (EPI == 0) yout[idx] = y;
            else gout[idx] = from_f32<TT>(y * silu_grad_f(to_f32(raw[idx])));
        }
        // the block's contribution, after its outputs used the state before it
        for (int a = 0; a < n; ++a) {
            const float vj = vs[a * D + j];
#pragma unroll
            for (int i = 0; i < D; ++i) R[i] += ks[a * D + i] * vj;
        }
        __syncthreads();
    }
}

// 8 consecutive fp32 values stored as fp32 or bf16
__device__ __forceinline__ void store8(float* p, const float (&x)[8]) {
    *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
}
__device__ __forceinline__ void store8(__bf16* p, const float (&x)[8]) {
    bf16x8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (__bf16)x[i];
    *reinterpret_cast<bf16x8*>(p) = v;
}
// the same with the non-temporal hint, for values nothing reads again
__device__ __forceinline__ void store8_nt(float* p, const float (&x)[8]) {
    __builtin_nontemporal_store(f32x4{x[0], x[1], x[2], x[3]}, reinterpret_cast<f32x4*>(p));
    __builtin_nontemporal_store(f32x4{x[4], x[5], x[6], x[7]}, reinterpret_cast<f32x4*>(p + 4));
}
__device__ __forceinline__ void store8_nt(__bf16* p, const float (&x)[8]) {
    bf16x8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (__bf16)x[i];
    __builtin_nontemporal_store(v, reinterpret_cast<bf16x8*>(p));
}

// 8 consecutive elements kept in their storage type (bf16 pieces take half
// the registers of fp32 ones), widened to fp32 where they are used
template <class T>
struct Piece;
template <>
struct Piece<float> {
    f32x4 a, b;
    __device__ __forceinline__ void load(const float* p) {
        a = *reinterpret_cast<const f32x4*>(p);
        b = *reinterpret_cast<const f32x4*>(p + 4);
    }
    __device__ __forceinline__ float operator[](int i) const { return i < 4 ? a[i] : b[i - 4]; }
    // taken as rewritten: values widened from it before this point are not reused after it
    __device__ __forceinline__ void fence() { asm volatile("" : "+v"(a), "+v"(b)); }
};
template <>
struct Piece<__bf16> {
    bf16x8 v;
    __device__ __forceinline__ void load(const __bf16* p) {
        v = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(p));
    }
    __device__ __forceinline__ float operator[](int i) const { return (float)v[i]; }
    __device__ __forceinline__ void fence() {
        f32x4 x = __builtin_bit_cast(f32x4, v);
        asm volatile("" : "+v"(x));
        v = __builtin_bit_cast(bf16x8, x);
    }
};

// Norm backward: one workgroup per tpb consecutive tokens.  Thread t
// holds the 8-element pieces t, t + 256, ... (CPT of them) of a token's H*D
// values in registers, in their storage type: one pass loads y, gate and
// dout, two block reductions give r and <a, yhat>, and the same registers
// give dy (DYT: fp32, or bf16 as an MFMA operand) and dgate (the gate's
// sigmoid is evaluated in both passes rather than kept, which keeps enough
// workgroups resident to have several tokens' loads in flight per CU).  dw
// is accumulated in LDS over the workgroup's tokens (each thread its own
// entries) and written as one partial sum row.
template <class TT, class DYT, class YT, int CPT>
__global__ __launch_bounds__(EW_THREADS) void norm_backward_kernel(
    const YT* __restrict__ y, const TT* __restrict__ g, const TT* __restrict__ w,
    const TT* __restrict__ dout, DYT* __restrict__ dy, TT* __restrict__ dg,
    float* __restrict__ dw_part, int64_t T, int64_t tpb, int HD, float eps) {
    __shared__ float red[2][EW_THREADS / 64];
    // this thread's dw sums, one column per thread (conflict-free)
    __shared__ float dwp[CPT][8][EW_THREADS];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int nch = HD >> 3;
    const int64_t t_begin = (int64_t)blockIdx.x * tpb;
    const int64_t t_end = min(T, t_begin + tpb);
    Piece<TT> wt[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        const int ch = tid + EW_THREADS * c;
#pragma unroll
        for (int i = 0; i < 8; ++i) dwp[c][i][tid] = 0.f;
        if (ch < nch) wt[c].load(w + 8 * ch);
    }
    for (int64_t t = t_begin; t < t_end; ++t) {
        const int64_t base = t * HD;
#pragma unroll
        for (int c = 0; c < CPT; ++c) wt[c].fence();  // widened per token, not held
        Piece<YT> yv[CPT];
        Piece<TT> gr[CPT], go[CPT];
        float ss = 0.f, ay = 0.f;
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const int ch = tid + EW_THREADS * c;
            if (ch < nch) {
                yv[c].load(y + base + 8 * ch);
                gr[c].load(g + base + 8 * ch);
                go[c].load(dout + base + 8 * ch);
            }
        }
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const int ch = tid + EW_THREADS * c;
            if (ch < nch) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float yy = yv[c][i];
                    ss += yy * yy;
                    ay += go[c][i] * wt[c][i] * sigmoid_f(gr[c][i]) * yy;
                }
            }
        }
        for (int off = 32; off > 0; off >>= 1) {
            ss += __shfl_xor(ss, off);
            ay += __shfl_xor(ay, off);
        }
        if (lane == 0) {
            red[0][wv] = ss;
            red[1][wv] = ay;
        }
        __syncthreads();
        ss = 0.f;
        ay = 0.f;
#pragma unroll
        for (int i = 0; i < EW_THREADS / 64; ++i) {
            ss += red[0][i];
            ay += red[1][i];
        }
        __syncthreads();
        const float r = __builtin_amdgcn_rsqf(ss / (float)HD + eps);
        const float m = ay * r / (float)HD;  // <a, yhat> / HD
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            yv[c].fence();
            gr[c].fence();
            go[c].fence();
            wt[c].fence();
        }
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const int ch = tid + EW_THREADS * c;
            if (ch < nch) {
                float d1[8], d2[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float sg = sigmoid_f(gr[c][i]);
                    const float yh = yv[c][i] * r;
                    const float gw = go[c][i] * wt[c][i] * sg;
                    d1[i] = r * (gw - yh * m);
                    d2[i] = gw * yh * (1.0f - sg);
                    dwp[c][i][tid] += go[c][i] * yh * sg;
                }
                store8(dy + base + 8 * ch, d1);
                store8_nt(dg + base + 8 * ch, d2);
            }
        }
    }
    float* part = dw_part + (int64_t)blockIdx.x * HD;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        const int ch = tid + EW_THREADS * c;
        if (ch < nch) {
            float x[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = dwp[c][i][tid];
            store8(part + 8 * ch, x);
        }
    }
}

// dw from the partial sum rows in one launch, in an order fixed by the row
// count alone: a workgroup owns DW_COLS columns; its thread (j, i), j < 8
// the column quad and i < DW_GROUPS the row group, adds rows i, i +
// DW_GROUPS, i + 2 DW_GROUPS, ... of its quad (all of a thread's loads in
// flight at once for up to 8 DW_GROUPS rows), then the row groups are added
// in LDS, 8 at a time and then the 16 results, in index order.
constexpr int DW_THREADS = 1024;
constexpr int DW_GROUPS = DW_THREADS / 8;  // 128 row groups
constexpr int DW_COLS = 32;                // 8 quads of 4 columns
__global__ __launch_bounds__(DW_THREADS) void dw_reduce_kernel(const float* __restrict__ part,
                                                               float* __restrict__ dw, int nparts,
                                                               int HD) {
    __shared__ float4 lv[DW_GROUPS][8];
    __shared__ float4 lv2[16][8];
    const int tid = threadIdx.x, j = tid & 7, i = tid >> 3;
    const int col = blockIdx.x * DW_COLS + 4 * j;  // HD is a multiple of 16
    const bool in = col < HD;
    float4 acc = {0.f, 0.f, 0.f, 0.f};
    if (in) {
        const float* p = part + col;
        int r = i;
        for (; r + 7 * DW_GROUPS < nparts; r += 8 * DW_GROUPS) {
            float4 x[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                x[u] = *reinterpret_cast<const float4*>(p + (int64_t)(r + u * DW_GROUPS) * HD);
#pragma unroll
            for (int u = 0; u < 8; ++u) acc += x[u];
        }
        for (; r < nparts; r += DW_GROUPS)
            acc += *reinterpret_cast<const float4*>(p + (int64_t)r * HD);
    }
    lv[i][j] = acc;
    __syncthreads();
    if (tid < 128) {
        const int g = tid >> 3;
        float4 s = lv[8 * g][j];
#pragma unroll
        for (int u = 1; u < 8; ++u) s += lv[8 * g + u][j];
        lv2[g][j] = s;
    }
    __syncthreads();
    if (tid < 8 && in) {
        float4 s = lv2[0][j];
#pragma unroll
        for (int u = 1; u < 16; ++u) s += lv2[u][j];
        dw[col] = s.x;  // the caller's dweight may be only 4-byte aligned
        dw[col + 1] = s.y;
        dw[col + 2] = s.z;
        dw[col + 3] = s.w;
    }
}

// Walk block: 16 tokens whatever the forward's block (the result does not
// depend on it beyond rounding); the small LDS footprint lets several
// workgroups share a CU.
constexpr int WALK_BK = 16;

unsigned ew_grid(int64_t n) {
    int64_t b = (n + EW_THREADS - 1) / EW_THREADS;
    return (unsigned)(b < 1 ? 1 : (b > 65536 ? 65536 : b));
}

template <class TT, int D, int BK, bool REV, bool TRS, int EPI>
hipError_t walk(const BackwardArgs& a, const float* X, const float* K, const float* V,
                const float* states, float* yout, const void* raw, void* gout) {
    const dim3 grid((unsigned)((int64_t)a.p.max_chunks * a.p.H));
    const size_t lds = sizeof(float) * (3 * BK * D + BK * BK);
    auto* fn = &lin_walk_kernel<TT, D, BK, REV, TRS, EPI>;
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(fn, grid, dim3(D), lds, a.stream, X, K, V, a.p.hdr, a.p.chunks, states,
                       yout, (const TT*)raw, (TT*)gout, a.p.H);
    return hipGetLastError();
}

hipError_t dw_reduce(const BackwardArgs& a, int HD) {
    const unsigned grid = (unsigned)((HD + DW_COLS - 1) / DW_COLS);
    hipLaunchKernelGGL(dw_reduce_kernel, dim3(grid), dim3(DW_THREADS), 0, a.stream, a.dw_part,
                       a.dw, a.n_tb, HD);
    return hipGetLastError();
}

// norm backward launch: CPT pieces of 8 per thread cover H*D <= 2048 CPT;
// y is stored as YT (fp32 on the portable path, bf16 on the MFMA path)
template <class TT, class DYT, class YT>
hipError_t norm_backward(const BackwardArgs& a, DYT* dy) {
    if (a.n_tb == 0) return hipSuccess;
    const PrefillArgs& p = a.p;
    const int HD = p.H * p.D;
    const int per = (HD / 8 + EW_THREADS - 1) / EW_THREADS;
    const dim3 grid((unsigned)a.n_tb), block(EW_THREADS);
#define LA_NB(C)                                                                                \
    hipLaunchKernelGGL((norm_backward_kernel<TT, DYT, YT, C>), grid, block, 0, a.stream,        \
                       (const YT*)a.y,                                                          \
                       (const TT*)p.g, (const TT*)p.w, (const TT*)a.dout, dy, (TT*)a.dg,        \
                       a.dw_part, p.total, backward_norm_tokens(p.total), HD, p.eps)
    if (per <= 1) LA_NB(1);
    else if (per <= 2) LA_NB(2);
    else if (per <= 4) LA_NB(4);
    else if (per <= 8) LA_NB(8);
    else if (per <= 16) LA_NB(16);
    else return hipErrorInvalidValue;
#undef LA_NB
    return hipGetLastError();
}

hipError_t reverse_scan(const BackwardArgs& a) {
    const int DD = a.p.D * a.p.D;
    const int tiles = (DD / 4 + RSCAN_THREADS - 1) / RSCAN_THREADS;
    const int64_t grid = (int64_t)a.p.nseq * a.p.H * tiles;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL(reverse_scan_kernel, dim3((unsigned)grid), dim3(RSCAN_THREADS), 0, a.stream,
                       a.gstates, a.p.segs, a.d_final, a.d_init, a.p.H, DD, tiles);
    return hipGetLastError();
}

// bf16 MFMA path (bf16, head_dim 128): chunk sums and walks on MFMA, the
// operands read from the activations with SiLU applied on load; dy is bf16.
hipError_t backward_mfma(const BackwardArgs& a) {
    // With an inline plan (uniform rows), the first chunk-sum launch writes
    // the plan tables that the later kernels read; the others take `p`.
    const PrefillArgs& first = a.p;
    PrefillArgs p = a.p;
    p.inline_plan = false;
    hipStream_t st = a.stream;
    const int HD = p.H * p.D;
    hipError_t e = hipSuccess;
    if (!a.saved) {
        if ((e = launch_chunk_sums_mfma(first, p.k, p.v, true, true, p.states, SumSkip::last,
                                        st)) != hipSuccess)
            return e;
        PrefillArgs s = p;
        s.final_state = nullptr;
        s.skip_last = true;
        if ((e = launch_state_scan(s, st)) != hipSuccess) return e;
        if ((e = launch_backward_walk_y(a)) != hipSuccess) return e;
    }
    if ((e = norm_backward<__bf16, __bf16, __bf16>(a, (__bf16*)a.dy)) != hipSuccess) return e;
    if ((e = dw_reduce(a, HD)) != hipSuccess) return e;
    // each sequence's first chunk sum only feeds dS0
    if ((e = launch_chunk_sums_mfma(a.saved ? first : p, p.q, a.dy, true, false, a.gstates,
                                    a.d_init ? SumSkip::none : SumSkip::first, st)) != hipSuccess)
        return e;
    if ((e = reverse_scan(a)) != hipSuccess) return e;
    return launch_backward_walks_grad(a);
}

template <class TT, int D, int BK>
hipError_t backward_db(const BackwardArgs& a) {
    const PrefillArgs& p = a.p;
    hipStream_t st = a.stream;
    float* dy = static_cast<float*>(a.dy);
    const int64_t n = p.total * p.H * D;
    const int HD = p.H * D;
    const dim3 cgrid((unsigned)((int64_t)p.max_chunks * p.H));
    hipError_t e = hipSuccess;
    // q~, k~, v~; forward chunk sums and the states entering the chunks
    hipLaunchKernelGGL((silu3_kernel<TT>), dim3(ew_grid(n)), dim3(EW_THREADS), 0, st,
                       (const TT*)p.q, (const TT*)p.k, (const TT*)p.v, a.qs, a.ks, a.vs, n);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((chunk_sum_kernel<D>), cgrid, dim3(D), 0, st, a.ks, a.vs, p.hdr, p.chunks,
                       p.states, p.H);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    {
        PrefillArgs s = p;
        s.final_state = nullptr;
        s.skip_last = false;
        if ((e = launch_state_scan(s, st)) != hipSuccess) return e;
    }
    // y, then the norm backward: dy, dgate, dw
    if ((e = walk<TT, D, BK, false, false, 0>(a, a.qs, a.ks, a.vs, p.states, a.y, nullptr,
                                               nullptr)) != hipSuccess)
        return e;
    if ((e = norm_backward<TT, float, float>(a, dy)) != hipSuccess) return e;
    if ((e = dw_reduce(a, HD)) != hipSuccess) return e;
    // reverse chunk sums of q~^T dy, G_exit and dS0
    hipLaunchKernelGGL((chunk_sum_kernel<D>), cgrid, dim3(D), 0, st, a.qs, dy, p.hdr, p.chunks,
                       a.gstates, p.H);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = reverse_scan(a)) != hipSuccess) return e;
    // the three input gradients
    if ((e = walk<TT, D, BK, false, true, 1>(a, dy, a.vs, a.ks, p.states, nullptr, p.q, a.dq)) !=
        hipSuccess)
        return e;
    if ((e = walk<TT, D, BK, true, true, 1>(a, a.vs, dy, a.qs, a.gstates, nullptr, p.k, a.dk)) !=
        hipSuccess)
        return e;
    return walk<TT, D, BK, true, false, 1>(a, a.ks, a.qs, dy, a.gstates, nullptr, p.v, a.dv);
}

template <class TT>
hipError_t backward_t(const BackwardArgs& a) {
    switch (a.p.D) {
        case 16: return backward_db<TT, 16, WALK_BK>(a);
        case 32: return backward_db<TT, 32, WALK_BK>(a);
        case 64: return backward_db<TT, 64, WALK_BK>(a);
        case 128: return backward_db<TT, 128, WALK_BK>(a);
    }
    return hipErrorInvalidValue;
}

}  // namespace

int64_t backward_norm_tokens(int64_t total) {
    const int64_t t = (total + NB_GROUPS - 1) / NB_GROUPS;
    return t > NB_TOKENS ? t : (int64_t)NB_TOKENS;
}
int backward_max_hd() { return 16 * 8 * EW_THREADS; }

// After the plan: every kernel of the backward.  With no token at all the
// token kernels find no chunk (or no token block) and return, dw comes out
// zero and dS0 = dS_final (or zero).
hipError_t launch_backward(const BackwardArgs& a) {
    if (a.p.max_chunks == 0) return hipSuccess;
    if (a.mfma) return backward_mfma(a);
    return a.p.bf16 ? backward_t<__bf16>(a) : backward_t<float>(a);
}

}  // namespace la
