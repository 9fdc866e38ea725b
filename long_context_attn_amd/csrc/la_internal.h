// Internal declarations of the Lightning Attention library (device helpers,
// workspace records and kernel launchers).  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// plan_body.h is plain C++, so that the plan can also be built and tested on
// the host; here its functions are compiled for both sides
#define LA_HD __host__ __device__
#include "plan_body.h"

namespace la {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

// ---------------------------------------------------------------- workspace
// PlanHeader, SegEntry, ChunkEntry and the plan's arithmetic: plan_body.h
// (included above, outside the namespace)

// --------------------------------------------------------- element helpers
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }
template <class TT> __device__ __forceinline__ TT from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

// logistic function 1 / (1 + e^-x) from its definition, on the hardware
// base-2 exponential and reciprocal (each ~1 ulp); saturates to 0 / 1.
__device__ __forceinline__ float sigmoid_f(float x) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * x));
}
// SiLU(x) = x * sigmoid(x)
__device__ __forceinline__ float silu_f(float x) { return x * sigmoid_f(x); }

// ---------------------------------------------------------------- launchers
// All launchers enqueue on `st` and return hipGetLastError().
struct PrefillArgs {
    const void *q, *k, *v, *g, *w;
    void* out;
    const float* init_state;  // [nseq][H][D][D] or null
    float* final_state;       // [nseq][H][D][D] or null
    const int32_t* cu;        // device cu_seqlens or null (uniform rows)
    int nseq;
    int64_t seqlen;           // rows' length when cu == null
    int64_t total;            // total tokens
    int H, D, block, chunk;
    float eps;
    bool bf16;
    int max_chunks;
    PlanHeader* hdr;
    SegEntry* segs;
    ChunkEntry* chunks;
    float* states;            // [max_chunks][H][D][D]: chunk sums, then (after the
                              // scan) the state entering each chunk
    // with skip_last the last chunk of each sequence is not summed (its sum is
    // neither computed nor read by the scan, and the scan writes no final
    // state: the MFMA walk forms it)
    bool skip_last;
    // MFMA path: q, k, v hold SiLU(q), SiLU(k), SiLU(v) already (applied by
    // the projection's epilogue)
    bool preact;
    // with preact: the gate holds sigmoid(gate) already (else it is raw)
    bool gate_act;
    // MFMA walk: also store y, the attention output before the norm (bf16,
    // [total][H][D]), for a later backward pass; null = not stored
    void* y_save;
    // MFMA prefill of uniform rows (cu == null): no plan kernel; the chunk-sum
    // kernel computes its chunks from (nseq, seqlen, chunk), and extra
    // workgroups of it write the plan tables and reset the header; the state
    // scan after it clears the exchange words
    bool inline_plan;
    // cross-head RMSNorm exchange of the fused MFMA walk, one slot per
    // (chunk, 64-token block): slot = chunk * (chunk_len / 64) + block.
    // Each word holds a float in its low half and 1 in its high half once
    // written (0 = not yet written); cleared on every call by the plan kernel
    // (or, for uniform rows, by the state scan).
    int n_slots;
    uint64_t* part;           // [n_slots][H][64] per-head sums of y^2 per token
    uint64_t* rsub;           // [n_slots][ceil(H / 16)][64] sums over groups of 16 heads
    // words zeroed on every call before the walk (exchange words)
    uint64_t* clear;
    int64_t clear_words;
};

// compute units of the current device (cached per device; 256 if unknown)
int device_cu_count();

hipError_t launch_plan(const PrefillArgs& a, hipStream_t st);
hipError_t launch_state_scan(const PrefillArgs& a, hipStream_t st);
hipError_t launch_norm_gate(const PrefillArgs& a, hipStream_t st);
// portable fp32 vector-ALU kernels (any supported shape)
hipError_t launch_chunk_state_valu(const PrefillArgs& a, hipStream_t st);
hipError_t launch_walk_valu(const PrefillArgs& a, hipStream_t st);
// bf16 MFMA prefill walk (D = 128, block = 64): every chunk walked from the
// scanned state entering it (states), with the RMSNorm fused
bool mfma_supported(const PrefillArgs& a);
hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t st);
// bf16 MFMA chunk states (D = 128, block = 64): the state-only calls and the
// first pass of the two-pass prefill
bool state_mfma_supported(const PrefillArgs& a);
hipError_t launch_chunk_state_mfma(const PrefillArgs& a, hipStream_t st);
// states[c][h] = sum over chunk c of f(x)^T g(y), f and g SiLU or the identity
// chunks a chunk-sum launch leaves out: none, each sequence's last (a forward
// scan never reads it) or each sequence's first (a reverse scan reads it only
// for the gradient of the initial state)
enum class SumSkip : int { none = 0, last = 1, first = 2 };
hipError_t launch_chunk_sums_mfma(const PrefillArgs& a, const void* x, const void* y, bool silu_x,
                                  bool silu_y, float* states, SumSkip skip, hipStream_t st);

// backward pass (portable fp32 kernels, any supported shape); the plan runs
// first with the chunk table
struct BackwardArgs {
    PrefillArgs p;            // forward inputs, plan, chunk states (forward sums / S_entry)
    hipStream_t stream;
    const void* dout;         // [T][H][D] gradient w.r.t. the output
    const float* d_final;     // [nseq][H][D][D] gradient w.r.t. the final states, or null
    void *dq, *dk, *dv, *dg;  // [T][H][D] outputs
    float* dw;                // [H*D] gradient w.r.t. the norm weight
    float* d_init;            // [nseq][H][D][D] gradient w.r.t. the initial states, or null
    // workspace: y [T][H][D] and dy [T][H][D] (fp32; bf16 on the MFMA path,
    // where y is read through a cast); q~, k~, v~ [T][H][D] fp32 (portable
    // path only); reverse chunk
    // sums / G_exit [max_chunks][H][D][D]; dw partial sums [n_tb][H*D]
    float *qs, *ks, *vs, *y, *gstates, *dw_part;
    void* dy;
    int n_tb;
    bool mfma;
    // y and the states entering the chunks (p.states) come from the prefill
    // (MFMA path): no chunk sums of k~^T v~, scan or y walk
    bool saved;
};
int64_t backward_norm_tokens(int64_t total);  // tokens per dw partial sum row
int backward_max_hd();        // largest heads * head_dim of the norm backward
hipError_t launch_backward(const BackwardArgs& a);
// bf16 MFMA walks of the backward (bf16, head_dim 128)
bool backward_mfma_supported(const PrefillArgs& a);
hipError_t launch_backward_walk_y(const BackwardArgs& a);
hipError_t launch_backward_walks_grad(const BackwardArgs& a);

// bf16 projection GEMMs on the library's own MFMA kernel: row-major
// Y_p [M][N] = act_p(X [M][K] W_p [K][N]) for p < P, W_p at w + p * wstride
// (rows N apart), Y_p at y + p * ystride (rows N apart); acts holds 2 bits per
// p (0 none, 1 SiLU, 2 logistic), applied to the fp32 accumulators.  Needs
// N % 8 == 0 and K % 64 == 0.
bool gemm_mfma_supported(int64_t M, int N, int K);
hipError_t gemm_bf16_mfma(const void* x, const void* w, void* y, int64_t M, int N, int K, int P,
                          int64_t wstride, int64_t ystride, unsigned acts, hipStream_t st);
// the same products on hipBLASLt (the baseline they are timed against):
// row-major y [rows][n] = act(x [rows][k] w [k][n])
enum class GemmAct { none, silu };
size_t gemm_workspace_bytes();
hipError_t gemm_bf16(const void* x, const void* w, void* y, int64_t rows, int n, int k, GemmAct act,
                     void* workspace, size_t workspace_bytes, hipStream_t st);

struct DecodeArgs {
    const void *q, *k, *v, *g, *w;
    void* out;
    float* state;
    int nseq, H, D;
    float eps;
    bool bf16;
    float* ybuf;   // [nseq][H*D]
    float* ssbuf;  // [nseq][H]
};
hipError_t launch_decode_state(const DecodeArgs& a, hipStream_t st);
hipError_t launch_decode_norm(const DecodeArgs& a, hipStream_t st);
// whether a decode of this shape runs the two-kernel path, which keeps y and
// the sums of squares in scratch memory (else one kernel per sequence, none)
bool decode_uses_workspace(int nseq, int H, int D);
// the fixed scratch of the no-allocation decode: its size, and the current
// device's address of it (looked up on the first call on each device)
size_t decode_scratch_bytes();
hipError_t decode_scratch(void** out);

// --------------------------------------------- softmax attention layer
// The hybrid's softmax layer: rotary embedding on the first rope_dim features,
// then causal softmax attention per sequence (bf16, head_dim 128).  The plan
// cuts the sequences into query tiles of SOFTMAX_TILE tokens.
constexpr int SOFTMAX_TILE = 128;
struct SoftmaxArgs {
    const void *q, *k, *v;
    void* out;
    int H, rope_dim;
    double rope_base;
    float scale;
    int max_tiles;
    PlanHeader* hdr;
    SegEntry* segs;
    ChunkEntry* tiles;   // query tiles, from the plan
    __bf16* kr;          // rotated k [total][H][128] (rope_dim > 0)
};
hipError_t launch_softmax_rope(const SoftmaxArgs& a, hipStream_t st);
hipError_t launch_softmax_fwd(const SoftmaxArgs& a, hipStream_t st);

// One decode step of the softmax layer against a KV cache: the new token's
// key (rotated at position len[s]) and value are appended at slot len[s], and
// its query (rotated likewise) attends over the len[s] + 1 keys.  Keys are
// split into ranges of SOFTMAX_DEC_SPLIT, each a workgroup's partial
// (max, sum, output); a second kernel combines them.
// 768 keys (192 KiB of one (sequence, head)'s keys, and as much of its values):
// with a power-of-two range (512 or 1024 keys: 128 or 256 KiB) the concurrent
// workgroups' streams start at addresses a power of two apart and the step ran
// at 5.5 TB/s; 768 keys gave 6.56 TB/s at 32 sequences x 64 heads with 1K-16K
// cached keys (640-1536 keys, 704 aside: 6.41-6.65 TB/s, measured on one MI355X).
#ifndef LA_SM_DEC_SPLIT
#define LA_SM_DEC_SPLIT 768
#endif
constexpr int SOFTMAX_DEC_SPLIT = LA_SM_DEC_SPLIT;
struct SoftmaxDecodeArgs {
    const void *q, *k, *v;    // [S][H][128] bf16, the new tokens
    void *k_cache, *v_cache;  // [S][H][max_len][128] bf16 (keys stored rotated)
    const int32_t* len;       // device [S]: tokens already cached
    void* out;                // [S][H][128] bf16
    int nseq, max_len, H, rope_dim;
    double rope_base;
    float scale;
    int nsplit;               // ceil(max_len / SOFTMAX_DEC_SPLIT)
    int32_t* status;          // device [S]: 1 where len is outside [0, max_len), else 0
    float* qr;                // [S][H][128] rotated queries, fp32
    float* part;              // [S][H][nsplit][2 + 128]: max, sum, output
};
hipError_t launch_softmax_decode(const SoftmaxDecodeArgs& a, hipStream_t st);

}  // namespace la
