// Projection GEMMs of the Lightning Attention layer on bf16 MFMA for gfx950.
//
// Mechanism step 1 of "Diving into MiniMax01 405B MoE" (section "Hybrid
// Modeling"): q, k, v and the gate are linear maps of the layer input x, and
// the attention output is mapped back to the hidden size.  One launch computes
//   Y_p [M][N] = act_p(X [M][K] W_p [K][N]),   p = 0 .. P-1,
// row-major, for P weight matrices that share X (the four input projections
// at once, or the output projection alone).  The activation of Mechanism step
// 2 is applied to the fp32 accumulators before the single rounding to bf16:
// SiLU for q, k and v, the logistic function for the gate (the attention
// then multiplies by it as it is), none for the output projection.
//
// Each 512-thread workgroup computes one 256 (n) x 256 (m) tile of
// Y_p^T = W_p^T X^T with v_mfma_f32_32x32x16_bf16 (fp32 accumulation):
//   - A operands (rows n, 16 k) come from the W tile, stored k-major as it
//     lies in memory (two GBK x 128 tiles in the XOR-swizzled layout of
//     mfma_common.h), through the gfx950 transposing LDS read;
//   - B operands (columns m, 16 k) are 16-byte row reads of the X tile, 256
//     rows of GBK features, swizzled so that the 16 rows a group of 16 lanes
//     reads sit on distinct banks.
// Tiles go from memory straight into LDS (buffer loads with the LDS as
// destination, no registers) in GNS stages of GBK = 32 k: the loads of the
// next GNS - 2 stages are in flight while the products of one stage run, and
// the stage after it is complete, so its first operands are read from LDS
// while this stage's last products run.
// Measured at 8192 x 6144 x 32768 (the four input projections): 32-wide
// stages in 4 buffers beat 64-wide ones in 2 by about 13%.
// Wave w owns n in [128 (w & 1), +128) and m in [64 (w >> 1), +64) of the
// tile: 4 x 2 accumulator tiles of 32 x 32 (128 fp32 per lane).  In the
// transposed product each lane ends with 4 consecutive n of one m per
// accumulator group, stored as one 8-byte write.
#include <type_traits>

#include "mfma_common.h"

#ifndef GEMM_BK
#define GEMM_BK 32
#endif
#ifndef GEMM_NS
#define GEMM_NS 4
#endif
#ifndef GEMM_GROUP_M
#define GEMM_GROUP_M 4
#endif
#ifndef GEMM_WAVES
#define GEMM_WAVES 8
#endif
#ifndef GEMM_XPF
#define GEMM_XPF 1
#endif

namespace la {

namespace {

constexpr int GW = GEMM_WAVES;  // waves per workgroup: 4 (128 x 128 each) or 8 (128 x 64)
constexpr int GT = 64 * GW;     // threads per workgroup
constexpr int WM = 512 / GW;    // tokens (m) per wave
constexpr int NJ = WM / 32;     // 32-token accumulator tiles per wave
constexpr int GBM = 256;      // m (tokens) per tile
constexpr int GBN = 256;      // n (output features) per tile
constexpr int GBK = GEMM_BK;  // k per LDS stage
constexpr int GNS = GEMM_NS;  // LDS stages (loads run GNS - 1 stages ahead)
constexpr int GXT = GBM * GBK;  // elements of an X stage tile
constexpr int GWT = GBK * MD;   // elements of one W half tile (GBK k x 128 n)
constexpr int GROUP_M = GEMM_GROUP_M;  // tile rows per raster group
constexpr int GCPR = GBK / 8;          // 16-byte chunks per X tile row
constexpr int GRPW = 128 / GBK;        // X tile rows per 256-byte span of banks

// The stage buffers are separate LDS variables, indexed by compile-time
// stage numbers: the compiler then knows that the loads in flight into one
// buffer do not alias the reads of another.  (In one array it has to wait for
// every load in flight before any LDS read, which serialises the loads with
// the products.)
static_assert(GNS >= 2 && GNS <= 4, "2 to 4 stages");
__shared__ __attribute__((aligned(16))) __bf16 gx0[GXT], gx1[GXT], gx2[GXT], gx3[GXT];
__shared__ __attribute__((aligned(16))) __bf16 gw0[2 * GWT], gw1[2 * GWT], gw2[2 * GWT],
    gw3[2 * GWT];
template <int S>
__device__ __forceinline__ __bf16* stage_x() {
    if constexpr (S == 0) return gx0;
    else if constexpr (S == 1) return gx1;
    else if constexpr (S == 2) return gx2;
    else return gx3;
}
template <int S>
__device__ __forceinline__ __bf16* stage_w() {
    if constexpr (S == 0) return gw0;
    else if constexpr (S == 1) return gw1;
    else if constexpr (S == 2) return gw2;
    else return gw3;
}

// element offset of (row, col) in an X stage tile: rows of GBK features;
// 16-byte chunk c of row r stored at chunk c ^ ((r / GRPW) % GCPR), so that
// the 16 rows a group of 16 lanes reads at one chunk fall on distinct banks
__device__ __forceinline__ int xswz(int row, int col) {
    return row * GBK + ((((col >> 3) ^ ((row / GRPW) % GCPR))) << 3) + (col & 7);
}

struct GemmParams {
    const __bf16* x;   // X [M][K], rows ldx elements apart
    const __bf16* w;   // W_p at w + p * wstride: [K][N], rows ldw apart
    __bf16* y;         // Y_p at y + p * ystride: [M][N], rows ldy apart
    int64_t ldx, ldw, wstride, ldy, ystride;
    int M, N, K, P;
    unsigned acts;     // 2 bits per p: 0 none, 1 SiLU, 2 logistic
    int tiles_m, tiles_n;  // tiles per Y_p
};

__device__ __forceinline__ float gemm_act(float v, unsigned act) {
    return act == 1 ? silu_f(v) : (act == 2 ? sigmoid_f(v) : v);
}

// s_waitcnt with vmcnt = n and the other counters left alone
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__global__ __launch_bounds__(GT) void gemm_bf16_kernel(const GemmParams a) {
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, g = lane >> 5;

    // ---- which tile: consecutive tiles on one XCD (workgroups are handed to
    // the 8 XCDs in turn), then groups of GROUP_M tile rows swept column by
    // column, so that the workgroups of an XCD share their X and W tiles in
    // its L2
    const int tn_all = a.tiles_n * a.P;
    const int total = a.tiles_m * tn_all;
    int t = blockIdx.x;
    if ((total & 7) == 0) t = (t & 7) * (total >> 3) + (t >> 3);
    const int per_group = GROUP_M * tn_all;
    const int grp = t / per_group;
    const int first_m = grp * GROUP_M;
    const int gm = min(GROUP_M, a.tiles_m - first_m);
    const int in = t - grp * per_group;
    const int tm = first_m + in % gm;
    const int tnp = in / gm;
    const int p = tnp / a.tiles_n;
    const int tn = tnp - p * a.tiles_n;
    const int m0 = tm * GBM, n0 = tn * GBN;
    const int mrows = min(GBM, a.M - m0);

    // buffer resources: X rows m0 .. m0 + mrows - 1 (rows past the end are
    // clamped to the last one: their products land in columns never stored);
    // W columns from n0 on, every k row (columns past N read the next row's
    // values, also never stored)
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.x + (int64_t)m0 * a.ldx), (short)0,
        __builtin_amdgcn_readfirstlane((int)(((int64_t)(mrows - 1) * a.ldx + a.K) * 2)), 0x00020000);
    const __bf16* wp = a.w + p * a.wstride + n0;
    const int wcols = min(GBN, a.N - n0);
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)wp, (short)0,
        __builtin_amdgcn_readfirstlane((int)(((int64_t)(a.K - 1) * a.ldw + wcols) * 2)), 0x00020000);

    // One stage: the X tile and the two W half tiles, in loads of 1 KiB (one
    // per wave instruction), GBK / 16 of each per wave; lane l of a load fills
    // physical chunk l of its rows with the logical chunk the swizzle puts
    // there.
    constexpr int XRPI = 1024 / (GBK * 2);  // X rows per load
    constexpr int XLPW = GBM / XRPI / GW;   // X loads per wave (as many W loads)
    constexpr int WLPH = GBK / 4;           // W loads per half tile (4 rows each)
    auto stage = [&](int kt, auto bufc) {
        constexpr int BUF = decltype(bufc)::value;
        __bf16* lx = stage_x<BUF>();
        __bf16* lw = stage_w<BUF>();
        const int k0 = kt * GBK;
#pragma unroll
        for (int ii = 0; ii < XLPW; ++ii) {
            const int e = XLPW * w + ii;
            const int row = XRPI * e + lane / GCPR;
            const int c = (lane % GCPR) ^ ((row / GRPW) % GCPR);
            const int r = min(row, mrows - 1);
            const int vo = (int)(((int64_t)r * a.ldx + k0 + 8 * c) * 2);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                xr, (__attribute__((address_space(3))) void*)(lx + XRPI * e * GBK), 16, vo, 0, 0,
                0);
        }
#pragma unroll
        for (int ii = 0; ii < XLPW; ++ii) {
            const int e = XLPW * w + ii;
            const int h = e / WLPH, row = 4 * (e % WLPH) + (lane >> 4);
            const int f = ((row & 3) << 2) | ((row >> 2) & 3);
            const int c = (lane & 15) ^ f;
            const int vo = (int)(((int64_t)(k0 + row) * a.ldw + MD * h + 8 * c) * 2);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                wr, (__attribute__((address_space(3))) void*)(lw + h * GWT + 4 * (e % WLPH) * MD),
                16, vo, 0, 0, 0);
        }
    };

    const int wn = w & 1, wm = w >> 1;
    f32x16 C[4][NJ] = {};
    const int nk = a.K / GBK;
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    // Step i issues the loads of stage i and computes stage i - (GNS - 1):
    // every load is issued inside the loop (loads issued before it, used only
    // by later passes, make the compiler drain every load at its top).  Each
    // step waits for this wave's loads of the stage it computes and of the
    // one after it (the later stages may still be in flight), then for
    // everyone's; the barrier also frees the buffer the products of the
    // previous step read, which this step's loads refill.  Past the last
    // stage the last one is loaded again, so that every step has the same
    // loads in flight.
    // Operand sets (double-buffered over the 16-k slices of a stage): A from
    // the W tile, B from the X tile of the stage in buffer SB.
    constexpr int KS = GBK / 16;  // 16-k slices per stage
    static_assert(KS % 2 == 0, "an even number of slices per stage");
    bf16x8 A[2][4], B[2][NJ];
    auto operands = [&](auto sbc, int s, int set) {
        constexpr int SB = decltype(sbc)::value;
        const __bf16* sw = stage_w<SB>() + wn * GWT;
        const __bf16* sx = stage_x<SB>();
#pragma unroll
        for (int i = 0; i < 4; ++i) A[set][i] = ld_tr_operand(sw, 16 * s, 32 * i, lane);
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            B[set][j] = *reinterpret_cast<const bf16x8*>(
                sx + xswz(WM * wm + 32 * j + l32, 16 * s + 8 * g));
    };
    // With XPF, a step waits for one more stage (the one computed next) and
    // reads that stage's first operands while its own last products run, so
    // no step starts with a wait on LDS: the loads then run GNS - 2 stages
    // ahead instead of GNS - 1.
    constexpr bool XPF = GEMM_XPF != 0;
    static_assert(!XPF || GNS >= 3, "the cross-stage operand read needs 3 stages");
    auto step = [&](int i, auto sc) {
        constexpr int S = decltype(sc)::value;  // buffer of stage i
        constexpr int SC = (S + 1) % GNS;       // buffer of stage i - (GNS - 1)
        constexpr int SN = (S + 2) % GNS;       // buffer of the stage after it
        const int kc = i - (GNS - 1);           // stage computed
        wait_vm<2 * XLPW * (XPF ? GNS - 3 : GNS - 2)>();
        // a bare barrier: nothing but these loads needs ordering, and a
        // barrier with a fence would also wait for the later stages' loads
        __builtin_amdgcn_s_barrier();
        stage(min(i, nk - 1), sc);
        if (kc < 0 || kc >= nk) return;
        if (!XPF || kc == 0) operands(std::integral_constant<int, SC>{}, 0, 0);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            // the next stage's first operands are read unconditionally (after
            // the last stage they read a buffer whose values go unused): with
            // the read under a condition, the compiler merged the two paths
            // and waited for every LDS read before the products that follow
            // (lgkmcnt 0-1 instead of 10-11), 1.5-2.5% of the layer call
            if (s + 1 < KS) operands(std::integral_constant<int, SC>{}, s + 1, (s + 1) & 1);
            else if (XPF) operands(std::integral_constant<int, SN>{}, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j) C[i][j] = mfma32(A[s & 1][i], B[s & 1][j], C[i][j]);
        }
    };
    // whole passes of GNS steps (the steps past the last computed stage only
    // load): with no step skipped inside a pass, the compiler sees the same
    // loads in flight on every path and keeps its waits partial
    const int steps = nk + GNS - 1;
    for (int i = 0; i < steps; i += GNS) {
        step(i, I0{});
        step(i + 1, I1{});
        if constexpr (GNS > 2) step(i + 2, I2{});
        if constexpr (GNS > 3) step(i + 3, I3{});
    }
    wait_vm<0>();

    // ---- epilogue: activation in fp32, 4 consecutive n per 8-byte store.
    // Every value and address is formed before the first store, and the
    // stored registers stay allocated to the end: a register a store is still
    // reading must not be rewritten (see put_word in mfma_common.h).
    const unsigned act = (a.acts >> (2 * p)) & 3u;
    __bf16* yp = a.y + p * a.ystride;
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    u32x2 data[4][NJ][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                data[i][j][q] = u32x2{
                    pack_bf16(gemm_act(C[i][j][4 * q], act), gemm_act(C[i][j][4 * q + 1], act)),
                    pack_bf16(gemm_act(C[i][j][4 * q + 2], act), gemm_act(C[i][j][4 * q + 3], act))};
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int m = m0 + WM * wm + 32 * j + l32;
        if (m < a.M) {
            __bf16* row = yp + (int64_t)m * a.ldy;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int n = n0 + MD * wn + 32 * i + 8 * q + 4 * g;
                    if (n < a.N) *reinterpret_cast<u32x2*>(row + n) = data[i][j][q];
                }
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) asm volatile("" ::"v"(data[i][j][q]));
}

}  // namespace

bool gemm_mfma_supported(int64_t M, int N, int K) {
    return M >= 0 && N > 0 && K > 0 && N % 8 == 0 && K % GBK == 0 &&
           (int64_t)GBM * K * 2 < ((int64_t)1 << 31) && (int64_t)K * N * 2 < ((int64_t)1 << 31);
}

hipError_t gemm_bf16_mfma(const void* x, const void* w, void* y, int64_t M, int N, int K, int P,
                          int64_t wstride, int64_t ystride, unsigned acts, hipStream_t st) {
    if (M == 0 || P == 0) return hipSuccess;
    if (!gemm_mfma_supported(M, N, K)) return hipErrorInvalidValue;
    GemmParams a{};
    a.x = (const __bf16*)x;
    a.w = (const __bf16*)w;
    a.y = (__bf16*)y;
    a.ldx = K;
    a.ldw = N;
    a.wstride = wstride;
    a.ldy = N;
    a.ystride = ystride;
    a.M = (int)M;
    a.N = N;
    a.K = K;
    a.P = P;
    a.acts = acts;
    a.tiles_m = (int)((M + GBM - 1) / GBM);
    a.tiles_n = (N + GBN - 1) / GBN;
    const int64_t grid = (int64_t)a.tiles_m * a.tiles_n * P;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(gemm_bf16_kernel, dim3((unsigned)grid), dim3(GT), 0, st, a);
    return hipGetLastError();
}

}  // namespace la
