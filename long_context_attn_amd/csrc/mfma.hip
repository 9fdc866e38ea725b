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
// global loads of the next block, SiLU in fp32, bf16 tiles in LDS, the final
// stores), waves 0-3 are consumers (the matrix products).  Each SIMD hosts
// one wave of each kind, so the vector-ALU SiLU work overlaps the matrix
// work, and the LDS tiles are double-buffered.
//
// Consumer wave w owns state columns dv in [32w, 32w+32) for all 128 key rows
// in four C tiles (64 fp32 registers per lane): the state never leaves
// registers during a walk, and the inter-block product reads it straight from
// the accumulators -- transposed, S^T is an A operand whose rows are the
// lane's own column dv, and the k permutation of the C layout is matched in
// the Q~ operand.
//
// LDS tiles are token-major, 64 rows of 128 bf16 (256 bytes) with the 16-byte
// chunk index of every row XOR-swizzled by f(row) = 4 (row & 3) + (row >> 2 & 3).
// Operands that reduce over features are read along rows (16 consecutive rows
// of one chunk: f is a bijection on them); operands that reduce over tokens
// (K~^T, V~^T) use the gfx950 transposing load, whose 16-lane groups read 4
// consecutive rows x 4 aligned chunks (f maps them to 16 distinct chunks).
// Both patterns are free of LDS bank conflicts.
#include "la_internal.h"

namespace la {

constexpr int MD = 128;        // head_dim
constexpr int MB = 64;         // block tokens
constexpr int NTHREADS = 512;  // 4 consumer + 4 producer waves
constexpr int TILE = MB * MD;  // elements of one swizzled tile
constexpr int PP = MB + 8;     // pitch of the score tile
constexpr int YP = MD + 8;     // pitch of the y staging tiles (rows 16-byte aligned)

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int RGRP = 16;       // heads per sub-reducer group of the RMSNorm exchange

// element offset of (row, col) in a swizzled 64 x 128 tile
__device__ __forceinline__ int swz(int row, int col) {
    const int f = ((row & 3) << 2) | ((row >> 2) & 3);
    return row * MD + ((((col >> 3) ^ f)) << 3) + (col & 7);
}

// gfx950 transposing LDS load: in each group of 16 lanes, lane 4j + r points
// at 4 features of token row0 + j, and lane i of the group receives feature
// c0 + i of tokens row0 .. row0 + 3.
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
__device__ __forceinline__ bf16x4 ld_tr(const __bf16* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}
// MFMA operand with rows = features f0 + lane % 32 and k = tokens
// t0 + 8 (lane / 32) + j, read transposed from a swizzled token-major tile.
__device__ __forceinline__ bf16x8 ld_tr_operand(const __bf16* tile, int t0, int f0, int lane) {
    const int grp = lane >> 4, i = lane & 15;
    const int row = t0 + 8 * (grp >> 1) + (i >> 2);
    const int col = f0 + 16 * (grp & 1) + 4 * (i & 3);
    const bf16x4 lo = ld_tr(tile + swz(row, col));
    const bf16x4 hi = ld_tr(tile + swz(row + 4, col));
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
// MFMA operand with rows = tokens and k = 8 consecutive features at col
__device__ __forceinline__ bf16x8 ld_row_operand(const __bf16* tile, int row, int col) {
    return *reinterpret_cast<const bf16x8*>(tile + swz(row, col));
}

__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
    return __builtin_bit_cast(unsigned, bf16x2{(__bf16)a, (__bf16)b});
}

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

// Buffer resource over rows 0 .. n-1 of a tile whose rows are HD elements
// apart.  The hardware range check makes loads beyond the last row return
// zeros and drops stores there, which handles a chunk's ragged last block
// without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const __bf16* base, int n, int HD) {
    const int bytes = n > 0 ? ((n - 1) * HD + MD) * 2 : 0;
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, bytes, 0x00020000);
}

// voff = byte offset of (row 4 rg, feature 8 cc); rows r are rstride bytes apart
__device__ __forceinline__ void load_tile(Tile& t, __amdgpu_buffer_rsrc_t rs, int voff, int rstride) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
        t.r[r] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, r * rstride, 0));
}

// a producer thread's four 16-byte pieces of a swizzled tile
__device__ __forceinline__ void store_rows(const bf16x8 (&x)[4], __bf16* tile, int cc, int rg) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
        *reinterpret_cast<bf16x8*>(tile + swz(4 * rg + r, 8 * cc)) = x[r];
}

// ------------------------------------------------------------ chunk state
// states[c][h][dk][dv] = sum over the chunk's tokens of k~_dk v~_dv.
// Chunks are visited in descending order so that the walk, which visits
// them in ascending order right after, finds the most recently read K and V
// still in the memory-side cache.
struct StateLds {
    __bf16 k[2][TILE];
    __bf16 v[2][TILE];
};

__global__ __launch_bounds__(NTHREADS) void chunk_state_mfma_kernel(
    const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const PlanHeader* __restrict__ hdr, const ChunkEntry* __restrict__ chunks,
    float* __restrict__ states, uint64_t* __restrict__ part, uint64_t* __restrict__ rsub, int H,
    int slots_per_chunk) {
    __shared__ __attribute__((aligned(16))) StateLds L;
    const int nch = hdr->n_chunks;
    const int cr = blockIdx.x / H, h = blockIdx.x - (blockIdx.x / H) * H;
    if (cr >= nch) return;
    const int c = nch - 1 - cr;
    const ChunkEntry ce = chunks[c];
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    // clear the walk's exchange words of this chunk: part[slot][h][*] of
    // this head, and the group-sum rows rsub[slot][gi][*] with gi % H == h
    const int G = (H + RGRP - 1) / RGRP;
    for (int i = tid; i < slots_per_chunk * MB; i += NTHREADS) {
        const int64_t slot = (int64_t)c * slots_per_chunk + i / MB;
        part[(slot * H + h) * MB + i % MB] = 0;
        for (int gi = h; gi < G; gi += H) rsub[(slot * G + gi) * MB + i % MB] = 0;
    }
    const int HD = H * MD;
    const int64_t off0 = ce.start * (int64_t)HD + (int64_t)h * MD;
    const int nblk = (ce.len + MB - 1) / MB;
    // Every wave loads, applies SiLU and multiplies: the SiLU work is a chain
    // of dependent transcendental operations, and two waves per SIMD hide its
    // latency where one could not.  Thread t loads rows t / 16 and t / 16 + 32
    // of a block, features 8 (t % 16) .. + 7; wave w accumulates the state
    // tiles dk in [64 (w / 4), +64), dv in [32 (w % 4), +32).
    const int cc = tid & 15, rg = tid >> 4;
    const int voff = (rg * HD + 8 * cc) * 2, rstride = 32 * HD * 2;
    // SPF register sets: block b is loaded into set b % SPF, SPF blocks
    // ahead.  Loads are issued unconditionally (blocks past the chunk's end
    // get an empty range and return zeros): a conditional load would make the
    // compiler copy registers that still have a load in flight.
    constexpr int SPF = 4;
    struct Rows {
        bf16x8 r[2];
    };
    Rows tk[SPF], tv[SPF];
    auto load_rows = [&](const __bf16* base, int b, Rows& t) {
        const int t0 = b * MB, n = max(0, min(MB, ce.len - t0));
        const __amdgpu_buffer_rsrc_t rs = tile_rsrc(base + off0 + (int64_t)t0 * HD, n, HD);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            t.r[j] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, j * rstride, 0));
    };
#pragma unroll
    for (int i = 0; i < SPF; ++i) {
        load_rows(k, i, tk[i]);
        load_rows(v, i, tv[i]);
    }
    const int l32 = lane & 31, g = lane >> 5;
    const int n = w & 3, m0 = 2 * (w >> 2);
    f32x16 acc[2] = {};
    for (int b0 = 0; b0 < nblk; b0 += SPF) {
#pragma unroll
        for (int i = 0; i < SPF; ++i) {
            const int b = b0 + i;  // block b goes to LDS buffer b & 1
            if (b >= nblk) break;
            __bf16* sK = L.k[b & 1];
            __bf16* sV = L.v[b & 1];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                *reinterpret_cast<bf16x8*>(sK + swz(rg + 32 * j, 8 * cc)) = silu8(tk[i].r[j]);
                *reinterpret_cast<bf16x8*>(sV + swz(rg + 32 * j, 8 * cc)) = silu8(tv[i].r[j]);
            }
            load_rows(k, b + SPF, tk[i]);
            load_rows(v, b + SPF, tv[i]);
            __syncthreads();
#pragma unroll
            for (int s = 0; s < MB / 16; ++s) {
                const bf16x8 bb = ld_tr_operand(sV, 16 * s, 32 * n, lane);
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[j] = mfma32(ld_tr_operand(sK, 16 * s, 32 * (m0 + j), lane), bb, acc[j]);
            }
        }
    }
    float* dst = states + ((int64_t)c * H + h) * MD * MD;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int dk = 32 * (m0 + j) + 8 * (r >> 2) + 4 * g + (r & 3);
            dst[dk * MD + 32 * n + l32] = acc[j][r];
        }
}

// --------------------------------------------- cross-workgroup exchange
// Exchange words carry a float in the low half and 1 in the high half once
// written.  They are stored and loaded as single 8-byte agent-scope atomics
// (coherent sc1 accesses on gfx950, seen by workgroups on every XCD), so a
// reader sees either the cleared word or the whole value: no fence or flag
// is needed, and a writer never waits for its store to complete.
// Returns the stored word: callers keep it live until their next barrier so
// that its registers are not the target of an LDS read while the store may
// still be waiting to read them.
__device__ __forceinline__ uint64_t put_word(uint64_t* p, float x) {
    const uint64_t word = (uint64_t(1) << 32) | __float_as_uint(x);
    __hip_atomic_store(p, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return word;
}
__device__ __forceinline__ void keep(uint64_t x) { asm volatile("" ::"v"(x)); }
__device__ __forceinline__ uint64_t get_word(uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool written(uint64_t x) { return (x >> 32) != 0; }
__device__ __forceinline__ float word_value(uint64_t x) { return __uint_as_float((uint32_t)x); }

// Bound on the polls of one cross-head wait (each poll is a coherent load,
// about a microsecond): a wait never legitimately lasts longer than one chunk
// walk, so reaching it means the workgroups of a chunk could not all run.
// The kernel then records error 3 in the plan header, every later wait gives
// up at once, and the launch finishes (with an unspecified output).
constexpr int WAIT_POLLS = 1 << 20;

// Called before each further poll of a wait: sleeps briefly and returns
// false once the wait is to be abandoned.
__device__ __forceinline__ bool poll_again(int& polls, PlanHeader* hdr) {
    __builtin_amdgcn_s_sleep(1);
    ++polls;
    if ((polls & 255) == 0 &&
        __hip_atomic_load(&hdr->error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 3)
        return false;
    if (polls >= WAIT_POLLS) {
        __hip_atomic_store(&hdr->error, 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return false;
    }
    return true;
}

// --------------------------------------------- fused chunk walk + RMSNorm
// Workgroups take (chunk, head) items in start order from a ticket, head
// fastest, so all heads of a chunk are started before any head of the next
// chunk: the per-block cross-head waits below only ever wait on workgroups
// that have started (or on earlier chunks that can always finish).
//
// Each iteration has two phases separated by workgroup barriers.  For the
// 64-token block j of chunk c (exchange slot s = c * slots_per_chunk + j):
//   * iteration j: the producers stage Q~, K~ (phase 1) and V~ (phase 2);
//   * iteration j + 1: the consumers compute S^T Q~^T and the scores
//     (phase 1), then V~^T P^T and the state update (phase 2); y is staged
//     as bf16 in LDS ring slot j % 3 and sum_dv y^2 per token is reduced over
//     the four waves; after the second barrier consumer wave 2 writes it to
//     part[s][h][t];
//   * iteration j + 2, phase 1: sub-reducer heads (s * G + g) % H, one per
//     group g of RGRP heads, wait for their group's words and write the
//     group sum to rsub[s][g][t];
//   * iteration j + 3: wave 2 issues the loads of rsub[s][*][t] in phase 1
//     and, at the end of phase 2, adds the G group sums in group order
//     (deterministic) and leaves 1 / sqrt(mean y^2 + eps) in LDS;
//   * iteration j + 4, phase 1: the producers write
//     out = y * rnorm * w * sigmoid(gate), freeing ring slot j % 3 before
//     block j + 3 is staged there in phase 2.
// Only wave 2 touches the exchange words (its score quadrant is empty), and
// no wave with global loads in flight ever waits on them.
constexpr int FIN = 4;      // iterations from a block's staging to its final store
constexpr int YRING = 3;    // y tiles in LDS
constexpr int RPRE = 4;     // group sums whose loads are issued a phase ahead

struct WalkLds {
    __bf16 q[2][TILE];        // Q~
    __bf16 k[2][TILE];        // K~
    __bf16 v[2][TILE];        // V~
    __bf16 y[YRING][MB * YP]; // y of the last blocks (bf16, padded rows), until finalised
    __bf16 p[MB * PP];        // masked scores P [t][t']
    float red[4][MB];         // per-wave sums of y^2 per token
    float rn[2][MB];          // norm factors of the block the producers finalise next
    int item;
};

__global__ __launch_bounds__(NTHREADS) void walk_norm_mfma_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ gate, const __bf16* __restrict__ wgt, __bf16* __restrict__ out,
    PlanHeader* __restrict__ hdr, const ChunkEntry* __restrict__ chunks,
    const float* __restrict__ states, uint64_t* __restrict__ part, uint64_t* __restrict__ rsub,
    int H, int slots_per_chunk, float eps) {
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
    const int iters = nblk + FIN;

    if (w >= 4) {
        // ------------------------------------------------------ producers
        const int ptid = tid - 256;
        const int cc = ptid & 15, rg = ptid >> 4;
        const int voff = (4 * rg * HD + 8 * cc) * 2, rstride = HD * 2;
        const bf16x8 wv = *reinterpret_cast<const bf16x8*>(wgt + h * MD + 8 * cc);
        // Two register sets: q, k, v of block b are loaded into set b & 1 two
        // iterations ahead, and so is the gate of the block that iteration b
        // finalises, so every load has two iterations to arrive.  Loads are
        // issued unconditionally (blocks outside the chunk get an empty range
        // and return zeros): a conditional load would make the compiler copy
        // registers that still have a load in flight.
        Tile q0, k0, v0, g0, q1, k1, v1, g1;
        auto tile_at = [&](const __bf16* base, int blk, Tile& t) {
            const int t0 = blk * MB;
            const int n = blk < 0 ? 0 : max(0, min(MB, ce.len - t0));
            load_tile(t, tile_rsrc(base + off0 + (int64_t)t0 * HD, n, HD), voff, rstride);
        };
        tile_at(q, 0, q0);
        tile_at(k, 0, k0);
        tile_at(v, 0, v0);
        tile_at(q, 1, q1);
        tile_at(k, 1, k1);
        tile_at(v, 1, v1);
        auto step = [&](int b, Tile& tq, Tile& tk, Tile& tv, Tile& tg) {
            const int buf = b & 1;
            // ---- phase 1: finalise block jf (its y in LDS, its norm factors
            // left by wave 2 in the previous iteration), then q, k of block b
            const int jf = b - FIN;
            if (jf >= 0 && jf < nblk) {
                // All LDS reads come before the first output store: an LDS
                // read returning into the data registers of a store that is
                // still waiting to issue has been seen to corrupt them.
                const __bf16* ys = L.y[jf % YRING];
                bf16x8 y[4];
                float rr[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 4 * rg + r;
                    y[r] = *reinterpret_cast<const bf16x8*>(ys + row * YP + 8 * cc);
                    rr[r] = L.rn[jf & 1][row];
                }
                bf16x8 o[4];
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        o[r][u] = (__bf16)((float)y[r][u] * rr[r] * (float)wv[u] *
                                           sigmoid_f((float)tg.r[r][u]));
                __builtin_amdgcn_sched_barrier(0);
                const __amdgpu_buffer_rsrc_t ro =
                    tile_rsrc(out + off0 + (int64_t)jf * MB * HD, min(MB, ce.len - jf * MB), HD);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o[r]), ro, voff,
                                                           r * rstride, 0);
            }
            tile_at(gate, jf + 2, tg);  // finalised in iteration b + 2, same register set
            if (b < nblk) {
                bf16x8 qs[4], ks[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    qs[r] = silu8(tq.r[r]);
                    ks[r] = silu8(tk.r[r]);
                }
                store_rows(qs, L.q[buf], cc, rg);
                store_rows(ks, L.k[buf], cc, rg);
            }
            tile_at(q, b + 2, tq);
            tile_at(k, b + 2, tk);
            __syncthreads();  // A
            // ---- phase 2: v of block b to LDS
            if (b < nblk) {
                bf16x8 vs[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) vs[r] = silu8(tv.r[r]);
                store_rows(vs, L.v[buf], cc, rg);
            }
            tile_at(v, b + 2, tv);
            __syncthreads();  // B
        };
        for (int b = 0; b < iters; b += 2) {
            step(b, q0, k0, v0, g0);
            if (b + 1 < iters) step(b + 1, q1, k1, v1, g1);
        }
        return;
    }

    // ---------------------------------------------------------- consumers
    const int l32 = lane & 31, g = lane >> 5;
    const float inv_hd = 1.0f / (float)HD;
    const int G = (H + RGRP - 1) / RGRP;  // group sums per token
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
    uint64_t held_pub = 0, held_red = 0;  // exchange words stored by wave 2, kept live
    for (int b = 0; b < iters; ++b) {
        const int jc = b - 1;  // block computed in this iteration
        const bool comp = jc >= 0 && jc < nblk;
        const int buf = jc & 1;
        const __bf16* sQ = L.q[buf];
        const __bf16* sK = L.k[buf];
        const __bf16* sV = L.v[buf];
        // ---- phase 1 (wave 2): issue the loads of block jn's group sums
        const int jn = b - 3;
        const bool fetch = w == 2 && jn >= 0 && jn < nblk;
        uint64_t* fsrc = rsub + (int64_t)(slot0 + jn) * G * MB + lane;
        uint64_t fx[RPRE];
        if (fetch) {
#pragma unroll
            for (int i = 0; i < RPRE; ++i) fx[i] = i < G ? get_word(fsrc + i * MB) : (uint64_t(1) << 32);
        }
        // ---- phase 1 (wave 2): sub-reduce block jr = b - 2 if this head is
        // one of its sub-reducers
        if (w == 2 && b - 2 >= 0 && b - 2 < nblk) {
            const int slot = slot0 + b - 2;
            const int gi = (int)(((int64_t)h - (int64_t)slot * G) % H + H) % H;  // group served
            if (gi < G) {
                const int h0 = gi * RGRP, n = min(RGRP, H - h0);
                uint64_t* src = part + ((int64_t)slot * H + h0) * MB + lane;
                uint64_t x[RGRP];
                int polls = 0;
                for (;;) {
                    bool all = true;
#pragma unroll
                    for (int i = 0; i < RGRP; ++i) {
                        x[i] = i < n ? get_word(src + i * MB) : (uint64_t(1) << 32);
                        all = all && written(x[i]);
                    }
                    if (all || !poll_again(polls, hdr)) break;
                }
                float tot = 0.f;
#pragma unroll
                for (int i = 0; i < RGRP; ++i) tot += word_value(x[i]);
                held_red = put_word(rsub + ((int64_t)slot * G + gi) * MB + lane, tot);
            }
        }
        // ---- phase 1: S^T Q~^T into O, and the scores of block jc (the
        // quadrant t' > t stays unread)
        f32x16 O[2] = {};
        if (comp) {
            // S^T as bf16 A operands: accumulator registers r0 .. r0 + 7 of
            // tile m hold dk = 16 s + 8 (j / 4) + 4 g + j % 4; one exchange
            // between the lane halves turns that into dk = 16 s + 8 g + j, so
            // that the matching Q~ operand is one 16-byte row read.
#pragma unroll
            for (int s = 0; s < MD / 16; ++s) {
                const int m = s >> 1, r0 = 8 * (s & 1);
                unsigned p0 = pack_bf16(S[m][r0 + 0], S[m][r0 + 1]);
                unsigned p1 = pack_bf16(S[m][r0 + 2], S[m][r0 + 3]);
                unsigned p2 = pack_bf16(S[m][r0 + 4], S[m][r0 + 5]);
                unsigned p3 = pack_bf16(S[m][r0 + 6], S[m][r0 + 7]);
                const auto x02 = __builtin_amdgcn_permlane32_swap(p0, p2, false, false);
                const auto x13 = __builtin_amdgcn_permlane32_swap(p1, p3, false, false);
                const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{x02[0], x13[0], x02[1], x13[1]});
#pragma unroll
                for (int tb = 0; tb < 2; ++tb)
                    O[tb] = mfma32(a, ld_row_operand(sQ, 32 * tb + l32, 16 * s + 8 * g), O[tb]);
            }
            if (!(qa == 1 && qb == 0)) {
                f32x16 pacc = {};
#pragma unroll
                for (int s = 0; s < MD / 16; ++s)
                    pacc = mfma32(ld_row_operand(sK, 32 * qa + l32, 16 * s + 8 * g),
                                  ld_row_operand(sQ, 32 * qb + l32, 16 * s + 8 * g), pacc);
                const int t = 32 * qb + l32;
#pragma unroll
                for (int qd = 0; qd < 4; ++qd) {
                    const int tp0 = 32 * qa + 8 * qd + 4 * g;
                    bf16x4 o;
#pragma unroll
                    for (int u = 0; u < 4; ++u) o[u] = (__bf16)(tp0 + u <= t ? pacc[4 * qd + u] : 0.f);
                    *reinterpret_cast<bf16x4*>(L.p + t * PP + tp0) = o;
                }
            }
        }
        __syncthreads();  // A
        keep(held_pub);
        keep(held_red);
        // ---- phase 2: V~^T P^T into O, state update, y staging
        if (comp) {
            bf16x8 vop[MB / 16];  // V~^T operands, shared by both tiles and the state update
#pragma unroll
            for (int s = 0; s < MB / 16; ++s) vop[s] = ld_tr_operand(sV, 16 * s, 32 * w, lane);
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                for (int s = 0; s < MB / 16; ++s) {
                    if (tb == 0 && s >= 2) continue;  // t < 32 sees only t' < 32
                    const bf16x8 bb = *reinterpret_cast<const bf16x8*>(L.p + (32 * tb + l32) * PP + 16 * s + 8 * g);
                    O[tb] = mfma32(vop[s], bb, O[tb]);
                }
#pragma unroll
            for (int s = 0; s < MB / 16; ++s)
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    S[m] = mfma32(ld_tr_operand(sK, 16 * s, 32 * m, lane), vop[s], S[m]);
            // per-token sum of y^2 over this wave's 32 columns; y staged as bf16
            __bf16* ys = L.y[jc % YRING];
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
                    *reinterpret_cast<bf16x4*>(ys + t * YP + 32 * w + 8 * qd + 4 * g) = y;
                }
            }
        }
        // ---- end of phase 2 (wave 2): norm factors of block jn for the
        // producers' next phase 1
        if (fetch) {
            float tot = 0.f;
            int polls = 0;
#pragma unroll
            for (int i = 0; i < RPRE; ++i) {
                while (!written(fx[i]) && poll_again(polls, hdr)) fx[i] = get_word(fsrc + i * MB);
                tot += word_value(fx[i]);
            }
            for (int i = RPRE; i < G; ++i) {
                uint64_t x = get_word(fsrc + i * MB);
                while (!written(x) && poll_again(polls, hdr)) x = get_word(fsrc + i * MB);
                tot += word_value(x);
            }
            L.rn[jn & 1][lane] = __builtin_amdgcn_rsqf(tot * inv_hd + eps);
        }
        __syncthreads();  // B
        // ---- after phase 2 (wave 2): publish block jc's sums of squares (the
        // store is not waited for)
        if (w == 2 && comp) {
            const float mine = L.red[0][lane] + L.red[1][lane] + L.red[2][lane] + L.red[3][lane];
            held_pub = put_word(part + ((int64_t)(slot0 + jc) * H + h) * MB + lane, mine);
        }
    }
}

bool mfma_supported(const PrefillArgs& a) { return a.bf16 && a.D == MD && a.block == MB; }

hipError_t launch_chunk_state_mfma(const PrefillArgs& a, hipStream_t st) {
    if (a.max_chunks == 0) return hipSuccess;
    const dim3 grid((unsigned)((int64_t)a.max_chunks * a.H));
    hipLaunchKernelGGL(chunk_state_mfma_kernel, grid, dim3(NTHREADS), 0, st, (const __bf16*)a.k,
                       (const __bf16*)a.v, a.hdr, a.chunks, a.states, a.part, a.rsub, a.H,
                       a.chunk / MB);
    return hipGetLastError();
}

hipError_t launch_walk_mfma(const PrefillArgs& a, hipStream_t st) {
    if (a.max_chunks == 0) return hipSuccess;
    const dim3 grid((unsigned)((int64_t)a.max_chunks * a.H));
    hipLaunchKernelGGL(walk_norm_mfma_kernel, grid, dim3(NTHREADS), 0, st, (const __bf16*)a.q,
                       (const __bf16*)a.k, (const __bf16*)a.v, (const __bf16*)a.g,
                       (const __bf16*)a.w, (__bf16*)a.out, a.hdr, a.chunks, a.states, a.part,
                       a.rsub, a.H, a.chunk / MB, a.eps);
    return hipGetLastError();
}

}  // namespace la
