// Device helpers shared by the bf16 MFMA prefill kernels for gfx950
// (head_dim 128, 64-token blocks): LDS tile layout and operand loads, the
// MFMA wrapper, SiLU on bf16 vectors, range-checked buffer tiles, and the
// tagged words and bounded waits of cross-workgroup exchanges.
//
// LDS tiles are token-major, 64 rows of 128 bf16 (256 bytes) with the 16-byte
// chunk index of every row XOR-swizzled by f(row) = 4 (row & 3) + (row >> 2 & 3).
// Operands that reduce over features are read along rows (16 consecutive rows
// of one chunk: f is a bijection on them); operands that reduce over tokens
// (K~^T, V~^T) use the gfx950 transposing load, whose 16-lane groups read 4
// consecutive rows x 4 aligned chunks (f maps them to 16 distinct chunks).
// Both patterns are free of LDS bank conflicts.
#pragma once

#include "la_internal.h"

namespace la {

constexpr int MD = 128;        // head_dim
constexpr int MB = 64;         // block tokens
constexpr int TILE = MB * MD;  // elements of one swizzled tile

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

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

// SiLU when ACT, else the value as it is (operands already activated)
template <bool ACT>
__device__ __forceinline__ bf16x8 act8(bf16x8 x);
__device__ __forceinline__ bf16x8 silu8(bf16x8 x) {
    bf16x8 o;
#pragma unroll
    for (int u = 0; u < 8; ++u) o[u] = (__bf16)silu_f((float)x[u]);
    return o;
}
template <bool ACT>
__device__ __forceinline__ bf16x8 act8(bf16x8 x) {
    if constexpr (ACT) return silu8(x);
    else return x;
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
// The byte count is read back into a scalar register: a clamp of a uniform
// value can be computed in a vector register, and a resource built from one
// is taken as divergent (every access then loops over the lanes).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const __bf16* base, int n, int HD) {
    const int bytes = __builtin_amdgcn_readfirstlane(n > 0 ? ((n - 1) * HD + MD) * 2 : 0);
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, bytes, 0x00020000);
}

// voff = byte offset of (row 4 rg, feature 8 cc); rows r are rstride bytes
// apart; AUX = cache policy bits of the loads
template <int AUX = 0>
__device__ __forceinline__ void load_tile(Tile& t, __amdgpu_buffer_rsrc_t rs, int voff, int rstride) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
        t.r[r] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, r * rstride, AUX));
}

// a producer thread's four 16-byte pieces of a swizzled tile
__device__ __forceinline__ void store_rows(const bf16x8 (&x)[4], __bf16* tile, int cc, int rg) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
        *reinterpret_cast<bf16x8*>(tile + swz(4 * rg + r, 8 * cc)) = x[r];
}

// --------------------------------------------- cross-workgroup exchange
// Exchange words carry a float in the low half and 1 in the high half once
// written.  They are stored and loaded as single 8-byte agent-scope atomics
// (coherent sc1 accesses on gfx950, seen by workgroups on every XCD), so a
// reader sees either the cleared word or the whole value: no fence or flag
// is needed, and a writer never waits for its store to complete.
// Returns the stored word: callers keep it live until their next barrier.
//
// A vector-memory store reads its data registers for some cycles after it
// issues, and a write to those registers in that window (a VALU result, an
// LDS or global load returning) has been seen to replace part of the stored
// data.  Every store's data therefore stays allocated, through keep(), until
// after the workgroup's next barrier.
__device__ __forceinline__ uint64_t put_word(uint64_t* p, float x) {
    const uint64_t word = (uint64_t(1) << 32) | __float_as_uint(x);
    __hip_atomic_store(p, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return word;
}
__device__ __forceinline__ void keep(uint64_t x) { asm volatile("" ::"v"(x)); }
__device__ __forceinline__ void keep(u32x4 x) { asm volatile("" ::"v"(x)); }
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
// false once the wait is to be abandoned.  The first wait to give up records
// its site, chunk and head in the plan header.
__device__ __forceinline__ bool poll_again(int& polls, PlanHeader* hdr, int site, int c, int h) {
    __builtin_amdgcn_s_sleep(1);
    ++polls;
    if ((polls & 255) == 0 &&
        __hip_atomic_load(&hdr->error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 3)
        return false;
    if (polls >= WAIT_POLLS) {
        int expected = 0;
        if (__hip_atomic_compare_exchange_strong(&hdr->error, &expected, 3, __ATOMIC_RELAXED,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
            __hip_atomic_store(&hdr->wait_site, site, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&hdr->wait_chunk, c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&hdr->wait_head, h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            __hip_atomic_store(&hdr->error, 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        return false;
    }
    return true;
}

// cache-policy operand of the buffer builtins selecting sc1 (device-coherent)
constexpr int SC1 = 16;

}  // namespace la
