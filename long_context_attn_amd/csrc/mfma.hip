// bf16 MFMA prefill walk of the Lightning Attention layer for gfx950
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
// The kernel runs 8 waves per workgroup: waves 4-7 are producers (16-byte
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
// the Q~ operand.  The LDS tile layout is described in mfma_common.h.
#include "mfma_common.h"

namespace la {

constexpr int NTHREADS = 512;  // 4 consumer + 4 producer waves
constexpr int PP = MB + 8;     // pitch of the score tile
constexpr int YP = MD + 8;     // pitch of the y staging tiles (rows 16-byte aligned)
constexpr int RGRP = 16;       // heads per sub-reducer group of the RMSNorm exchange

// --------------------------------------------- prefill walk
// Second pass of the two-pass prefill.  The plan cut the sequences into
// chunks; chunk_state_mfma_kernel summed K~^T V~ over every chunk but each
// sequence's last, and state_scan_kernel turned those sums into the state
// entering each chunk, entry[c][h] ([dk][dv] layout, the initial state
// included).  Every (chunk, head) item then walks its chunk from that state.
// Workgroups take items in start order from a ticket, chunk major and head
// fastest, so all heads of a chunk are started before any head of the next
// one: the cross-head RMSNorm exchange only ever waits on started items.
//
// An item runs nblk + FIN iterations of two phases (barriers A and B).  Per
// 64-token block j of the chunk (exchange slot s = c * slots_per_chunk + j):
//   - iteration j: the producers stage Q~, K~ (phase 1) and V~ (phase 2);
//   - iteration j + 1: the consumers compute S^T Q~^T and the scores (phase
//     1), then V~^T P^T and the state update (phase 2); y is staged as bf16
//     in LDS ring slot j % 3, sum_dv y^2 per token is reduced over the four
//     waves, and after barrier B consumer wave 2 writes it to part[s][h][t];
//   - iteration j + 2, phase 1: sub-reducer heads (s * G + g) % H, one per
//     group g of RGRP heads, wait for their group's words and write the group
//     sum to rsub[s][g][t];
//   - iteration j + 3: wave 2 issues the loads of rsub[s][*][t] in phase 1
//     and, at the end of phase 2, adds the G group sums in group order
//     (deterministic) and leaves 1 / sqrt(mean y^2 + eps) in LDS;
//   - iteration j + 4, phase 1: the producers write
//     out = y * rnorm * w * sigmoid(gate), freeing ring slot j % 3 before
//     block j + 3 is staged there in phase 2.
// The state enters the consumers' registers in phase 2 of iteration 0.  Only
// wave 2 touches the exchange words (its score quadrant is empty), and no
// wave with global loads in flight waits on them.  Q, K, V and the gate are
// streamed with the non-temporal hint, and so is the output.
constexpr int FIN = 4;      // iterations from a block's staging to its final store
constexpr int YRING = 3;    // y tiles in LDS
constexpr int RPRE = 4;     // group sums whose loads are issued a phase ahead
constexpr int NT = 2;       // cache policy of streamed loads and stores: non-temporal

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

// ACT: apply SiLU to q, k, v on load; without it they arrive activated (a
// projection whose epilogue applied SiLU).  GSIG: apply the logistic function
// to the gate when the outputs are finalised; without it the gate arrives as
// sigmoid(gate) (the projection's epilogue applied it).
template <bool ACT, bool GSIG>
__global__ __launch_bounds__(NTHREADS) void prefill_mfma_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ gate, const __bf16* __restrict__ wgt, __bf16* __restrict__ out,
    __bf16* __restrict__ y_save, PlanHeader* __restrict__ hdr, const SegEntry* __restrict__ segs,
    const ChunkEntry* __restrict__ chunks, const float* __restrict__ init_state,
    float* __restrict__ final_state, const float* __restrict__ entry,
    uint64_t* __restrict__ part, uint64_t* __restrict__ rsub, int H, int nseq,
    int slots_per_chunk, float eps) {
    __shared__ __attribute__((aligned(16))) WalkLds L;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    if (tid == 0) L.item = atomicAdd(&hdr->ticket, 1);
    __syncthreads();
    // uniform across the workgroup: read into a scalar register, so that
    // everything derived from it (chunk, head, buffer resources) is scalar too
    // (an LDS value is otherwise taken as divergent, and every buffer access
    // built from it becomes a loop over lanes)
    const int64_t item = __builtin_amdgcn_readfirstlane(L.item);
    const int64_t n_items = (int64_t)hdr->n_chunks * H;
    const int64_t DD = (int64_t)MD * MD;
    if (item >= n_items) {
        // tickets past the chunk items: final states of empty sequences
        const int64_t s = item - n_items;
        if (final_state != nullptr && s < nseq && segs[s].count == 0)
            for (int64_t i = tid; i < H * DD; i += NTHREADS)
                final_state[s * H * DD + i] = init_state ? init_state[s * H * DD + i] : 0.f;
        return;
    }
    const int c = (int)(item / H), h = (int)(item - (int64_t)c * H);
    const ChunkEntry ce = chunks[c];
    const SegEntry se = segs[ce.seg];
    const bool last = c == se.first + se.count - 1;
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
        // Two register sets: the tiles of block i are loaded into set i & 1
        // two iterations ahead, and so is the gate of the block that
        // iteration i finalises.  Loads are issued unconditionally (blocks
        // outside the chunk get an empty range and return zeros): a
        // conditional load would make the compiler copy registers that still
        // have a load in flight.
        auto rows = [&](int blk) { return blk < 0 ? 0 : max(0, min(MB, ce.len - blk * MB)); };
        auto load = [&](const __bf16* base, int blk, Tile& t) {
            load_tile<NT>(t, tile_rsrc(base + off0 + (int64_t)max(blk, 0) * MB * HD, rows(blk), HD),
                          voff, rstride);
        };
        Tile q0, k0, v0, g0, q1, k1, v1, g1;
        load(q, 0, q0);
        load(k, 0, k0);
        load(v, 0, v0);
        load(q, 1, q1);
        load(k, 1, k1);
        load(v, 1, v1);
        auto step = [&](int it, Tile& tq, Tile& tk, Tile& tv, Tile& tg) {
            const int buf = it & 1;
            const int b = it;  // block staged in this iteration
            // ---- phase 1: finalise block jf (its y in LDS, its norm factors
            // left by wave 2 in the previous iteration), then stage q and k
            const int jf = b - FIN;
            u32x4 od[4];  // stored output, kept live until barrier A
            u32x4 oy[4];  // stored y (y_save), likewise
            if (jf >= 0 && jf < nblk) {
                // All LDS reads come before the first output store (their
                // results must not land in registers a store is reading).
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
                                           (GSIG ? sigmoid_f((float)tg.r[r][u])
                                                 : (float)tg.r[r][u]));
                __builtin_amdgcn_sched_barrier(0);
                const __amdgpu_buffer_rsrc_t ro =
                    tile_rsrc(out + off0 + (int64_t)jf * MB * HD, rows(jf), HD);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    od[r] = __builtin_bit_cast(u32x4, o[r]);
                    __builtin_amdgcn_raw_buffer_store_b128(od[r], ro, voff, r * rstride, NT);
                }
                if (y_save != nullptr) {
                    const __amdgpu_buffer_rsrc_t ry =
                        tile_rsrc(y_save + off0 + (int64_t)jf * MB * HD, rows(jf), HD);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        oy[r] = __builtin_bit_cast(u32x4, y[r]);
                        __builtin_amdgcn_raw_buffer_store_b128(oy[r], ry, voff, r * rstride, NT);
                    }
                }
            }
            load(gate, jf + 2, tg);  // finalised in iteration it + 2, same register set
            if (b < nblk) {
                bf16x8 qs[4], ks[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    qs[r] = act8<ACT>(tq.r[r]);
                    ks[r] = act8<ACT>(tk.r[r]);
                }
                store_rows(qs, L.q[buf], cc, rg);
                store_rows(ks, L.k[buf], cc, rg);
            }
            load(q, it + 2, tq);
            load(k, it + 2, tk);
            __syncthreads();  // A
            if (jf >= 0 && jf < nblk) {
#pragma unroll
                for (int r = 0; r < 4; ++r) keep(od[r]);
                if (y_save != nullptr)
#pragma unroll
                    for (int r = 0; r < 4; ++r) keep(oy[r]);
            }
            // ---- phase 2: stage V~
            if (b < nblk) {
                bf16x8 vs[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) vs[r] = act8<ACT>(tv.r[r]);
                store_rows(vs, L.v[buf], cc, rg);
            }
            load(v, it + 2, tv);
            __syncthreads();  // B
        };
        for (int it = 0; it < iters; it += 2) {
            step(it, q0, k0, v0, g0);
            if (it + 1 < iters) step(it + 1, q1, k1, v1, g1);
        }
        return;
    }

    // ---------------------------------------------------------- consumers
    const int l32 = lane & 31, g = lane >> 5;
    const float inv_hd = 1.0f / (float)HD;
    const int G = (H + RGRP - 1) / RGRP;  // group sums per token
    // accumulator register r of tile m in this lane holds state entry
    // dk = 32 m + 8 (r / 4) + 4 g + r % 4, dv = 32 w + l32
    const int dv = 32 * w + l32;
    // the walk's running state (this wave's 32 columns)
    f32x16 S[4] = {};
    const int qa = w >> 1, qb = w & 1;  // score quadrant: t' in [32 qa, +32), t in [32 qb, +32)
    uint64_t held_pub = 0, held_red = 0;  // exchange words stored by wave 2, kept live
    for (int it = 0; it < iters; ++it) {
        const int b = it;
        const int jc = b - 1;   // block computed in this iteration
        const bool comp = jc >= 0 && jc < nblk;
        const int buf = (it - 1) & 1;  // tiles staged in the previous iteration
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
        // ---- phase 1 (wave 2): sub-reduce block b - 2 if this head is one of
        // its sub-reducers
        if (w == 2 && b - 2 >= 0 && b - 2 < nblk) {
            const int slot = slot0 + b - 2;
            const int gi = (int)(((int64_t)h - (int64_t)slot * G) % H + H) % H;  // group served
            if (gi < G) {
                const int h0 = gi * RGRP, n = min(RGRP, H - h0);
                uint64_t* src = part + ((int64_t)slot * H + h0) * MB + lane;
                // loads are issued in one batch (one round trip); a batch with
                // a word not yet written is reloaded
                uint64_t x[RGRP];
                int polls = 0;
                for (;;) {
                    bool all = true;
#pragma unroll
                    for (int i = 0; i < RGRP; ++i) {
                        x[i] = i < n ? get_word(src + i * MB) : (uint64_t(1) << 32);
                        all = all && written(x[i]);
                    }
                    if (all || !poll_again(polls, hdr, 1, c, h)) break;
                }
                float tot = 0.f;
#pragma unroll
                for (int i = 0; i < RGRP; ++i) tot += word_value(x[i]);
                held_red = put_word(rsub + ((int64_t)slot * G + gi) * MB + lane, tot);
            }
        }
        // ---- phase 1: walk: S^T Q~^T into O, and the scores of block jc
        // (the quadrant t' > t stays unread)
        f32x16 O[2] = {};
        if (comp) {
            // S^T as bf16 A operands: accumulator registers r0 .. r0 + 7 of
            // tile m hold dk = 16 s + 8 (j / 4) + 4 g + j % 4; one exchange
            // between the lane halves turns that into dk = 16 s + 8 g + j, so
            // that the matching Q~ operand is one 16-byte row read.
            // (Q~ operands loaded half of the features at a time)
            bf16x8 qo[MD / 32][2];
#pragma unroll
            for (int s = 0; s < MD / 16; ++s) {
                if (s % (MD / 32) == 0) {
#pragma unroll
                    for (int i = 0; i < MD / 32; ++i)
#pragma unroll
                        for (int tb = 0; tb < 2; ++tb)
                            qo[i][tb] = ld_row_operand(sQ, 32 * tb + l32, 16 * (s + i) + 8 * g);
                    __builtin_amdgcn_sched_barrier(0);
                }
                const int m = s >> 1, r0 = 8 * (s & 1);
                unsigned p0 = pack_bf16(S[m][r0 + 0], S[m][r0 + 1]);
                unsigned p1 = pack_bf16(S[m][r0 + 2], S[m][r0 + 3]);
                unsigned p2 = pack_bf16(S[m][r0 + 4], S[m][r0 + 5]);
                unsigned p3 = pack_bf16(S[m][r0 + 6], S[m][r0 + 7]);
                const auto x02 = __builtin_amdgcn_permlane32_swap(p0, p2, false, false);
                const auto x13 = __builtin_amdgcn_permlane32_swap(p1, p3, false, false);
                const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{x02[0], x13[0], x02[1], x13[1]});
#pragma unroll
                for (int tb = 0; tb < 2; ++tb) O[tb] = mfma32(a, qo[s % (MD / 32)][tb], O[tb]);
            }
            if (!(qa == 1 && qb == 0)) {
                bf16x8 kr[MD / 16], qr[MD / 16];
#pragma unroll
                for (int s = 0; s < MD / 16; ++s) {
                    kr[s] = ld_row_operand(sK, 32 * qa + l32, 16 * s + 8 * g);
                    qr[s] = ld_row_operand(sQ, 32 * qb + l32, 16 * s + 8 * g);
                }
                __builtin_amdgcn_sched_barrier(0);
                f32x16 pacc = {};
#pragma unroll
                for (int s = 0; s < MD / 16; ++s) pacc = mfma32(kr[s], qr[s], pacc);
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
        // ---- phase 2, iteration 0: the state entering the chunk
        if (it == 0) {
            const __amdgpu_buffer_rsrc_t er = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(entry + ((int64_t)c * H + h) * DD), (short)0, (int)(DD * 4), 0x00020000);
            const int ioff = (4 * g * MD + dv) * 4;
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    S[m][r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                        er, ioff, (32 * m + 8 * (r >> 2) + (r & 3)) * MD * 4, 0));
        }
        // ---- phase 2: walk: V~^T P^T into O, state update, y staging
        if (comp) {
            bf16x8 vop[MB / 16];     // V~^T operands, shared by both tiles and the state update
            bf16x8 pb[MB / 16][2];   // P^T operands (tile tb = 0 needs s < 2 only)
            bf16x8 ko[2][4];         // K~^T operands, half of the tokens at a time
#pragma unroll
            for (int s = 0; s < MB / 16; ++s) {
                vop[s] = ld_tr_operand(sV, 16 * s, 32 * w, lane);
#pragma unroll
                for (int tb = 0; tb < 2; ++tb)
                    if (tb == 1 || s < 2)
                        pb[s][tb] = *reinterpret_cast<const bf16x8*>(L.p + (32 * tb + l32) * PP + 16 * s + 8 * g);
            }
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int m = 0; m < 4; ++m) ko[s][m] = ld_tr_operand(sK, 16 * s, 32 * m, lane);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                for (int s = 0; s < MB / 16; ++s)
                    if (tb == 1 || s < 2)  // t < 32 sees only t' < 32
                        O[tb] = mfma32(vop[s], pb[s][tb], O[tb]);
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int m = 0; m < 4; ++m) S[m] = mfma32(ko[s][m], vop[s], S[m]);
#pragma unroll
            for (int s = 2; s < MB / 16; ++s)
#pragma unroll
                for (int m = 0; m < 4; ++m) ko[s - 2][m] = ld_tr_operand(sK, 16 * s, 32 * m, lane);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 2; s < MB / 16; ++s)
#pragma unroll
                for (int m = 0; m < 4; ++m) S[m] = mfma32(ko[s - 2][m], vop[s], S[m]);
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
                while (!written(fx[i]) && poll_again(polls, hdr, 4, c, h)) fx[i] = get_word(fsrc + i * MB);
                tot += word_value(fx[i]);
            }
            for (int i = RPRE; i < G; ++i) {
                uint64_t x = get_word(fsrc + i * MB);
                while (!written(x) && poll_again(polls, hdr, 4, c, h)) x = get_word(fsrc + i * MB);
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
    // the sequence's final state, from the walk's registers
    if (last && final_state != nullptr) {
        const __amdgpu_buffer_rsrc_t fr = __builtin_amdgcn_make_buffer_rsrc(
            final_state + ((int64_t)ce.seg * H + h) * DD, (short)0, (int)(DD * 4), 0x00020000);
        const int ioff = (4 * g * MD + dv) * 4;
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                // (bit_cast of a vector-element lvalue would read element 0)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(S[m][r]), fr, ioff,
                                                      (32 * m + 8 * (r >> 2) + (r & 3)) * MD * 4, 0);
    }
}

bool mfma_supported(const PrefillArgs& a) { return a.bf16 && a.D == MD && a.block == MB; }

hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t st) {
    if (a.max_chunks == 0 && a.nseq == 0) return hipSuccess;
    const dim3 grid((unsigned)((int64_t)a.max_chunks * a.H + a.nseq));
    auto* fn = a.preact ? (a.gate_act ? &prefill_mfma_kernel<false, false>
                                      : &prefill_mfma_kernel<false, true>)
                        : &prefill_mfma_kernel<true, true>;
    hipLaunchKernelGGL(fn, grid, dim3(NTHREADS), 0, st, (const __bf16*)a.q, (const __bf16*)a.k,
                       (const __bf16*)a.v, (const __bf16*)a.g, (const __bf16*)a.w, (__bf16*)a.out,
                       (__bf16*)a.y_save, a.hdr, a.segs, a.chunks, a.init_state, a.final_state, a.states, a.part,
                       a.rsub, a.H, a.nseq, a.chunk / MB, a.eps);
    return hipGetLastError();
}

}  // namespace la
