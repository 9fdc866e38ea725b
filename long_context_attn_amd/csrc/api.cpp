// C ABI of the Lightning Attention library: host-side validation, workspace
// layout and kernel dispatch.  See include/lightning_attn.h for the contract.
#include "lightning_attn.h"

#include <hip/hip_runtime.h>

#include <cmath>

#include "la_internal.h"

namespace {

constexpr size_t ALIGN = 256;
inline size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

bool supported_dim(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool supported_block(int b) { return b == 16 || b == 32 || b == 64; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Chunk length when the caller leaves it to the library: the longest power
// of two (up to 8192 tokens) that still gives about 256 (chunk, head) work
// items, one per CU.  Both prefill walks hold one workgroup per CU, and
// every chunk costs a D*D*4-byte state per head that is written and read
// back, so fewer, longer chunks are cheaper as long as the CUs stay busy.
int auto_chunk(int64_t total, int nseq, int heads, int block) {
    const int64_t target_items = 256;
    int64_t per = total * heads / target_items;
    int64_t c = block;
    while (c * 2 <= per && c < 8192) c *= 2;
    (void)nseq;
    return (int)c;
}

struct Layout {
    bool fused = false; // chunked MFMA walk with the RMSNorm exchange inside
    int chunk = 0;
    int max_chunks = 0;
    int n_slots = 0;
    size_t off_segs = 0, off_chunks = 0, off_states = 0, off_part = 0, off_rsub = 0,
           off_clear_end = 0, bytes = 0;
};

// the bf16 MFMA path (walk + RMSNorm in one kernel)
bool fused_path(int head_dim, int block, la_dtype dtype) {
    return dtype == LA_DTYPE_BF16 && head_dim == 128 && block == 64;
}

// The fused walk's cross-head RMSNorm exchange waits, inside the kernel, on
// the workgroups of every head of a chunk, one workgroup per CU.  Those waits
// can only end if all `heads` workgroups of a chunk are resident at once, so
// the fused walk is taken only when heads <= the device's compute units;
// wider calls run the portable kernels (walk, then a separate norm kernel),
// which have no cross-workgroup wait.
bool fused_fits(int heads) { return heads <= la::device_cu_count(); }

// Workspace: [PlanHeader][SegEntry x nseq][ChunkEntry x max_chunks], then
// per-chunk states [max_chunks][H][D][D] fp32 (chunk sums, then the states
// entering the chunks), then on the fused MFMA path the words cleared on every call before the walk (by the plan
//    kernel, or for uniform rows by the chunk-sum kernel), the
//    per-(chunk, block) RMSNorm exchange part [n_slots][H][64] and
//    rsub [n_slots][ceil(H/16)][64].
bool plan_layout(int64_t total, int nseq, int heads, int head_dim, int block, int chunk_tokens,
                 bool fused, Layout* L) {
    if (total < 0 || nseq < 0 || heads < 1 || !supported_dim(head_dim) || !supported_block(block))
        return false;
    fused = fused && fused_fits(heads);
    if (chunk_tokens < 0) return false;
    int chunk = chunk_tokens;
    // Both paths: about one (chunk, head) item per CU.  For the MFMA walk
    // that is 2048-token chunks at 8192 tokens x 64 heads, the fastest
    // measured there (1024: 236 us, 2048: 211 us per call); at 1M tokens
    // longer chunks (8192) spread the per-item fill and drain over more
    // blocks.
    if (chunk == 0) chunk = auto_chunk(total, nseq, heads, block);
    if (chunk < block || chunk % block != 0) return false;
    const int64_t maxc = total / chunk + nseq;  // >= sum over sequences of ceil(L_s / chunk)
    // work-item tickets (chunk items + one per sequence) are 32-bit
    if (maxc > (int64_t)0x7fffffff / 2 || maxc * heads + nseq > (int64_t)0x7fffffffLL) return false;
    L->chunk = chunk;
    L->max_chunks = (int)maxc;
    size_t off = align_up(sizeof(la::PlanHeader));
    L->off_segs = off;
    off = align_up(off + sizeof(la::SegEntry) * (size_t)nseq);
    L->off_chunks = off;
    off = align_up(off + sizeof(la::ChunkEntry) * (size_t)maxc);
    L->off_states = off;
    off = align_up(off + sizeof(float) * (size_t)maxc * heads * head_dim * head_dim);
    if (!fused) {
        L->bytes = off;
        return true;
    }
    const int64_t slots = maxc * (chunk / block);
    if (slots > (int64_t)0x7fffffff) return false;
    L->fused = true;
    L->n_slots = (int)slots;
    L->off_part = off;
    off = align_up(off + sizeof(uint64_t) * (size_t)slots * heads * block);
    L->off_rsub = off;
    off = align_up(off + sizeof(uint64_t) * (size_t)slots * ((heads + 15) / 16) * block);
    L->off_clear_end = off;
    L->bytes = off;
    return true;
}

// Backward workspace: [PlanHeader][SegEntry x nseq][ChunkEntry x max_chunks],
// the forward chunk states and the reverse ones [max_chunks][H][D][D] fp32,
// y and dy [total][H][D] (bf16 on the MFMA path, else fp32), on the portable
// path q~, k~, v~ [total][H][D] fp32, and the dw partial sums
// [ceil(total / norm tokens)][H*D] fp32.  Automatic chunks: the
// MFMA walks (one workgroup per CU) take the prefill's choice; the
// portable walks, a workgroup of only head_dim threads each, the longest
// power of two (at least the block) that gives about 8 walks per CU.
bool backward_mfma_path(int head_dim, la_dtype dtype) {
    return dtype == LA_DTYPE_BF16 && head_dim == 128;
}

struct BwdLayout {
    bool mfma = false;
    int chunk = 0, max_chunks = 0, n_tb = 0;
    size_t off_segs = 0, off_chunks = 0, off_states = 0, off_gstates = 0, off_qs = 0, off_ks = 0,
           off_vs = 0, off_y = 0, off_dy = 0, off_dw = 0, bytes = 0;
};

bool backward_layout(int64_t total, int nseq, int heads, int head_dim, int block, int chunk_tokens,
                     la_dtype dtype, BwdLayout* L) {
    if (total < 0 || nseq < 0 || heads < 1 || chunk_tokens < 0 || !supported_dim(head_dim) ||
        !supported_block(block) || (int64_t)heads * head_dim > la::backward_max_hd())
        return false;
    L->mfma = backward_mfma_path(head_dim, dtype);
    int chunk = chunk_tokens;
    if (chunk == 0 && L->mfma) {
        chunk = auto_chunk(total, nseq, heads, block);
    } else if (chunk == 0) {
        const int64_t per = total * heads / (8 * (int64_t)la::device_cu_count());
        int64_t c = block;
        while (c * 2 <= per && c < 8192) c *= 2;
        chunk = (int)c;
    }
    if (chunk < block || chunk % block != 0) return false;
    const int64_t maxc = total / chunk + nseq;
    if (maxc * heads > (int64_t)0x7fffffff) return false;
    const int64_t tpb = la::backward_norm_tokens(total);
    const int64_t ntb = (total + tpb - 1) / tpb;
    if (ntb > (int64_t)0x7fffffff) return false;
    L->chunk = chunk;
    L->max_chunks = (int)maxc;
    L->n_tb = (int)ntb;
    const size_t DD = (size_t)head_dim * head_dim;
    const size_t act = sizeof(float) * (size_t)total * heads * head_dim;
    size_t off = align_up(sizeof(la::PlanHeader));
    L->off_segs = off;
    off = align_up(off + sizeof(la::SegEntry) * (size_t)nseq);
    L->off_chunks = off;
    off = align_up(off + sizeof(la::ChunkEntry) * (size_t)maxc);
    L->off_states = off;
    off = align_up(off + sizeof(float) * (size_t)maxc * heads * DD);
    L->off_gstates = off;
    off = align_up(off + sizeof(float) * (size_t)maxc * heads * DD);
    L->off_y = off;
    off = align_up(off + (L->mfma ? act / 2 : act));  // y: bf16 on the MFMA path
    L->off_dy = off;
    off = align_up(off + (L->mfma ? act / 2 : act));
    if (!L->mfma) {
        size_t* acts[3] = {&L->off_qs, &L->off_ks, &L->off_vs};
        for (size_t* o : acts) {
            *o = off;
            off = align_up(off + act);
        }
    }
    L->off_dw = off;
    off = align_up(off + sizeof(float) * (size_t)ntb * heads * head_dim);
    L->bytes = off;
    return true;
}

// Activations a prefill keeps for lightning_attn_backward_saved: y (the
// attention output before the norm, bf16 [total][H][D]) and then the fp32
// state entering every chunk ([max_chunks][H][D][D]), in the chunk layout that
// both passes derive from the same arguments.  Only the fused bf16 MFMA path
// (head_dim 128, block 64, heads <= CUs) saves them.
struct SavedLayout {
    int chunk = 0, max_chunks = 0;
    size_t off_states = 0, bytes = 0;
};

bool saved_layout(int64_t total, int nseq, int heads, int head_dim, int block, int chunk_tokens,
                  la_dtype dtype, SavedLayout* S) {
    if (!fused_path(head_dim, block, dtype)) return false;
    Layout L;
    if (!plan_layout(total, nseq, heads, head_dim, block, chunk_tokens, true, &L) || !L.fused)
        return false;
    BwdLayout B;
    if (!backward_layout(total, nseq, heads, head_dim, block, chunk_tokens, dtype, &B) ||
        !B.mfma || B.chunk != L.chunk || B.max_chunks != L.max_chunks)
        return false;
    S->chunk = L.chunk;
    S->max_chunks = L.max_chunks;
    S->off_states = align_up(sizeof(uint16_t) * (size_t)total * heads * head_dim);
    S->bytes = S->off_states + sizeof(float) * (size_t)L.max_chunks * heads * head_dim * head_dim;
    return true;
}

// Checks a saved-activations buffer for a call with these arguments.
la_status check_saved(const void* saved, size_t saved_bytes, int64_t total, int nseq, int heads,
                      int head_dim, int block, int chunk_tokens, la_dtype dtype,
                      SavedLayout* S) {
    if (!saved_layout(total, nseq, heads, head_dim, block, chunk_tokens, dtype, S))
        return LA_ERR_UNSUPPORTED;
    if (!saved) return LA_ERR_NULL_POINTER;
    if (!aligned16(saved)) return LA_ERR_MISALIGNED;
    if (saved_bytes < S->bytes) return LA_ERR_WORKSPACE_TOO_SMALL;
    return LA_OK;
}

la_status check_dtype(la_dtype dtype) {
    return (dtype == LA_DTYPE_F32 || dtype == LA_DTYPE_BF16) ? LA_OK : LA_ERR_UNSUPPORTED;
}

const char* const kPrefillStages[] = {"plan", "chunk_state", "state_scan", "walk", "norm_gate"};
constexpr int kPrefillStageCount = 5;
const char* const kDecodeStages[] = {"decode_state", "decode_norm"};
constexpr int kDecodeStageCount = 2;

// Records events[i] (if any) on the stream; returns false on a HIP error.
struct Marks {
    hipEvent_t* ev = nullptr;
    int n = 0;
    int next = 0;
    hipError_t mark(hipStream_t st) {
        if (ev == nullptr) return hipSuccess;
        return hipEventRecord(ev[next++], st);
    }
};

la_status run_prefill(la::PrefillArgs& a, const Layout& L, void* workspace, hipStream_t stream,
                      Marks marks = Marks()) {
    char* ws = static_cast<char*>(workspace);
    a.chunk = L.chunk;
    a.max_chunks = L.max_chunks;
    a.hdr = reinterpret_cast<la::PlanHeader*>(ws);
    a.segs = reinterpret_cast<la::SegEntry*>(ws + L.off_segs);
    a.chunks = reinterpret_cast<la::ChunkEntry*>(ws + L.off_chunks);
    // (states already set: the caller keeps them, in a saved-activations buffer)
    if (a.states == nullptr) a.states = reinterpret_cast<float*>(ws + L.off_states);
    // the layout decided the kernels: the fused MFMA walk needs its exchange
    // words, which only a fused layout holds
    const bool mfma = L.fused && la::mfma_supported(a);
    if (a.preact && !mfma) return LA_ERR_UNSUPPORTED;
    if (mfma) {
        a.skip_last = true;
        a.n_slots = L.n_slots;
        a.part = reinterpret_cast<uint64_t*>(ws + L.off_part);
        a.rsub = reinterpret_cast<uint64_t*>(ws + L.off_rsub);
        a.clear = a.part;
        a.clear_words = (int64_t)((L.off_clear_end - L.off_part) / sizeof(uint64_t));
    }
    // uniform rows on the MFMA path: the chunk-sum kernel writes the plan
    a.inline_plan = mfma && a.cu == nullptr && a.seqlen > 0;
    hipError_t e = marks.mark(stream);
    if (e == hipSuccess && !a.inline_plan) e = la::launch_plan(a, stream);
    if (e == hipSuccess) e = marks.mark(stream);
    if (mfma) {
        // chunk sums (every chunk but each sequence's last), the scan of the
        // states entering the chunks, then every chunk's walk with the
        // RMSNorm fused (the norm_gate mark stays empty)
        if (e == hipSuccess) e = la::launch_chunk_state_mfma(a, stream);
        if (e == hipSuccess) e = marks.mark(stream);
        if (e == hipSuccess) e = la::launch_state_scan(a, stream);
        if (e == hipSuccess) e = marks.mark(stream);
        if (e == hipSuccess) e = la::launch_prefill_mfma(a, stream);
        if (e == hipSuccess) e = marks.mark(stream);
    } else {
        if (e == hipSuccess) e = la::launch_chunk_state_valu(a, stream);
        if (e == hipSuccess) e = marks.mark(stream);
        if (e == hipSuccess) e = la::launch_state_scan(a, stream);
        if (e == hipSuccess) e = marks.mark(stream);
        if (e == hipSuccess) e = la::launch_walk_valu(a, stream);
        if (e == hipSuccess) e = marks.mark(stream);
        if (e == hipSuccess) e = la::launch_norm_gate(a, stream);
    }
    if (e == hipSuccess) e = marks.mark(stream);
    return e == hipSuccess ? LA_OK : LA_ERR_HIP;
}

la_status check_ptrs(const void* q, const void* k, const void* v, const void* g, const void* w,
                     const void* out) {
    if (!q || !k || !v || !g || !w || !out) return LA_ERR_NULL_POINTER;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned16(w) ||
        !aligned16(out))
        return LA_ERR_MISALIGNED;
    return LA_OK;
}

// Softmax attention workspace: [PlanHeader][SegEntry x nseq][ChunkEntry x
// max_tiles] (128-token query tiles), then the rotated k (bf16 [total][H][D])
// when rope_dim > 0.
struct SoftmaxLayout {
    int max_tiles = 0;
    size_t off_segs = 0, off_tiles = 0, off_kr = 0, bytes = 0;
};

bool softmax_layout(int64_t total, int nseq, int heads, int head_dim, int rope_dim,
                    SoftmaxLayout* L) {
    if (total < 0 || nseq < 0 || heads < 1 || head_dim != 128) return false;
    if (rope_dim < 0 || rope_dim > head_dim || rope_dim % 8 != 0) return false;
    const int64_t tiles = total / la::SOFTMAX_TILE + nseq;
    // one workgroup per (tile, head), counted in 32 bits
    if (tiles * heads > (int64_t)0x7fffffff) return false;
    L->max_tiles = (int)tiles;
    size_t off = align_up(sizeof(la::PlanHeader));
    L->off_segs = off;
    off = align_up(off + sizeof(la::SegEntry) * (size_t)nseq);
    L->off_tiles = off;
    off = align_up(off + sizeof(la::ChunkEntry) * (size_t)tiles);
    const size_t act = rope_dim > 0 ? sizeof(uint16_t) * (size_t)total * heads * head_dim : 0;
    L->off_kr = off;
    off = align_up(off + act);
    L->bytes = off;
    return true;
}

la_status softmax_checks(const void* q, const void* k, const void* v, const void* out,
                         int64_t total, int heads, int head_dim, int rope_dim, double rope_base,
                         float scale, la_dtype dtype) {
    if (heads < 1 || !(scale > 0.0f) || !std::isfinite(scale)) return LA_ERR_BAD_SHAPE;
    if (rope_dim > 0 && (!(rope_base > 0.0) || !std::isfinite(rope_base))) return LA_ERR_BAD_SHAPE;
    if (dtype != LA_DTYPE_BF16 || head_dim != 128 || rope_dim < 0 || rope_dim > head_dim ||
        rope_dim % 8 != 0)
        return LA_ERR_UNSUPPORTED;
    if (total > 0) {
        if (!q || !k || !v || !out) return LA_ERR_NULL_POINTER;
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
            return LA_ERR_MISALIGNED;
    }
    return LA_OK;
}

// plan (query tiles of SOFTMAX_TILE tokens) -> rotate q, k -> attention
la_status run_softmax(const void* q, const void* k, const void* v, void* out, const int32_t* cu,
                      int nseq, int64_t seqlen, int64_t total, int heads, int rope_dim,
                      double rope_base, float scale, const SoftmaxLayout& L, void* workspace,
                      hipStream_t stream) {
    char* ws = static_cast<char*>(workspace);
    la::PrefillArgs p{};
    p.cu = cu;
    p.nseq = nseq;
    p.seqlen = seqlen;
    p.total = total;
    p.H = heads;
    p.D = 128;
    p.chunk = la::SOFTMAX_TILE;
    p.max_chunks = L.max_tiles;
    p.hdr = reinterpret_cast<la::PlanHeader*>(ws);
    p.segs = reinterpret_cast<la::SegEntry*>(ws + L.off_segs);
    p.chunks = reinterpret_cast<la::ChunkEntry*>(ws + L.off_tiles);
    p.clear = nullptr;
    p.clear_words = 0;
    la::SoftmaxArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.H = heads;
    a.rope_dim = rope_dim;
    a.rope_base = rope_base;
    a.scale = scale;
    a.max_tiles = L.max_tiles;
    a.hdr = p.hdr;
    a.segs = p.segs;
    a.tiles = p.chunks;
    a.kr = reinterpret_cast<__bf16*>(ws + L.off_kr);
    hipError_t e = la::launch_plan(p, stream);
    if (e == hipSuccess && rope_dim > 0) e = la::launch_softmax_rope(a, stream);
    if (e == hipSuccess) e = la::launch_softmax_fwd(a, stream);
    return e == hipSuccess ? LA_OK : LA_ERR_HIP;
}

}  // namespace

extern "C" {

const char* lightning_attn_status_string(la_status s) {
    switch (s) {
        case LA_OK: return "ok";
        case LA_ERR_NULL_POINTER: return "a required pointer is NULL";
        case LA_ERR_BAD_SHAPE: return "invalid or inconsistent sizes";
        case LA_ERR_UNSUPPORTED: return "unsupported head_dim, block, chunk or dtype";
        case LA_ERR_MISALIGNED: return "a pointer is not 16-byte aligned";
        case LA_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than the required size";
        case LA_ERR_HIP: return "the HIP runtime reported an error while enqueueing";
        case LA_ERR_SCRATCH_TOO_SMALL:
            return "sizes exceed the fixed scratch of the no-allocation entry point";
    }
    return "unknown status";
}

la_status lightning_attn_workspace_status(const void* workspace, size_t workspace_bytes,
                                          int32_t* status, hipStream_t stream) {
    if (!workspace || !status) return LA_ERR_NULL_POINTER;
    if (!aligned16(workspace)) return LA_ERR_MISALIGNED;
    if (workspace_bytes < sizeof(la::PlanHeader)) return LA_ERR_WORKSPACE_TOO_SMALL;
    la::PlanHeader h{};
    if (hipMemcpyAsync(&h, workspace, sizeof(h), hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return LA_ERR_HIP;
    status[0] = h.error;
    status[1] = h.wait_site;
    status[2] = h.wait_chunk;
    status[3] = h.wait_head;
    return LA_OK;
}

size_t lightning_attn_prefill_workspace_size(int64_t total_tokens, int nseq, int heads,
                                             int head_dim, int block, int chunk_tokens,
                                             la_dtype dtype) {
    if (check_dtype(dtype) != LA_OK) return 0;
    Layout L;
    if (!plan_layout(total_tokens, nseq, heads, head_dim, block, chunk_tokens,
                     fused_path(head_dim, block, dtype), &L))
        return 0;
    return L.bytes;
}

static la_status prefill_impl(const void* q, const void* k, const void* v, const void* gate,
                              const void* norm_weight, void* out, const float* initial_state,
                              float* final_state, int batch, int64_t seqlen, int heads,
                              int head_dim, int block, int chunk_tokens, float eps,
                              la_dtype dtype, void* workspace, size_t workspace_bytes,
                              hipStream_t stream, Marks marks, void* saved = nullptr,
                              size_t saved_bytes = 0, bool save = false) {
    if (batch < 0 || seqlen < 0 || heads < 1 || !(eps >= 0.0f)) return LA_ERR_BAD_SHAPE;
    if (chunk_tokens < 0) return LA_ERR_BAD_SHAPE;
    if (check_dtype(dtype) != LA_OK || !supported_dim(head_dim) || !supported_block(block))
        return LA_ERR_UNSUPPORTED;
    if (batch > 0 && seqlen > ((int64_t)1 << 40) / batch) return LA_ERR_BAD_SHAPE;
    const int64_t total = (int64_t)batch * seqlen;
    if (total > 0) {
        la_status s = check_ptrs(q, k, v, gate, norm_weight, out);
        if (s != LA_OK) return s;
    }
    if (initial_state && !aligned16(initial_state)) return LA_ERR_MISALIGNED;
    if (final_state && !aligned16(final_state)) return LA_ERR_MISALIGNED;
    Layout L;
    if (!plan_layout(total, batch, heads, head_dim, block, chunk_tokens,
                     fused_path(head_dim, block, dtype), &L))
        return LA_ERR_UNSUPPORTED;
    if (!workspace) return LA_ERR_NULL_POINTER;
    if (!aligned16(workspace)) return LA_ERR_MISALIGNED;
    if (workspace_bytes < L.bytes) return LA_ERR_WORKSPACE_TOO_SMALL;
    SavedLayout S;
    if (save) {
        const la_status st = check_saved(saved, saved_bytes, total, batch, heads, head_dim, block,
                                         chunk_tokens, dtype, &S);
        if (st != LA_OK) return st;
    }
    if (batch == 0) return LA_OK;
    la::PrefillArgs a{};
    if (save) {
        a.y_save = saved;
        a.states = reinterpret_cast<float*>(static_cast<char*>(saved) + S.off_states);
    }
    a.q = q; a.k = k; a.v = v; a.g = gate; a.w = norm_weight; a.out = out;
    a.init_state = initial_state;
    a.final_state = final_state;
    a.cu = nullptr;
    a.nseq = batch;
    a.seqlen = seqlen;
    a.total = total;
    a.H = heads; a.D = head_dim; a.block = block;
    a.eps = eps;
    a.bf16 = dtype == LA_DTYPE_BF16;
    return run_prefill(a, L, workspace, stream, marks);
}

la_status lightning_attn_prefill(const void* q, const void* k, const void* v, const void* gate,
                                 const void* norm_weight, void* out, const float* initial_state,
                                 float* final_state, int batch, int64_t seqlen, int heads,
                                 int head_dim, int block, int chunk_tokens, float eps,
                                 la_dtype dtype, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
    return prefill_impl(q, k, v, gate, norm_weight, out, initial_state, final_state, batch, seqlen,
                        heads, head_dim, block, chunk_tokens, eps, dtype, workspace,
                        workspace_bytes, stream, Marks());
}

la_status lightning_attn_prefill_profiled(
    const void* q, const void* k, const void* v, const void* gate, const void* norm_weight,
    void* out, const float* initial_state, float* final_state, int batch, int64_t seqlen,
    int heads, int head_dim, int block, int chunk_tokens, float eps, la_dtype dtype,
    void* workspace, size_t workspace_bytes, hipStream_t stream, hipEvent_t* events,
    int n_events) {
    Marks m;
    if (n_events != 0) {
        if (events == nullptr) return LA_ERR_NULL_POINTER;
        if (n_events < kPrefillStageCount + 1) return LA_ERR_BAD_SHAPE;
        m.ev = events;
        m.n = n_events;
    }
    return prefill_impl(q, k, v, gate, norm_weight, out, initial_state, final_state, batch, seqlen,
                        heads, head_dim, block, chunk_tokens, eps, dtype, workspace,
                        workspace_bytes, stream, m);
}

int lightning_attn_prefill_stage_count(void) { return kPrefillStageCount; }
const char* lightning_attn_prefill_stage_name(int stage) {
    return (stage >= 0 && stage < kPrefillStageCount) ? kPrefillStages[stage] : nullptr;
}
int lightning_attn_decode_stage_count(void) { return kDecodeStageCount; }
const char* lightning_attn_decode_stage_name(int stage) {
    return (stage >= 0 && stage < kDecodeStageCount) ? kDecodeStages[stage] : nullptr;
}

static la_status prefill_varlen_impl(const void* q, const void* k, const void* v,
                                     const void* gate, const void* norm_weight, void* out,
                                     const int32_t* cu_seqlens, int nseq, int64_t total_tokens,
                                     const float* initial_state, float* final_state, int heads,
                                     int head_dim, int block, int chunk_tokens, float eps,
                                     la_dtype dtype, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream, void* saved, size_t saved_bytes,
                                     bool save) {
    if (nseq < 0 || total_tokens < 0 || total_tokens > 0x7fffffffLL || heads < 1 ||
        !(eps >= 0.0f) || chunk_tokens < 0)
        return LA_ERR_BAD_SHAPE;
    if (check_dtype(dtype) != LA_OK || !supported_dim(head_dim) || !supported_block(block))
        return LA_ERR_UNSUPPORTED;
    if (nseq == 0 && total_tokens != 0) return LA_ERR_BAD_SHAPE;
    if (total_tokens > 0) {
        la_status s = check_ptrs(q, k, v, gate, norm_weight, out);
        if (s != LA_OK) return s;
    }
    if (nseq > 0 && !cu_seqlens) return LA_ERR_NULL_POINTER;
    if (cu_seqlens && (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u)) return LA_ERR_MISALIGNED;
    if (initial_state && !aligned16(initial_state)) return LA_ERR_MISALIGNED;
    if (final_state && !aligned16(final_state)) return LA_ERR_MISALIGNED;
    Layout L;
    if (!plan_layout(total_tokens, nseq, heads, head_dim, block, chunk_tokens,
                     fused_path(head_dim, block, dtype), &L))
        return LA_ERR_UNSUPPORTED;
    if (!workspace) return LA_ERR_NULL_POINTER;
    if (!aligned16(workspace)) return LA_ERR_MISALIGNED;
    if (workspace_bytes < L.bytes) return LA_ERR_WORKSPACE_TOO_SMALL;
    SavedLayout S;
    if (save) {
        const la_status st = check_saved(saved, saved_bytes, total_tokens, nseq, heads, head_dim,
                                         block, chunk_tokens, dtype, &S);
        if (st != LA_OK) return st;
    }
    if (nseq == 0) return LA_OK;
    la::PrefillArgs a{};
    if (save) {
        a.y_save = saved;
        a.states = reinterpret_cast<float*>(static_cast<char*>(saved) + S.off_states);
    }
    a.q = q; a.k = k; a.v = v; a.g = gate; a.w = norm_weight; a.out = out;
    a.init_state = initial_state;
    a.final_state = final_state;
    a.cu = cu_seqlens;
    a.nseq = nseq;
    a.seqlen = 0;
    a.total = total_tokens;
    a.H = heads; a.D = head_dim; a.block = block;
    a.eps = eps;
    a.bf16 = dtype == LA_DTYPE_BF16;
    return run_prefill(a, L, workspace, stream);
}

la_status lightning_attn_prefill_varlen(const void* q, const void* k, const void* v,
                                        const void* gate, const void* norm_weight, void* out,
                                        const int32_t* cu_seqlens, int nseq, int64_t total_tokens,
                                        const float* initial_state, float* final_state, int heads,
                                        int head_dim, int block, int chunk_tokens, float eps,
                                        la_dtype dtype, void* workspace, size_t workspace_bytes,
                                        hipStream_t stream) {
    return prefill_varlen_impl(q, k, v, gate, norm_weight, out, cu_seqlens, nseq, total_tokens,
                               initial_state, final_state, heads, head_dim, block, chunk_tokens,
                               eps, dtype, workspace, workspace_bytes, stream, nullptr, 0, false);
}

size_t lightning_attn_saved_size(int64_t total_tokens, int nseq, int heads, int head_dim,
                                 int block, int chunk_tokens, la_dtype dtype) {
    if (check_dtype(dtype) != LA_OK || chunk_tokens < 0) return 0;
    SavedLayout S;
    if (!saved_layout(total_tokens, nseq, heads, head_dim, block, chunk_tokens, dtype, &S))
        return 0;
    return S.bytes;
}

la_status lightning_attn_prefill_save(const void* q, const void* k, const void* v,
                                      const void* gate, const void* norm_weight, void* out,
                                      const float* initial_state, float* final_state, int batch,
                                      int64_t seqlen, int heads, int head_dim, int block,
                                      int chunk_tokens, float eps, la_dtype dtype, void* saved,
                                      size_t saved_bytes, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
    return prefill_impl(q, k, v, gate, norm_weight, out, initial_state, final_state, batch, seqlen,
                        heads, head_dim, block, chunk_tokens, eps, dtype, workspace,
                        workspace_bytes, stream, Marks(), saved, saved_bytes, true);
}

la_status lightning_attn_prefill_varlen_save(
    const void* q, const void* k, const void* v, const void* gate, const void* norm_weight,
    void* out, const int32_t* cu_seqlens, int nseq, int64_t total_tokens,
    const float* initial_state, float* final_state, int heads, int head_dim, int block,
    int chunk_tokens, float eps, la_dtype dtype, void* saved, size_t saved_bytes,
    void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return prefill_varlen_impl(q, k, v, gate, norm_weight, out, cu_seqlens, nseq, total_tokens,
                               initial_state, final_state, heads, head_dim, block, chunk_tokens,
                               eps, dtype, workspace, workspace_bytes, stream, saved, saved_bytes,
                               true);
}

size_t lightning_attn_state_workspace_size(int64_t total_tokens, int nseq, int heads,
                                           int head_dim, int block, int chunk_tokens,
                                           la_dtype dtype) {
    if (check_dtype(dtype) != LA_OK || chunk_tokens < 0) return 0;
    Layout L;
    if (!plan_layout(total_tokens, nseq, heads, head_dim, block, chunk_tokens, false, &L)) return 0;
    return L.bytes;
}

// State-only pass: plan, per-chunk sums of k~^T v~, then the scan, which
// writes initial state + all chunk sums of each sequence as its final state.
static la_status run_state(la::PrefillArgs& a, const Layout& L, void* workspace,
                           hipStream_t stream) {
    char* ws = static_cast<char*>(workspace);
    a.chunk = L.chunk;
    a.max_chunks = L.max_chunks;
    a.hdr = reinterpret_cast<la::PlanHeader*>(ws);
    a.segs = reinterpret_cast<la::SegEntry*>(ws + L.off_segs);
    a.chunks = reinterpret_cast<la::ChunkEntry*>(ws + L.off_chunks);
    a.states = reinterpret_cast<float*>(ws + L.off_states);
    a.clear = nullptr;
    a.clear_words = 0;
    // uniform rows on the MFMA path: the chunk-sum kernel writes the plan
    const bool mfma = la::state_mfma_supported(a);
    a.inline_plan = mfma && a.cu == nullptr && a.seqlen > 0;
    hipError_t e = a.inline_plan ? hipSuccess : la::launch_plan(a, stream);
    if (e == hipSuccess)
        e = mfma ? la::launch_chunk_state_mfma(a, stream) : la::launch_chunk_state_valu(a, stream);
    if (e == hipSuccess) e = la::launch_state_scan(a, stream);
    return e == hipSuccess ? LA_OK : LA_ERR_HIP;
}

static la_status state_checks(const void* k, const void* v, const float* initial_state,
                              float* final_state, int64_t total, int nseq, int heads,
                              int head_dim, int block, int chunk_tokens, la_dtype dtype,
                              void* workspace, size_t workspace_bytes, Layout* L) {
    if (heads < 1 || chunk_tokens < 0) return LA_ERR_BAD_SHAPE;
    if (check_dtype(dtype) != LA_OK || !supported_dim(head_dim) || !supported_block(block))
        return LA_ERR_UNSUPPORTED;
    if (total > 0) {
        if (!k || !v) return LA_ERR_NULL_POINTER;
        if (!aligned16(k) || !aligned16(v)) return LA_ERR_MISALIGNED;
    }
    if (nseq > 0 && !final_state) return LA_ERR_NULL_POINTER;
    if (final_state && !aligned16(final_state)) return LA_ERR_MISALIGNED;
    if (initial_state && !aligned16(initial_state)) return LA_ERR_MISALIGNED;
    if (!plan_layout(total, nseq, heads, head_dim, block, chunk_tokens, false, L))
        return LA_ERR_UNSUPPORTED;
    if (!workspace) return LA_ERR_NULL_POINTER;
    if (!aligned16(workspace)) return LA_ERR_MISALIGNED;
    if (workspace_bytes < L->bytes) return LA_ERR_WORKSPACE_TOO_SMALL;
    return LA_OK;
}

la_status lightning_attn_state(const void* k, const void* v, const float* initial_state,
                               float* final_state, int batch, int64_t seqlen, int heads,
                               int head_dim, int block, int chunk_tokens, la_dtype dtype,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (batch < 0 || seqlen < 0) return LA_ERR_BAD_SHAPE;
    if (batch > 0 && seqlen > ((int64_t)1 << 40) / batch) return LA_ERR_BAD_SHAPE;
    const int64_t total = (int64_t)batch * seqlen;
    Layout L;
    la_status s = state_checks(k, v, initial_state, final_state, total, batch, heads, head_dim,
                               block, chunk_tokens, dtype, workspace, workspace_bytes, &L);
    if (s != LA_OK || batch == 0) return s;
    la::PrefillArgs a{};
    a.k = k; a.v = v;
    a.init_state = initial_state;
    a.final_state = final_state;
    a.cu = nullptr;
    a.nseq = batch;
    a.seqlen = seqlen;
    a.total = total;
    a.H = heads; a.D = head_dim; a.block = block;
    a.bf16 = dtype == LA_DTYPE_BF16;
    return run_state(a, L, workspace, stream);
}

la_status lightning_attn_state_varlen(const void* k, const void* v, const int32_t* cu_seqlens,
                                      int nseq, int64_t total_tokens, const float* initial_state,
                                      float* final_state, int heads, int head_dim, int block,
                                      int chunk_tokens, la_dtype dtype, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
    if (nseq < 0 || total_tokens < 0 || total_tokens > 0x7fffffffLL) return LA_ERR_BAD_SHAPE;
    if (nseq == 0 && total_tokens != 0) return LA_ERR_BAD_SHAPE;
    if (nseq > 0 && !cu_seqlens) return LA_ERR_NULL_POINTER;
    if (cu_seqlens && (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u)) return LA_ERR_MISALIGNED;
    Layout L;
    la_status s = state_checks(k, v, initial_state, final_state, total_tokens, nseq, heads,
                               head_dim, block, chunk_tokens, dtype, workspace, workspace_bytes, &L);
    if (s != LA_OK || nseq == 0) return s;
    la::PrefillArgs a{};
    a.k = k; a.v = v;
    a.init_state = initial_state;
    a.final_state = final_state;
    a.cu = cu_seqlens;
    a.nseq = nseq;
    a.seqlen = 0;
    a.total = total_tokens;
    a.H = heads; a.D = head_dim; a.block = block;
    a.bf16 = dtype == LA_DTYPE_BF16;
    return run_state(a, L, workspace, stream);
}

size_t lightning_attn_backward_workspace_size(int64_t total_tokens, int nseq, int heads,
                                              int head_dim, int block, int chunk_tokens,
                                              la_dtype dtype) {
    if (check_dtype(dtype) != LA_OK) return 0;
    BwdLayout L;
    if (!backward_layout(total_tokens, nseq, heads, head_dim, block, chunk_tokens, dtype, &L))
        return 0;
    return L.bytes;
}

// Shared checks and launch of the backward (batch rows when cu == null).
static la_status backward_impl(const void* q, const void* k, const void* v, const void* gate,
                               const void* norm_weight, const void* dout,
                               const float* initial_state, const float* d_final_state, void* dq,
                               void* dk, void* dv, void* dgate, float* dweight,
                               float* d_initial_state, const int32_t* cu, int nseq,
                               int64_t seqlen, int64_t total, int heads, int head_dim, int block,
                               int chunk_tokens, float eps, la_dtype dtype, void* workspace,
                               size_t workspace_bytes, hipStream_t stream,
                               const void* saved = nullptr, size_t saved_bytes = 0,
                               bool use_saved = false) {
    if (heads < 1 || chunk_tokens < 0 || !(eps >= 0.0f)) return LA_ERR_BAD_SHAPE;
    if (check_dtype(dtype) != LA_OK || !supported_dim(head_dim) || !supported_block(block))
        return LA_ERR_UNSUPPORTED;
    if (total > 0) {
        la_status st = check_ptrs(q, k, v, gate, norm_weight, dout);
        if (st != LA_OK) return st;
        st = check_ptrs(dq, dk, dv, dgate, dweight, dweight);
        if (st != LA_OK) return st;
    }
    if (nseq > 0 && !dweight) return LA_ERR_NULL_POINTER;
    if (dweight && !aligned16(dweight)) return LA_ERR_MISALIGNED;
    if (initial_state && !aligned16(initial_state)) return LA_ERR_MISALIGNED;
    if (d_final_state && !aligned16(d_final_state)) return LA_ERR_MISALIGNED;
    if (d_initial_state && !aligned16(d_initial_state)) return LA_ERR_MISALIGNED;
    BwdLayout L;
    if (!backward_layout(total, nseq, heads, head_dim, block, chunk_tokens, dtype, &L))
        return LA_ERR_UNSUPPORTED;
    if (!workspace) return LA_ERR_NULL_POINTER;
    if (!aligned16(workspace)) return LA_ERR_MISALIGNED;
    if (workspace_bytes < L.bytes) return LA_ERR_WORKSPACE_TOO_SMALL;
    SavedLayout S;
    if (use_saved) {
        const la_status st = check_saved(saved, saved_bytes, total, nseq, heads, head_dim, block,
                                         chunk_tokens, dtype, &S);
        if (st != LA_OK) return st;
    }
    if (nseq == 0) return LA_OK;
    char* ws = static_cast<char*>(workspace);
    la::BackwardArgs a{};
    la::PrefillArgs& p = a.p;
    p.q = q; p.k = k; p.v = v; p.g = gate; p.w = norm_weight;
    p.init_state = initial_state;
    p.cu = cu;
    p.nseq = nseq;
    p.seqlen = seqlen;
    p.total = total;
    p.H = heads; p.D = head_dim; p.block = block;
    p.eps = eps;
    p.bf16 = dtype == LA_DTYPE_BF16;
    p.chunk = L.chunk;
    p.max_chunks = L.max_chunks;
    p.hdr = reinterpret_cast<la::PlanHeader*>(ws);
    p.segs = reinterpret_cast<la::SegEntry*>(ws + L.off_segs);
    p.chunks = reinterpret_cast<la::ChunkEntry*>(ws + L.off_chunks);
    p.states = reinterpret_cast<float*>(ws + L.off_states);
    a.stream = stream;
    a.dout = dout;
    a.d_final = d_final_state;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dgate;
    a.dw = dweight;
    a.d_init = d_initial_state;
    a.mfma = L.mfma;
    a.gstates = reinterpret_cast<float*>(ws + L.off_gstates);
    if (!L.mfma) {
        a.qs = reinterpret_cast<float*>(ws + L.off_qs);
        a.ks = reinterpret_cast<float*>(ws + L.off_ks);
        a.vs = reinterpret_cast<float*>(ws + L.off_vs);
    }
    a.y = reinterpret_cast<float*>(ws + L.off_y);
    if (use_saved) {
        // y and the states entering the chunks come from the prefill
        a.saved = true;
        a.y = static_cast<float*>(const_cast<void*>(saved));
        p.states = reinterpret_cast<float*>(static_cast<char*>(const_cast<void*>(saved)) +
                                            S.off_states);
    }
    a.dy = ws + L.off_dy;
    a.dw_part = reinterpret_cast<float*>(ws + L.off_dw);
    a.n_tb = L.n_tb;
    // uniform rows on the MFMA path: the first chunk-sum kernel writes the plan
    p.inline_plan = L.mfma && cu == nullptr && seqlen > 0;
    hipError_t e = p.inline_plan ? hipSuccess : la::launch_plan(p, stream);
    if (e == hipSuccess) e = la::launch_backward(a);
    return e == hipSuccess ? LA_OK : LA_ERR_HIP;
}

la_status lightning_attn_backward(const void* q, const void* k, const void* v, const void* gate,
                                  const void* norm_weight, const void* dout,
                                  const float* initial_state, const float* d_final_state,
                                  void* dq, void* dk, void* dv, void* dgate, float* dweight,
                                  float* d_initial_state, int batch, int64_t seqlen, int heads,
                                  int head_dim, int block, int chunk_tokens, float eps,
                                  la_dtype dtype, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
    if (batch < 0 || seqlen < 0) return LA_ERR_BAD_SHAPE;
    if (batch > 0 && seqlen > ((int64_t)1 << 40) / batch) return LA_ERR_BAD_SHAPE;
    return backward_impl(q, k, v, gate, norm_weight, dout, initial_state, d_final_state, dq, dk,
                         dv, dgate, dweight, d_initial_state, nullptr, batch, seqlen,
                         (int64_t)batch * seqlen, heads, head_dim, block, chunk_tokens, eps, dtype,
                         workspace, workspace_bytes, stream);
}

la_status lightning_attn_backward_varlen(
    const void* q, const void* k, const void* v, const void* gate, const void* norm_weight,
    const void* dout, const int32_t* cu_seqlens, int nseq, int64_t total_tokens,
    const float* initial_state, const float* d_final_state, void* dq, void* dk, void* dv,
    void* dgate, float* dweight, float* d_initial_state, int heads, int head_dim, int block,
    int chunk_tokens, float eps, la_dtype dtype, void* workspace, size_t workspace_bytes,
    hipStream_t stream) {
    if (nseq < 0 || total_tokens < 0 || total_tokens > 0x7fffffffLL) return LA_ERR_BAD_SHAPE;
    if (nseq == 0 && total_tokens != 0) return LA_ERR_BAD_SHAPE;
    if (nseq > 0 && !cu_seqlens) return LA_ERR_NULL_POINTER;
    if (cu_seqlens && (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u)) return LA_ERR_MISALIGNED;
    return backward_impl(q, k, v, gate, norm_weight, dout, initial_state, d_final_state, dq, dk,
                         dv, dgate, dweight, d_initial_state, cu_seqlens, nseq, 0, total_tokens,
                         heads, head_dim, block, chunk_tokens, eps, dtype, workspace,
                         workspace_bytes, stream);
}

la_status lightning_attn_backward_saved(
    const void* q, const void* k, const void* v, const void* gate, const void* norm_weight,
    const void* dout, const float* initial_state, const float* d_final_state, void* dq, void* dk,
    void* dv, void* dgate, float* dweight, float* d_initial_state, int batch, int64_t seqlen,
    int heads, int head_dim, int block, int chunk_tokens, float eps, la_dtype dtype,
    const void* saved, size_t saved_bytes, void* workspace, size_t workspace_bytes,
    hipStream_t stream) {
    if (batch < 0 || seqlen < 0) return LA_ERR_BAD_SHAPE;
    if (batch > 0 && seqlen > ((int64_t)1 << 40) / batch) return LA_ERR_BAD_SHAPE;
    return backward_impl(q, k, v, gate, norm_weight, dout, initial_state, d_final_state, dq, dk,
                         dv, dgate, dweight, d_initial_state, nullptr, batch, seqlen,
                         (int64_t)batch * seqlen, heads, head_dim, block, chunk_tokens, eps, dtype,
                         workspace, workspace_bytes, stream, saved, saved_bytes, true);
}

la_status lightning_attn_backward_varlen_saved(
    const void* q, const void* k, const void* v, const void* gate, const void* norm_weight,
    const void* dout, const int32_t* cu_seqlens, int nseq, int64_t total_tokens,
    const float* initial_state, const float* d_final_state, void* dq, void* dk, void* dv,
    void* dgate, float* dweight, float* d_initial_state, int heads, int head_dim, int block,
    int chunk_tokens, float eps, la_dtype dtype, const void* saved, size_t saved_bytes,
    void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (nseq < 0 || total_tokens < 0 || total_tokens > 0x7fffffffLL) return LA_ERR_BAD_SHAPE;
    if (nseq == 0 && total_tokens != 0) return LA_ERR_BAD_SHAPE;
    if (nseq > 0 && !cu_seqlens) return LA_ERR_NULL_POINTER;
    if (cu_seqlens && (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u)) return LA_ERR_MISALIGNED;
    return backward_impl(q, k, v, gate, norm_weight, dout, initial_state, d_final_state, dq, dk,
                         dv, dgate, dweight, d_initial_state, cu_seqlens, nseq, 0, total_tokens,
                         heads, head_dim, block, chunk_tokens, eps, dtype, workspace,
                         workspace_bytes, stream, saved, saved_bytes, true);
}

// Layer workspace: the prefill's (automatic chunks), then SiLU(q), SiLU(k),
// SiLU(v), the gate projection and the attention output [total][H*D] bf16
// each, then the GEMM workspace.
struct LayerLayout {
    Layout pre;
    size_t off_act = 0, off_attn = 0, off_gemm = 0, bytes = 0;
};

static bool layer_layout(int64_t total, int nseq, int hidden, int heads, int head_dim,
                         LayerLayout* L) {
    if (hidden < 1 || head_dim != 128) return false;
    // the attention reads activated q, k, v, which only the fused walk takes
    if (!plan_layout(total, nseq, heads, head_dim, 64, 0, true, &L->pre) || !L->pre.fused)
        return false;
    const size_t act = sizeof(uint16_t) * (size_t)total * heads * head_dim;
    size_t off = align_up(L->pre.bytes);
    L->off_act = off;
    off = align_up(off + 4 * act);
    L->off_attn = off;
    off = align_up(off + act);
    L->off_gemm = off;
    off = align_up(off + la::gemm_workspace_bytes());
    L->bytes = off;
    return true;
}

size_t lightning_attn_layer_workspace_size(int64_t total_tokens, int nseq, int hidden, int heads,
                                           int head_dim) {
    LayerLayout L;
    if (total_tokens < 0 || nseq < 0 || heads < 1 ||
        !layer_layout(total_tokens, nseq, hidden, heads, head_dim, &L))
        return 0;
    return L.bytes;
}

la_status lightning_attn_layer_prefill(const void* x, const void* w_qkvg, const void* norm_weight,
                                       const void* w_out, void* out, const float* initial_state,
                                       float* final_state, int batch, int64_t seqlen, int hidden,
                                       int heads, int head_dim, la_gemm gemm, float eps,
                                       void* workspace, size_t workspace_bytes,
                                       hipStream_t stream) {
    if (batch < 0 || seqlen < 0 || heads < 1 || hidden < 1 || !(eps >= 0.0f))
        return LA_ERR_BAD_SHAPE;
    if (batch > 0 && seqlen > ((int64_t)1 << 40) / batch) return LA_ERR_BAD_SHAPE;
    if (head_dim != 128) return LA_ERR_UNSUPPORTED;
    if (gemm != LA_GEMM_MFMA && gemm != LA_GEMM_HIPBLASLT) return LA_ERR_UNSUPPORTED;
    // the library's GEMM: hidden is the reduction of the input projections
    // (a multiple of its 64-wide k steps) and the width of the output one
    if (gemm == LA_GEMM_MFMA && !la::gemm_mfma_supported((int64_t)batch * seqlen,
                                                         heads * head_dim, hidden))
        return LA_ERR_UNSUPPORTED;
    if (gemm == LA_GEMM_MFMA && !la::gemm_mfma_supported((int64_t)batch * seqlen, hidden,
                                                         heads * head_dim))
        return LA_ERR_UNSUPPORTED;
    const int64_t total = (int64_t)batch * seqlen;
    if (total > 0) {
        la_status s = check_ptrs(x, w_qkvg, w_out, norm_weight, out, out);
        if (s != LA_OK) return s;
    }
    if (initial_state && !aligned16(initial_state)) return LA_ERR_MISALIGNED;
    if (final_state && !aligned16(final_state)) return LA_ERR_MISALIGNED;
    LayerLayout L;
    if (!layer_layout(total, batch, hidden, heads, head_dim, &L)) return LA_ERR_UNSUPPORTED;
    if (!workspace) return LA_ERR_NULL_POINTER;
    if (!aligned16(workspace)) return LA_ERR_MISALIGNED;
    if (workspace_bytes < L.bytes) return LA_ERR_WORKSPACE_TOO_SMALL;
    if (batch == 0) return LA_OK;
    char* ws = static_cast<char*>(workspace);
    const int HD = heads * head_dim;
    const size_t act = sizeof(uint16_t) * (size_t)total * HD;
    char* acts = ws + L.off_act;
    void* attn = ws + L.off_attn;
    void* gws = ws + L.off_gemm;
    const size_t gbytes = la::gemm_workspace_bytes();
    const size_t wmat = sizeof(uint16_t) * (size_t)hidden * HD;
    hipError_t e = hipSuccess;
    const bool own = gemm == LA_GEMM_MFMA;
    if (own) {
        // one launch for the four input projections: SiLU on q, k, v and the
        // logistic function on the gate in the epilogue (2 bits per projection)
        const unsigned acts_qkvg = 1u | (1u << 2) | (1u << 4) | (2u << 6);
        e = la::gemm_bf16_mfma(x, w_qkvg, acts, total, HD, hidden, 4, (int64_t)hidden * HD,
                               (int64_t)total * HD, acts_qkvg, stream);
    } else {
        // hipBLASLt: SiLU in the epilogue of the q, k, v projections; the gate
        // stays raw (its sigmoid is applied by the attention when it finalises
        // the outputs)
        const la::GemmAct acts_of[4] = {la::GemmAct::silu, la::GemmAct::silu, la::GemmAct::silu,
                                       la::GemmAct::none};
        for (int i = 0; i < 4 && e == hipSuccess; ++i)
            e = la::gemm_bf16(x, static_cast<const char*>(w_qkvg) + i * wmat, acts + i * act,
                              total, HD, hidden, acts_of[i], gws, gbytes, stream);
    }
    if (e != hipSuccess) return LA_ERR_HIP;
    la::PrefillArgs a{};
    a.q = acts; a.k = acts + act; a.v = acts + 2 * act; a.g = acts + 3 * act;
    a.w = norm_weight; a.out = attn;
    a.init_state = initial_state;
    a.final_state = final_state;
    a.cu = nullptr;
    a.nseq = batch;
    a.seqlen = seqlen;
    a.total = total;
    a.H = heads; a.D = head_dim; a.block = 64;
    a.eps = eps;
    a.bf16 = true;
    a.preact = true;
    a.gate_act = own;
    la_status s = run_prefill(a, L.pre, workspace, stream);
    if (s != LA_OK) return s;
    e = own ? la::gemm_bf16_mfma(attn, w_out, out, total, hidden, HD, 1, 0, 0, 0u, stream)
            : la::gemm_bf16(attn, w_out, out, total, hidden, HD, la::GemmAct::none, gws, gbytes,
                            stream);
    return e == hipSuccess ? LA_OK : LA_ERR_HIP;
}

size_t lightning_attn_softmax_workspace_size(int64_t total_tokens, int nseq, int heads,
                                             int head_dim, int rope_dim) {
    SoftmaxLayout L;
    if (!softmax_layout(total_tokens, nseq, heads, head_dim, rope_dim, &L)) return 0;
    return L.bytes;
}

la_status lightning_attn_softmax_prefill(const void* q, const void* k, const void* v, void* out,
                                         int batch, int64_t seqlen, int heads, int head_dim,
                                         int rope_dim, double rope_base, float scale,
                                         la_dtype dtype, void* workspace, size_t workspace_bytes,
                                         hipStream_t stream) {
    if (batch < 0 || seqlen < 0) return LA_ERR_BAD_SHAPE;
    if (batch > 0 && seqlen > ((int64_t)1 << 40) / batch) return LA_ERR_BAD_SHAPE;
    const int64_t total = (int64_t)batch * seqlen;
    la_status s = softmax_checks(q, k, v, out, total, heads, head_dim, rope_dim, rope_base, scale,
                                 dtype);
    if (s != LA_OK) return s;
    SoftmaxLayout L;
    if (!softmax_layout(total, batch, heads, head_dim, rope_dim, &L)) return LA_ERR_UNSUPPORTED;
    if (!workspace) return LA_ERR_NULL_POINTER;
    if (!aligned16(workspace)) return LA_ERR_MISALIGNED;
    if (workspace_bytes < L.bytes) return LA_ERR_WORKSPACE_TOO_SMALL;
    if (total == 0) return LA_OK;
    return run_softmax(q, k, v, out, nullptr, batch, seqlen, total, heads, rope_dim, rope_base,
                       scale, L, workspace, stream);
}

la_status lightning_attn_softmax_prefill_varlen(const void* q, const void* k, const void* v,
                                                void* out, const int32_t* cu_seqlens, int nseq,
                                                int64_t total_tokens, int heads, int head_dim,
                                                int rope_dim, double rope_base, float scale,
                                                la_dtype dtype, void* workspace,
                                                size_t workspace_bytes, hipStream_t stream) {
    if (nseq < 0 || total_tokens < 0 || total_tokens > ((int64_t)1 << 40)) return LA_ERR_BAD_SHAPE;
    if (nseq == 0 && total_tokens != 0) return LA_ERR_BAD_SHAPE;
    la_status s = softmax_checks(q, k, v, out, total_tokens, heads, head_dim, rope_dim, rope_base,
                                 scale, dtype);
    if (s != LA_OK) return s;
    if (!cu_seqlens) return LA_ERR_NULL_POINTER;
    SoftmaxLayout L;
    if (!softmax_layout(total_tokens, nseq, heads, head_dim, rope_dim, &L))
        return LA_ERR_UNSUPPORTED;
    if (!workspace) return LA_ERR_NULL_POINTER;
    if (!aligned16(workspace)) return LA_ERR_MISALIGNED;
    if (workspace_bytes < L.bytes) return LA_ERR_WORKSPACE_TOO_SMALL;
    if (total_tokens == 0 || nseq == 0) return LA_OK;
    return run_softmax(q, k, v, out, cu_seqlens, nseq, 0, total_tokens, heads, rope_dim, rope_base,
                       scale, L, workspace, stream);
}

// Softmax decode workspace: status [S] int32, rotated queries [S][H][128]
// fp32, partials [S][H][nsplit][130] fp32.
static bool softmax_decode_layout(int nseq, int max_len, int heads, int head_dim, size_t* off_q,
                                  size_t* off_part, size_t* bytes, int* nsplit) {
    if (nseq < 0 || max_len < 1 || heads < 1 || head_dim != 128) return false;
    const int ns = (max_len + la::SOFTMAX_DEC_SPLIT - 1) / la::SOFTMAX_DEC_SPLIT;
    if ((int64_t)nseq * heads * ns > (int64_t)0x7fffffff) return false;
    size_t off = align_up(sizeof(int32_t) * (size_t)nseq);
    *off_q = off;
    off = align_up(off + sizeof(float) * (size_t)nseq * heads * head_dim);
    *off_part = off;
    off = align_up(off + sizeof(float) * (size_t)nseq * heads * ns * (2 + head_dim));
    *bytes = off;
    *nsplit = ns;
    return true;
}

size_t lightning_attn_softmax_decode_workspace_size(int nseq, int max_len, int heads,
                                                    int head_dim) {
    size_t oq, op, bytes;
    int ns;
    if (!softmax_decode_layout(nseq, max_len, heads, head_dim, &oq, &op, &bytes, &ns)) return 0;
    return bytes;
}

la_status lightning_attn_softmax_decode(const void* q, const void* k, const void* v,
                                        void* k_cache, void* v_cache, const int32_t* cache_len,
                                        void* out, int nseq, int max_len, int heads, int head_dim,
                                        int rope_dim, double rope_base, float scale,
                                        la_dtype dtype, void* workspace, size_t workspace_bytes,
                                        hipStream_t stream) {
    if (nseq < 0 || max_len < 1) return LA_ERR_BAD_SHAPE;
    la_status st = softmax_checks(q, k, v, out, nseq, heads, head_dim, rope_dim, rope_base, scale,
                                  dtype);
    if (st != LA_OK) return st;
    if (nseq > 0) {
        if (!k_cache || !v_cache || !cache_len) return LA_ERR_NULL_POINTER;
        if (!aligned16(k_cache) || !aligned16(v_cache)) return LA_ERR_MISALIGNED;
    }
    size_t off_q, off_part, bytes;
    int ns;
    if (!softmax_decode_layout(nseq, max_len, heads, head_dim, &off_q, &off_part, &bytes, &ns))
        return LA_ERR_UNSUPPORTED;
    if (!workspace) return LA_ERR_NULL_POINTER;
    if (!aligned16(workspace)) return LA_ERR_MISALIGNED;
    if (workspace_bytes < bytes) return LA_ERR_WORKSPACE_TOO_SMALL;
    if (nseq == 0) return LA_OK;
    char* ws = static_cast<char*>(workspace);
    la::SoftmaxDecodeArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.len = cache_len;
    a.out = out;
    a.nseq = nseq;
    a.max_len = max_len;
    a.H = heads;
    a.rope_dim = rope_dim;
    a.rope_base = rope_base;
    a.scale = scale;
    a.nsplit = ns;
    a.status = reinterpret_cast<int32_t*>(ws);
    a.qr = reinterpret_cast<float*>(ws + off_q);
    a.part = reinterpret_cast<float*>(ws + off_part);
    return la::launch_softmax_decode(a, stream) == hipSuccess ? LA_OK : LA_ERR_HIP;
}

size_t lightning_attn_decode_workspace_size(int nseq, int heads, int head_dim) {
    if (nseq < 0 || heads < 1 || !supported_dim(head_dim)) return 0;
    return align_up(sizeof(float) * (size_t)nseq * heads * head_dim) +
           align_up(sizeof(float) * (size_t)nseq * heads);
}

static la_status decode_impl(const void* q, const void* k, const void* v, const void* gate,
                             const void* norm_weight, void* out, float* state, int nseq, int heads,
                             int head_dim, float eps, la_dtype dtype, void* workspace,
                             size_t workspace_bytes, hipStream_t stream, Marks marks) {
    if (nseq < 0 || heads < 1 || !(eps >= 0.0f)) return LA_ERR_BAD_SHAPE;
    if (check_dtype(dtype) != LA_OK || !supported_dim(head_dim)) return LA_ERR_UNSUPPORTED;
    if ((int64_t)nseq * heads > 0x7fffffffLL) return LA_ERR_BAD_SHAPE;
    if (nseq > 0) {
        la_status s = check_ptrs(q, k, v, gate, norm_weight, out);
        if (s != LA_OK) return s;
        if (!state) return LA_ERR_NULL_POINTER;
        if (!aligned16(state)) return LA_ERR_MISALIGNED;
    }
    const size_t need = lightning_attn_decode_workspace_size(nseq, heads, head_dim);
    if (!workspace) return LA_ERR_NULL_POINTER;
    if (!aligned16(workspace)) return LA_ERR_MISALIGNED;
    if (workspace_bytes < need) return LA_ERR_WORKSPACE_TOO_SMALL;
    if (nseq == 0) return LA_OK;
    la::DecodeArgs a{};
    a.q = q; a.k = k; a.v = v; a.g = gate; a.w = norm_weight; a.out = out;
    a.state = state;
    a.nseq = nseq; a.H = heads; a.D = head_dim;
    a.eps = eps;
    a.bf16 = dtype == LA_DTYPE_BF16;
    a.ybuf = static_cast<float*>(workspace);
    a.ssbuf = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                       align_up(sizeof(float) * (size_t)nseq * heads * head_dim));
    hipError_t e = marks.mark(stream);
    if (e == hipSuccess) e = la::launch_decode_state(a, stream);
    if (e == hipSuccess) e = marks.mark(stream);
    if (e == hipSuccess) e = la::launch_decode_norm(a, stream);
    if (e == hipSuccess) e = marks.mark(stream);
    return e == hipSuccess ? LA_OK : LA_ERR_HIP;
}

la_status lightning_attn_decode(const void* q, const void* k, const void* v, const void* gate,
                                const void* norm_weight, void* out, float* state, int nseq,
                                int heads, int head_dim, float eps, la_dtype dtype,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return decode_impl(q, k, v, gate, norm_weight, out, state, nseq, heads, head_dim, eps, dtype,
                       workspace, workspace_bytes, stream, Marks());
}

la_status lightning_attn_decode_noalloc(const void* q, const void* k, const void* v,
                                        const void* gate, const void* norm_weight, void* out,
                                        float* state, int nseq, int heads, int head_dim, float eps,
                                        la_dtype dtype, hipStream_t stream) {
    if (nseq < 0 || heads < 1 || !(eps >= 0.0f)) return LA_ERR_BAD_SHAPE;
    if (check_dtype(dtype) != LA_OK || !supported_dim(head_dim)) return LA_ERR_UNSUPPORTED;
    if ((int64_t)nseq * heads > 0x7fffffffLL) return LA_ERR_BAD_SHAPE;
    if (nseq == 0) return LA_OK;
    const size_t need = lightning_attn_decode_workspace_size(nseq, heads, head_dim);
    const bool scratch = la::decode_uses_workspace(nseq, heads, head_dim);
    if (scratch && need > la::decode_scratch_bytes()) return LA_ERR_SCRATCH_TOO_SMALL;
    // the shapes that run one kernel per sequence read no workspace: decode_impl
    // still validates one, so it gets the scratch's address and a size that passes
    void* ws = nullptr;
    if (la::decode_scratch(&ws) != hipSuccess) return LA_ERR_HIP;
    return decode_impl(q, k, v, gate, norm_weight, out, state, nseq, heads, head_dim, eps, dtype,
                       ws, scratch ? la::decode_scratch_bytes() : need, stream, Marks());
}

la_status lightning_attn_decode_profiled(
    const void* q, const void* k, const void* v, const void* gate, const void* norm_weight,
    void* out, float* state, int nseq, int heads, int head_dim, float eps, la_dtype dtype,
    void* workspace, size_t workspace_bytes, hipStream_t stream, hipEvent_t* events,
    int n_events) {
    Marks m;
    if (n_events != 0) {
        if (events == nullptr) return LA_ERR_NULL_POINTER;
        if (n_events < kDecodeStageCount + 1) return LA_ERR_BAD_SHAPE;
        m.ev = events;
        m.n = n_events;
    }
    return decode_impl(q, k, v, gate, norm_weight, out, state, nseq, heads, head_dim, eps, dtype,
                       workspace, workspace_bytes, stream, m);
}

}  // extern "C"
