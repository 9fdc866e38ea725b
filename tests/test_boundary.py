"""The C-ABI library on a host without a GPU: it loads, exports every symbol
include/lightning_attn.h declares, and rejects bad arguments on the host
before any HIP call (no compute is launched here)."""
import ctypes
import os
import re
import subprocess

import pytest
import torch

from long_context_attn_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lightning_attn.h")

OK, NULLP, SHAPE, UNSUP, MISAL, WS, HIPERR = range(7)
F32, BF16 = 0, 1
A = 0x10000  # a fake 16-byte aligned "device" address: never dereferenced


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ops.LIB_PATH):
        from long_context_attn_amd import build
        build.build()
    return ops.library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"LA_API\s+[\w\s\*]+?\b(lightning_attn_\w+)\s*\(", text)))


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("lightning_attn_prefill", "lightning_attn_prefill_varlen", "lightning_attn_decode"):
        assert n in names
    for n in ("lightning_attn_prefill_profiled", "lightning_attn_decode_profiled",
              "lightning_attn_state", "lightning_attn_state_varlen",
              "lightning_attn_state_workspace_size", "lightning_attn_backward",
              "lightning_attn_backward_varlen", "lightning_attn_backward_workspace_size",
              "lightning_attn_layer_prefill", "lightning_attn_layer_workspace_size",
              "lightning_attn_softmax_prefill", "lightning_attn_softmax_prefill_varlen",
              "lightning_attn_softmax_workspace_size", "lightning_attn_softmax_decode",
              "lightning_attn_softmax_decode_workspace_size", "lightning_attn_workspace_status",
              "lightning_attn_decode_noalloc", "lightning_attn_saved_size",
              "lightning_attn_prefill_save", "lightning_attn_prefill_varlen_save",
              "lightning_attn_backward_saved", "lightning_attn_backward_varlen_saved"):
        assert n in names
    assert len(names) == 32


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", ops.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(\w+)", out))
    for n in declared_functions():
        assert n in exported, n
        assert hasattr(lib, n)
    # nothing else leaks out of the library under the API's prefix
    assert {e for e in exported if e.startswith("lightning_attn")} == set(declared_functions())


def test_status_strings(lib):
    assert ops.status_string(0) == "ok"
    for s in range(1, 8):
        assert len(ops.status_string(s)) > 10
    assert ops.status_string(99) == "unknown status"


def test_prefill_workspace_size(lib):
    ws = ops.prefill_workspace_size(8192, 1, 64, 128, 64, 1024)
    # bf16 MFMA path, 8 chunks of 1024 tokens (+ one spare per sequence): a 64 heads x
    # 128 x 128 fp32 state per chunk (chunk sum, then the state entering the chunk), and
    # per (chunk, 64-token block) the RMSNorm exchange: 64 heads x 64 tokens of partial
    # sums and 64 sums for each group of 16 heads, each an 8-byte {value, written} word
    slots = 9 * (1024 // 64)
    need = 9 * 64 * 128 * 128 * 4 + slots * (64 * 64 * 8 + 4 * 64 * 8)
    assert need <= ws < need + 65536
    # the automatic choice is the chunked prefill with about 256 (chunk, head) items:
    # 2048-token chunks for 64 heads, 128-token chunks for 4 heads
    slots = (4 + 1) * (2048 // 64)
    need = 5 * 64 * 128 * 128 * 4 + slots * (64 * 64 * 8 + 4 * 64 * 8)
    assert need <= ops.prefill_workspace_size(8192, 1, 64, 128, 64, 0) < need + 65536
    slots = (64 + 1) * (128 // 64)
    need = 65 * 4 * 128 * 128 * 4 + slots * (4 * 64 * 8 + 1 * 64 * 8)
    assert need <= ops.prefill_workspace_size(8192, 1, 4, 128, 64, 0) < need + 65536
    # negative chunk sizes are refused
    assert ops.prefill_workspace_size(8192, 1, 64, 128, 64, -1) == 0
    assert ops.prefill_workspace_size(8192, 1, 64, 128, 64, -2) == 0
    ws32 = ops.prefill_workspace_size(8192, 1, 64, 128, 64, 1024, dtype=torch.float32)
    assert 9 * 64 * 128 * 128 * 4 <= ws32 < 9 * 64 * 128 * 128 * 4 + 65536
    assert ops.prefill_workspace_size(8192, 1, 64, 96, 64, 0) == 0      # head_dim
    assert ops.prefill_workspace_size(8192, 1, 64, 128, 48, 0) == 0     # block
    assert ops.prefill_workspace_size(8192, 1, 64, 128, 64, 100) == 0   # chunk % block
    assert ops.prefill_workspace_size(8192, 1, 64, 128, 64, 32) == 0    # chunk < block
    assert ops.prefill_workspace_size(0, 0, 64, 128, 64, 0) > 0
    # varlen: one extra chunk per sequence at most
    assert ops.prefill_workspace_size(1000, 3, 2, 64, 32, 64) >= (1000 // 64 + 3) * 2 * 64 * 64 * 4
    assert ops.decode_workspace_size(256, 64, 128) >= 256 * 64 * 128 * 4 + 256 * 64 * 4


def test_fused_walk_needs_heads_within_cus(lib):
    """The fused walk's cross-head exchange waits on the workgroups of every head
    of a chunk (one per CU), so it is taken only for heads <= CUs (256 without a
    GPU); wider calls get the portable kernels' workspace (no exchange words),
    the same size as for fp32, and the layer (fused walk only) is refused."""
    for heads in (255, 256):
        bf = ops.prefill_workspace_size(8192, 1, heads, 128, 64, 1024)
        f32 = ops.prefill_workspace_size(8192, 1, heads, 128, 64, 1024, dtype=torch.float32)
        assert bf > f32  # + exchange words
    for heads in (257, 512):
        bf = ops.prefill_workspace_size(8192, 1, heads, 128, 64, 1024)
        f32 = ops.prefill_workspace_size(8192, 1, heads, 128, 64, 1024, dtype=torch.float32)
        assert bf == f32 > 0
        assert ops.layer_workspace_size(8192, 1, 6144, heads, 128) == 0
    assert ops.layer_workspace_size(8192, 1, 6144, 256, 128) > 0
    assert lib.lightning_attn_layer_prefill(A, A, A, A, A, None, None, 1, 100, 256, 257, 128, 0,
                                            1e-6, A, 1 << 40, None) == UNSUP


def test_workspace_status_validation(lib):
    st = (ctypes.c_int32 * 4)()
    assert lib.lightning_attn_workspace_status(None, 1 << 20, st, None) == NULLP
    assert lib.lightning_attn_workspace_status(A, 1 << 20, None, None) == NULLP
    assert lib.lightning_attn_workspace_status(A + 8, 1 << 20, st, None) == MISAL
    assert lib.lightning_attn_workspace_status(A, 32, st, None) == WS


def _prefill(lib, q=A, k=A, v=A, g=A, w=A, out=A, init=None, fin=None, batch=1, seqlen=128,
             heads=2, d=64, block=32, chunk=0, eps=1e-6, dtype=F32, ws=A, ws_bytes=1 << 40):
    return lib.lightning_attn_prefill(q, k, v, g, w, out, init, fin, batch, seqlen, heads, d,
                                      block, chunk, eps, dtype, ws, ws_bytes, None)


def test_prefill_validation(lib):
    assert _prefill(lib, q=None) == NULLP
    assert _prefill(lib, out=None) == NULLP
    assert _prefill(lib, ws=None) == NULLP
    assert _prefill(lib, k=A + 8) == MISAL
    assert _prefill(lib, init=A + 4) == MISAL
    assert _prefill(lib, fin=A + 4) == MISAL
    assert _prefill(lib, ws=A + 8) == MISAL
    assert _prefill(lib, d=96) == UNSUP
    assert _prefill(lib, block=48) == UNSUP
    assert _prefill(lib, chunk=48) == UNSUP
    assert _prefill(lib, dtype=7) == UNSUP
    assert _prefill(lib, batch=-1) == SHAPE
    assert _prefill(lib, seqlen=-5) == SHAPE
    assert _prefill(lib, heads=0) == SHAPE
    assert _prefill(lib, eps=-1.0) == SHAPE
    assert _prefill(lib, eps=float("nan")) == SHAPE
    assert _prefill(lib, chunk=-64) == SHAPE
    assert _prefill(lib, chunk=-1) == SHAPE
    assert _prefill(lib, d=128, block=64, dtype=BF16, chunk=-1) == SHAPE
    assert _prefill(lib, ws_bytes=100) == WS
    # empty batch: valid, nothing to enqueue
    assert _prefill(lib, batch=0, q=None, k=None, v=None, g=None, w=None, out=None) == OK


def test_varlen_validation(lib):
    def call(q=A, cu=A, nseq=2, total=100, d=64, block=32, ws=A, ws_bytes=1 << 40, eps=1e-6):
        return lib.lightning_attn_prefill_varlen(q, A, A, A, A, A, cu, nseq, total, None, None, 2,
                                                 d, block, 0, eps, F32, ws, ws_bytes, None)
    assert call(q=None) == NULLP
    assert call(cu=None) == NULLP
    assert call(cu=A + 2) == MISAL
    assert call(nseq=-1) == SHAPE
    assert call(total=-1) == SHAPE
    assert call(total=1 << 31) == SHAPE
    assert call(nseq=0, total=10) == SHAPE
    assert call(d=48) == UNSUP
    assert lib.lightning_attn_prefill_varlen(A, A, A, A, A, A, A, 2, 100, None, None, 2, 64, 32,
                                             -1, 1e-6, F32, A, 1 << 40, None) == SHAPE
    assert call(ws_bytes=64) == WS
    assert call(nseq=0, total=0, q=None, cu=None) == OK


def test_state_workspace_size(lib):
    # the plan and one fp32 state per (chunk, head)
    for args in ((8192, 1, 64, 128, 64, 0), (1000, 3, 2, 64, 32, 64)):
        assert ops.state_workspace_size(*args) > 0
    assert ops.state_workspace_size(1000, 3, 2, 64, 32, 64) >= (1000 // 64 + 3) * 2 * 64 * 64 * 4
    st = ops.state_workspace_size(8192, 1, 64, 128, 64, 1024)
    # room for total / chunk + nseq chunks (a sequence's last chunk may be partial)
    assert 9 * 64 * 128 * 128 * 4 <= st < 9 * 64 * 128 * 128 * 4 + 65536
    assert ops.state_workspace_size(8192, 1, 64, 128, 64, -1) == 0
    assert ops.state_workspace_size(8192, 1, 64, 96, 64, 0) == 0
    assert ops.state_workspace_size(8192, 1, 64, 128, 64, 100) == 0
    assert ops.state_workspace_size(0, 0, 64, 128, 64, 0) > 0


def test_state_validation(lib):
    def call(k=A, v=A, init=None, fin=A, batch=2, seqlen=100, heads=2, d=64, block=32, chunk=0,
             dtype=BF16, ws=A, ws_bytes=1 << 40):
        return lib.lightning_attn_state(k, v, init, fin, batch, seqlen, heads, d, block, chunk,
                                        dtype, ws, ws_bytes, None)
    assert call(k=None) == NULLP
    assert call(fin=None) == NULLP          # the final state is the only output
    assert call(ws=None) == NULLP
    assert call(v=A + 8) == MISAL
    assert call(init=A + 4) == MISAL
    assert call(fin=A + 4) == MISAL
    assert call(d=96) == UNSUP
    assert call(block=48) == UNSUP
    assert call(dtype=3) == UNSUP
    assert call(chunk=-1) == SHAPE
    assert call(batch=-1) == SHAPE
    assert call(heads=0) == SHAPE
    assert call(ws_bytes=100) == WS
    assert call(batch=0, k=None, v=None, fin=None) == OK

    def vcall(k=A, cu=A, nseq=2, total=100, fin=A, ws_bytes=1 << 40):
        return lib.lightning_attn_state_varlen(k, A, cu, nseq, total, None, fin, 2, 64, 32, 0, F32,
                                               A, ws_bytes, None)
    assert vcall(cu=None) == NULLP
    assert vcall(fin=None) == NULLP
    assert vcall(cu=A + 2) == MISAL
    assert vcall(nseq=0, total=10) == SHAPE
    assert vcall(total=1 << 31) == SHAPE
    assert vcall(ws_bytes=8) == WS
    assert vcall(nseq=0, total=0, k=None, cu=None, fin=None) == OK


def test_backward_workspace_size(lib):
    # plan + two states per chunk + y and dy + dw partial sums per 8 tokens,
    # at most 2048 rows;
    # bf16 at head_dim 128 (MFMA walks): y and dy in bf16 and no other copies;
    # otherwise y, dy and q~, k~, v~ in fp32
    T, H, D = 8192, 64, 128
    act = T * H * D * 4
    states = 2 * (T // 256 + 1) * H * D * D * 4
    parts = (T // 8) * H * D * 4
    need = act + states + parts
    assert need <= ops.backward_workspace_size(T, 1, H, D, 64, 256) < need + 65536
    need = 5 * act + states + parts
    ws = ops.backward_workspace_size(T, 1, H, D, 64, 256, dtype=torch.float32)
    assert need <= ws < need + 65536
    # automatic chunks: 2048 tokens on the MFMA path (about one walk per CU)
    need = act + 2 * (T // 2048 + 1) * H * D * D * 4 + parts
    assert need <= ops.backward_workspace_size(T, 1, H, D, 64, 0) < need + 65536
    assert ops.backward_workspace_size(T, 1, H, 96, 64, 0) == 0
    assert ops.backward_workspace_size(T, 1, 257, D, 64, 0) == 0  # heads * head_dim > 32768
    assert ops.backward_workspace_size(T, 1, H, D, 64, 100) == 0
    assert ops.backward_workspace_size(T, 1, H, D, 64, -1) == 0
    assert ops.backward_workspace_size(0, 0, H, D, 64, 0) > 0
    # 1M tokens: the dw partial rows stop at 2048 (512 tokens each)
    T = 1 << 20
    act = T * H * D * 4
    need = act + 2 * (T // 8192 + 1) * H * D * D * 4 + 2048 * H * D * 4
    assert need <= ops.backward_workspace_size(T, 1, H, D, 64, 8192) < need + 65536


def test_backward_validation(lib):
    def call(q=A, dq=A, dw=A, init=None, dfin=None, dinit=None, batch=2, seqlen=100, heads=2,
             d=64, block=32, chunk=0, eps=1e-6, dtype=F32, ws=A, ws_bytes=1 << 40):
        return lib.lightning_attn_backward(q, A, A, A, A, A, init, dfin, dq, A, A, A, dw, dinit,
                                           batch, seqlen, heads, d, block, chunk, eps, dtype, ws,
                                           ws_bytes, None)
    assert call(q=None) == NULLP
    assert call(dq=None) == NULLP
    assert call(dw=None) == NULLP
    assert call(ws=None) == NULLP
    assert call(q=A + 8) == MISAL
    assert call(dfin=A + 4) == MISAL
    assert call(dinit=A + 4) == MISAL
    assert call(d=96) == UNSUP
    assert call(block=48) == UNSUP
    assert call(chunk=48) == UNSUP
    assert call(dtype=9) == UNSUP
    assert call(chunk=-1) == SHAPE
    assert call(batch=-1) == SHAPE
    assert call(eps=-1.0) == SHAPE
    assert call(ws_bytes=64) == WS
    assert call(batch=0, q=None, dq=None, dw=None) == OK

    def vcall(cu=A, nseq=2, total=100, ws_bytes=1 << 40):
        return lib.lightning_attn_backward_varlen(A, A, A, A, A, A, cu, nseq, total, None, None, A,
                                                  A, A, A, A, None, 2, 64, 32, 0, 1e-6, F32, A,
                                                  ws_bytes, None)
    assert vcall(cu=None) == NULLP
    assert vcall(cu=A + 2) == MISAL
    assert vcall(nseq=0, total=5) == SHAPE
    assert vcall(total=1 << 31) == SHAPE
    assert vcall(ws_bytes=8) == WS


def test_layer_workspace_and_validation(lib):
    # the prefill's workspace, 5 bf16 activations of T x H*D, 64 MiB for the GEMMs
    T, H, D, hidden = 8192, 64, 128, 6144
    ws = ops.layer_workspace_size(T, 1, hidden, H, D)
    pre = ops.prefill_workspace_size(T, 1, H, D, 64, 0)
    need = pre + 5 * T * H * D * 2 + (64 << 20)
    assert need <= ws < need + 65536
    assert ops.layer_workspace_size(T, 1, hidden, H, 64) == 0   # head_dim 128 only
    assert ops.layer_workspace_size(T, 1, 0, H, D) == 0

    def call(x=A, w=A, out=A, batch=2, seqlen=100, hidden=256, heads=2, d=128, gemm=0, eps=1e-6,
             ws=A, ws_bytes=1 << 40):
        return lib.lightning_attn_layer_prefill(x, w, A, A, out, None, None, batch, seqlen, hidden,
                                                heads, d, gemm, eps, ws, ws_bytes, None)
    assert call(x=None) == NULLP
    assert call(out=None) == NULLP
    assert call(ws=None) == NULLP
    assert call(w=A + 8) == MISAL
    assert call(d=64) == UNSUP
    assert call(batch=-1) == SHAPE
    assert call(hidden=0) == SHAPE
    assert call(eps=-1.0) == SHAPE
    assert call(ws_bytes=1024) == WS
    assert call(batch=0, x=None, w=None, out=None) == OK
    assert call(gemm=2) == UNSUP                     # no such GEMM backend
    assert call(hidden=200) == UNSUP                 # the library's GEMM: hidden % 64
    assert call(hidden=200, gemm=1, ws_bytes=8) == WS  # hipBLASLt takes any hidden


def test_softmax_workspace_and_validation(lib):
    # plan (header, sequences, 128-token query tiles) + rotated k
    T, H, D = 8192, 64, 128
    ws = ops.softmax_workspace_size(T, 1, H, D, 64)
    assert T * H * D * 2 <= ws < T * H * D * 2 + 65536
    assert ops.softmax_workspace_size(T, 1, H, D, 0) < 65536   # no rotation: no copies
    assert ops.softmax_workspace_size(T, 1, H, 64, 32) == 0    # head_dim 128 only
    assert ops.softmax_workspace_size(T, 1, H, D, 12) == 0     # rope_dim a multiple of 8
    assert ops.softmax_workspace_size(T, 1, H, D, 136) == 0    # rope_dim <= head_dim
    D64 = ctypes.c_double

    def call(q=A, out=A, batch=2, seqlen=100, heads=2, d=128, rd=64, base=1e7, scale=0.088,
             dtype=BF16, ws=A, ws_bytes=1 << 40):
        return lib.lightning_attn_softmax_prefill(q, A, A, out, batch, seqlen, heads, d, rd,
                                                  D64(base), scale, dtype, ws, ws_bytes, None)
    assert call(q=None) == NULLP
    assert call(out=None) == NULLP
    assert call(ws=None) == NULLP
    assert call(q=A + 8) == MISAL
    assert call(d=64) == UNSUP
    assert call(dtype=F32) == UNSUP
    assert call(rd=12) == UNSUP
    assert call(batch=-1) == SHAPE
    assert call(heads=0) == SHAPE
    assert call(scale=0.0) == SHAPE
    assert call(scale=float("nan")) == SHAPE
    assert call(base=0.0) == SHAPE
    assert call(base=0.0, rd=0, ws_bytes=16) == WS  # the base is unused without rotation
    assert call(ws_bytes=1024) == WS
    assert call(batch=0, q=None, out=None) == OK

    def vcall(cu=A, nseq=3, total=100, ws_bytes=1 << 40):
        return lib.lightning_attn_softmax_prefill_varlen(A, A, A, A, cu, nseq, total, 2, 128, 64,
                                                         D64(1e7), 0.088, BF16, A, ws_bytes, None)
    assert vcall(cu=None) == NULLP
    assert vcall(nseq=-1) == SHAPE
    assert vcall(nseq=0) == SHAPE
    assert vcall(ws_bytes=10) == WS
    assert vcall(nseq=0, total=0) == OK


def test_softmax_decode_workspace_and_validation(lib):
    # status words, fp32 rotated queries, (2 + 128)-float partials per 512-key range
    S, L, H, D = 4, 1000, 8, 128
    ws = ops.softmax_decode_workspace_size(S, L, H, D)
    need = S * 4 + S * H * D * 4 + S * H * 2 * (2 + D) * 4
    assert need <= ws < need + 1024
    assert ops.softmax_decode_workspace_size(S, 0, H, D) == 0
    assert ops.softmax_decode_workspace_size(S, L, H, 64) == 0
    D64 = ctypes.c_double

    def call(q=A, kc=A, ln=A, out=A, nseq=4, max_len=1000, heads=8, d=128, rd=64, scale=0.088,
             dtype=BF16, ws=A, ws_bytes=1 << 40):
        return lib.lightning_attn_softmax_decode(q, A, A, kc, A, ln, out, nseq, max_len, heads,
                                                 d, rd, D64(1e7), scale, dtype, ws, ws_bytes,
                                                 None)
    assert call(q=None) == NULLP
    assert call(kc=None) == NULLP
    assert call(ln=None) == NULLP
    assert call(out=None) == NULLP
    assert call(ws=None) == NULLP
    assert call(kc=A + 8) == MISAL
    assert call(d=64) == UNSUP
    assert call(dtype=F32) == UNSUP
    assert call(nseq=-1) == SHAPE
    assert call(max_len=0) == SHAPE
    assert call(scale=-1.0) == SHAPE
    assert call(ws_bytes=100) == WS
    assert call(nseq=0, q=None, kc=None, ln=None, out=None) == OK


def test_decode_validation(lib):
    def call(q=A, state=A, nseq=4, heads=2, d=64, ws=A, ws_bytes=1 << 30, dtype=BF16):
        return lib.lightning_attn_decode(q, A, A, A, A, A, state, nseq, heads, d, 1e-6, dtype, ws,
                                         ws_bytes, None)
    assert call(q=None) == NULLP
    assert call(state=None) == NULLP
    assert call(state=A + 4) == MISAL
    assert call(ws=None) == NULLP
    assert call(nseq=-1) == SHAPE
    assert call(heads=0) == SHAPE
    assert call(d=100) == UNSUP
    assert call(dtype=5) == UNSUP
    assert call(ws_bytes=16) == WS
    assert call(nseq=0, q=None, state=None) == OK


def test_decode_noalloc_validation(lib):
    """Host-side checks of the no-allocation decode (nothing reaches HIP)."""
    def call(q=A, state=A, nseq=8, heads=4, d=64, eps=1e-6, dtype=F32):
        return lib.lightning_attn_decode_noalloc(q, A, A, A, A, A, state, nseq, heads, d, eps,
                                                 dtype, None)
    assert call(nseq=-1) == SHAPE
    assert call(heads=0) == SHAPE
    assert call(eps=-1.0) == SHAPE
    assert call(d=96) == UNSUP
    assert call(dtype=5) == UNSUP
    assert call(nseq=0, q=None, state=None) == OK
    # y of 255 sequences x 64 heads x 128 (fewer sequences than the 256 CUs assumed
    # without a GPU: the two-kernel path) needs 8.2 MB, more than the fixed 4 MiB + 64 KiB
    assert call(nseq=255, heads=64, d=128, dtype=BF16) == 7
    assert ops.status_string(7).startswith("sizes exceed the fixed scratch")


def test_stage_names_and_profiled_validation(lib):
    assert lib.lightning_attn_prefill_stage_count() == 5
    lib.lightning_attn_prefill_stage_name.restype = ctypes.c_char_p
    lib.lightning_attn_decode_stage_name.restype = ctypes.c_char_p
    names = [lib.lightning_attn_prefill_stage_name(i) for i in range(5)]
    assert names == [b"plan", b"chunk_state", b"state_scan", b"walk", b"norm_gate"]
    assert lib.lightning_attn_prefill_stage_name(5) is None
    assert lib.lightning_attn_decode_stage_count() == 2
    assert lib.lightning_attn_decode_stage_name(0) == b"decode_state"
    assert lib.lightning_attn_decode_stage_name(-1) is None
    f = lib.lightning_attn_prefill_profiled
    f.argtypes = [ctypes.c_void_p] * 8 + [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_int,
                                          ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_int]
    ev = (ctypes.c_void_p * 8)()
    args = [A] * 6 + [None, None, 1, 128, 2, 64, 32, 0, 1e-6, F32, A, 1 << 40, None]
    assert f(*args, None, 6) == NULLP          # events missing
    assert f(*args, ev, 3) == SHAPE            # too few events
    assert f(*(args[:9] + [-1] + args[10:]), ev, 6) == SHAPE  # validation still applies
    d = lib.lightning_attn_decode_profiled
    d.argtypes = [ctypes.c_void_p] * 7 + [ctypes.c_int] * 3 + [ctypes.c_float, ctypes.c_int,
                                                                ctypes.c_void_p, ctypes.c_size_t,
                                                                ctypes.c_void_p, ctypes.c_void_p,
                                                                ctypes.c_int]
    dargs = [A] * 7 + [4, 2, 64, 1e-6, F32, A, 1 << 30, None]
    assert d(*dargs, ev, 2) == SHAPE
    assert d(*dargs, None, 3) == NULLP


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(ops, "_lib", None)
    monkeypatch.setattr(ops, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        ops.library()


def test_product_path_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "long_context_attn_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.replace("CPU oracle", ""), os.path.join(dirpath, f)


def test_saved_activations_validation(lib):
    """Saving (and starting the backward from saved activations) is only for
    the fused bf16 path; the buffer is checked like a workspace."""
    sz = lib.lightning_attn_saved_size
    y = 8192 * 64 * 128 * 2
    assert y + 5 * 64 * 128 * 128 * 4 <= sz(8192, 1, 64, 128, 64, 0, BF16) < y + 5 * 64 * 128 * 128 * 4 + 4096
    assert sz(8192, 1, 64, 128, 64, 0, F32) == 0          # fp32: portable kernels, no save
    assert sz(8192, 1, 64, 64, 64, 0, BF16) == 0          # head_dim 64
    assert sz(8192, 1, 64, 128, 32, 0, BF16) == 0         # block 32
    assert sz(8192, 1, 257, 128, 64, 0, BF16) == 0        # more heads than CUs
    assert sz(8192, 1, 64, 128, 64, -1, BF16) == 0
    need = sz(1000, 2, 3, 128, 64, 0, BF16)
    assert need > 0

    def pre(saved=A, saved_bytes=1 << 40, dtype=BF16, d=128, block=64):
        return lib.lightning_attn_prefill_save(A, A, A, A, A, A, None, None, 2, 500, 3, d, block,
                                               0, 1e-6, dtype, saved, saved_bytes, A, 1 << 40, None)
    assert pre(saved=None) == NULLP
    assert pre(saved=A + 8) == MISAL
    assert pre(saved_bytes=need - 1) == WS
    assert pre(dtype=F32) == UNSUP
    assert pre(d=64) == UNSUP
    assert pre(block=32) == UNSUP

    def bwd(saved=A, saved_bytes=1 << 40, dtype=BF16):
        return lib.lightning_attn_backward_saved(A, A, A, A, A, A, None, None, A, A, A, A, A, None,
                                                 2, 500, 3, 128, 64, 0, 1e-6, dtype, saved,
                                                 saved_bytes, A, 1 << 40, None)
    assert bwd(saved=None) == NULLP
    assert bwd(saved_bytes=need - 1) == WS
    assert bwd(dtype=F32) == UNSUP

    def vpre(saved=A, saved_bytes=1 << 40, cu=A):
        return lib.lightning_attn_prefill_varlen_save(A, A, A, A, A, A, cu, 2, 1000, None, None, 3,
                                                      128, 64, 0, 1e-6, BF16, saved, saved_bytes,
                                                      A, 1 << 40, None)
    assert vpre(saved=None) == NULLP
    assert vpre(saved_bytes=need - 1) == WS
    assert vpre(cu=None) == NULLP

    def vbwd(saved=A, saved_bytes=1 << 40):
        return lib.lightning_attn_backward_varlen_saved(A, A, A, A, A, A, A, 2, 1000, None, None, A,
                                                        A, A, A, A, None, 3, 128, 64, 0, 1e-6,
                                                        BF16, saved, saved_bytes, A, 1 << 40, None)
    assert vbwd(saved=None) == NULLP
    assert vbwd(saved_bytes=need - 1) == WS
