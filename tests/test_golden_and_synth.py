"""Golden fixtures and the seeded input generator (no GPU)."""
import json
import os
import sys

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))
import oracle  # noqa: E402
from long_context_attn_amd import synth  # noqa: E402
import make_golden  # noqa: E402


def test_oracle_regression_fixture():
    doc = json.load(open(os.path.join(HERE, "golden", "oracle_regression.json")))
    q, k, v, g, w, s0 = make_golden.inputs()
    out, st = oracle.prefill(q, k, v, g, w, cu_seqlens=doc["seg"], eps=doc["eps"],
                             init_state=s0, return_state=True)
    np.testing.assert_allclose(out.reshape(-1), doc["out"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(st.reshape(-1), doc["final_state"], rtol=1e-12, atol=1e-12)


def test_page_facts_match_workloads():
    facts = json.load(open(os.path.join(HERE, "golden", "page_facts.json")))
    import bench
    assert bench.PREFILL_8K["heads"] == facts["attention_heads"]
    assert bench.PREFILL_8K["head_dim"] == facts["attention_head_dim"]
    assert bench.PREFILL_1M["seqlen"] >= facts["training_context_tokens"]


def test_round_bf16_matches_torch():
    import torch
    x = synth.stream((1, 2, 3), 100000) * np.float32(3.7)
    x = np.concatenate([x, np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0,
                                     65504.0, 1e-30], np.float32)])
    ours = synth.round_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(ours, ref)
    # ties go to even
    assert synth.round_bf16(np.array([1.0 + 2 ** -8], np.float32))[0] == 1.0
    assert synth.round_bf16(np.array([1.0 + 3 * 2 ** -8], np.float32))[0] == 1.0 + 2 ** -6


def test_stream_is_prefix_consistent_and_chunked():
    a = synth.stream((5, 6), 1000)
    b = synth.stream((5, 6), 300)
    assert np.array_equal(a[:300], b)
    H, D = 2, 8
    full = synth.token_tensor(1, synth.Q, 0, 70000, H, D, 1.0)
    part = synth.token_tensor(1, synth.Q, 65000, 66000, H, D, 1.0)
    assert np.array_equal(full[65000:66000], part)
    thr = synth.token_tensor(1, synth.Q, 0, 70000, H, D, 1.0, threads=4)
    assert np.array_equal(full, thr)


def test_block_tensor_windows_and_heads_agree():
    """Per-(1024-token block, head) streams: any window or head subset is the
    same slice of the whole tensor, with or without threads."""
    D = 8
    full = synth.block_tensor(5, synth.K, 0, 3000, range(4), D, 0.5)
    assert full.shape == (3000, 4, D)
    assert np.array_equal(synth.block_tensor(5, synth.K, 1000, 2100, [1, 3], D, 0.5),
                          full[1000:2100][:, [1, 3]])
    assert np.array_equal(synth.block_tensor(5, synth.K, 0, 3000, range(4), D, 0.5, threads=3),
                          full)
    # other tensors and workloads are other streams; values are bf16-representable
    assert not np.array_equal(synth.block_tensor(5, synth.V, 0, 3000, range(4), D, 0.5), full)
    assert np.array_equal(synth.round_bf16(full), full)
    assert synth.pick(3, 20, 4) == synth.pick(3, 20, 4) and len(set(synth.pick(5, 8, 4))) == 5


def test_varlen_lengths():
    lens = synth.varlen_lengths(1 << 20)
    assert sum(lens) == 1 << 20
    assert all(1 <= L < 131072 for L in lens)
    assert all(L >= 1024 for L in lens[:-1])
    lens2 = synth.varlen_lengths(1 << 20)
    assert lens == lens2


def test_distributions():
    q, k, v, g, w = synth.layer_inputs(2, 64, 4, 128, "minimax")
    assert abs(np.std(q) - 1 / np.sqrt(128)) < 0.01
    assert abs(np.mean(w) - 1.0) < 0.01 and 0.01 < np.std(w) < 0.03
    q, k, v, g, w = synth.layer_inputs(1, 64, 2, 64, "unit", bf16=False)
    assert np.all(w == 1.0) and abs(np.std(g) - 1.0) < 0.05
