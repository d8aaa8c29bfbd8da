"""The oracle pinned to facts outside itself (CPU only).

Closed forms, invariants, brute force, torch's float64 SDPA and hand-worked
cases under tests/golden/ (the pages print no worked example).  Also the
split-softmax merge identity that the v2a split-KV path relies on, and the
stream pairing of the four attentions.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from tests import pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def oracle_attn(q, k, v, kv_len):
    return oracle.attention(q, k, v, kv_len=kv_len, threads=2)


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(oracle_attn)


def test_hand_worked_cases():
    with open(os.path.join(GOLDEN, "hand_worked.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        q = np.array(c["q"], np.float32)[None, :, None, :]
        k = np.array(c["k"], np.float32)[None, :, None, :]
        v = np.array(c["v"], np.float32)[None, :, None, :]
        o = oracle.attention(q, k, v, kv_len=c["kv_len"])
        want = np.array(c["o"], np.float64)
        assert np.max(np.abs(o[0, :, 0, :] - want)) < 1e-14, c["name"]


def test_lse_brute_force():
    """lse = log sum_j exp(s_j), checked against math.fsum without max subtraction."""
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 3, 2, 8)).astype(np.float32)
    k = rng.standard_normal((1, 6, 2, 8)).astype(np.float32)
    v = rng.standard_normal((1, 6, 2, 8)).astype(np.float32)
    _, lse = oracle.attention(q, k, v, kv_len=5, return_lse=True)
    for i in range(3):
        for h in range(2):
            s = [math.fsum(float(q[0, i, h, d]) * float(k[0, j, h, d]) for d in range(8)) / math.sqrt(8)
                 for j in range(5)]
            assert abs(lse[0, i, h] - math.log(math.fsum(math.exp(x) for x in s))) < 1e-13


@pytest.mark.parametrize("splits", [[0, 1, 40], [0, 13, 26, 40], [0, 7, 8, 30, 31, 40]])
def test_split_softmax_merge_identity(splits):
    """Partial attentions over disjoint key ranges, merged by their log-sum-exp,
    give the unsplit result: O = sum_r exp(lse_r - LSE) O_r, LSE = log sum_r exp(lse_r).
    This is the per-rank softmax-statistics merge of the context-parallel v2a
    (TensorRT-Model-Connect PR #1586, the commit onboarding LTX-2.5), done here
    across chunks of one key range."""
    rng = np.random.default_rng(4)
    q = (rng.standard_normal((2, 5, 2, 16)) * 2).astype(np.float32)
    k = (rng.standard_normal((2, 40, 2, 16)) * 2).astype(np.float32)
    v = rng.standard_normal((2, 40, 2, 16)).astype(np.float32)
    o_full, lse_full = oracle.attention(q, k, v, return_lse=True)
    parts = []
    for a, b in zip(splits[:-1], splits[1:]):
        o_r, lse_r = oracle.attention(q, np.ascontiguousarray(k[:, a:b]),
                                      np.ascontiguousarray(v[:, a:b]), return_lse=True)
        parts.append((o_r, lse_r))
    M = np.max([p[1] for p in parts], axis=0)
    L = sum(np.exp(p[1] - M) for p in parts)
    lse = M + np.log(L)
    o = sum(np.exp(p[1] - lse)[..., None] * p[0] for p in parts)
    assert np.max(np.abs(lse - lse_full)) < 1e-13
    assert np.max(np.abs(o - o_full)) < 1e-13


def test_rows_match_full():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((2, 9, 3, 8)).astype(np.float32)
    k = rng.standard_normal((2, 12, 3, 8)).astype(np.float32)
    v = rng.standard_normal((2, 12, 3, 8)).astype(np.float32)
    full, lse = oracle.attention(q, k, v, kv_len=10, return_lse=True)
    rows = np.array([[0, 0, 0], [1, 2, 8], [0, 1, 4], [1, 0, 3]])
    o, l = oracle.attention_rows(q, k, v, rows, kv_len=10, return_lse=True)
    for n, (b, h, i) in enumerate(rows):
        assert np.array_equal(o[n], full[b, i, h])
        assert l[n] == lse[b, i, h]


def test_thread_count_does_not_change_result():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((1, 33, 2, 16)).astype(np.float32)
    k = rng.standard_normal((1, 50, 2, 16)).astype(np.float32)
    v = rng.standard_normal((1, 50, 2, 16)).astype(np.float32)
    a = oracle.attention(q, k, v, threads=1)
    b = oracle.attention(q, k, v, threads=7)
    assert np.array_equal(a, b)


def test_block_pairing():
    """video_self: video Q over video K/V; audio_self: audio over valid audio keys;
    a2v: video Q over audio K/V; v2a: audio Q over video K/V (PR #16228, "Description")."""
    rng = np.random.default_rng(7)
    H, D, Sv, La, L = 2, 8, 11, 6, 4
    mk = lambda S: rng.standard_normal((1, S, H, D)).astype(np.float32)
    inp = {"video_q": mk(Sv), "video_k": mk(Sv), "video_v": mk(Sv),
           "audio_q": mk(La), "audio_k": mk(La), "audio_v": mk(La)}
    inp["audio_k"][:, L:] = 4.0
    inp["audio_v"][:, L:] = 64.0
    out = oracle.block_attention(inp, L)
    assert out["video_self"].shape == (1, Sv, H, D)
    assert out["a2v"].shape == (1, Sv, H, D)
    assert out["audio_self"].shape == (1, La, H, D)
    assert out["v2a"].shape == (1, La, H, D)
    A = oracle.attention
    assert np.array_equal(out["a2v"], A(inp["video_q"], inp["audio_k"][:, :L].copy(), inp["audio_v"][:, :L].copy()))
    assert np.array_equal(out["v2a"], A(inp["audio_q"], inp["video_k"], inp["video_v"]))
    assert np.array_equal(out["audio_self"], A(inp["audio_q"], inp["audio_k"][:, :L].copy(), inp["audio_v"][:, :L].copy()))
    # no masked (poisoned, V = 64) key leaks into any output
    assert max(np.abs(o).max() for o in out.values()) < 10


def test_bad_sizes_rejected():
    z = np.zeros((1, 4, 1, 8), np.float32)
    with pytest.raises(ValueError):
        oracle.attention(z, z, z, kv_len=0)
    with pytest.raises(ValueError):
        oracle.attention(z, z, z, kv_len=5)


# ---------------------------------------------------------------- output gate
def _gate_case(seed=9):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((2, 7, 3, 8)).astype(np.float32)
    k = rng.standard_normal((2, 11, 3, 8)).astype(np.float32)
    v = rng.standard_normal((2, 11, 3, 8)).astype(np.float32)
    return q, k, v


def test_gate_closed_forms():
    """All-ones leaves the output unchanged, all-zeros clears it, a gate of 2
    doubles it exactly (a power of two), in every row and channel."""
    q, k, v = _gate_case()
    base = oracle.attention(q, k, v, kv_len=9)
    shape = base.shape
    assert np.array_equal(oracle.attention(q, k, v, kv_len=9, gate=np.ones(shape, np.float32)), base)
    assert np.array_equal(oracle.attention(q, k, v, kv_len=9, gate=np.zeros(shape, np.float32)),
                          np.zeros(shape))
    assert np.array_equal(oracle.attention(q, k, v, kv_len=9, gate=np.full(shape, 2, np.float32)), 2 * base)


def test_gate_follows_query_row_and_channel():
    """A gate that is 1 on some (query row, head, channel) cells and 0 on the
    others keeps exactly those cells of the ungated output; the rows entry
    point applies the same cells."""
    q, k, v = _gate_case(10)
    base = oracle.attention(q, k, v, kv_len=11)
    B, Sq, H, D = base.shape
    b, i, h, d = np.meshgrid(*[np.arange(n) for n in (B, Sq, H, D)], indexing="ij")
    gate = ((b + 2 * i + 3 * h + 5 * d) % 3 == 0).astype(np.float32)
    got = oracle.attention(q, k, v, kv_len=11, gate=gate)
    assert np.array_equal(got, np.where(gate == 1, base, 0.0))
    rows = np.array([[0, 0, 0], [1, 2, 6], [0, 1, 3], [1, 0, 5]])
    o = oracle.attention_rows(q, k, v, rows, kv_len=11, gate=gate)
    for n, (bb, hh, ii) in enumerate(rows):
        assert np.array_equal(o[n], got[bb, ii, hh])


def test_gate_on_the_wrong_axis_is_caught():
    """A mistaken reading that gates by key position instead of query row fails
    the row pin above (so that pin can tell the two apart)."""
    q, k, v = _gate_case(11)
    base = oracle.attention(q, k, v, kv_len=11)
    B, Sq, H, D = base.shape
    gate = np.zeros((B, Sq, H, D), np.float32)
    gate[:, 0] = 1.0                                   # keep query row 0 only
    right = oracle.attention(q, k, v, kv_len=11, gate=gate)
    # the mutant: weight the values of key 0 only (the same index, read as a key)
    vm = np.zeros_like(v)
    vm[:, 0] = v[:, 0]
    wrong = oracle.attention(q, k, vm, kv_len=11)
    assert np.array_equal(right[:, 0], base[:, 0]) and not np.allclose(wrong[:, 0], base[:, 0])
