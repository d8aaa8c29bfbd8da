"""Checks that pin an attention implementation to facts outside itself.

Each ``check_*`` takes ``attn(q, k, v, kv_len) -> o`` (float32 inputs in
[B, S, H, D], float64 output) and raises AssertionError when the
implementation breaks the fact.  The facts come from the definition of
softmax attention, softmax(Q K^T / sqrt(D)) V, and from mathematics:
closed forms, invariants, brute force on tiny inputs and an independent
library routine.  ``test_oracle_pins.py`` applies them to the oracle and
``test_oracle_mutants.py`` shows that plausible mistakes fail them.
"""

from __future__ import annotations

import math

import numpy as np

TIGHT = 1e-12


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _grid(rng, shape, denom=8, lo=-16, hi=16):
    """Random multiples of 1/denom: exact in float32, so sums and shifts stay exact."""
    return (rng.integers(lo, hi + 1, size=shape) / denom).astype(np.float32)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max abs error {err:.3e} > {tol:.1e}"


# --------------------------------------------------------------- closed forms
def check_single_key(attn):
    """Sk = 1: the only weight is 1, so O equals V_0 for every query."""
    rng = _rng(11)
    q = rng.standard_normal((2, 5, 3, 16)).astype(np.float32)
    k = rng.standard_normal((2, 1, 3, 16)).astype(np.float32)
    v = rng.standard_normal((2, 1, 3, 16)).astype(np.float32)
    o = attn(q, k, v, 1)
    _close(o, np.broadcast_to(v, o.shape), TIGHT, "single key")


def check_two_keys_logistic(attn):
    """Two keys: w_0 = logistic((s_0 - s_1)), s_j = q.k_j / sqrt(D).

    D = 4 and 64 make a wrong scale (1, 1/D, sqrt(D)) visible.
    """
    for D in (1, 4, 64):
        q = np.zeros((1, 3, 1, D), np.float32)
        k = np.zeros((1, 2, 1, D), np.float32)
        v = np.zeros((1, 2, 1, D), np.float32)
        qs = [1.0, 2.0, -1.5]
        q[0, :, 0, 0] = qs
        k[0, 0, 0, 0] = 1.25
        k[0, 1, 0, 0] = -0.5
        if D > 1:
            k[0, 1, 0, 1] = 3.0     # orthogonal to q: no effect on the logit
        v[0, 0, 0, :] = 1.0
        v[0, 1, 0, :] = -2.0
        o = attn(q, k, v, 2)
        for i, qi in enumerate(qs):
            delta = qi * (1.25 - (-0.5)) / math.sqrt(D)
            w0 = 1.0 / (1.0 + math.exp(-delta))
            want = w0 * 1.0 + (1.0 - w0) * (-2.0)
            _close(o[0, i, 0, :], np.full(D, want), 1e-14, f"logistic D={D} row {i}")


def check_equal_keys_mean(attn):
    """All keys equal: uniform weights, O = mean of the valid V rows."""
    rng = _rng(12)
    B, Sq, Sk, H, D = 2, 4, 9, 2, 8
    q = rng.standard_normal((B, Sq, H, D)).astype(np.float32)
    k = np.broadcast_to(rng.standard_normal((B, 1, H, D)).astype(np.float32), (B, Sk, H, D)).copy()
    v = rng.standard_normal((B, Sk, H, D)).astype(np.float32)
    for L in (Sk, 5, 1):
        o = attn(q, k, v, L)
        want = v[:, :L].astype(np.float64).mean(axis=1, keepdims=True)
        _close(o, np.broadcast_to(want, o.shape), 1e-14, f"equal keys L={L}")


def check_needle(attn):
    """One key aligned with the query by a huge margin: its weight is 1 to
    within exp(-margin) (here exp(-64) < 2e-28), so O equals that key's V."""
    D, Sk = 16, 37
    for pos in (0, 17, Sk - 1):
        q = np.zeros((1, 1, 1, D), np.float32)
        k = np.zeros((1, Sk, 1, D), np.float32)
        q[0, 0, 0, 0] = 16.0
        k[0, pos, 0, 0] = 16.0          # s = 256 / 4 = 64 for the needle, 0 elsewhere
        v = np.arange(Sk * D, dtype=np.float32).reshape(1, Sk, 1, D) / 64.0
        o = attn(q, k, v, Sk)
        _close(o[0, 0, 0], v[0, pos, 0], 1e-13, f"needle at {pos}")


# ----------------------------------------------------------------- invariants
def check_rows_sum_to_one(attn):
    """V = 1 everywhere: O = sum_j w_j = 1.  O lies in the hull of valid V."""
    rng = _rng(13)
    B, Sq, Sk, H, D = 1, 6, 11, 2, 8
    q = rng.standard_normal((B, Sq, H, D)).astype(np.float32) * 2
    k = rng.standard_normal((B, Sk, H, D)).astype(np.float32) * 2
    ones = np.ones((B, Sk, H, D), np.float32)
    _close(attn(q, k, ones, Sk), np.ones((B, Sq, H, D)), 1e-14, "rows sum to 1")
    v = rng.standard_normal((B, Sk, H, D)).astype(np.float32)
    L = 7
    o = attn(q, k, v, L)
    lo = v[:, :L].min(axis=1, keepdims=True) - 1e-14
    hi = v[:, :L].max(axis=1, keepdims=True) + 1e-14
    assert np.all(o >= lo) and np.all(o <= hi), "output outside the hull of valid V rows"


def check_joint_permutation(attn):
    """Permuting K and V rows together (within the valid keys) leaves O unchanged;
    permuting query rows permutes O rows."""
    rng = _rng(14)
    B, Sq, Sk, H, D = 2, 5, 13, 3, 8
    q = rng.standard_normal((B, Sq, H, D)).astype(np.float32)
    k = rng.standard_normal((B, Sk, H, D)).astype(np.float32)
    v = rng.standard_normal((B, Sk, H, D)).astype(np.float32)
    L = 10
    o = attn(q, k, v, L)
    perm = np.concatenate([rng.permutation(L), np.arange(L, Sk)])
    _close(attn(q, k[:, perm], v[:, perm], L), o, 1e-13, "joint K/V permutation")
    qp = rng.permutation(Sq)
    _close(attn(q[:, qp], k, v, L), o[:, qp], 1e-13, "query permutation")


def check_key_shift(attn):
    """Adding one vector c to every key adds q.c/sqrt(D) to every logit of a row:
    the softmax is unchanged.  Grid values keep K + c exact in float32."""
    rng = _rng(15)
    B, Sq, Sk, H, D = 1, 4, 9, 2, 8
    q = _grid(rng, (B, Sq, H, D))
    k = _grid(rng, (B, Sk, H, D))
    v = _grid(rng, (B, Sk, H, D))
    c = _grid(rng, (B, 1, H, D), denom=4, lo=-8, hi=8)
    _close(attn(q, k + c, v, Sk), attn(q, k, v, Sk), 1e-13, "key shift")


def check_affine_in_v(attn):
    """O(a V + b) = a O(V) + b, because the weights sum to one."""
    rng = _rng(16)
    B, Sq, Sk, H, D = 1, 4, 9, 2, 8
    q = _grid(rng, (B, Sq, H, D))
    k = _grid(rng, (B, Sk, H, D))
    v = _grid(rng, (B, Sk, H, D))
    b = _grid(rng, (1, 1, H, D))
    o = attn(q, k, v, Sk)
    _close(attn(q, k, 2 * v + b, Sk), 2 * o + b, 1e-13, "affine in V")


def check_qk_rescale(attn):
    """Scaling Q by 2 and K by 1/2 leaves every logit, hence O, unchanged,
    while scaling Q alone by 2 changes O (the logits enter non-linearly)."""
    rng = _rng(17)
    q = _grid(rng, (1, 4, 2, 8))
    k = _grid(rng, (1, 9, 2, 8))
    v = _grid(rng, (1, 9, 2, 8))
    o = attn(q, k, v, 9)
    _close(attn(2 * q, k / 2, v, 9), o, 1e-13, "Q*2, K/2")
    assert np.max(np.abs(attn(2 * q, k, v, 9) - o)) > 1e-3, "temperature has no effect"


def check_padding_is_truncation(attn):
    """Keys j >= kv_len take no part: the padded buffer equals the truncated
    problem, whatever the padding rows hold (here poison: K = 4, V = 64)."""
    rng = _rng(18)
    B, Sq, H, D = 2, 5, 2, 8
    for L, Sk in ((1, 4), (5, 8), (126, 128), (252, 256)):
        q = rng.standard_normal((B, Sq, H, D)).astype(np.float32)
        k = rng.standard_normal((B, Sk, H, D)).astype(np.float32)
        v = rng.standard_normal((B, Sk, H, D)).astype(np.float32)
        k[:, L:] = 4.0
        v[:, L:] = 64.0
        want = attn(np.ascontiguousarray(q), np.ascontiguousarray(k[:, :L]),
                    np.ascontiguousarray(v[:, :L]), L)
        _close(attn(q, k, v, L), want, 1e-14, f"padding L={L} Sk={Sk}")


def check_slices_independent(attn):
    """Each (batch, head) slice is its own problem."""
    rng = _rng(19)
    B, Sq, Sk, H, D = 2, 3, 6, 3, 4
    q = rng.standard_normal((B, Sq, H, D)).astype(np.float32)
    k = rng.standard_normal((B, Sk, H, D)).astype(np.float32)
    v = rng.standard_normal((B, Sk, H, D)).astype(np.float32)
    o = attn(q, k, v, Sk)
    for b in range(B):
        for h in range(H):
            ob = attn(np.ascontiguousarray(q[b:b + 1, :, h:h + 1]),
                      np.ascontiguousarray(k[b:b + 1, :, h:h + 1]),
                      np.ascontiguousarray(v[b:b + 1, :, h:h + 1]), Sk)
            _close(ob[0, :, 0], o[b, :, h], 1e-15, f"slice b={b} h={h}")


# ---------------------------------------------------------------- brute force
def brute_force(q, k, v, kv_len):
    """softmax(q k^T / sqrt(D)) v written without max subtraction, each sum
    taken with math.fsum (correctly rounded): a second formulation."""
    B, Sq, H, D = q.shape
    out = np.zeros((B, Sq, H, D))
    for b in range(B):
        for h in range(H):
            for i in range(Sq):
                e = []
                for j in range(kv_len):
                    s = math.fsum(float(q[b, i, h, d]) * float(k[b, j, h, d]) for d in range(D))
                    e.append(math.exp(s / math.sqrt(D)))
                den = math.fsum(e)
                for d in range(D):
                    out[b, i, h, d] = math.fsum(e[j] * float(v[b, j, h, d])
                                                for j in range(kv_len)) / den
    return out


def check_brute_force(attn):
    rng = _rng(20)
    for (B, Sq, Sk, L, H, D) in ((1, 1, 1, 1, 1, 1), (2, 3, 5, 5, 2, 4),
                                 (1, 5, 7, 4, 2, 8), (2, 4, 8, 8, 1, 8)):
        q = rng.standard_normal((B, Sq, H, D)).astype(np.float32)
        k = rng.standard_normal((B, Sk, H, D)).astype(np.float32)
        v = rng.standard_normal((B, Sk, H, D)).astype(np.float32)
        _close(attn(q, k, v, L), brute_force(q, k, v, L), 1e-13, f"brute force {B,Sq,Sk,L,H,D}")


def check_torch_sdpa(attn):
    """Against torch's own float64 scaled_dot_product_attention on the CPU
    (a library routine; default scale is 1/sqrt(D)); padding as a boolean mask."""
    import torch
    rng = _rng(21)
    for (B, Sq, Sk, L, H, D) in ((1, 17, 40, 33, 3, 64), (2, 9, 16, 16, 2, 128)):
        q = rng.standard_normal((B, Sq, H, D)).astype(np.float32)
        k = rng.standard_normal((B, Sk, H, D)).astype(np.float32)
        v = rng.standard_normal((B, Sk, H, D)).astype(np.float32)
        t = lambda x: torch.from_numpy(x.astype(np.float64)).permute(0, 2, 1, 3)
        mask = torch.zeros(Sq, Sk, dtype=torch.bool)
        mask[:, :L] = True
        ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=mask)
        ref = ref.permute(0, 2, 1, 3).numpy()
        _close(attn(q, k, v, L), ref, 1e-13, f"torch sdpa {B,Sq,Sk,L,H,D}")


ALL_CHECKS = [
    check_single_key, check_two_keys_logistic, check_equal_keys_mean, check_needle,
    check_rows_sum_to_one, check_joint_permutation, check_key_shift, check_affine_in_v,
    check_qk_rescale, check_padding_is_truncation, check_slices_independent,
    check_brute_force, check_torch_sdpa,
]
