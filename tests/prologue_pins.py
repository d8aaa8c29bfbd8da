"""Checks that pin a QK-norm + rotary prologue to facts outside itself.

Each ``check_*`` takes ``pro(x, w, cos, sin, eps, pairing) -> z`` (x float32
[B, S, H, D], w float32 [D], cos/sin float32 [S, D/2], z float64 before any
rounding) and raises AssertionError when the implementation breaks the fact.
The facts come from what the two steps are: an RMS norm of each (token,
head) row over its D channels with a per-channel weight, then a rotation of
channel pairs by an angle per pair and token (the keys and queries of the
LTX-2.5 DiT arrive normed and rotated, TensorRT-Model-Connect PR #1586, the
commit onboarding LTX-2.5; its RoPE tables are per-grid data, "The DiT plan
serves both grids").  Invariants, closed forms and the relative-position
property of rotary embeddings; ``test_oracle_prologue.py`` applies them to
the oracle and shows that plausible mistakes fail them.
"""

from __future__ import annotations

import numpy as np

TIGHT = 1e-12


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _close(a, b, tol, what):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max abs error {err:.3e} > {tol:.1e}"


def _tables(S, P, angle):
    """cos/sin tables [S, P] of angle(s, i), as float32."""
    s = np.arange(S)[:, None]
    i = np.arange(P)[None, :]
    th = angle(s, i)
    return np.cos(th).astype(np.float32), np.sin(th).astype(np.float32)


def _zero_angle(S, P):
    return np.ones((S, P), np.float32), np.zeros((S, P), np.float32)


def _pairs(D, pairing):
    P = D // 2
    if pairing == "half":
        return np.arange(P), np.arange(P) + P
    return 2 * np.arange(P), 2 * np.arange(P) + 1


# ------------------------------------------------------------------ the norm
def check_unit_rms(pro):
    """Weight 1, eps 0, no rotation: every row comes out with root mean square
    exactly 1 over its D channels, and parallel to the input (one positive
    factor per row)."""
    rng = _rng(21)
    B, S, H, D = 2, 5, 3, 16
    x = rng.standard_normal((B, S, H, D)).astype(np.float32)
    c, s = _zero_angle(S, D // 2)
    z = pro(x, np.ones(D, np.float32), c, s, 0.0, "half")
    _close(np.sqrt(np.mean(z * z, axis=-1)), np.ones((B, S, H)), TIGHT, "row RMS")
    ratio = z / x.astype(np.float64)
    _close(ratio, np.broadcast_to(ratio[..., :1], ratio.shape), TIGHT, "one factor per row")
    assert np.all(ratio > 0), "negative factor"


def check_scale_invariant(pro):
    """eps 0: scaling a row by any c > 0 leaves the output unchanged (powers of
    two keep the float32 inputs exact)."""
    rng = _rng(22)
    B, S, H, D = 1, 4, 2, 32
    x = rng.standard_normal((B, S, H, D)).astype(np.float32)
    c, s = _tables(S, D // 2, lambda s, i: 0.3 * s + 0.1 * i)
    w = (1 + 0.25 * rng.standard_normal(D)).astype(np.float32)
    z = pro(x, w, c, s, 0.0, "half")
    for f in (0.125, 8.0, 1024.0):
        _close(pro(x * np.float32(f), w, c, s, 0.0, "half"), z, TIGHT, f"scale {f}")


def check_eps_in_mean_square(pro):
    """A row of ones with eps = 3: mean square 1, so the factor is 1/sqrt(1 + 3)
    = 1/2 for every channel (eps is added to the mean of the squares, inside
    the root)."""
    B, S, H, D = 1, 2, 2, 8
    x = np.ones((B, S, H, D), np.float32)
    c, s = _zero_angle(S, D // 2)
    z = pro(x, np.ones(D, np.float32), c, s, 3.0, "half")
    _close(z, np.full(z.shape, 0.5), TIGHT, "eps")


def check_per_head_statistics(pro):
    """The statistics are per (token, head): scaling one head's channels by 8
    changes nothing in any head's output (eps 0)."""
    rng = _rng(23)
    B, S, H, D = 1, 3, 4, 8
    x = rng.standard_normal((B, S, H, D)).astype(np.float32)
    c, s = _tables(S, D // 2, lambda s, i: 0.7 * s - 0.2 * i)
    w = np.ones(D, np.float32)
    z = pro(x, w, c, s, 0.0, "half")
    x2 = x.copy()
    x2[:, :, 1] *= 8
    _close(pro(x2, w, c, s, 0.0, "half"), z, TIGHT, "per-head statistics")


def check_weight_per_channel_before_rotation(pro):
    """Rows of +-1 have root mean square 1, so with eps 0 the norm alone gives
    the row times the weight.  A weight of 2 on channel j only and zero
    angles leaves 2 x_j there and zeros elsewhere; with angle pi/2 the weighted
    channel moves to its partner (the weight applies before the rotation)."""
    rng = _rng(24)
    B, S, H, D = 1, 2, 2, 8
    x = rng.choice(np.array([-1.0, 1.0], np.float32), size=(B, S, H, D))
    for pairing in ("half", "interleaved"):
        a, cc = _pairs(D, pairing)
        for j in range(D):
            w = np.zeros(D, np.float32)
            w[j] = 2.0
            c0, s0 = _zero_angle(S, D // 2)
            want = np.zeros(x.shape)
            want[..., j] = 2 * x[..., j]
            _close(pro(x, w, c0, s0, 0.0, pairing), want, TIGHT, f"weight on {j} ({pairing})")
            c1, s1 = np.zeros((S, D // 2), np.float32), np.ones((S, D // 2), np.float32)
            want = np.zeros(x.shape)
            i = int(np.nonzero((a == j) | (cc == j))[0][0])
            if a[i] == j:       # (y_a, 0) -> (0, y_a)
                want[..., cc[i]] = 2 * x[..., j]
            else:               # (0, y_c) -> (-y_c, 0)
                want[..., a[i]] = -2 * x[..., j]
            _close(pro(x, w, c1, s1, 0.0, pairing), want, TIGHT, f"weight on {j}, quarter turn ({pairing})")


# -------------------------------------------------------------- the rotation
def check_quarter_turn(pro):
    """Angle pi/2 on every pair (cos 0, sin 1) maps (y_a, y_c) to (-y_c, y_a);
    rows of +-1 with weight 1 and eps 0 make y the input itself."""
    rng = _rng(25)
    B, S, H, D = 2, 3, 2, 16
    x = rng.choice(np.array([-1.0, 1.0], np.float32), size=(B, S, H, D))
    c, s = np.zeros((S, D // 2), np.float32), np.ones((S, D // 2), np.float32)
    for pairing in ("half", "interleaved"):
        a, cc = _pairs(D, pairing)
        want = np.empty(x.shape)
        want[..., a] = -x[..., cc]
        want[..., cc] = x[..., a]
        _close(pro(x, np.ones(D, np.float32), c, s, 0.0, pairing), want, TIGHT, f"quarter turn ({pairing})")


def check_table_row_is_the_token(pro):
    """Token s is rotated by the table's row s: with s quarter turns in row s
    (tables of 0 and +-1 only) and rows of +-1, token s's pairs (a, c) come out
    as (a, c), (-c, a), (-a, -c), (c, -a) for s = 0, 1, 2, 3 (mod 4)."""
    rng = _rng(29)
    B, S, H, D = 2, 7, 2, 8
    P = D // 2
    x = rng.choice(np.array([-1.0, 1.0], np.float32), size=(B, S, H, D))
    th = (np.pi / 2) * np.arange(S)[:, None] * np.ones((1, P))
    c = np.rint(np.cos(th)).astype(np.float32)
    s_ = np.rint(np.sin(th)).astype(np.float32)
    for pairing in ("half", "interleaved"):
        a, cc = _pairs(D, pairing)
        z = pro(x, np.ones(D, np.float32), c, s_, 0.0, pairing)
        for t in range(S):
            xa, xc = x[:, t, :, a].astype(np.float64), x[:, t, :, cc].astype(np.float64)
            want_a, want_c = [(xa, xc), (-xc, xa), (-xa, -xc), (xc, -xa)][t % 4]
            _close(z[:, t, :, a], want_a, TIGHT, f"token {t} row ({pairing})")
            _close(z[:, t, :, cc], want_c, TIGHT, f"token {t} row ({pairing})")


def check_pair_lengths_kept(pro):
    """A rotation keeps the length of every channel pair: rotating (a, b) by a
    table entry (c, s) multiplies its squared length by c^2 + s^2 (1 up to the
    float32 rounding of the table), so the output's pair lengths are those of
    the output with zero angles times that factor."""
    rng = _rng(26)
    B, S, H, D = 2, 6, 2, 32
    x = rng.standard_normal((B, S, H, D)).astype(np.float32)
    w = (1 + 0.3 * rng.standard_normal(D)).astype(np.float32)
    c0, s0 = _zero_angle(S, D // 2)
    c, s = _tables(S, D // 2, lambda s, i: 1.3 * s + 0.37 * i * i)
    for pairing in ("half", "interleaved"):
        a, cc = _pairs(D, pairing)
        y = pro(x, w, c0, s0, 1e-6, pairing)
        z = pro(x, w, c, s, 1e-6, pairing)
        f = (c.astype(np.float64) ** 2 + s.astype(np.float64) ** 2)[None, :, None, :]
        _close(z[..., a] ** 2 + z[..., cc] ** 2, (y[..., a] ** 2 + y[..., cc] ** 2) * f, 1e-12,
               f"pair lengths ({pairing})")


def check_relative_position(pro):
    """Rotary tables theta_i(p) = p * omega_i: the dot product of a query at
    position p with a key at position p' depends only on p - p' -- shifting
    both positions by t leaves it unchanged.  Exactly, with quarter-turn
    frequencies whose tables hold only 0 and +-1; to the float32 rounding of
    the tables (1e-5 relative), with omega_i = 10000^(-2i/D)."""
    rng = _rng(27)
    D, S = 32, 40
    P = D // 2
    quarter = lambda p, i: p * (np.pi / 2) * (1 + i % 3)
    cq = np.rint(np.cos(quarter(np.arange(S)[:, None], np.arange(P)[None, :]))).astype(np.float32)
    sq = np.rint(np.sin(quarter(np.arange(S)[:, None], np.arange(P)[None, :]))).astype(np.float32)
    cg, sg = _tables(S, P, lambda p, i: p * 10000.0 ** (-2.0 * i / D))
    for c, s, tol in ((cq, sq, 1e-12), (cg, sg, 1e-5)):
        _relative_position(pro, rng, D, S, c, s, tol)


def _relative_position(pro, rng, D, S, c, s, tol):
    q1 = rng.standard_normal((1, 1, 1, D)).astype(np.float32)
    k1 = rng.standard_normal((1, 1, 1, D)).astype(np.float32)
    w = (1 + 0.2 * rng.standard_normal(D)).astype(np.float32)
    for pairing in ("half", "interleaved"):
        def at(v, p):
            # the same vector at every position; row p rotated by theta(p)
            return pro(np.broadcast_to(v, (1, S, 1, D)).copy(), w, c, s, 1e-6, pairing)[0, p, 0]
        for p, pk, t in ((3, 17, 5), (20, 2, 11), (0, 0, 30)):
            d0 = float(np.dot(at(q1, p), at(k1, pk)))
            d1 = float(np.dot(at(q1, p + t), at(k1, pk + t)))
            assert abs(d0 - d1) <= tol * max(1.0, abs(d0)), f"relative position ({pairing}) {p},{pk},{t}: {d0} vs {d1}"


def check_pairings_are_a_permutation_apart(pro):
    """Interleaved pairs (2i, 2i+1) are rotate-half pairs (i, i + D/2) after
    moving channel 2i to i and 2i+1 to i + D/2 (weights moved alike)."""
    rng = _rng(28)
    B, S, H, D = 1, 5, 2, 16
    P = D // 2
    x = rng.standard_normal((B, S, H, D)).astype(np.float32)
    w = (1 + 0.3 * rng.standard_normal(D)).astype(np.float32)
    c, s = _tables(S, P, lambda s, i: 0.9 * s + 0.4 * i)
    perm = np.concatenate([2 * np.arange(P), 2 * np.arange(P) + 1])   # half position -> interleaved channel
    zi = pro(x, w, c, s, 1e-5, "interleaved")
    zh = pro(np.ascontiguousarray(x[..., perm]), np.ascontiguousarray(w[perm]), c, s, 1e-5, "half")
    _close(zh, zi[..., perm], 1e-12, "pairings")


ALL_CHECKS = [check_unit_rms, check_scale_invariant, check_eps_in_mean_square, check_per_head_statistics,
              check_weight_per_channel_before_rotation, check_quarter_turn, check_table_row_is_the_token,
              check_pair_lengths_kept,
              check_relative_position, check_pairings_are_a_permutation_apart]
