"""The pins are sharp: plausible mistakes in an attention implementation fail
at least one of them (mistakes are planted in CPU copies written here, never
in the HIP path).  A correct NumPy formulation passes all of them, which
shows the harness itself is sound."""

import numpy as np
import pytest

from tests import pins


def _numpy_attn(q, k, v, kv_len, scale=None, over="keys", use_v=None, keys=None,
                head_mix=False, dtype=np.float64):
    q = q.astype(dtype)
    k = k.astype(dtype)
    v = (use_v if use_v is not None else v).astype(dtype)
    L = kv_len if keys is None else keys(kv_len, k.shape[1])
    k, v = k[:, :L], v[:, :L]
    if head_mix:
        k = np.broadcast_to(k[:, :, :1], k.shape)
    D = q.shape[-1]
    sc = (1 / np.sqrt(D)) if scale is None else scale(D)
    s = np.einsum("bihd,bjhd->bhij", q, k) * dtype(sc)
    axis = -1 if over == "keys" else -2
    w = np.exp(s - s.max(axis=axis, keepdims=True))
    w = w / w.sum(axis=axis, keepdims=True)
    return np.einsum("bhij,bjhd->bihd", w, v).astype(np.float64)


MUTANTS = {
    "scale 1/D": lambda q, k, v, L: _numpy_attn(q, k, v, L, scale=lambda D: 1.0 / D),
    "no scale": lambda q, k, v, L: _numpy_attn(q, k, v, L, scale=lambda D: 1.0),
    "scale sqrt(D)": lambda q, k, v, L: _numpy_attn(q, k, v, L, scale=lambda D: np.sqrt(D)),
    "padding ignored": lambda q, k, v, L: _numpy_attn(q, k, v, L, keys=lambda L, S: S),
    "last valid key dropped": lambda q, k, v, L: _numpy_attn(q, k, v, L, keys=lambda L, S: max(L - 1, 1)),
    "one key too many": lambda q, k, v, L: _numpy_attn(q, k, v, L, keys=lambda L, S: min(L + 1, S)),
    "softmax over queries": lambda q, k, v, L: _numpy_attn(q, k, v, L, over="queries"),
    "K used as V": lambda q, k, v, L: _numpy_attn(q, k, v, L, use_v=k),
    "heads mixed": lambda q, k, v, L: _numpy_attn(q, k, v, L, head_mix=True),
    "float32 arithmetic": lambda q, k, v, L: _numpy_attn(q, k, v, L, dtype=np.float32),
    "sign of logits flipped": lambda q, k, v, L: _numpy_attn(q, k, v, L, scale=lambda D: -1 / np.sqrt(D)),
}


def _failures(fn):
    failed = []
    for check in pins.ALL_CHECKS:
        try:
            check(fn)
        except AssertionError:
            failed.append(check.__name__)
    return failed


def test_correct_numpy_passes_every_pin():
    assert _failures(lambda q, k, v, L: _numpy_attn(q, k, v, L)) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    assert _failures(MUTANTS[name]), f"mutant '{name}' passes every pin"
