"""Double-precision CPU oracle for the LTX-2 per-block attention set.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does.  It
shares no code with the HIP library and imports nothing from it.

The arithmetic lives in ``ltxattn_oracle.c`` (softmax(Q K^T / sqrt(D)) V in
IEEE double, one row at a time).  This module only marshals arrays and
applies the stream pairing of the four attentions that every block of the
joint video+audio DiT runs (TensorRT-LLM PR #16228 "LTX-2: replicate audio
stream across Ulysses ranks by default", section "Description"):

============  =========  ==========  =====================
kind          queries    keys/values  valid keys
============  =========  ==========  =====================
video_self    video      video       all video tokens
audio_self    audio      audio       ``audio_kv_len``
a2v           video      audio       ``audio_kv_len``
v2a           audio      video       all video tokens
============  =========  ==========  =====================

Audio keys at or beyond ``audio_kv_len`` are padding (the audio stream is
padded, same PR, "Description") and get weight exactly zero.

Two optional per-kind steps, both computed in the C file too:

* gated attention (named among the DiT's parts by TensorRT-Model-Connect PR
  #1586, the commit onboarding LTX-2.5, which gives no gate formula): a gate
  of the output's shape, taken as given (already activated), multiplies the
  output elementwise;
* the QK-norm + rotary prologue (the same commit: keys are normed and
  rotated before the context-parallel gather, with fp32 norm and RoPE
  islands in a bf16 network): ``qk_prologue`` -- per-(token, head) RMS norm
  with a per-channel weight, then a rotation of channel pairs by the
  caller's per-position cos/sin tables, rounded to the bf16 the attention
  reads.  ``block_attention(prologues=...)`` applies it to a kind's Q and K
  before the attention.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ltxattn_oracle.c")
_LIB = os.path.join(_HERE, "libltxattn_oracle.so")
_lib = None

KINDS = ("video_self", "audio_self", "a2v", "v2a")


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (-O2, no fast-math).  Returns the .so path."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                        "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        lib = ctypes.CDLL(_LIB)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        lib.ltxattn_oracle_attention.argtypes = [p, p, p, p, i64, i64, i64, i64, i64, i64,
                                                 p, p, ctypes.c_int]
        lib.ltxattn_oracle_attention.restype = ctypes.c_int
        lib.ltxattn_oracle_attention_rows.argtypes = [p, p, p, p, i64, i64, i64, i64, i64, i64,
                                                      p, i64, p, p, ctypes.c_int]
        lib.ltxattn_oracle_attention_rows.restype = ctypes.c_int
        lib.ltxattn_oracle_qk_prologue.argtypes = [p, i64, i64, i64, i64, p, p, p, ctypes.c_double,
                                                   ctypes.c_int, p, p]
        lib.ltxattn_oracle_qk_prologue.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    """Host threads the oracle uses: the CPUs this process may run on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _as_f32(x: np.ndarray) -> np.ndarray:
    """bf16 bits (uint16) are widened to float32 exactly; float arrays must
    already hold the values to use."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32)
    if x.dtype == np.float32:
        return np.ascontiguousarray(x)
    if x.dtype == np.float64:
        f = x.astype(np.float32)
        if not np.array_equal(f.astype(np.float64), x):
            raise ValueError("float64 input is not exactly representable in float32")
        return f
    raise TypeError(f"unsupported dtype {x.dtype}")


def _shapes(q, k, v, kv_len):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, S, H, D]")
    B, Sq, H, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2:] != (H, D):
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    Sk = k.shape[1]
    kv_len = Sk if kv_len is None else int(kv_len)
    if not 1 <= kv_len <= Sk:
        raise ValueError(f"kv_len {kv_len} outside [1, {Sk}]")
    return B, Sq, Sk, kv_len, H, D


def _gate(gate, shape):
    """The gate as float32 values of the output's shape, or None."""
    if gate is None:
        return None
    g = _as_f32(gate)
    if g.shape != shape:
        raise ValueError(f"gate shape {g.shape}, expected {shape}")
    return np.ascontiguousarray(g)


def attention(q, k, v, kv_len=None, threads=None, return_lse=False, gate=None):
    """softmax(q k^T / sqrt(D)) v over keys j < kv_len, in double, times
    ``gate`` elementwise if given.

    q: [B, Sq, H, D]; k, v: [B, Sk, H, D]; gate: [B, Sq, H, D] (bf16 bits or
    float32 values).  Returns o [B, Sq, H, D] float64 (and lse [B, Sq, H] if
    asked; the lse is the ungated softmax's).
    """
    q, k, v = _as_f32(q), _as_f32(k), _as_f32(v)
    B, Sq, Sk, L, H, D = _shapes(q, k, v, kv_len)
    g = _gate(gate, (B, Sq, H, D))
    out = np.empty((B, Sq, H, D), dtype=np.float64)
    lse = np.empty((B, Sq, H), dtype=np.float64) if return_lse else None
    rc = _load().ltxattn_oracle_attention(
        q.ctypes.data, k.ctypes.data, v.ctypes.data, g.ctypes.data if g is not None else None,
        B, Sq, Sk, L, H, D, out.ctypes.data, lse.ctypes.data if lse is not None else None,
        threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle failed with {rc}")
    return (out, lse) if return_lse else out


def attention_rows(q, k, v, rows, kv_len=None, threads=None, return_lse=False, gate=None):
    """Same as :func:`attention` for selected rows only.

    rows: int array [n, 3] of (b, h, i).  Returns o [n, D] float64 (and lse [n]).
    """
    q, k, v = _as_f32(q), _as_f32(k), _as_f32(v)
    B, Sq, Sk, L, H, D = _shapes(q, k, v, kv_len)
    g = _gate(gate, (B, Sq, H, D))
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
    n = rows.shape[0]
    out = np.empty((n, D), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64) if return_lse else None
    rc = _load().ltxattn_oracle_attention_rows(
        q.ctypes.data, k.ctypes.data, v.ctypes.data, g.ctypes.data if g is not None else None,
        B, Sq, Sk, L, H, D, rows.ctypes.data, n, out.ctypes.data,
        lse.ctypes.data if lse is not None else None, threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle failed with {rc}")
    return (out, lse) if return_lse else out


PAIRINGS = {"half": 0, "interleaved": 1}


def qk_prologue(x, weight, cos, sin, eps, pairing="half", round_bf16=True):
    """RMS norm of every (token, head) row of x [B, S, H, D] over its D
    channels with the per-channel weight [D], then the rotation of channel
    pairs by cos/sin [S, D/2] of the row's token; pairing "half" pairs
    channels i and i + D/2, "interleaved" 2i and 2i + 1.  Returns the bf16
    bits (uint16) the attention reads, or with round_bf16=False the float64
    values before rounding."""
    x = _as_f32(x)
    if x.ndim != 4:
        raise ValueError("x must be [B, S, H, D]")
    B, S, H, D = x.shape
    w = np.ascontiguousarray(_as_f32(weight).reshape(-1))
    c = np.ascontiguousarray(_as_f32(cos))
    s = np.ascontiguousarray(_as_f32(sin))
    if w.shape != (D,) or c.shape != (S, D // 2) or s.shape != (S, D // 2):
        raise ValueError(f"weight {w.shape}, cos {c.shape}, sin {s.shape} for x {x.shape}")
    out = np.empty(x.shape, np.float64) if not round_bf16 else None
    bits = np.empty(x.shape, np.uint16) if round_bf16 else None
    rc = _load().ltxattn_oracle_qk_prologue(
        x.ctypes.data, B, S, H, D, w.ctypes.data, c.ctypes.data, s.ctypes.data, float(eps),
        PAIRINGS[pairing], out.ctypes.data if out is not None else None,
        bits.ctypes.data if bits is not None else None)
    if rc != 0:
        raise RuntimeError(f"oracle prologue failed with {rc}")
    return bits if round_bf16 else out


def apply_prologue(q, k, pro):
    """(q, k) of one attention after its prologue: pro holds q_weight,
    k_weight, q_cos, q_sin, k_cos, k_sin, eps and pairing."""
    return (qk_prologue(q, pro["q_weight"], pro["q_cos"], pro["q_sin"], pro["eps"], pro["pairing"]),
            qk_prologue(k, pro["k_weight"], pro["k_cos"], pro["k_sin"], pro["eps"], pro["pairing"]))


def pairing(kind: str, inputs: dict, audio_kv_len: int):
    """(q, k, v, kv_len) of attention ``kind`` from the six stream tensors."""
    vq, vk, vv = inputs["video_q"], inputs["video_k"], inputs["video_v"]
    aq, ak, av = inputs["audio_q"], inputs["audio_k"], inputs["audio_v"]
    if kind == "video_self":
        return vq, vk, vv, vk.shape[1]
    if kind == "audio_self":
        return aq, ak, av, audio_kv_len
    if kind == "a2v":
        return vq, ak, av, audio_kv_len
    if kind == "v2a":
        return aq, vk, vv, vk.shape[1]
    raise ValueError(kind)


def block_attention(inputs: dict, audio_kv_len: int, kinds=KINDS, threads=None, gates=None,
                    prologues=None):
    """All four attentions of one block; returns {kind: o float64 [B, Sq, H, D]}.
    gates: optional {kind: gate [B, Sq, H, D]}; prologues: optional {kind:
    QK-norm + rotary parameters (see apply_prologue)}."""
    out = {}
    for kind in kinds:
        q, k, v, L = pairing(kind, inputs, audio_kv_len)
        if prologues and kind in prologues:
            q, k = apply_prologue(q, k, prologues[kind])
        out[kind] = attention(q, k, v, kv_len=L, threads=threads, gate=(gates or {}).get(kind))
    return out


def block_attention_rows(inputs: dict, audio_kv_len: int, rows: dict, threads=None, gates=None,
                         prologues=None):
    """Selected rows of each attention: rows = {kind: int array [n, 3] of (b, h, i)};
    gates and prologues as for block_attention."""
    out = {}
    for kind, r in rows.items():
        q, k, v, L = pairing(kind, inputs, audio_kv_len)
        if prologues and kind in prologues:
            q, k = apply_prologue(q, k, prologues[kind])
        out[kind] = attention_rows(q, k, v, r, kv_len=L, threads=threads, gate=(gates or {}).get(kind))
    return out
