"""Python binding of the ``ltxattn`` C ABI (``include/ltxattn.h``).

Argument marshalling only: every step of the attention runs in the HIP
kernels of ``libltxattn.so``.  PyTorch provides device memory and streams.
If the library is missing this module raises on import; there is no
fallback of any kind.

The functions keep the C names (``ltxattn_create``, ``ltxattn_block_attention``,
...).  :class:`BlockAttention` wraps them for torch tensors.
"""

from __future__ import annotations

import ctypes
import os

# torch ships its own HIP runtime (libamdhip64.so.7).  Load it before the
# library so that libltxattn.so binds to that same runtime instead of pulling
# a second copy from /opt/rocm into the process: device pointers and streams
# handed over from torch then belong to the runtime the kernels launch on.
import torch  # noqa: F401  (imported for its HIP runtime)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libltxattn.so")

LTXATTN_OK = 0
LTXATTN_ERR_INVALID_ARG = -1
LTXATTN_ERR_UNSUPPORTED = -2
LTXATTN_ERR_HIP = -3
LTXATTN_ERR_OOM = -4
LTXATTN_ERR_SCRATCH = -5

LTXATTN_VIDEO_SELF = 0
LTXATTN_AUDIO_SELF = 1
LTXATTN_A2V = 2
LTXATTN_V2A = 3
LTXATTN_NUM_KINDS = 4
LTXATTN_PROFILE_FLOATS = 9
LTXATTN_ROPE_HALF = 0
LTXATTN_ROPE_INTERLEAVED = 1
PAIRINGS = {"half": LTXATTN_ROPE_HALF, "interleaved": LTXATTN_ROPE_INTERLEAVED}
KIND_NAMES = ("video_self", "audio_self", "a2v", "v2a")
KIND_INDEX = {n: i for i, n in enumerate(KIND_NAMES)}


class ltxattn_config(ctypes.Structure):
    _fields_ = [("device", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("max_batch", ctypes.c_int32),
                ("max_video_len", ctypes.c_int32), ("max_audio_len", ctypes.c_int32),
                ("qk_prologue", ctypes.c_int32)]


class ltxattn_tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("stride_b", ctypes.c_int64),
                ("stride_s", ctypes.c_int64), ("stride_h", ctypes.c_int64)]


class ltxattn_qk_prologue(ctypes.Structure):
    _fields_ = [("q_weight", ctypes.c_void_p), ("k_weight", ctypes.c_void_p),
                ("q_cos", ctypes.c_void_p), ("q_sin", ctypes.c_void_p),
                ("k_cos", ctypes.c_void_p), ("k_sin", ctypes.c_void_p),
                ("eps", ctypes.c_float), ("pairing", ctypes.c_int32)]


class ltxattn_attn_io(ctypes.Structure):
    _fields_ = [("q", ltxattn_tensor), ("k", ltxattn_tensor),
                ("v", ltxattn_tensor), ("o", ltxattn_tensor),
                ("gate", ltxattn_tensor),        # gate.data = None: no output gate
                ("prologue", ltxattn_qk_prologue)]   # prologue.q_weight = None: none


class ltxattn_block_io(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("video_len", ctypes.c_int32),
                ("audio_len", ctypes.c_int32), ("audio_kv_len", ctypes.c_int32),
                ("attn", ltxattn_attn_io * LTXATTN_NUM_KINDS)]


class LtxattnError(RuntimeError):
    def __init__(self, status: int, what: str, hip_error: int = 0):
        msg = f"{what}: {ltxattn_status_string(status)} ({status})"
        if hip_error:
            msg += f", hipError_t {hip_error}"
        super().__init__(msg)
        self.status = status
        self.hip_error = hip_error


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run "
                          "`python -m video_audio_diffusion_ltxattn_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    sig = {
        "ltxattn_create": ([ctypes.POINTER(ltxattn_config), ctypes.POINTER(P)], ctypes.c_int),
        "ltxattn_block_attention": ([P, ctypes.POINTER(ltxattn_block_io), P], ctypes.c_int),
        "ltxattn_block_attention_overlap": ([P, ctypes.POINTER(ltxattn_block_io), P], ctypes.c_int),
        "ltxattn_block_attention_noalloc": ([ctypes.POINTER(ltxattn_config), ctypes.POINTER(ltxattn_block_io), P],
                                            ctypes.c_int),
        "ltxattn_check_block": ([ctypes.POINTER(ltxattn_config), ctypes.POINTER(ltxattn_block_io)],
                                ctypes.c_int),
        "ltxattn_destroy": ([P], ctypes.c_int),
        "ltxattn_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "ltxattn_last_hip_error": ([P], ctypes.c_int),
        "ltxattn_profile_begin": ([P, ctypes.c_int32], ctypes.c_int),
        "ltxattn_profile_begin_kinds": ([P, ctypes.c_int32, ctypes.c_uint32], ctypes.c_int),
        "ltxattn_profile_read": ([P, ctypes.POINTER(ctypes.c_float), ctypes.c_int32,
                                  ctypes.POINTER(ctypes.c_int32)], ctypes.c_int),
        "ltxattn_profile_end": ([P], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


_lib = _load()
EXPORTED = ("ltxattn_create", "ltxattn_block_attention", "ltxattn_block_attention_overlap",
            "ltxattn_block_attention_noalloc",
            "ltxattn_check_block",
            "ltxattn_destroy", "ltxattn_status_string", "ltxattn_last_hip_error",
            "ltxattn_profile_begin", "ltxattn_profile_begin_kinds", "ltxattn_profile_read",
            "ltxattn_profile_end")


# ------------------------------------------------------------- C-named calls
def ltxattn_status_string(status: int) -> str:
    return _lib.ltxattn_status_string(int(status)).decode()


def ltxattn_create(cfg: ltxattn_config) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    rc = _lib.ltxattn_create(ctypes.byref(cfg), ctypes.byref(h))
    if rc != LTXATTN_OK:
        raise LtxattnError(rc, "ltxattn_create", _lib.ltxattn_last_hip_error(None))
    return h


def ltxattn_block_attention(h, io: ltxattn_block_io, stream: int) -> None:
    rc = _lib.ltxattn_block_attention(h, ctypes.byref(io), ctypes.c_void_p(stream))
    if rc != LTXATTN_OK:
        raise LtxattnError(rc, "ltxattn_block_attention",
                           _lib.ltxattn_last_hip_error(h) if rc == LTXATTN_ERR_HIP else 0)


def ltxattn_block_attention_overlap(h, io: ltxattn_block_io, stream: int) -> None:
    rc = _lib.ltxattn_block_attention_overlap(h, ctypes.byref(io), ctypes.c_void_p(stream))
    if rc != LTXATTN_OK:
        raise LtxattnError(rc, "ltxattn_block_attention_overlap",
                           _lib.ltxattn_last_hip_error(h) if rc == LTXATTN_ERR_HIP else 0)


def ltxattn_block_attention_noalloc(cfg: ltxattn_config, io: ltxattn_block_io, stream: int) -> None:
    rc = _lib.ltxattn_block_attention_noalloc(ctypes.byref(cfg), ctypes.byref(io), ctypes.c_void_p(stream))
    if rc != LTXATTN_OK:
        raise LtxattnError(rc, "ltxattn_block_attention_noalloc",
                           _lib.ltxattn_last_hip_error(None) if rc == LTXATTN_ERR_HIP else 0)


def ltxattn_check_block(cfg: ltxattn_config, io: ltxattn_block_io) -> int:
    """Status the block call would get from argument validation (no device use)."""
    return _lib.ltxattn_check_block(ctypes.byref(cfg), ctypes.byref(io))


def ltxattn_destroy(h) -> None:
    rc = _lib.ltxattn_destroy(h)
    if rc != LTXATTN_OK:
        raise LtxattnError(rc, "ltxattn_destroy")


def ltxattn_last_hip_error(h) -> int:
    return _lib.ltxattn_last_hip_error(h)


def ltxattn_profile_begin(h, max_calls: int) -> None:
    rc = _lib.ltxattn_profile_begin(h, int(max_calls))
    if rc != LTXATTN_OK:
        raise LtxattnError(rc, "ltxattn_profile_begin")


def ltxattn_profile_begin_kinds(h, max_calls: int, kinds) -> None:
    """Record events for the named kinds only (others, and 'total' unless all
    four are named, read as NaN)."""
    mask = 0
    for k in kinds:
        mask |= 1 << KIND_INDEX[k]
    rc = _lib.ltxattn_profile_begin_kinds(h, int(max_calls), mask)
    if rc != LTXATTN_OK:
        raise LtxattnError(rc, "ltxattn_profile_begin_kinds")


def ltxattn_profile_read(h, max_calls: int):
    """Per recorded call: {kind: ms of all its kernels, 'total': ms,
    'kernel': {kind: ms of the attention kernels only}}; NaN where not recorded."""
    nf = LTXATTN_PROFILE_FLOATS
    buf = (ctypes.c_float * (nf * max_calls))()
    n = ctypes.c_int32()
    rc = _lib.ltxattn_profile_read(h, buf, int(max_calls), ctypes.byref(n))
    if rc != LTXATTN_OK:
        raise LtxattnError(rc, "ltxattn_profile_read")
    out = []
    for c in range(n.value):
        d = {KIND_NAMES[k]: buf[c * nf + k] for k in range(4)}
        d["total"] = buf[c * nf + 4]
        d["kernel"] = {KIND_NAMES[k]: buf[c * nf + 5 + k] for k in range(4)}
        out.append(d)
    return out


def ltxattn_profile_end(h) -> None:
    rc = _lib.ltxattn_profile_end(h)
    if rc != LTXATTN_OK:
        raise LtxattnError(rc, "ltxattn_profile_end")


# ------------------------------------------------------------ torch wrapper
def _f32_ptr(t, what: str) -> int:
    import torch
    if t.dtype != torch.float32 or not t.is_contiguous():
        raise TypeError(f"{what}: expected a contiguous float32 tensor")
    return t.data_ptr()


def prologue_desc(p: dict) -> ltxattn_qk_prologue:
    """The QK-norm + rotary prologue of one kind from a dict: q_weight, k_weight
    (float32 [D]), q_cos, q_sin, k_cos, k_sin (float32 [rows, D/2]), eps and
    pairing ("half" or "interleaved")."""
    return ltxattn_qk_prologue(*(_f32_ptr(p[n], n) for n in ("q_weight", "k_weight", "q_cos", "q_sin",
                                                              "k_cos", "k_sin")),
                               float(p["eps"]), PAIRINGS[p["pairing"]])


def tensor_desc(t) -> ltxattn_tensor:
    """Describe a torch bf16 tensor [B, S, H, D] (D contiguous) for the ABI."""
    import torch
    if t.dtype != torch.bfloat16:
        raise TypeError(f"expected bfloat16, got {t.dtype}")
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("expected [B, S, H, D] with D contiguous")
    sb, ss, sh, _ = t.stride()
    return ltxattn_tensor(t.data_ptr(), sb, ss, sh)


class BlockAttention:
    """The four per-block attentions of the joint video+audio DiT on one GPU.

    ``__call__`` takes the video and audio Q/K/V streams ([B, S, H, D] bf16 on
    the handle's device) and the number of valid audio keys, and returns the
    four outputs.  Work is enqueued on the current torch stream.
    """

    def __init__(self, heads: int, head_dim: int, max_batch: int, max_video_len: int,
                 max_audio_len: int, device: int = 0, qk_prologue: bool = False):
        self.cfg = ltxattn_config(device, heads, head_dim, max_batch, max_video_len, max_audio_len,
                                  int(qk_prologue))
        self.device = device
        self.handle = ltxattn_create(self.cfg)

    def close(self):
        if self.handle is not None and self.handle.value:
            ltxattn_destroy(self.handle)
        self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def make_io(self, streams: dict, audio_kv_len: int, outs: dict, inputs: dict = None,
                gates: dict = None, prologues: dict = None) -> ltxattn_block_io:
        """streams: video_q/k/v, audio_q/k/v tensors; outs: {kind name: output tensor};
        inputs: optional {kind name: (q, k, v)} replacing that kind's stream tensors;
        gates: optional {kind name: gate tensor of that output's shape};
        prologues: optional {kind name: QK-norm + rotary parameters (prologue_desc)}.
        The struct holds raw device pointers: every tensor named here must stay
        alive until the work enqueued with it has completed."""
        vq, vk, vv = streams["video_q"], streams["video_k"], streams["video_v"]
        aq, ak, av = streams["audio_q"], streams["audio_k"], streams["audio_v"]
        io = ltxattn_block_io()
        io.batch, io.video_len = vq.shape[0], vq.shape[1]
        io.audio_len, io.audio_kv_len = aq.shape[1], int(audio_kv_len)
        pairs = {"video_self": (vq, vk, vv), "audio_self": (aq, ak, av),
                 "a2v": (vq, ak, av), "v2a": (aq, vk, vv)}
        pairs.update(inputs or {})
        for name, o in outs.items():
            q, k, v = pairs[name]
            g = (gates or {}).get(name)
            pro = (prologues or {}).get(name)
            io.attn[KIND_INDEX[name]] = ltxattn_attn_io(tensor_desc(q), tensor_desc(k), tensor_desc(v),
                                                        tensor_desc(o),
                                                        tensor_desc(g) if g is not None else ltxattn_tensor(),
                                                        prologue_desc(pro) if pro else ltxattn_qk_prologue())
        return io

    def __call__(self, streams: dict, audio_kv_len: int, kinds=KIND_NAMES, outs: dict = None,
                 stream=None, overlap: bool = False, gates: dict = None, prologues: dict = None) -> dict:
        import torch
        if outs is None:
            vq, aq = streams["video_q"], streams["audio_q"]
            outs = {k: torch.empty_like(vq if k in ("video_self", "a2v") else aq) for k in kinds}
        io = self.make_io(streams, audio_kv_len, outs, gates=gates, prologues=prologues)
        s = stream if stream is not None else torch.cuda.current_stream(self.device)
        call = ltxattn_block_attention_overlap if overlap else ltxattn_block_attention
        call(self.handle, io, s.cuda_stream)
        return outs
