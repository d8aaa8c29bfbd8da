"""Seeded synthetic inputs for the LTX-2 per-block attention set.

This module only draws and packs numbers; it holds none of the attention
arithmetic.  Both the double-precision oracle (used by the tests) and the
HIP path consume the arrays it returns, so the two sides always see the
same bits.

Shapes are token-major ``[B, S, H, D]`` with ``D`` contiguous, the packed
layout of the joint video/audio DiT.  The workloads stand in for the clips
the pages measure:

* the tiny block used for bring-up (video 256 / audio 16, 4 heads of 64);
* stage 1 of the two-stage recipe at half resolution, 3840 video tokens
  (SGLang cookbook "LTX2.5", sec. 4.4; TensorRT-Model-Connect PR #1586,
  "Background");
* the 768x1280x121 clip, 15360 video / 126 audio tokens, audio padded to 128
  (TensorRT-LLM PR #16228 "LTX-2: replicate audio stream across Ulysses
  ranks by default", "Description" and "Test Coverage");
* the same at batch 2 (the guided and unguided branches, SGLang cookbook
  sec. 3.3 "CFG parallel");
* the 1280x704x241 clip, 27280 video tokens (PR #1586, "Two-stage phase
  breakdown"), 252 audio tokens padded to 256, with a shared rank-4 spike
  added to Q and K so that the softmax is peaky.

Recipe (all normals are ``numpy.random.Generator(PCG64(seed))``
``standard_normal(..., float32)``, then rounded to bf16 round-to-nearest-even):

* tensor seed = 1000*cfg + 10*tensor_id + b with tensor_id 0..5 =
  video q, k, v, audio q, k, v and b the batch index;
* cfg 2 scales K of both streams by 0.5 before rounding;
* cfg 5 draws, per batch, U[h] in R^{D x 4} (seed 1000*cfg + 900 + b) shared
  by the video and audio Q and K, and per tensor A[h] in R^{S x 4}
  (seed 1000*cfg + 500 + 10*tensor_id + b), then adds 1.5 * A[h] U[h]^T to
  that Q or K before rounding (each spike element has standard deviation 3);
* audio K/V rows at or beyond the valid audio length are poisoned with
  K = +4.0 and V = +64.0 (both exact in bf16), so that a leaked masked key
  shows up as a large error.
"""

from __future__ import annotations

import dataclasses

import numpy as np

VIDEO_Q, VIDEO_K, VIDEO_V, AUDIO_Q, AUDIO_K, AUDIO_V = range(6)
TENSOR_NAMES = ("video_q", "video_k", "video_v", "audio_q", "audio_k", "audio_v")

POISON_K = 4.0
POISON_V = 64.0


@dataclasses.dataclass(frozen=True)
class Workload:
    """One block-attention workload: sizes plus the input recipe knobs."""

    cfg: int            # seed namespace (1..5 for the named workloads)
    name: str
    batch: int
    heads: int
    head_dim: int
    video_len: int      # Sv, video tokens
    audio_len: int      # audio buffer rows (padded length)
    audio_kv_len: int   # valid audio keys (<= audio_len)
    k_scale: float = 1.0
    spike_rank: int = 0
    spike_amp: float = 0.0

    def with_sizes(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    1: Workload(1, "tiny: video 256 / audio 16, H4 D64, B1", 1, 4, 64, 256, 16, 16),
    2: Workload(2, "two-stage stage-1: video 3840 / audio 126, H32 D128, B1, K*0.5",
                1, 32, 128, 3840, 126, 126, k_scale=0.5),
    3: Workload(3, "768x1280x121: video 15360 / audio 126 (pad 128), H32 D128, B1",
                1, 32, 128, 15360, 128, 126),
    4: Workload(4, "768x1280x121 CFG batch: video 15360 / audio 126 (pad 128), H32 D128, B2",
                2, 32, 128, 15360, 128, 126),
    5: Workload(5, "1280x704x241: video 27280 / audio 252 (pad 256), H32 D128, B1, rank-4 spike",
                1, 32, 128, 27280, 256, 252, spike_rank=4, spike_amp=3.0),
}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round to nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bits to float32 (exact)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _normals(seed: int, shape) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.standard_normal(shape, dtype=np.float32)


def _seq_len(w: Workload, tid: int) -> int:
    return w.video_len if tid in (VIDEO_Q, VIDEO_K, VIDEO_V) else w.audio_len


def make_tensor(w: Workload, tid: int) -> np.ndarray:
    """bf16 bits, shape [B, S, H, D], for tensor ``tid`` of workload ``w``."""
    S = _seq_len(w, tid)
    out = np.empty((w.batch, S, w.heads, w.head_dim), dtype=np.uint16)
    for b in range(w.batch):
        x = _normals(1000 * w.cfg + 10 * tid + b, (S, w.heads, w.head_dim))
        if tid in (VIDEO_K, AUDIO_K) and w.k_scale != 1.0:
            x *= np.float32(w.k_scale)
        if w.spike_rank and tid in (VIDEO_Q, VIDEO_K, AUDIO_Q, AUDIO_K):
            u = _normals(1000 * w.cfg + 900 + b, (w.heads, w.head_dim, w.spike_rank))
            a = _normals(1000 * w.cfg + 500 + 10 * tid + b, (w.heads, S, w.spike_rank))
            amp = np.float32(w.spike_amp / np.sqrt(w.spike_rank))
            x += amp * np.einsum("hsr,hdr->shd", a, u).astype(np.float32)
        if tid in (AUDIO_K, AUDIO_V) and w.audio_kv_len < w.audio_len:
            x[w.audio_kv_len:] = POISON_K if tid == AUDIO_K else POISON_V
        out[b] = bf16_bits(x)
    return out


def make_block_inputs(w: Workload) -> dict:
    """All six stream tensors as bf16 bits, keyed by ``TENSOR_NAMES``."""
    return {name: make_tensor(w, tid) for tid, name in enumerate(TENSOR_NAMES)}


def attention_flops(w: Workload) -> dict:
    """Algorithmic FLOPs per attention kind: 4*B*H*Sq*Sk_valid*D (two GEMMs)."""
    B, H, D = w.batch, w.heads, w.head_dim
    Sv, La, Lk = w.video_len, w.audio_len, w.audio_kv_len
    return {
        "video_self": 4.0 * B * H * Sv * Sv * D,
        "audio_self": 4.0 * B * H * La * Lk * D,
        "a2v": 4.0 * B * H * Sv * Lk * D,
        "v2a": 4.0 * B * H * La * Sv * D,
    }


def attention_bytes(w: Workload) -> dict:
    """Algorithmic HBM bytes per kind: bf16 Q, K, V read once and O written once."""
    row = 2 * w.heads * w.head_dim * w.batch
    Sv, La = w.video_len, w.audio_len
    return {
        "video_self": row * 4 * Sv,
        "audio_self": row * 4 * La,
        "a2v": row * (2 * Sv + 2 * La),
        "v2a": row * (2 * La + 2 * Sv),
    }


# ------------------------------------------- QK-norm + rotary prologue inputs
# The caller's side of the prologue: RMS-norm weights near 1 (as trained
# norm weights are) and rotary tables per token position.  The pages bake
# the tables of each latent grid into the DiT plan and give no frequencies;
# these stand in for them: video tokens at (frame, row, column) of a latent
# grid 40 columns wide and 24 rows high (the 768x1280 grid; other lengths
# wrap the same way), the D/2 channel pairs split into three groups that
# rotate with the frame, the row and the column; audio tokens along one
# axis.  Angles theta = position * 10000^(-j/n) for pair j of a group of n.
GRID_W, GRID_H = 40, 24


def _angles_1d(pos: np.ndarray, n: int) -> np.ndarray:
    return pos[:, None].astype(np.float64) * 10000.0 ** (-np.arange(n) / n)[None, :]


def rope_tables(S: int, D: int, video: bool):
    """cos, sin float32 [S, D/2] for S tokens of the video or the audio stream."""
    P = D // 2
    s = np.arange(S)
    if video:
        n_y = n_x = P // 3
        n_t = P - n_y - n_x
        th = np.concatenate([_angles_1d(s // (GRID_W * GRID_H), n_t),
                             _angles_1d((s // GRID_W) % GRID_H, n_y),
                             _angles_1d(s % GRID_W, n_x)], axis=1)
    else:
        th = _angles_1d(s, P)
    return np.cos(th).astype(np.float32), np.sin(th).astype(np.float32)


def make_prologues(w: Workload, pairing: str = "half", eps: float = 1e-6, shared_k: bool = False,
                   seed: int = 0) -> dict:
    """Per kind: q_weight, k_weight (float32 [D], 1 + 0.1 N(0,1), drawn per kind
    and tensor, seed 1000*cfg + 700 + seed), the rotary tables of its query and
    key streams, eps and the pairing.  shared_k: the kinds that read the same
    keys (video self and v2a; audio self and a2v) share one k weight."""
    rng = np.random.Generator(np.random.PCG64(1000 * w.cfg + 700 + seed))
    D = w.head_dim
    tabs = {"video": rope_tables(w.video_len, D, True), "audio": rope_tables(w.audio_len, D, False)}
    q_of = {"video_self": "video", "audio_self": "audio", "a2v": "video", "v2a": "audio"}
    kv_of = {"video_self": "video", "audio_self": "audio", "a2v": "audio", "v2a": "video"}
    weight = lambda: (1 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    k_weights = {"video": weight(), "audio": weight()}
    out = {}
    for kind in ("video_self", "audio_self", "a2v", "v2a"):
        qs, ks = q_of[kind], kv_of[kind]
        out[kind] = {"q_weight": weight(), "k_weight": k_weights[ks] if shared_k else weight(),
                     "q_cos": tabs[qs][0], "q_sin": tabs[qs][1], "k_cos": tabs[ks][0], "k_sin": tabs[ks][1],
                     "eps": eps, "pairing": pairing}
    return out
