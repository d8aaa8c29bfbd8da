"""HIP path vs the double-precision oracle, element by element, through the C ABI.

* the tiny block and ragged multi-tile blocks: every output element;
* the four full-size workloads (3840, 15360 at batch 1 and 2, 27280 video
  tokens): sampled rows the oracle computes one by one, plus properties
  that hold for every row (finite, inside the hull of the valid V rows, so
  no masked poison key leaks);
* needles at every tile / split / padding boundary, strided layouts, guard
  bands around outputs, bit-identical reruns.
"""

import numpy as np
import pytest

import oracle
from tests.gpu_util import compare, log, to_device, to_numpy
from video_audio_diffusion_ltxattn_amd import synth

pytestmark = pytest.mark.gpu

KINDS = ("video_self", "audio_self", "a2v", "v2a")


@pytest.fixture(scope="module")
def torch():
    import torch as _torch
    if not _torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    return _torch


@pytest.fixture(scope="module")
def lt(torch):
    # Raises (does not skip) if the HIP library is missing.
    from video_audio_diffusion_ltxattn_amd import ltxattn
    return ltxattn


def run_block(lt, torch, w, inputs, kinds=KINDS, gates=None):
    log(f"  GPU block: {w.name} B{w.batch} H{w.heads} D{w.head_dim} Sv{w.video_len} "
        f"La{w.audio_len} Lk{w.audio_kv_len} kinds={list(kinds)}{' gated' if gates else ''}")
    dev = {n: to_device(a) for n, a in inputs.items()}
    dev_gates = {k: to_device(g) for k, g in gates.items()} if gates else None
    ba = lt.BlockAttention(w.heads, w.head_dim, w.batch, w.video_len, w.audio_len)
    outs = ba(dev, w.audio_kv_len, kinds=kinds, gates=dev_gates)
    torch.cuda.synchronize()
    res = {k: to_numpy(v) for k, v in outs.items()}
    ba.close()
    return res


RAGGED = [
    # several query and key tiles, ragged tails, split-KV v2a, masked audio keys
    synth.Workload(11, "ragged D128", 2, 3, 128, 1000, 77, 70),
    # D = 64, split v2a, one masked audio key
    synth.Workload(12, "ragged D64", 1, 2, 64, 2100, 130, 129),
    # a single valid audio key
    synth.Workload(13, "one audio key", 1, 2, 64, 300, 33, 1),
    # the smallest block
    synth.Workload(14, "one token", 1, 1, 128, 1, 1, 1),
    # exactly one tile everywhere, no mask
    synth.Workload(15, "whole tiles", 1, 2, 128, 128, 64, 64),
    # scaled keys, spike
    synth.Workload(16, "spiky", 1, 2, 128, 700, 96, 90, k_scale=0.5, spike_rank=4, spike_amp=3.0),
    # Video self-attention on the 256-query ring kernel with a ragged last
    # query tile and a ragged last key tile; the ring's 4-step unroll leaves
    # 2, 3 and 1 tiles over (18, 19 and 17 key tiles).  v2a parts of 3..5 tiles.
    synth.Workload(17, "ring ragged", 2, 2, 128, 1100, 77, 70),
    synth.Workload(18, "ring remainder 3", 1, 1, 128, 1215, 130, 129),
    synth.Workload(19, "ring remainder 1", 1, 3, 128, 1030, 16, 16),
    # The two-tile pass of the resident-key kernel at its mask boundaries:
    # one key into the second tile, and one key short of both tiles.
    synth.Workload(20, "audio keys 65", 1, 2, 128, 300, 96, 65),
    synth.Workload(22, "audio keys 127", 1, 2, 128, 300, 128, 127),
]


@pytest.mark.parametrize("w", [synth.WORKLOADS[1]] + RAGGED, ids=lambda w: w.name)
def test_block_full_oracle(lt, torch, w):
    inputs = synth.make_block_inputs(w)
    got = run_block(lt, torch, w, inputs)
    want = oracle.block_attention(inputs, w.audio_kv_len)
    for k in KINDS:
        compare(got[k], want[k], f"{w.name} {k}")


def sample_rows(rng, B, H, Sq, n_random=24):
    special = {0, 1, 31, 32, 63, 64, 127, 128, 129, Sq - 2, Sq - 1, Sq // 2}
    special = sorted(i for i in special if 0 <= i < Sq)
    rows = []
    for n, i in enumerate(special):
        rows.append((n % B, (7 * n) % H, i))
    for _ in range(n_random):
        rows.append((int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(Sq))))
    return np.array(rows, dtype=np.int64)


def item_rows(rng, B, H, Sq, tile, per_tile=1):
    """per_tile random rows of every (b, h, query tile of `tile` rows), plus the
    first and last row of every (b, h): every work item of a kind whose items are
    whole tiles of `tile` rows (or a multiple of it) has rows among them, its
    split parts included (a split item's rows are finished from all its parts)."""
    rows = []
    for b in range(B):
        for h in range(H):
            rows += [(b, h, 0), (b, h, Sq - 1)]
            for t0 in range(0, Sq, tile):
                hi = min(Sq, t0 + tile)
                rows += [(b, h, int(i)) for i in rng.integers(t0, hi, per_tile)]
    return np.array(rows, dtype=np.int64)


def block_item_rows(rng, w, video_tile=256, audio_tile=128, audio_per_tile=4):
    """Rows covering every work item of every kind: video-query kinds (video self,
    a2v) run 256-query items at these sizes (or 128), audio-query kinds 128."""
    return {k: (item_rows(rng, w.batch, w.heads, w.video_len, video_tile)
                if k in ("video_self", "a2v") else
                item_rows(rng, w.batch, w.heads, w.audio_len, audio_tile, audio_per_tile))
            for k in KINDS}


def check_rows(got, want_rows, rows, what):
    for k in want_rows:
        r = rows[k]
        compare(got[k][r[:, 0], r[:, 2], r[:, 1], :], want_rows[k], f"{what} {k}")


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_full_size_sampled(lt, torch, cfg):
    """The full-size workloads: one oracle row from every work item of every
    kind (every (b, h, query tile), split last-round items and v2a included),
    fixed rows at tile edges, and properties of every row."""
    w = synth.WORKLOADS[cfg]
    inputs = synth.make_block_inputs(w)
    got = run_block(lt, torch, w, inputs)
    rng = np.random.default_rng(100 + cfg)
    rows = block_item_rows(rng, w)
    for k in KINDS:
        Sq = w.video_len if k in ("video_self", "a2v") else w.audio_len
        rows[k] = np.concatenate([rows[k], sample_rows(rng, w.batch, w.heads, Sq, n_random=0)])
    log(f"  oracle rows: " + ", ".join(f"{k} {len(r)}" for k, r in rows.items()))
    want = oracle.block_attention_rows(inputs, w.audio_kv_len, rows)
    check_rows(got, want, rows, f"cfg{cfg} every item")
    # every row: finite and inside the hull of the valid V rows of its (b, h)
    vv = synth.bits_to_f32(inputs["video_v"])
    av = synth.bits_to_f32(inputs["audio_v"])[:, :w.audio_kv_len]
    bound = {"video_self": vv, "v2a": vv, "audio_self": av, "a2v": av}
    for k in KINDS:
        o = got[k]
        assert np.all(np.isfinite(o)), k
        hi = bound[k].max(axis=1, keepdims=True) + 2e-2
        lo = bound[k].min(axis=1, keepdims=True) - 2e-2
        assert np.all(o <= hi) and np.all(o >= lo), f"cfg{cfg} {k}: output outside hull of valid V"


# Blocks that reach launch configurations the workloads above do not, each
# compared with the full oracle (every element):
EDGE_BLOCKS = [
    # v2a at its most parts: 2 items of 128 audio queries on 256 CUs -> 16
    # parts of 256 video keys
    synth.Workload(51, "v2a at 16 parts", 1, 2, 128, 4096, 128, 128),
    # v2a in 5 parts of 320 keys whose last holds one key: its second key group
    # sees no valid key at all (m stays at its start, merge weight 0); video
    # self-attention with one valid row in its last query tile and one valid
    # key in its last key tile
    synth.Workload(52, "v2a one-key last part", 1, 1, 128, 1281, 64, 60),
]


@pytest.mark.parametrize("w", EDGE_BLOCKS, ids=lambda w: w.name)
def test_edge_blocks_full_oracle(lt, torch, w):
    inputs = synth.make_block_inputs(w)
    got = run_block(lt, torch, w, inputs)
    want = oracle.block_attention(inputs, w.audio_kv_len)
    for k in KINDS:
        compare(got[k], want[k], f"{w.name} {k}")


# 200 valid audio keys of 256 (128 KB of K/V in LDS: no room for row-staged
# Q/O): a2v on 8 register-Q waves (256-query items fill the 256 CUs), audio
# self-attention on 4.  Gated and ungated.
RESIDENT_200 = synth.Workload(53, "resident 200 audio keys", 1, 32, 128, 2048, 256, 200)


@pytest.mark.parametrize("gated", [False, True])
def test_resident_keys_unstaged(lt, torch, gated):
    w = RESIDENT_200
    inputs = synth.make_block_inputs(w)
    gates = make_gates(w, 530) if gated else None
    got = run_block(lt, torch, w, inputs, gates=gates)
    for k in ("a2v", "audio_self", "v2a"):
        q, kk, v, L = oracle.pairing(k, inputs, w.audio_kv_len)
        want = oracle.attention(q, kk, v, kv_len=L, gate=gates[k] if gated else None)
        compare(got[k], want, f"{w.name}{' gated' if gated else ''} {k}")
    rng = np.random.default_rng(53)
    rows = {"video_self": item_rows(rng, 1, w.heads, w.video_len, 256)}
    want = oracle.block_attention_rows(inputs, w.audio_kv_len, rows,
                                       gates={"video_self": gates["video_self"]} if gated else None)
    check_rows(got, want, rows, f"{w.name}{' gated' if gated else ''} every item")


# More than 256 valid audio keys: a2v and audio self-attention leave the
# resident-key kernel for the two-buffer kernel, while video self-attention
# (288 items of 256 queries) splits its last round -- in the concurrent call
# the audio side then runs beside that split on the other stream.
LONG_AUDIO = [synth.Workload(54, "600 audio keys", 1, 8, 128, 9216, 640, 600),
              synth.Workload(55, "300 audio keys", 1, 8, 128, 9216, 320, 300)]


@pytest.mark.parametrize("w", LONG_AUDIO, ids=lambda w: w.name)
def test_long_audio_sequential_and_overlap(lt, torch, w):
    inputs = synth.make_block_inputs(w)
    dev = {n: to_device(a) for n, a in inputs.items()}
    ba = lt.BlockAttention(w.heads, w.head_dim, w.batch, w.video_len, w.audio_len)
    log(f"  GPU block: {w.name}, sequential and overlap")
    seq = ba(dev, w.audio_kv_len)
    ovl = ba(dev, w.audio_kv_len, overlap=True)
    torch.cuda.synchronize()
    seq = {k: to_numpy(v) for k, v in seq.items()}
    ovl = {k: to_numpy(v) for k, v in ovl.items()}
    ba.close()
    rng = np.random.default_rng(w.cfg)
    rows = block_item_rows(rng, w)
    want = oracle.block_attention_rows(inputs, w.audio_kv_len, rows)
    check_rows(seq, want, rows, f"{w.name} sequential")
    check_rows(ovl, want, rows, f"{w.name} overlap")
    for k in KINDS:
        assert np.array_equal(seq[k], ovl[k]), k


TAIL_SPLITS = [
    # 8 heads x 9216 video queries = 288 work items of 256 queries.  On a
    # 256-CU MI355X each XCD's group holds one head's 36 items and runs 32 at
    # a time, so the last 4 query tiles of each head (rows 8192..9215) run as
    # 8 key-range parts, dealt after the whole items.
    (synth.Workload(31, "tail split, 8 parts", 1, 8, 128, 9216, 64, 64), range(8), (8192, 9216)),
    # 16 heads x 6144 = 384 items, 48 per XCD group: its last 16 (query tiles
    # 8..23 of the odd heads, rows 2048..6143) run as two key halves on half
    # of the group's CUs, the first halves dealt before the whole items and
    # the second halves after them.
    (synth.Workload(32, "tail split, 2 parts staggered", 1, 16, 128, 6144, 64, 64), range(1, 16, 2),
     (2048, 6144)),
    # D = 64 takes fa_fwd_kernel (128-query items, two workgroups per CU): 8
    # heads x 72 items, one head per XCD group of 64 slots, so each head's last
    # 8 query tiles (rows 8192..9215) run as 8 key-range parts.
    (synth.Workload(33, "tail split, D64 two-buffer kernel", 1, 8, 64, 9216, 64, 64), range(8), (8192, 9216)),
]


@pytest.mark.parametrize("w,split_heads,split_rows", TAIL_SPLITS, ids=lambda x: getattr(x, "name", None))
def test_tail_round_split(lt, torch, w, split_heads, split_rows):
    """Rows of the split items and of whole items must match the oracle."""
    inputs = synth.make_block_inputs(w)
    got = run_block(lt, torch, w, inputs, kinds=("video_self",))
    rng = np.random.default_rng(w.cfg)
    lo, hi = split_rows
    rows = []
    for h in range(w.heads):
        if h in split_heads:
            picks = list(rng.integers(lo, hi, 6)) + [lo, hi - 1]
            if lo > 0:
                picks.append(int(rng.integers(0, lo)))
        else:
            picks = list(rng.integers(0, w.video_len, 3))
        rows += [(0, h, int(i)) for i in picks]
    rows = np.array(rows, np.int64)
    want = oracle.block_attention_rows(inputs, w.audio_kv_len, {"video_self": rows})["video_self"]
    compare(got["video_self"][rows[:, 0], rows[:, 2], rows[:, 1], :], want, "tail-split rows")


def needle_inputs(B, H, D, Sv, La, Lk, video_pos, audio_pos, seed=7):
    """Q = 16 e_0 everywhere; K ~ 0.25 N(0,1) with K[pos_h, h, 0] = 64 (logit 90 at
    D = 128 for the needle), V ~ N(0,1)/16 (outputs on the scale of the real
    workloads, so the absolute tolerance means the same).  Masked audio rows get the needle value
    too, with V = 64: any leak of a masked key shows."""
    rng = np.random.default_rng(seed)
    def q(S):
        x = np.zeros((B, S, H, D), np.float32)
        x[..., 0] = 16.0
        return synth.bf16_bits(x)
    def kv(S, pos):
        k = (0.25 * rng.standard_normal((B, S, H, D))).astype(np.float32)
        v = (rng.standard_normal((B, S, H, D)) / 16).astype(np.float32)
        for h in range(H):
            k[:, pos[h % len(pos)], h, 0] = 64.0
        return k, v
    vk, vv = kv(Sv, video_pos)
    ak, av = kv(La, audio_pos)
    ak[:, Lk:, :, 0] = 64.0
    av[:, Lk:] = 64.0
    return {"video_q": q(Sv), "video_k": synth.bf16_bits(vk), "video_v": synth.bf16_bits(vv),
            "audio_q": q(La), "audio_k": synth.bf16_bits(ak), "audio_v": synth.bf16_bits(av)}


def test_needles_at_boundaries(lt, torch):
    B, H, D, Sv, La, Lk = 1, 16, 128, 2000, 100, 90
    # tile edges (64), query-tile edges (128), split edges of the v2a pass
    # (2000 keys in 7 splits of 320), the last key
    video_pos = [0, 63, 64, 127, 128, 319, 320, 639, 640, 959, 1919, 1920, 1983, 1984, 1998, 1999]
    audio_pos = [0, 31, 32, 63, 64, 88, 89, 1]
    inputs = needle_inputs(B, H, D, Sv, La, Lk, video_pos, audio_pos)
    w = synth.Workload(0, "needles", B, H, D, Sv, La, Lk)
    got = run_block(lt, torch, w, inputs)
    rng = np.random.default_rng(9)
    rows = {k: sample_rows(rng, B, H, Sv if k in ("video_self", "a2v") else La, n_random=40)
            for k in KINDS}
    # make sure every head is sampled
    for k in KINDS:
        extra = np.array([[0, h, (37 * h) % (Sv if k in ("video_self", "a2v") else La)]
                          for h in range(H)], np.int64)
        rows[k] = np.concatenate([rows[k], extra])
    want = oracle.block_attention_rows(inputs, Lk, rows)
    for k in KINDS:
        r = rows[k]
        # the needle dominates, so O ~ V[needle]: a dropped or misplaced tile is an O(1) error
        compare(got[k][r[:, 0], r[:, 2], r[:, 1], :], want[k], f"needle {k}", guard=False)


def test_degenerate_logits(lt, torch):
    """Q = 0: every logit is equal, so each output row is the mean of the valid V
    rows (a closed form, computed here independently of the oracle).  Q and K
    scaled by 30 (logits of several hundred): every output is finite and inside
    the hull of the valid V rows, and rows whose top logit leads the next by more
    than 20 (all but ~1e-9 of the weight on one key) match the oracle."""
    w = synth.Workload(41, "degenerate", 1, 2, 128, 1100, 77, 70)   # ring kernel, ragged tails
    base = synth.make_block_inputs(w)
    Lk = w.audio_kv_len
    v = {"video": synth.bits_to_f32(base["video_v"]).astype(np.float64),
         "audio": synth.bits_to_f32(base["audio_v"]).astype(np.float64)[:, :Lk]}
    keys_of = {"video_self": "video", "audio_self": "audio", "a2v": "audio", "v2a": "video"}

    flat = dict(base)
    flat["video_q"] = np.zeros_like(base["video_q"])
    flat["audio_q"] = np.zeros_like(base["audio_q"])
    got = run_block(lt, torch, w, flat)
    for k in KINDS:
        mean = v[keys_of[k]].mean(axis=1, keepdims=True)
        compare(got[k], np.broadcast_to(mean, got[k].shape), f"Q = 0 {k}")

    big = dict(base)
    for n in ("video_q", "video_k", "audio_q", "audio_k"):
        big[n] = synth.bf16_bits(synth.bits_to_f32(base[n]) * 30)
    got = run_block(lt, torch, w, big)
    want = oracle.block_attention(big, Lk)
    q_of = {"video_self": "video", "audio_self": "audio", "a2v": "video", "v2a": "audio"}
    for k in KINDS:
        g = got[k]
        assert np.isfinite(g).all(), k
        vv = v[keys_of[k]]
        lo, hi = vv.min(axis=1, keepdims=True), vv.max(axis=1, keepdims=True)
        assert (g >= lo - 1e-2).all() and (g <= hi + 1e-2).all(), k
        q = synth.bits_to_f32(big[q_of[k] + "_q"]).astype(np.float64)
        kk = synth.bits_to_f32(big[keys_of[k] + "_k"]).astype(np.float64)
        if keys_of[k] == "audio":
            kk = kk[:, :Lk]
        logits = np.einsum("bihd,bjhd->bhij", q, kk) / np.sqrt(w.head_dim)
        top2 = np.sort(logits, axis=-1)[..., -2:]
        sel = np.argwhere(top2[..., 1] - top2[..., 0] > 20)   # (b, h, i)
        assert len(sel) > 0.5 * logits.shape[0] * logits.shape[1] * logits.shape[2], k
        b, h, i = sel[:, 0], sel[:, 1], sel[:, 2]
        compare(g[b, i, h], want[k][b, i, h], f"30x logits, one-hot rows {k}")


def test_distinct_tensors_per_kind(lt, torch):
    """Each kind with its own Q/K/V (the ABI accepts per-kind tensors, not only
    the two shared stream triples): every kind matches the oracle on its own
    inputs, so no kind reads another kind's tensors."""
    w = synth.Workload(42, "distinct per kind", 1, 2, 128, 1100, 77, 70)   # ring path, split v2a
    stream = synth.make_block_inputs(w)
    rng = np.random.default_rng(42)
    rows = {"video": w.video_len, "audio": w.audio_len}
    q_of = {"video_self": "video", "audio_self": "audio", "a2v": "video", "v2a": "audio"}
    kv_of = {"video_self": "video", "audio_self": "audio", "a2v": "audio", "v2a": "video"}
    shape = lambda s: (w.batch, rows[s], w.heads, w.head_dim)
    own = {}
    for k in KINDS:
        own[k] = tuple(synth.bf16_bits(rng.standard_normal(shape(s)).astype(np.float32))
                       for s in (q_of[k], kv_of[k], kv_of[k]))
    dev = {n: to_device(a) for n, a in stream.items()}
    ba = lt.BlockAttention(w.heads, w.head_dim, w.batch, w.video_len, w.audio_len)
    outs = {k: torch.empty_like(dev[q_of[k] + "_q"]) for k in KINDS}
    own_dev = {k: tuple(to_device(a) for a in own[k]) for k in KINDS}   # alive until the sync below
    io = ba.make_io(dev, w.audio_kv_len, outs, inputs=own_dev)
    lt.ltxattn_block_attention(ba.handle, io, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    del own_dev
    for k in KINDS:
        q, kk, vv = own[k]
        want = oracle.attention(q, kk, vv, kv_len=w.audio_kv_len if kv_of[k] == "audio" else None)
        compare(to_numpy(outs[k]), want, f"distinct inputs {k}")
    ba.close()


def make_gates(w, seed):
    """A gate per kind, uniform in (0, 1) like an activated gate, bf16."""
    rng = np.random.default_rng(seed)
    rows = {"video_self": w.video_len, "audio_self": w.audio_len, "a2v": w.video_len, "v2a": w.audio_len}
    return {k: synth.bf16_bits(rng.uniform(0, 1, (w.batch, rows[k], w.heads, w.head_dim)).astype(np.float32))
            for k in KINDS}


@pytest.mark.parametrize("w", [synth.WORKLOADS[1]] + [r for r in RAGGED if r.cfg in (11, 12, 17)],
                         ids=lambda w: w.name)
def test_gated_outputs(lt, torch, w):
    """Gated attention (o = gate * attention, per channel) on every output path:
    the two-buffer kernel at D = 128 and 64, the ring kernel, v2a and its
    combine, the resident-key kernel with and without row staging."""
    inputs = synth.make_block_inputs(w)
    gates = make_gates(w, 100 + w.cfg)
    got = run_block(lt, torch, w, inputs, gates=gates)
    want = oracle.block_attention(inputs, w.audio_kv_len, gates=gates)
    for k in KINDS:
        compare(got[k], want[k], f"{w.name} gated {k}")


def test_gated_split_tail(lt, torch):
    """The gate on the split last-round items of video self-attention (applied
    by the combine kernel), in the staggered dealing order."""
    w, split_heads, (lo, hi) = TAIL_SPLITS[1]
    inputs = synth.make_block_inputs(w)
    gates = make_gates(w, 132)
    got = run_block(lt, torch, w, inputs, kinds=("video_self",), gates={"video_self": gates["video_self"]})
    rng = np.random.default_rng(7)
    rows = np.array([(0, h, int(i)) for h in split_heads for i in list(rng.integers(lo, hi, 4)) + [lo, hi - 1]]
                    + [(0, h, int(rng.integers(0, lo))) for h in range(w.heads)], np.int64)
    want = oracle.block_attention_rows(inputs, w.audio_kv_len, {"video_self": rows},
                                       gates={"video_self": gates["video_self"]})["video_self"]
    compare(got["video_self"][rows[:, 0], rows[:, 2], rows[:, 1], :], want, "gated tail-split rows")


def test_strided_layouts_and_guard_bands(lt, torch):
    """Inputs in [B, H, S, D] storage, outputs inside larger buffers: the
    kernels honour every stride and write nothing outside the output view."""
    w = synth.Workload(21, "strided", 2, 3, 128, 333, 40, 37)
    inputs = synth.make_block_inputs(w)
    dev = {}
    for n, a in inputs.items():
        t = to_device(np.ascontiguousarray(a.transpose(0, 2, 1, 3)))   # [B, H, S, D] storage
        dev[n] = t.permute(0, 2, 1, 3)                                 # [B, S, H, D] view
    sentinel = 123.0
    outs, bigs = {}, {}
    for k in KINDS:
        S = w.video_len if k in ("video_self", "a2v") else w.audio_len
        big = torch.full((w.batch, S + 2, w.heads + 1, w.head_dim + 16), sentinel,
                         dtype=torch.bfloat16, device="cuda:0")
        bigs[k] = big
        outs[k] = big[:, 1:S + 1, :w.heads, 8:8 + w.head_dim]
    log("  GPU block: strided layouts + guard bands")
    ba = lt.BlockAttention(w.heads, w.head_dim, w.batch, w.video_len, w.audio_len)
    ba(dev, w.audio_kv_len, outs=outs)
    torch.cuda.synchronize()
    want = oracle.block_attention(inputs, w.audio_kv_len)
    for k in KINDS:
        compare(to_numpy(outs[k]), want[k], f"strided {k}")
        big = to_numpy(bigs[k])
        mask = np.ones(big.shape, bool)
        mask[:, 1:-1, :w.heads, 8:8 + w.head_dim] = False
        assert np.all(big[mask] == sentinel), f"{k}: write outside the output view"
    ba.close()


def test_bit_identical_reruns(lt, torch):
    w = synth.WORKLOADS[3]
    inputs = synth.make_block_inputs(w)
    dev = {n: to_device(a) for n, a in inputs.items()}
    log("  GPU block: cfg3 twice for bit identity")
    ba = lt.BlockAttention(w.heads, w.head_dim, w.batch, w.video_len, w.audio_len)
    o1 = ba(dev, w.audio_kv_len)
    o1 = {k: v.clone() for k, v in o1.items()}
    o2 = ba(dev, w.audio_kv_len)
    torch.cuda.synchronize()
    for k in KINDS:
        assert torch.equal(o1[k].view(torch.int16), o2[k].view(torch.int16)), k
    ba.close()


def test_kinds_are_independent(lt, torch):
    """Running a subset of kinds gives the same bits as the full block."""
    w = RAGGED[0]
    inputs = synth.make_block_inputs(w)
    full = run_block(lt, torch, w, inputs)
    for k in KINDS:
        one = run_block(lt, torch, w, inputs, kinds=(k,))
        assert np.array_equal(one[k], full[k]), k


@pytest.mark.parametrize("overlap", [False, True])
def test_profile_events(lt, torch, overlap):
    w = RAGGED[[r.cfg for r in RAGGED].index(17)]
    dev = {n: to_device(a) for n, a in synth.make_block_inputs(w).items()}
    ba = lt.BlockAttention(w.heads, w.head_dim, w.batch, w.video_len, w.audio_len)
    lt.ltxattn_profile_begin(ba.handle, 4)
    for _ in range(2):
        ba(dev, w.audio_kv_len, overlap=overlap)
    rec = lt.ltxattn_profile_read(ba.handle, 4)
    lt.ltxattn_profile_end(ba.handle)
    assert len(rec) == 2
    for r in rec:
        assert all(r[k] > 0 for k in KINDS)
        for k in KINDS:   # the attention kernel alone is part of its kind
            assert 0 < r["kernel"][k] <= r[k] + 1e-3
            assert r[k] <= r["total"] + 1e-3
        if not overlap:   # one stream: the kinds add up within the call
            assert r["total"] + 1e-3 >= sum(r[k] for k in KINDS)
        else:             # two streams: the call lasts at least its longer side
            side = r["v2a"] + r["a2v"] + r["audio_self"]
            assert r["total"] + 1e-3 >= max(r["video_self"], side)
    ba.close()


@pytest.mark.parametrize("overlap", [False, True])
@pytest.mark.parametrize("kinds", [("video_self",), ("a2v", "v2a"), ("audio_self",)])
def test_profile_selected_kinds(lt, torch, kinds, overlap):
    """Recording a subset of kinds: those read as times, the rest and the
    whole-call figure as NaN; a kind after an unrecorded one gets its own start."""
    w = RAGGED[[r.cfg for r in RAGGED].index(17)]
    dev = {n: to_device(a) for n, a in synth.make_block_inputs(w).items()}
    ba = lt.BlockAttention(w.heads, w.head_dim, w.batch, w.video_len, w.audio_len)
    lt.ltxattn_profile_begin_kinds(ba.handle, 3, kinds)
    for _ in range(3):
        ba(dev, w.audio_kv_len, overlap=overlap)
    rec = lt.ltxattn_profile_read(ba.handle, 3)
    lt.ltxattn_profile_end(ba.handle)
    assert len(rec) == 3
    for r in rec:
        assert np.isnan(r["total"])
        for k in KINDS:
            if k in kinds:
                assert 0 < r["kernel"][k] <= r[k] + 1e-3
            else:
                assert np.isnan(r[k]) and np.isnan(r["kernel"][k])
    with pytest.raises(lt.LtxattnError):
        lt.ltxattn_profile_begin_kinds(ba.handle, 3, [])
    ba.close()


def test_create_on_missing_device(lt, torch):
    cfg = lt.ltxattn_config(99, 4, 64, 1, 16, 16)
    with pytest.raises(lt.LtxattnError) as e:
        lt.ltxattn_create(cfg)
    assert e.value.status == lt.LTXATTN_ERR_INVALID_ARG


@pytest.mark.parametrize("cfg", [1, 3, 17])
def test_overlap_matches_sequential(lt, torch, cfg):
    """ltxattn_block_attention_overlap runs the audio side on the handle's
    second stream; the kernels are the same, so every output must equal the
    sequential call's bit for bit."""
    w = RAGGED[[r.cfg for r in RAGGED].index(cfg)] if cfg > 10 else synth.WORKLOADS[cfg]
    inputs = synth.make_block_inputs(w)
    dev = {n: to_device(a) for n, a in inputs.items()}
    ba = lt.BlockAttention(w.heads, w.head_dim, w.batch, w.video_len, w.audio_len)
    log(f"  overlap vs sequential: {w.name}")
    seq = ba(dev, w.audio_kv_len)
    ovl = ba(dev, w.audio_kv_len, overlap=True)
    gates = {k: to_device(g) for k, g in make_gates(w, 200 + cfg).items()}
    seq_g = ba(dev, w.audio_kv_len, gates=gates)
    ovl_g = ba(dev, w.audio_kv_len, overlap=True, gates=gates)
    torch.cuda.synchronize()
    for k in KINDS:
        assert torch.equal(seq[k].view(torch.int16), ovl[k].view(torch.int16)), k
        assert torch.equal(seq_g[k].view(torch.int16), ovl_g[k].view(torch.int16)), k
    # and the concurrent call's outputs against the oracle itself
    host_gates = make_gates(w, 200 + cfg)
    if w.video_len <= 2048:
        want = oracle.block_attention(inputs, w.audio_kv_len)
        want_g = oracle.block_attention(inputs, w.audio_kv_len, gates=host_gates)
        for k in KINDS:
            compare(to_numpy(ovl[k]), want[k], f"overlap {w.name} {k}")
            compare(to_numpy(ovl_g[k]), want_g[k], f"overlap gated {w.name} {k}")
    else:
        rows = block_item_rows(np.random.default_rng(cfg), w)
        want = oracle.block_attention_rows(inputs, w.audio_kv_len, rows)
        want_g = oracle.block_attention_rows(inputs, w.audio_kv_len, rows, gates=host_gates)
        check_rows({k: to_numpy(v) for k, v in ovl.items()}, want, rows, f"overlap {w.name}")
        check_rows({k: to_numpy(v) for k, v in ovl_g.items()}, want_g, rows, f"overlap gated {w.name}")
    ba.close()


@pytest.mark.parametrize("overlap", [False, True])
def test_graph_capture_replays(lt, torch, overlap):
    """The block call captured into a HIP graph from the caller's stream
    (with overlap, the side stream joins the capture through the fork event)
    and replayed three times, with eager work and synchronisation between
    the replays: every replay equals the eager result bit for bit."""
    w = RAGGED[[r.cfg for r in RAGGED].index(17)]
    inputs = synth.make_block_inputs(w)
    dev = {n: to_device(a) for n, a in inputs.items()}
    ba = lt.BlockAttention(w.heads, w.head_dim, w.batch, w.video_len, w.audio_len)
    want = ba(dev, w.audio_kv_len, overlap=overlap)
    torch.cuda.synchronize()
    outs = {k: torch.empty_like(v) for k, v in want.items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    log(f"  graph capture, overlap={overlap}")
    with torch.cuda.graph(g, stream=s):
        ba(dev, w.audio_kv_len, outs=outs, stream=s, overlap=overlap)
    torch.cuda.synchronize()
    oracle_out = oracle.block_attention(inputs, w.audio_kv_len)
    for rep in range(3):
        for o in outs.values():
            o.zero_()                      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in KINDS:
            assert torch.equal(outs[k].view(torch.int16), want[k].view(torch.int16)), (rep, k)
            compare(to_numpy(outs[k]), oracle_out[k], f"graph replay {rep} overlap={overlap} {k}")
    del g
    ba.close()
