"""The allocation-free block call, ltxattn_block_attention_noalloc, through the
C ABI: it keeps the split parts in the library's static device scratch instead
of a handle's workspace.  Two calls in a row, the second with a smaller block
(so it runs on what the first left in the scratch), each checked against
ltxattn_block_attention's outputs bit for bit and against the oracle within
the tolerance; then the call captured into a HIP graph and replayed."""

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
    from video_audio_diffusion_ltxattn_amd import ltxattn
    return ltxattn


def _outs(torch, dev):
    return {k: torch.empty_like(dev["video_q"] if k in ("video_self", "a2v") else dev["audio_q"]) for k in KINDS}


def _oracle_check(w, inputs, got, what):
    if w.video_len <= 2048:
        want = oracle.block_attention(inputs, w.audio_kv_len)
        for k in KINDS:
            compare(got[k], want[k], f"{what} {k}")
        return
    rng = np.random.default_rng(w.cfg)
    rows = {}
    for k in KINDS:
        Sq = w.video_len if k in ("video_self", "a2v") else w.audio_len
        tile = 256 if k in ("video_self", "a2v") else 32
        rows[k] = np.array([(b, h, int(rng.integers(t0, min(Sq, t0 + tile))))
                            for b in range(w.batch) for h in range(w.heads)
                            for t0 in range(0, Sq, tile)], np.int64)
    want = oracle.block_attention_rows(inputs, w.audio_kv_len, rows)
    for k in KINDS:
        r = rows[k]
        compare(got[k][r[:, 0], r[:, 2], r[:, 1], :], want[k], f"{what} {k} rows")


def test_noalloc_two_calls_match_the_handle_call(lt, torch):
    # The headline block (its video self-attention splits the last round, v2a
    # splits into 8 parts: both scratch regions in use), then a smaller one
    # (v2a in 3 to 5 parts, no split last round).
    blocks = [synth.WORKLOADS[3], synth.Workload(17, "ring ragged", 2, 2, 128, 1100, 77, 70)]
    stream = torch.cuda.current_stream()
    for n, w in enumerate(blocks):
        log(f"  no-alloc call {n + 1}: {w.name}")
        inputs = synth.make_block_inputs(w)
        dev = {k: to_device(a) for k, a in inputs.items()}
        ba = lt.BlockAttention(w.heads, w.head_dim, w.batch, w.video_len, w.audio_len)
        ref = ba(dev, w.audio_kv_len)
        outs = _outs(torch, dev)
        io = ba.make_io(dev, w.audio_kv_len, outs)
        cfg = lt.ltxattn_config(0, w.heads, w.head_dim, w.batch, w.video_len, w.audio_len)
        lt.ltxattn_block_attention_noalloc(cfg, io, stream.cuda_stream)
        torch.cuda.synchronize()
        for k in KINDS:
            assert torch.equal(outs[k].view(torch.int16), ref[k].view(torch.int16)), (w.name, k)
        _oracle_check(w, inputs, {k: to_numpy(v) for k, v in outs.items()}, f"no-alloc {w.name}")
        # a request beyond cfg is refused before anything is enqueued
        small = lt.ltxattn_config(0, w.heads, w.head_dim, w.batch, w.video_len - 1, w.audio_len)
        with pytest.raises(lt.LtxattnError) as e:
            lt.ltxattn_block_attention_noalloc(small, io, stream.cuda_stream)
        assert e.value.status == lt.LTXATTN_ERR_INVALID_ARG
        ba.close()


def test_noalloc_graph_replays(lt, torch):
    """Captured into a HIP graph (after one eager call) and replayed three
    times with eager work between the replays: every replay equals the eager
    result bit for bit."""
    w = synth.Workload(17, "ring ragged", 2, 2, 128, 1100, 77, 70)
    inputs = synth.make_block_inputs(w)
    dev = {k: to_device(a) for k, a in inputs.items()}
    cfg = lt.ltxattn_config(0, w.heads, w.head_dim, w.batch, w.video_len, w.audio_len)
    ba = lt.BlockAttention(w.heads, w.head_dim, w.batch, w.video_len, w.audio_len)   # only for make_io
    want = _outs(torch, dev)
    lt.ltxattn_block_attention_noalloc(cfg, ba.make_io(dev, w.audio_kv_len, want),
                                       torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    outs = _outs(torch, dev)
    io = ba.make_io(dev, w.audio_kv_len, outs)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    log("  no-alloc call under graph capture")
    with torch.cuda.graph(g, stream=s):
        lt.ltxattn_block_attention_noalloc(cfg, io, s.cuda_stream)
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs.values():
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in KINDS:
            assert torch.equal(outs[k].view(torch.int16), want[k].view(torch.int16)), (rep, k)
    del g
    ba.close()
