"""The C ABI without a GPU: the library loads, exports every function the
header declares, and rejects bad requests before touching a device."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

lt = pytest.importorskip("video_audio_diffusion_ltxattn_amd.ltxattn",
                         reason="libltxattn.so not built")


def declared_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(ltxattn_\w+)\s*\(", text))
    return names


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"ltxattn_create", "ltxattn_block_attention", "ltxattn_destroy"} <= names
    lib = ctypes.CDLL(lt.LIB_PATH)
    for n in sorted(names):
        assert hasattr(lib, n), f"{n} declared in include/ but not exported"
    assert set(lt.EXPORTED) == names


def test_status_strings():
    assert lt.ltxattn_status_string(0) == "ok"
    for s in (-1, -2, -3, -4, -5):
        assert lt.ltxattn_status_string(s) not in ("ok", "unknown status")
    assert lt.ltxattn_status_string(7) == "unknown status"


def test_create_rejects_before_device():
    h = ctypes.c_void_p(1234)
    assert lt._lib.ltxattn_create(None, ctypes.byref(h)) == lt.LTXATTN_ERR_INVALID_ARG
    assert h.value is None
    bad = [((0, 32, 96, 1, 16, 16), lt.LTXATTN_ERR_UNSUPPORTED),
           ((0, 0, 128, 1, 16, 16), lt.LTXATTN_ERR_UNSUPPORTED),
           ((0, 32, 128, 0, 16, 16), lt.LTXATTN_ERR_INVALID_ARG),
           ((0, 32, 128, 1, 0, 16), lt.LTXATTN_ERR_INVALID_ARG),
           ((-1, 32, 128, 1, 16, 16), lt.LTXATTN_ERR_INVALID_ARG)]
    for args, want in bad:
        cfg = lt.ltxattn_config(*args)
        assert lt._lib.ltxattn_create(ctypes.byref(cfg), ctypes.byref(h)) == want, args
    assert lt._lib.ltxattn_create(ctypes.byref(lt.ltxattn_config(0, 1, 64, 1, 1, 1)), None) \
        == lt.LTXATTN_ERR_INVALID_ARG


def test_null_handles():
    io = lt.ltxattn_block_io()
    assert lt._lib.ltxattn_block_attention(None, ctypes.byref(io), None) == lt.LTXATTN_ERR_INVALID_ARG
    assert lt._lib.ltxattn_block_attention_overlap(None, ctypes.byref(io), None) == lt.LTXATTN_ERR_INVALID_ARG
    assert lt._lib.ltxattn_destroy(None) == lt.LTXATTN_OK
    assert lt._lib.ltxattn_profile_begin(None, 4) == lt.LTXATTN_ERR_INVALID_ARG
    assert lt._lib.ltxattn_profile_begin_kinds(None, 4, 1) == lt.LTXATTN_ERR_INVALID_ARG
    assert lt._lib.ltxattn_last_hip_error(None) == 0
    assert lt._lib.ltxattn_block_attention_noalloc(None, ctypes.byref(io), None) == lt.LTXATTN_ERR_INVALID_ARG
    cfg = lt.ltxattn_config(0, 4, 64, 1, 16, 16)
    assert lt._lib.ltxattn_block_attention_noalloc(ctypes.byref(cfg), None, None) == lt.LTXATTN_ERR_INVALID_ARG
    for bad, want in (((0, 4, 96, 1, 16, 16), lt.LTXATTN_ERR_UNSUPPORTED), ((0, 0, 64, 1, 16, 16), lt.LTXATTN_ERR_UNSUPPORTED),
                      ((-1, 4, 64, 1, 16, 16), lt.LTXATTN_ERR_INVALID_ARG), ((0, 4, 64, 0, 16, 16), lt.LTXATTN_ERR_INVALID_ARG)):
        cfg = lt.ltxattn_config(*bad)
        assert lt._lib.ltxattn_block_attention_noalloc(ctypes.byref(cfg), ctypes.byref(io), None) == want, bad


# ------------------------------------------------------------ block checks
H, D = 4, 64
Sv, La, Lk, B = 256, 16, 13, 2
ROW = H * D


def _t(addr, S, sb=None, ss=ROW, sh=D):
    return lt.ltxattn_tensor(addr, S * ROW if sb is None else sb, ss, sh)


def make_io(**over):
    """A valid request with fake (never dereferenced) 16-byte-aligned addresses;
    every tensor occupies its own 1 GiB window."""
    base = 1 << 40
    win = 1 << 30
    io = lt.ltxattn_block_io()
    io.batch, io.video_len, io.audio_len, io.audio_kv_len = B, Sv, La, Lk
    vq, vk, vv = _t(base, Sv), _t(base + win, Sv), _t(base + 2 * win, Sv)
    aq, ak, av = _t(base + 3 * win, La), _t(base + 4 * win, La), _t(base + 5 * win, La)
    outs = [_t(base + (6 + k) * win, Sv if k in (0, 2) else La) for k in range(4)]
    io.attn[0] = lt.ltxattn_attn_io(vq, vk, vv, outs[0])
    io.attn[1] = lt.ltxattn_attn_io(aq, ak, av, outs[1])
    io.attn[2] = lt.ltxattn_attn_io(vq, ak, av, outs[2])
    io.attn[3] = lt.ltxattn_attn_io(aq, vk, vv, outs[3])
    for k, v in over.items():
        setattr(io, k, v)
    return io


CFG = lt.ltxattn_config(0, H, D, B, Sv, La)


def check(io, cfg=CFG):
    return lt.ltxattn_check_block(cfg, io)


def test_valid_request_passes():
    assert check(make_io()) == lt.LTXATTN_OK
    io = make_io()
    io.attn[1].o.data = None     # skipped kind: its tensors are not looked at
    io.attn[1].q.data = None
    assert check(io) == lt.LTXATTN_OK


@pytest.mark.parametrize("field,value", [
    ("batch", 0), ("batch", B + 1), ("video_len", 0), ("video_len", Sv + 1),
    ("audio_len", 0), ("audio_len", La + 1), ("audio_kv_len", 0), ("audio_kv_len", La + 1),
])
def test_sizes_out_of_range(field, value):
    assert check(make_io(**{field: value})) == lt.LTXATTN_ERR_INVALID_ARG


def test_audio_kv_len_equal_to_buffer_is_fine():
    assert check(make_io(audio_kv_len=La)) == lt.LTXATTN_OK


@pytest.mark.parametrize("kind", range(4))
@pytest.mark.parametrize("which", ["q", "k", "v", "o"])
def test_bad_tensor(kind, which):
    for mutate in ("null", "misaligned", "stride_s_small", "stride_odd", "stride_h_small"):
        io = make_io()
        t = getattr(io.attn[kind], which)
        if mutate == "null":
            if which == "o":
                continue              # a null output means "skip", not an error
            t.data = None
        elif mutate == "misaligned":
            t.data = t.data + 8
        elif mutate == "stride_s_small":
            t.stride_s = D - 8
        elif mutate == "stride_odd":
            t.stride_s = ROW + 4
        elif mutate == "stride_h_small":
            t.stride_h = 8
        setattr(io.attn[kind], which, t)
        assert check(io) == lt.LTXATTN_ERR_INVALID_ARG, (kind, which, mutate)


def test_output_aliasing_rejected():
    io = make_io()
    o = io.attn[0].o
    o.data = io.attn[3].k.data          # video self output on top of v2a's video K
    io.attn[0].o = o
    assert check(io) == lt.LTXATTN_ERR_INVALID_ARG
    io = make_io()
    o = io.attn[2].o
    o.data = io.attn[0].o.data + 4096   # two outputs overlapping
    io.attn[2].o = o
    assert check(io) == lt.LTXATTN_ERR_INVALID_ARG


def test_head_major_layout_accepted():
    """[B, H, S, D] strides are a valid description of the same tensors."""
    io = make_io()
    for k in range(4):
        for which in "qkvo":
            t = getattr(io.attn[k], which)
            S = t.stride_b // ROW
            setattr(io.attn[k], which, lt.ltxattn_tensor(t.data, S * ROW, D, S * D))
    assert check(io) == lt.LTXATTN_OK


def test_unsupported_config():
    assert check(make_io(), lt.ltxattn_config(0, H, 96, B, Sv, La)) == lt.LTXATTN_ERR_UNSUPPORTED
    assert check(make_io(), lt.ltxattn_config(0, 0, D, B, Sv, La)) == lt.LTXATTN_ERR_UNSUPPORTED


def test_huge_slice_unsupported():
    """A (batch, head) slice beyond 32-bit byte offsets is refused, not mis-addressed."""
    big = 1 << 21
    cfg = lt.ltxattn_config(0, H, D, 1, big, La)
    io = make_io(batch=1, video_len=big)
    for k in (0,):
        for which in "qkvo":
            t = getattr(io.attn[k], which)
            setattr(io.attn[k], which, lt.ltxattn_tensor(t.data + (k + 1) * (1 << 36) * ("qkvo".index(which) + 1),
                                                        big * 1024, 1024, 64))
    io.attn[1].o.data = io.attn[2].o.data = io.attn[3].o.data = None
    assert check(io, cfg) == lt.LTXATTN_ERR_UNSUPPORTED


# ------------------------------------------------------------ output gates
def _gated_io():
    """make_io() with a gate on every kind, each in a window of its own."""
    io = make_io()
    base, win = 1 << 40, 1 << 30
    for k in range(4):
        io.attn[k].gate = _t(base + (10 + k) * win, Sv if k in (0, 2) else La)
    return io


def test_gates_pass_and_may_alias_inputs():
    assert check(_gated_io()) == lt.LTXATTN_OK
    io = _gated_io()
    io.attn[0].gate = io.attn[0].q          # a gate is an input: it may be any input tensor
    io.attn[3].gate = io.attn[1].q
    assert check(io) == lt.LTXATTN_OK


@pytest.mark.parametrize("kind", range(4))
def test_bad_gate(kind):
    for mutate in ("misaligned", "stride_s_small", "stride_odd", "short", "overlaps_own_output",
                   "overlaps_other_output"):
        io = _gated_io()
        g = io.attn[kind].gate
        if mutate == "misaligned":
            g.data = g.data + 8
        elif mutate == "stride_s_small":
            g.stride_s = D - 8
        elif mutate == "stride_odd":
            g.stride_s = ROW + 4
        elif mutate == "short":                      # rows of this kind's output beyond 32-bit reach
            g.stride_s = 1 << 24
        elif mutate == "overlaps_own_output":
            io.attn[kind].gate = io.attn[kind].o
        else:
            io.attn[kind].gate = io.attn[(kind + 1) % 4].o
        want = lt.LTXATTN_ERR_UNSUPPORTED if mutate == "short" else lt.LTXATTN_ERR_INVALID_ARG
        assert check(io) == want, (kind, mutate)


def test_struct_layouts_match_the_header(tmp_path):
    """The binding's ctypes structs have the C header's sizes and field offsets
    (a C program built against include/ltxattn.h prints them)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    fields = {"ltxattn_config": [f for f, _ in lt.ltxattn_config._fields_],
              "ltxattn_tensor": [f for f, _ in lt.ltxattn_tensor._fields_],
              "ltxattn_qk_prologue": [f for f, _ in lt.ltxattn_qk_prologue._fields_],
              "ltxattn_attn_io": [f for f, _ in lt.ltxattn_attn_io._fields_],
              "ltxattn_block_io": [f for f, _ in lt.ltxattn_block_io._fields_]}
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "ltxattn.h"', "int main(void) {"]
    for st, fs in fields.items():
        lines.append(f'  printf("{st} %zu\\n", sizeof({st}));')
        for f in fs:
            lines.append(f'  printf("{st}.{f} %zu\\n", offsetof({st}, {f}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-I", os.path.join(root, "include"), "-o", str(exe), str(src)], check=True)
    got = dict(ln.split() for ln in subprocess.run([str(exe)], capture_output=True, text=True,
                                                     check=True).stdout.splitlines())
    for st, fs in fields.items():
        cls = getattr(lt, st)
        assert int(got[st]) == ctypes.sizeof(cls), st
        for f in fs:
            assert int(got[f"{st}.{f}"]) == getattr(cls, f).offset, (st, f)


# ------------------------------------------------- outputs with shared rows
@pytest.mark.parametrize("case", ["s_and_h_same_stride", "batch_stride_zero", "h_inside_s_span",
                                  "s_inside_b_span"])
def test_output_rows_sharing_memory_rejected(case):
    """Distinct (b, s, h) rows of an output must not share bytes; the same
    strides on an input are accepted (a kernel only reads them)."""
    for kind in range(4):
        S = Sv if kind in (0, 2) else La
        io = make_io()
        o = io.attn[kind].o
        if case == "s_and_h_same_stride":
            o.stride_s, o.stride_h = D, D
        elif case == "batch_stride_zero":
            o.stride_b = 0
        elif case == "h_inside_s_span":            # head-major, heads closer than S rows apart
            o.stride_s, o.stride_h, o.stride_b = D, (S - 1) * D, S * ROW
        else:                                      # batches closer than one batch's span
            o.stride_b = S * ROW - D
        io.attn[kind].o = o
        assert check(io) == lt.LTXATTN_ERR_INVALID_ARG, (case, kind)
        io = make_io()
        q = io.attn[kind].q
        q.stride_b, q.stride_s, q.stride_h = o.stride_b, o.stride_s, o.stride_h
        io.attn[kind].q = q
        assert check(io) == lt.LTXATTN_OK, (case, kind)


def test_output_dims_of_extent_one_take_any_stride():
    """A dimension of extent 1 spans nothing: its stride does not matter."""
    cfg = lt.ltxattn_config(0, 1, D, 1, Sv, La)
    io = make_io(batch=1)
    for k in range(4):
        for which in "qkvo":
            t = getattr(io.attn[k], which)
            t.stride_h = D                          # one head: the head stride is never used
            t.stride_s = ROW
            setattr(io.attn[k], which, t)
    assert check(io, cfg) == lt.LTXATTN_OK


# ------------------------------------------------ workspace of split parts
def test_split_parts_fit_the_workspace_at_any_size():
    """ltxattn_check_block also plans every kind for a 256-CU device and checks
    the rows its split parts need (video self-attention's incomplete last
    round, v2a's key ranges) against the workspace a handle has: over a sweep
    of shapes up to and past the headline sizes, every request fits."""
    import numpy as np
    rng = np.random.default_rng(5)
    shapes = [(1, 32, 128, 15360, 128, 126), (2, 32, 128, 15360, 128, 126), (1, 32, 128, 27280, 256, 252),
              (1, 32, 128, 3840, 126, 126), (1, 8, 128, 9216, 640, 600), (1, 2, 128, 4096, 128, 128),
              (1, 1, 128, 1281, 64, 64), (4, 48, 128, 40000, 1024, 1000), (1, 256, 64, 5000, 8, 8)]
    for _ in range(60):
        D_ = int(rng.choice([64, 128]))
        La_ = int(rng.integers(1, 1200))
        shapes.append((int(rng.integers(1, 5)), int(rng.integers(1, 65)), D_, int(rng.integers(1, 40001)),
                       La_, int(rng.integers(1, La_ + 1))))
    base, win = 1 << 44, 1 << 38
    for B_, H_, D_, Sv_, La_, Lk_ in shapes:
        row = H_ * D_
        def t(i, S):
            return lt.ltxattn_tensor(base + i * win, S * row, row, D_)
        io = lt.ltxattn_block_io()
        io.batch, io.video_len, io.audio_len, io.audio_kv_len = B_, Sv_, La_, Lk_
        vq, vk, vv, aq, ak, av = t(0, Sv_), t(1, Sv_), t(2, Sv_), t(3, La_), t(4, La_), t(5, La_)
        io.attn[0] = lt.ltxattn_attn_io(vq, vk, vv, t(6, Sv_))
        io.attn[1] = lt.ltxattn_attn_io(aq, ak, av, t(7, La_))
        io.attn[2] = lt.ltxattn_attn_io(vq, ak, av, t(8, Sv_))
        io.attn[3] = lt.ltxattn_attn_io(aq, vk, vv, t(9, La_))
        cfg = lt.ltxattn_config(0, H_, D_, B_, Sv_, La_)
        assert lt.ltxattn_check_block(cfg, io) == lt.LTXATTN_OK, (B_, H_, D_, Sv_, La_, Lk_)


# ------------------------------------------- QK-norm + rotary prologue
def _prologue(base=1 << 41):
    """A prologue whose six arrays are 16-byte aligned fake addresses."""
    return lt.ltxattn_qk_prologue(base, base + 4096, base + 8192, base + 12288, base + 16384, base + 20480,
                                  1e-6, lt.LTXATTN_ROPE_HALF)


CFG_PRO = lt.ltxattn_config(0, H, D, B, Sv, La, 1)


def test_prologue_accepted_with_workspace_only():
    io = make_io()
    for k in range(4):
        io.attn[k].prologue = _prologue()
    assert check(io, CFG_PRO) == lt.LTXATTN_OK
    assert check(io, CFG) == lt.LTXATTN_ERR_UNSUPPORTED        # handle without the key workspace
    io.attn[2].prologue = lt.ltxattn_qk_prologue()             # q_weight NULL: no prologue for a2v
    assert check(io, CFG_PRO) == lt.LTXATTN_OK


@pytest.mark.parametrize("kind", range(4))
@pytest.mark.parametrize("mutate", ["null", "misaligned", "eps_zero", "eps_negative", "eps_inf", "eps_nan",
                                    "pairing"])
def test_bad_prologue(kind, mutate):
    fields = ["k_weight", "q_cos", "q_sin", "k_cos", "k_sin"]
    cases = []
    if mutate in ("null", "misaligned"):
        for f in fields:
            p = _prologue()
            setattr(p, f, None if mutate == "null" else getattr(p, f) + 4)
            cases.append(p)
        if mutate == "misaligned":
            p = _prologue()
            p.q_weight += 8
            cases.append(p)
    else:
        p = _prologue()
        if mutate == "pairing":
            p.pairing = 2
        else:
            p.eps = {"eps_zero": 0.0, "eps_negative": -1e-6, "eps_inf": float("inf"), "eps_nan": float("nan")}[mutate]
        cases.append(p)
    for p in cases:
        io = make_io()
        io.attn[kind].prologue = p
        assert check(io, CFG_PRO) == lt.LTXATTN_ERR_INVALID_ARG, (kind, mutate)
