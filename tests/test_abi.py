"""C-ABI tests that need no GPU: the library loads, exports every function
include/lorabwd.h declares, and rejects bad arguments with the documented
status codes before any HIP call.

Every call below carries at least one invalid argument, so none reaches a
kernel launch (the fake pointers are never dereferenced).
"""
import ctypes
import os
import re

import pytest

import layer_backward_pass_amd as lbp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lorabwd.h")

OK, ENULL, ESHAPE, EALIGN, EDTYPE, EWS, ESTEP, EALIAS, EHIP, EARG = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9

# fake, 16-byte-aligned, non-overlapping "device" addresses (never touched)
BASE = 1 << 40
SPAN = 1 << 32


def fake(i):
    return BASE + i * SPAN


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(lbp.lib_path()):
        import __graft_entry__
        __graft_entry__.build()
    return lbp.load_library()


def declared_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(lorabwd_\w+)\s*\(", src, re.M)))


def test_header_declares_the_six_entry_points():
    names = declared_functions()
    for f in ("lorabwd_attn_backward", "lorabwd_ffn_backward", "lorabwd_rmsnorm_backward",
              "lorabwd_rope_backward", "lorabwd_lora_grad_adamw", "lorabwd_layer_backward"):
        assert f in names


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert set(lbp.EXPORTS) <= set(names)


def test_status_strings_and_version(lib):
    assert lib.lorabwd_abi_version() == 6
    for code in (OK, ENULL, ESHAPE, EALIGN, EDTYPE, EWS, ESTEP, EALIAS, EHIP, EARG):
        s = lib.lorabwd_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.lorabwd_status_string(12345).decode() == "unknown status"


# ---------------------------------------------------------------- RMSNorm
def test_rmsnorm_validation(lib):
    f = lib.lorabwd_rmsnorm_backward
    x, g, dy, dx = fake(0), fake(1), fake(2), fake(3)
    assert f(4, 64, x, g, dy, dx, 1e-6, 0, 7, None) == EDTYPE
    assert f(4, 60, x, g, dy, dx, 1e-6, 0, 0, None) == ESHAPE       # n % 8
    assert f(-1, 64, x, g, dy, dx, 1e-6, 0, 0, None) == ESHAPE
    assert f(4, 64, x, g, dy, dx, -1.0, 0, 0, None) == EARG
    assert f(4, 64, x, g, dy, dx, float("nan"), 0, 0, None) == EARG
    assert f(4, 64, x, g, dy, dx, 1e-6, 2, 0, None) == EARG
    assert f(4, 64, None, g, dy, dx, 1e-6, 0, 0, None) == ENULL
    assert f(4, 64, x + 4, g, dy, dx, 1e-6, 0, 0, None) == EALIGN
    assert f(4, 64, x, g, dy, dy + 16, 1e-6, 0, 0, None) == EALIAS   # partial overlap
    assert f(4, 64, x, g, dy, x, 1e-6, 0, 0, None) == EALIAS         # dx over x
    assert f(0, 64, None, None, None, None, 1e-6, 0, 0, None) == OK  # empty: no-op


def test_rope_validation(lib):
    f = lib.lorabwd_rope_backward
    a, b = fake(0), fake(1)
    assert f(2, 4, 24, a, b, 0, 1e4, None) == ESHAPE    # head_dim not supported
    assert f(2, 0, 16, a, b, 0, 1e4, None) == ESHAPE
    assert f(2, 4, 16, a, b, -1, 1e4, None) == ESHAPE
    assert f(2, 4, 16, a, b, 0, 0.0, None) == EARG
    assert f(2, 4, 16, None, b, 0, 1e4, None) == ENULL
    assert f(2, 4, 16, a, a + 64, 0, 1e4, None) == EALIAS
    assert f(2, 4, 16, a, b + 8, 0, 1e4, None) == EALIGN
    assert f(0, 4, 16, None, None, 0, 1e4, None) == OK


def test_attn_validation(lib):
    f = lib.lorabwd_attn_backward
    p = [fake(i) for i in range(8)]
    ws = lib.lorabwd_attn_workspace_size(64, 64, 4, 2, 64, 0)
    assert ws > 0

    def call(s_q=64, s_kv=64, hq=4, hkv=2, d=64, dctx=p[0], P=p[1], K=p[2], V=p[3], ctx=p[4],
             dq=p[5], dv=p[6], scale=0.125, causal=1, dt=0, w=p[7], wsb=ws):
        return f(s_q, s_kv, hq, hkv, d, dctx, P, K, V, ctx, dq, dv, scale, causal, dt, w, wsb, None)
    assert call(hq=4, hkv=3) == ESHAPE              # Hq % Hkv
    assert call(d=48) == ESHAPE
    assert call(s_q=65, s_kv=64) == ESHAPE          # causal needs s_q <= s_kv
    assert call(dt=3) == EDTYPE
    assert call(causal=2) == EARG
    assert call(scale=float("inf")) == EARG
    assert call(K=None) == ENULL
    assert call(dq=None) == ENULL
    assert call(V=p[3] + 2) == EALIGN
    assert call(dq=p[1]) == EALIAS                  # dq over P
    assert call(dv=p[5] + 256) == EALIAS            # dv over dq
    assert call(wsb=ws - 1) == EWS
    assert call(w=None) == EWS
    assert call(s_q=0, dv=None) == OK               # nothing to do


def test_ffn_validation(lib):
    f = lib.lorabwd_ffn_backward
    p = [fake(i) for i in range(14)]
    ws = lib.lorabwd_ffn_workspace_size(16, 64, 256, 0)
    assert ws > 0

    def call(rows=16, dim=64, ffn=256, act=0, d_out=p[0], wd=p[1], wg=p[2], wu=p[3], g=p[4],
             u=p[5], hp=None, gs=None, r1=p[6], gf=p[7], dres=p[8], eps=1e-6, dt=0, w=p[9],
             wsb=ws):
        return f(rows, dim, ffn, act, d_out, wd, wg, wu, g, u, hp, gs, r1, gf, dres, eps, dt, w,
                 wsb, None)
    assert call(act=5) == EDTYPE
    assert call(dt=9) == EDTYPE
    assert call(ffn=250) == ESHAPE
    assert call(eps=-1.0) == EARG
    assert call(wg=None) == ENULL
    assert call(hp=p[10]) == ENULL                  # sub-norm input without its gamma
    assert call(g=p[4] + 4) == EALIGN
    assert call(dres=p[0] + 16) == EALIAS           # partial overlap with d_out
    assert call(dres=p[6]) == EALIAS                # over resid1
    assert call(wsb=ws - 256) == EWS
    assert call(w=None) == EWS
    assert call(rows=0) == OK


def test_lora_validation(lib):
    f = lib.lorabwd_lora_grad_adamw
    p = [fake(i) for i in range(13)]
    ws = lib.lorabwd_lora_workspace_size(16, 64, 64, 4)

    def call(rows=16, i=64, o=64, r=4, dy=p[0], x=p[1], h=p[2], A=p[3], B=p[4], ma=p[5], va=p[6],
             mb=p[7], vb=p[8], ga=None, gb=None, gn=None, alpha=8.0, lra=1e-4, lrb=1.6e-3,
             b1=0.9, b2=0.999, eps=1e-8, wd=0.01, step=1, dt=0, w=p[9], wsb=ws):
        return f(rows, i, o, r, dy, x, h, A, B, ma, va, mb, vb, ga, gb, gn, alpha, lra, lrb, b1, b2,
                 eps, wd, step, dt, w, wsb, None)
    assert call(step=0) == ESTEP
    assert call(r=0) == ESHAPE
    assert call(r=65) == ESHAPE
    assert call(dt=2) == EDTYPE
    assert call(b1=1.0) == EARG
    assert call(lra=float("nan")) == EARG
    assert call(B=None) == ENULL
    assert call(dy=None) == ENULL
    assert call(ma=p[5] + 8) == EALIGN
    assert call(va=p[5]) == EALIAS                  # v_a over m_a
    assert call(ga=p[0]) == EALIAS                  # grad_a over dy
    assert call(gn=p[3] + 16) == EALIAS             # gnorm inside A
    assert call(wsb=ws - 1) == EWS


def test_layer_validation(lib):
    d = lbp.make_desc(16, 16, 64, 256, 4, 2, 16, lora_alpha=8.0)
    ws = lib.lorabwd_layer_workspace_size(ctypes.byref(d))
    assert ws > 0
    bad = lbp.make_desc(16, 16, 64, 256, 4, 3, 16)
    assert lib.lorabwd_layer_workspace_size(ctypes.byref(bad)) == 0
    w = lbp.LayerWeights(*[fake(i) for i in range(4)], fake(4), None, None)
    a = lbp.LayerSaved(*[fake(10 + i) for i in range(11)])
    st = lbp.LoraState(4, *[fake(30 + i) for i in range(6)])
    hp = lbp.AdamW(1e-4, 1.6e-3, 0.9, 0.999, 1e-8, 0.01, 0)
    f = lib.lorabwd_layer_backward
    r = ctypes.byref
    dh = fake(50)
    assert f(r(bad), r(w), r(a), None, None, None, None, dh, None, None, None, fake(60), ws, None) == ESHAPE
    assert f(r(d), r(w), r(a), r(st), None, r(hp), None, dh, None, None, None, fake(60), ws, None) == ESTEP
    hp.step = 1
    assert f(r(d), r(w), r(a), r(st), None, None, None, dh, None, None, None, fake(60), ws, None) == ENULL
    sub = lbp.make_desc(16, 16, 64, 256, 4, 2, 16, sub_norms=True)
    assert f(r(sub), r(w), r(a), None, None, None, None, dh, None, None, None, fake(60), ws, None) == ENULL
    assert f(r(d), r(w), r(a), r(st), None, r(hp), None, dh, None, None, None, fake(60), ws - 1, None) == EWS
    assert f(r(d), r(w), r(a), r(st), None, r(hp), None, dh, fake(50) + 64, None, None, fake(60), ws,
             None) == EALIAS
    # a separate input must not overlap the output
    assert f(r(d), r(w), r(a), None, None, None, fake(50) + 256, dh, None, None, None, fake(60), ws,
             None) == EALIAS
    qn = lbp.make_desc(16, 16, 64, 256, 4, 2, 16, qk_norm=True)  # QK-norm without gamma_q
    assert f(r(qn), r(w), r(a), None, None, None, None, dh, None, None, None, fake(60), ws, None) == ENULL
    qn.qk_norm, qn.input_grad = 0, 2
    assert f(r(qn), r(w), r(a), None, None, None, None, dh, None, None, None, fake(60), ws, None) == EARG
    d.kv_len = 8                                  # kv_len < seq
    assert f(r(d), r(w), r(a), None, None, None, None, dh, None, None, None, fake(60), ws, None) == ESHAPE


def far(i):
    # fake addresses 4 TiB apart, for the multi-gigabyte shapes below
    return (1 << 46) + i * (1 << 42)


def test_size_limits_and_kernel_limits_are_validated(lib):
    # Row counts and feature sizes above 2^20, more than 4096 heads, and
    # shapes within those caps that a kernel still cannot take (a 1 GiB buffer
    # range, the single-token attention's LDS) are refused with ESHAPE by the
    # validation and checking pass, before any HIP call: with no GPU here a
    # call that got as far as a launch would report EHIP instead.
    p = [far(i) for i in range(13)]
    big = (1 << 20) + 8
    f = lib.lorabwd_rmsnorm_backward
    assert f(big, 64, p[0], p[1], p[2], p[3], 1e-6, 0, 0, None) == ESHAPE
    assert f(4, big, p[0], p[1], p[2], p[3], 1e-6, 0, 0, None) == ESHAPE
    assert lib.lorabwd_rope_backward(big, 4, 16, p[0], p[1], 0, 1e4, None) == ESHAPE
    assert lib.lorabwd_rope_backward(4, 8192, 128, p[0], p[1], 0, 1e4, None) == ESHAPE

    def attn(s_q, s_kv, hq, hkv, d):
        ws = lib.lorabwd_attn_workspace_size(s_q, s_kv, hq, hkv, d, 0)
        return lib.lorabwd_attn_backward(s_q, s_kv, hq, hkv, d, p[0], p[1], p[2], p[3], p[4],
                                         p[5], p[6], 0.1, 1, 0, p[7], max(ws, 256), None)
    assert attn(4, big, 4, 2, 64) == ESHAPE              # rows cap
    assert attn(1, 4096, 8192, 1024, 16) == ESHAPE       # more than 4096 heads
    assert attn(1, 4096, 1024, 1024, 128) == ESHAPE      # K/V cache range of 2 GiB

    def ffn(rows, dim, ffn_dim):
        ws = lib.lorabwd_ffn_workspace_size(rows, dim, ffn_dim, 0)
        return lib.lorabwd_ffn_backward(rows, dim, ffn_dim, 0, p[0], p[1], p[2], p[3], p[4], p[5],
                                        None, None, p[6], p[7], p[8], 1e-6, 0, p[9],
                                        max(ws, 256), None)
    assert ffn(4, big, 1024) == ESHAPE
    assert ffn(1, 1 << 20, 1024) == ESHAPE               # one GEMV chunk of weight rows > 1 GiB
    assert ffn(1, 1024, 1 << 20) == ESHAPE

    def lora(rows, out_dim):
        ws = lib.lorabwd_lora_workspace_size(rows, 64, out_dim, 4)
        return lib.lorabwd_lora_grad_adamw(rows, 64, out_dim, 4, p[0], p[1], p[2], p[3], p[4],
                                           p[5], p[6], p[7], p[8], None, None, None, 8.0, 1e-4,
                                           1.6e-3, 0.9, 0.999, 1e-8, 0.01, 1, 0, p[9], ws, None)
    assert lora(big, 64) == ESHAPE
    assert lora(512, 1 << 20) == ESHAPE                  # a row slice of dy > 1 GiB

    # a one-token layer whose cache range is beyond the kernels' limit
    d = lbp.make_desc(1, 4096, 1024, 2048, 1024, 1024, 128, act=lbp.ACT_RELU2, pos0=4095)
    ws = lib.lorabwd_layer_workspace_size(ctypes.byref(d))
    w = lbp.LayerWeights(*[far(i) for i in range(4)], far(4), None, None)
    a = lbp.LayerSaved(*[far(10 + i) for i in range(11)])
    r = ctypes.byref
    assert lib.lorabwd_layer_backward(r(d), r(w), r(a), None, None, None, None, far(40), None,
                                      None, None, far(50), ws, None) == ESHAPE
    d.seq, d.kv_len = big, big
    assert lib.lorabwd_layer_backward(r(d), r(w), r(a), None, None, None, None, far(40), None,
                                      None, None, far(50), ws, None) == ESHAPE


def test_noalloc_validation(lib):
    # the allocation-free layer: a layer whose workspace exceeds the static
    # scratch is refused with EWS before any HIP call; invalid descriptors
    # with their usual codes
    assert lbp.NOALLOC_SCRATCH_BYTES == 16 << 20
    big = lbp.make_desc(512, 512, 2560, 9728, 32, 8, 128, lora_alpha=32.0)
    assert lib.lorabwd_layer_workspace_size(ctypes.byref(big)) > lbp.NOALLOC_SCRATCH_BYTES
    w = lbp.LayerWeights(*[far(i) for i in range(4)], far(4), None, None)
    a = lbp.LayerSaved(*[far(10 + i) for i in range(11)])
    r = ctypes.byref
    f = lib.lorabwd_layer_backward_noalloc
    assert f(r(big), r(w), r(a), None, None, None, None, far(40), None, None, None, None) == EWS
    bad = lbp.make_desc(16, 16, 64, 256, 4, 3, 16)
    assert f(r(bad), r(w), r(a), None, None, None, None, far(40), None, None, None, None) == ESHAPE
    d = lbp.make_desc(16, 16, 64, 256, 4, 2, 16)
    assert f(r(d), r(w), r(a), None, None, None, None, None, None, None, None, None) == ENULL


def test_pack_ternary_validation(lib):
    f = lib.lorabwd_pack_ternary
    assert lib.lorabwd_ternary_packed_bytes(3, 16) == 12
    assert lib.lorabwd_ternary_packed_bytes(3, 12) == 0          # cols % 8
    assert f(3, 12, fake(0), 0, fake(1), None) == ESHAPE
    assert f(3, 16, fake(0), 5, fake(1), None) == EDTYPE
    assert f(3, 16, None, 0, fake(1), None) == ENULL
    assert f(3, 16, fake(0) + 4, 0, fake(1), None) == EALIGN
    assert f(3, 16, fake(0), 0, fake(0) + 16, None) == EALIAS     # output over the input
    assert f(0, 16, None, 0, None, None) == OK
    # packed weights are for the single-token layer only, with finite scales
    d = lbp.make_desc(16, 16, 64, 256, 4, 2, 16, weight_format=1)
    w = lbp.LayerWeights(*[fake(i) for i in range(4)], fake(4), *([None] * 8),
                         *([0.02] * 4))
    a = lbp.LayerSaved(*[fake(10 + i) for i in range(11)])
    r = ctypes.byref
    ws = 1 << 30
    fl = lib.lorabwd_layer_backward
    assert fl(r(d), r(w), r(a), None, None, None, None, fake(50), None, None, None, fake(60), ws,
              None) == ESHAPE
    one = lbp.make_desc(1, 64, 64, 256, 4, 2, 16, act=lbp.ACT_RELU2, weight_format=1, pos0=63)
    w.scale_up = float("nan")
    assert fl(r(one), r(w), r(a), None, None, None, None, fake(50), None, None, None, fake(60), ws,
              None) == EARG


def test_lm_head_validation(lib):
    f = lib.lorabwd_lm_head_backward
    p = [fake(i) for i in range(12)]
    S, H, V = 16, 64, 1000
    ws = lib.lorabwd_lm_head_workspace_size(S, H, V)
    assert ws >= S * V * 4 + S * 4
    assert lib.lorabwd_lm_head_workspace_size(S, H, 1002) == 0     # vocab % 4
    assert lib.lorabwd_lm_head_workspace_size(S, 60, V) == 0       # hidden % 8
    assert lib.lorabwd_lm_head_workspace_size(S, H, (1 << 20) + 4) == 0

    def call(rows=S, hid=H, voc=V, h=p[0], z=p[1], lab=p[2], W=p[3], m=p[4], v=p[5], gh=p[6],
             loss=p[7], gw=None, lr=1e-3, b1=0.9, b2=0.999, eps=1e-8, wd=0.01, step=1, w=p[9],
             wsb=ws):
        return f(rows, hid, voc, h, z, lab, W, m, v, gh, loss, gw, lr, b1, b2, eps, wd, step, w,
                 wsb, None)
    assert call(voc=1002) == ESHAPE
    assert call(voc=0) == ESHAPE
    assert call(hid=60) == ESHAPE
    assert call(rows=-1) == ESHAPE
    assert call(rows=(1 << 20) + 1) == ESHAPE
    assert call(step=0) == ESTEP
    assert call(b2=1.0) == EARG
    assert call(lr=float("inf")) == EARG
    assert call(W=None) == ENULL
    assert call(loss=None) == ENULL
    assert call(lab=None) == ENULL
    assert call(h=p[0] + 8) == EALIGN
    assert call(lab=p[2] + 2) == EALIGN
    assert call(gh=p[0]) == EALIAS                  # grad_hidden over h
    assert call(m=p[3] + 64) == EALIAS              # m inside W
    assert call(loss=p[1] + 16) == EALIAS           # loss inside the logits
    assert call(gw=p[5]) == EALIAS                  # grad_w over v
    assert call(wsb=ws - 1) == EWS
    assert call(w=None) == EWS
    # the timed variant validates the same way
    ft = lib.lorabwd_lm_head_backward_timed
    assert ft(S, H, V, *p[:8], None, 1e-3, 0.9, 0.999, 1e-8, 0.01, 0, p[9], ws, None, None, None,
              0, None) == ESTEP
    assert ft(S, H, V, *p[:8], None, 1e-3, 0.9, 0.999, 1e-8, 0.01, 1, p[9], ws, None, None, None,
              -1, None) == EARG


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(OSError):
        lbp.load_library(str(tmp_path / "missing.so"))
