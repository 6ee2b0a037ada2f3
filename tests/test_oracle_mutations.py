"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
the pins catch every one: a dropped term, a wrong sign, a wrong index, a
transposed operand, a wrong constant.

Each mutation rewrites one expression of oracle/backward.py, loads the result
as a throw-away module, and runs the pin checks against it; at least one check
must fail.
"""
import os
import types

import numpy as np
import pytest

import synth
from oracle import forward as F
from oracle import fd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "backward.py")
FWD_SRC = os.path.join(ROOT, "oracle", "forward.py")

MUTATIONS = [
    # (old, new) - each old string must occur in oracle/backward.py
    ("return (g - x * dot / (n * r * r)) / r", "return g / r"),                      # dropped term
    ("return (g - x * dot / (n * r * r)) / r", "return (g - x * dot / (n * r)) / r"),  # wrong power
    ("dx[..., half:] = -lo * s + hi * c", "dx[..., half:] = lo * s + hi * c"),      # sign
    ("dx[..., :half] = lo * c + hi * s", "dx[..., :half] = lo * c - hi * s"),       # forward rotation
    ("inv_freq = np.power(float(base), -2.0 * d / head_dim)",
     "inv_freq = np.power(float(base), -1.0 * d / head_dim)"),                      # constant
    ("return dh * up * 2.0 * r, dh * r * r", "return dh * up * r, dh * r * r"),     # factor 2
    ("dsilu = sig * (1.0 + gate - silu)", "dsilu = sig * (1.0 - silu)"),            # dropped term
    ("return P * (dA - delta)", "return P * dA"),                                    # no delta
    ("g = h // grp", "g = h % n_kv_heads"),                                          # GQA map
    ("dQ[:, h * D:(h + 1) * D] = scale * (dS @ Kg)", "dQ[:, h * D:(h + 1) * D] = dS @ Kg"),
    ("dV[:, g * D:(g + 1) * D] += P[h].T @ dC", "dV[:, g * D:(g + 1) * D] += P[h] @ dC"),
    ("g = s * (dy @ B)", "g = dy @ B"),                                              # dropped scaling
    ("dB = s * (dy.T @ h)", "dB = s * (h.T @ dy).T * 0 + s * (dy.T @ h) / 2"),       # halved
    ("v = beta2 * v + (1.0 - beta2) * g * g", "v = beta2 * v + (1.0 - beta2) * g"),
    ("p = p - lr * ((m * bc1) / (np.sqrt(v * bc2) + eps) + wd * p)",
     "p = p - lr * ((m * bc1) / (np.sqrt(v * bc2) + eps)) - wd * p"),               # decay not scaled by lr
    ("dh1 = d_out + rmsnorm_bwd(resid1, gamma_ffn, dn2, eps)",
     "dh1 = rmsnorm_bwd(resid1, gamma_ffn, dn2, eps)"),                              # dropped residual
    ("dn2 = dgate @ np.asarray(W_gate, np.float64) + dup @ np.asarray(W_up, np.float64)",
     "dn2 = dgate @ np.asarray(W_up, np.float64) + dup @ np.asarray(W_gate, np.float64)"),
    ("dq_pre = rope_bwd(dq, cfg.n_heads, cfg.head_dim, cfg.pos0 + np.arange(rows),",
     "dq_pre = rope_bwd(dq, cfg.n_heads, cfg.head_dim, np.arange(rows),"),           # positions
    ('res["gnorm_sq"] += float(np.sum(dA * dA))',
     'res["gnorm_sq"] += float(np.sum(dA * dA) + np.sum(dB * dB))'),                 # gnorm of B too
    ("dv[dv.shape[0] - rows:]", "dv[:rows]"),                                        # prefix rows
    ('dq_pre = head_rmsnorm_bwd(saved["q_raw"], cfg.n_heads, w["gamma_q"], dq_pre, cfg.eps)',
     'dq_pre = head_rmsnorm_bwd(saved["q_raw"], cfg.n_heads, w["gamma_k"], dq_pre, cfg.eps)'),
    ("dx = rmsnorm_bwd(x.reshape(rows, n_heads, -1), gamma,",
     "dx = rmsnorm_bwd(x.reshape(rows, -1, n_heads).transpose(0, 2, 1), gamma,"),     # head layout
    ("dK[:, g * D:(g + 1) * D] += scale * (dS.T @", "dK[:, g * D:(g + 1) * D] += (dS.T @"),  # scale
    ("kpos = cfg.pos0 - (L - S) + np.arange(L)", "kpos = cfg.pos0 + np.arange(L)"),  # key positions
    ("+ dv_cur @ np.asarray(w[\"W_v\"], np.float64))", ")"),                         # dropped dV term
    ("dxa = dxa + (float(cfg.alpha) / A.shape[0]) * ((dy @ Bm) @ A)", "dxa = dxa"),  # adapters
    ("dx = dh1 + rmsnorm_bwd(saved[\"x\"], w[\"gamma_attn\"], dxa, cfg.eps)",
     "dx = dh1 + dxa"),                                                              # no norm bwd
]


def _load_mutant(old, new, path=SRC):
    src = open(path).read()
    assert src.count(old) == 1, old
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new, 1), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _checks(B):
    """Pin checks that do not depend on which module is under test; each
    returns True when the module passes."""
    cfg = synth.get_config("tiny")
    out = []
    # golden-style closed forms
    x = np.array([[3.0, 4.0]])
    out.append(np.allclose(B.rmsnorm_bwd(x, np.ones(2), np.array([[1.0, 0.0]]), 0.0)[0],
                           [0.18101933598375617, -0.13576450198781713], atol=1e-15))
    out.append(np.allclose(B.rope_bwd(np.array([[1.0, 0, 0, 0]]), 1, 4, [1], 100.0)[0],
                           [np.cos(1.0), 0, -np.sin(1.0), 0], atol=1e-15))
    out.append(np.allclose(B.rope_bwd(np.array([[0, 0, 0, 1.0]]), 1, 4, [1], 100.0)[0],
                           [0, np.sin(0.1), 0, np.cos(0.1)], atol=1e-15))
    dg, du = B.relu2_mul_bwd(np.array([-1, 0, 0.5, 2.0]), np.array([3, 1, -2, 0.5]),
                             np.array([1, 1, 1, 2.0]))
    out.append(np.array_equal(dg, [0, 0, -2, 4]) and np.array_equal(du, [0, 0, 0.25, 8]))
    out.append(np.array_equal(B.softmax_bwd(np.array([0.5, 0.5, 0]), np.array([1.0, 3, 7])),
                              [-0.5, 0.5, 0]))
    p, m, v = B.adamw(0.5, 0.2, 0.0, 0.0, 1e-3, 0.9, 0.999, 1e-8, 0.01, 1)
    out.append(abs(p - 0.49899500004999997) < 1e-15 and abs(v - 4e-5) < 1e-18)
    # whole-layer finite differences (SwiGLU + LoRA)
    d = synth.draw_layer(cfg)
    w, saved, lora = F.make_layer(cfg, d)
    res = B.layer_bwd(cfg, w, saved, d["d_out"], lora)
    x0 = d["x"]

    def L(**kw):
        o, _ = F.layer_forward(cfg, w, kw.pop("x", x0), x_attn=x0, **kw)
        return float(np.sum(d["d_out"] * o))
    idx = range(0, x0.size, 37)
    num = fd.grad(lambda z: L(x=z, lora=lora), x0, idx=idx)
    out.append(fd.rel_err(res["d_hidden"].reshape(-1)[list(idx)], num.reshape(-1)[list(idx)]) < 1e-5)
    for k in ("A_q", "B_q", "A_v", "B_v"):
        def Lk(z, k=k):
            l2 = dict(lora)
            l2[k] = z
            return L(lora=l2)
        ii = range(0, lora[k].size, 5)
        num = fd.grad(Lk, lora[k], idx=ii, rel_step=1e-5)
        out.append(fd.rel_err(res["d" + k].reshape(-1)[list(ii)], num.reshape(-1)[list(ii)]) < 1e-5)
    # A-only gradient norm and the AdamW step-1 closed form on B (LoRA+)
    out.append(abs(res["gnorm_sq"] - float(np.sum(res["dA_q"] ** 2) + np.sum(res["dA_v"] ** 2)))
               <= 1e-15 * res["gnorm_sq"])
    g = res["dB_q"]
    b0 = np.asarray(lora["B_q"], np.float64)
    want = b0 - cfg.lr_b * (g / (np.abs(g) + cfg.adam_eps) + cfg.weight_decay * b0)
    out.append(np.allclose(res["B_q"], want, rtol=1e-13))
    # GQA attention FD with 4 query heads on 2 KV heads
    r = np.random.default_rng(3)
    q = r.standard_normal((5, 4 * 4))
    kk = r.standard_normal((5, 2 * 4))
    vv = r.standard_normal((5, 2 * 4))
    P, ctx = F.attention(q, kk, vv, 4, 2, 4, 0.5, True)
    dctx = r.standard_normal(ctx.shape)
    dq, dv = B.attention_bwd(dctx, P, kk, vv, 4, 2, 0.5)
    out.append(fd.rel_err(dq, fd.grad(lambda z: float(np.sum(dctx * F.attention(z, kk, vv, 4, 2, 4, 0.5, True)[1])), q)) < 1e-7)
    out.append(fd.rel_err(dv, fd.grad(lambda z: float(np.sum(dctx * F.attention(q, kk, z, 4, 2, 4, 0.5, True)[1])), vv)) < 1e-7)
    # decode-like layer (pos0 = 11, ReLU^2 x up, sub-norms): FD of dQpre and dX
    cd = synth.get_config("decode").with_(hidden=16, ffn=24, n_heads=2, n_kv_heads=1,
                                         head_dim=8, kv_len=12, pos0=11)
    dd = synth.draw_layer(cd)
    wd_, sd_, _ = F.make_layer(cd, dd)
    rd = B.layer_bwd(cd, wd_, sd_, dd["d_out"], None)

    def Ld(**kw):
        o, _ = F.layer_forward(cd, wd_, kw.pop("x", dd["x"]), x_attn=dd["x"], **kw)
        return float(np.sum(dd["d_out"] * o))
    out.append(fd.rel_err(rd["dq_pre"], fd.grad(lambda z: Ld(q_pre=z), sd_["q_pre"])) < 1e-5)
    out.append(fd.rel_err(rd["d_hidden"], fd.grad(lambda z: Ld(x=z), dd["x"])) < 1e-5)
    # the input gradient without the stop-gradient: FD of the layer in x,
    # plain and after a cached prefix with QK-norm
    for over in ({}, {"seq": 5, "kv_len": 11, "pos0": 6, "qk_norm": True}):
        ci = cfg.with_(input_grad=True, **over)
        di = synth.draw_layer(ci)
        wi, si, li = F.make_layer(ci, di)
        ri = B.layer_bwd(ci, wi, si, di["d_out"], li)

        def Li(z, ci=ci, wi=wi, li=li, di=di):
            o, _ = F.layer_forward(ci, wi, z, lora=li)
            return float(np.sum(di["d_out"] * o))
        out.append(fd.rel_err(ri["d_hidden"], fd.grad(Li, di["x"])) < 1e-5)
    # QK-norm: FD of dQpre with respect to the Q projection output
    cq = cfg.with_(qk_norm=True, pos0=5)
    dq_ = synth.draw_layer(cq)
    wq, sq, lq = F.make_layer(cq, dq_)
    rq = B.layer_bwd(cq, wq, sq, dq_["d_out"], lq)

    def Lq(z):
        o, _ = F.layer_forward(cq, wq, dq_["x"], lora=lq, q_pre=z)
        return float(np.sum(dq_["d_out"] * o))
    out.append(fd.rel_err(rq["dq_pre"], fd.grad(Lq, sq["q_raw"])) < 1e-5)
    # a chunk after a cached prefix: the V adapter sees the chunk's dV rows
    cp = cfg.with_(seq=5, kv_len=11, pos0=6)
    dp = synth.draw_layer(cp)
    wp, sp, lp = F.make_layer(cp, dp)
    rp = B.layer_bwd(cp, wp, sp, dp["d_out"], lp)

    def Lp(z):
        l2 = dict(lp)
        l2["B_v"] = z
        o, _ = F.layer_forward(cp, wp, dp["x"], lora=l2)
        return float(np.sum(dp["d_out"] * o))
    out.append(fd.rel_err(rp["dB_v"], fd.grad(Lp, lp["B_v"], rel_step=1e-5)) < 1e-5)
    # multi-step AdamW v update against its definition through a second step
    p2, m2, v2 = B.adamw(np.array([1.0]), np.array([0.5]), np.array([0.1]), np.array([0.04]),
                         1e-3, 0.9, 0.999, 1e-8, 0.0, 2)
    out.append(abs(v2[0] - (0.999 * 0.04 + 0.001 * 0.25)) < 1e-15)
    return out


def test_unmutated_oracle_passes_all_checks():
    from oracle import backward as B
    assert all(_checks(B))


@pytest.mark.parametrize("i", range(len(MUTATIONS)))
def test_mutation_is_caught(i):
    old, new = MUTATIONS[i]
    B = _load_mutant(old, new)
    try:
        ok = all(_checks(B))
    except (ValueError, IndexError):  # a shape error also exposes the mistake
        ok = False
    assert not ok, "mutation not caught: %r -> %r" % (old, new)


# Mutations of oracle/forward.py context() (the apply step that builds ctx for
# the whole-stack parity inputs); each old string occurs once in that file.
CONTEXT_MUTATIONS = [
    ("        g = h // grp\n        ctx[:, h * D:(h + 1) * D] = P[h] @ V[:, g * D:(g + 1) * D]\n    return ctx",
     "        g = h % n_kv_heads\n        ctx[:, h * D:(h + 1) * D] = P[h] @ V[:, g * D:(g + 1) * D]\n    return ctx"),
    ("        ctx[:, h * D:(h + 1) * D] = P[h] @ V[:, g * D:(g + 1) * D]\n    return ctx",
     "        ctx[:, h * D:(h + 1) * D] = P[h].T @ V[:, g * D:(g + 1) * D]\n    return ctx"),
    ("    grp = n_heads // n_kv_heads\n    ctx = np.zeros((P.shape[1], n_heads * D))",
     "    grp = n_kv_heads\n    ctx = np.zeros((P.shape[1], n_heads * D))"),
]


def _context_checks(Fm):
    """The pins of test_oracle_pins.test_context_is_the_apply_step, run on
    the module under test (square and GQA 6:2 cases)."""
    ok = []
    for s_q, s_kv, Hq, Hkv in ((5, 5, 4, 2), (4, 4, 6, 2)):
        r = np.random.default_rng(5 + Hq)
        D = 3
        P = r.random((Hq, s_q, s_kv))
        V = r.standard_normal((s_kv, Hkv * D))
        ctx = Fm.context(P, V, Hq, Hkv)
        loops = np.zeros((s_q, Hq * D))
        for h in range(Hq):
            g = h // (Hq // Hkv)
            for i in range(s_q):
                for d in range(D):
                    loops[i, h * D + d] = sum(P[h, i, j] * V[j, g * D + d] for j in range(s_kv))
        ok.append(np.allclose(ctx, loops, rtol=1e-13, atol=1e-15))
    return ok


def test_unmutated_context_passes():
    assert all(_context_checks(F))


@pytest.mark.parametrize("i", range(len(CONTEXT_MUTATIONS)))
def test_context_mutation_is_caught(i):
    old, new = CONTEXT_MUTATIONS[i]
    Fm = _load_mutant(old, new, FWD_SRC)
    try:
        ok = all(_context_checks(Fm))
    except (ValueError, IndexError):
        ok = False
    assert not ok, "mutation not caught: %r -> %r" % (old, new)


# Mutations of oracle/bitlinear.py (the packed ternary weight format).
BL_SRC = os.path.join(ROOT, "oracle", "bitlinear.py")
BITLINEAR_MUTATIONS = [
    ("CODE = {0: 0b00, 1: 0b01, -1: 0b11}", "CODE = {0: 0b00, 1: 0b01, -1: 0b10}"),     # code of -1
    ("out[r, c // 4] |= np.uint8(code << (2 * (c % 4)))",
     "out[r, c // 4] |= np.uint8(code << (2 * (3 - c % 4)))"),                        # bit order
    ("return float(scale) * (np.asarray(dy, np.float64) @ unpack_ternary(packed, cols))",
     "return (np.asarray(dy, np.float64) @ unpack_ternary(packed, cols))"),            # scale dropped
]


def _bitlinear_checks(M):
    g = {}
    with open(os.path.join(ROOT, "tests", "golden", "ternary_pack_example.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = (s.strip() for s in line.split("=", 1))
                g[k] = np.array([float(t) for t in v.split()])
    w = np.stack([g["w_row0"], g["w_row1"]])
    ok = [np.array_equal(M.pack_ternary(w).reshape(-1), g["packed"].astype(np.uint8))]
    r = np.random.default_rng(9)
    t = r.integers(-1, 2, size=(5, 16))
    dy = r.standard_normal((2, 5))
    ok.append(np.allclose(M.bitlinear_t(dy, M.pack_ternary(0.02 * t), 0.02, 16), dy @ (0.02 * t)))
    return ok


def test_unmutated_bitlinear_passes():
    from oracle import bitlinear
    assert all(_bitlinear_checks(bitlinear))


@pytest.mark.parametrize("i", range(len(BITLINEAR_MUTATIONS)))
def test_bitlinear_mutation_is_caught(i):
    old, new = BITLINEAR_MUTATIONS[i]
    M = _load_mutant(old, new, BL_SRC)
    try:
        ok = all(_bitlinear_checks(M))
    except (ValueError, IndexError, KeyError):
        ok = False
    assert not ok, "mutation not caught: %r -> %r" % (old, new)


# Mutations of oracle/lmhead.py.
LM_SRC = os.path.join(ROOT, "oracle", "lmhead.py")
LM_MUTATIONS = [
    ("dlogits = (p - y) / S", "dlogits = p - y"),                                # mean dropped
    ("dlogits = (p - y) / S", "dlogits = (y - p) / S"),                          # sign
    ("    p[~ok] = 0.0\n", ""),                                                  # ignored rows kept
    ("S = max(len(rows), 1)", "S = max(len(ok), 1)"),                            # mean over all rows
    ("dW = dlogits.T @ h", "dW = dlogits.T @ h[::-1]"),                          # rows paired wrongly
    ("\n    lse = mx + np.log(np.exp(z - mx[:, None]).sum(axis=-1))",
     "\n    lse = np.log(np.exp(z - mx[:, None]).sum(axis=-1))"),                 # max dropped
]


def _lm_checks(M):
    from oracle import fd as FD
    r = np.random.default_rng(4)
    h = r.standard_normal((3, 5))
    W = 0.3 * r.standard_normal((7, 5))
    labels = np.array([1, 6, 1, -100])
    h = np.vstack([h, r.standard_normal((1, 5))])
    res = M.lm_head_bwd(h, h @ W.T, labels, W, np.zeros_like(W), np.zeros_like(W),
                        1e-3, 0.9, 0.999, 1e-8, 0.01, 1)
    loss = lambda h_, W_: float(np.mean(  # noqa: E731  (the labelled rows 0..2)
        np.log(np.exp(h_[:3] @ W_.T).sum(-1)) - (h_[:3] @ W_.T)[np.arange(3), labels[:3]]))
    return [abs(res["loss"] - loss(h, W)) < 1e-12,
            FD.rel_err(res["grad_hidden"], FD.grad(lambda z: loss(z, W), h)) < 1e-8,
            FD.rel_err(res["dW"], FD.grad(lambda z: loss(h, z), W)) < 1e-8]


def test_unmutated_lmhead_passes():
    from oracle import lmhead
    assert all(_lm_checks(lmhead))


@pytest.mark.parametrize("i", range(len(LM_MUTATIONS)))
def test_lmhead_mutation_is_caught(i):
    old, new = LM_MUTATIONS[i]
    src = open(LM_SRC).read().replace("from .backward import adamw", "from oracle.backward import adamw")
    assert src.count(old) == 1, old
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new, 1), "oracle_mutant", "exec"), mod.__dict__)
    try:
        ok = all(_lm_checks(mod))
    except (ValueError, IndexError):
        ok = False
    assert not ok, "mutation not caught: %r -> %r" % (old, new)
