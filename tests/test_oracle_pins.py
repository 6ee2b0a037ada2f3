"""Pins of the float64 oracle against what the pages and mathematics fix.

Each test checks the oracle against something other than itself: hand-worked
examples of the pages' closed forms (tests/golden), central finite differences
of the forward it differentiates, invariants (softmax-backward rows sum to
zero, RoPE is a rotation), textbook Jacobians, and library routines
(torch.optim.AdamW in float64 on the CPU).
"""
import os

import numpy as np
import pytest

import synth
from oracle import backward as B
from oracle import forward as F
from oracle import fd

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = (s.strip() for s in line.split("=", 1))
            vals = [float(t) for t in v.split()]
            out[k] = np.array(vals) if len(vals) > 1 else vals[0]
    return out


def rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- RMSNorm
def test_rmsnorm_bwd_golden():
    g = load_golden("rmsnorm_bwd_example.txt")
    dx = B.rmsnorm_bwd(g["x"][None], g["gamma"], g["dy"][None], g["eps"])[0]
    np.testing.assert_allclose(dx, g["dx"], rtol=0, atol=1e-15)


@pytest.mark.parametrize("n,eps", [(1, 0.25), (2, 1e-6), (7, 1e-6), (64, 1e-6), (64, 0.5)])
def test_rmsnorm_bwd_fd(n, eps):
    # (n = 1 with a tiny eps is nearly constant, so it is probed with a large eps)
    r = rng(n)
    x = r.standard_normal((3, n))
    gam = 1 + 0.1 * r.standard_normal(n)
    w = r.standard_normal((3, n))
    an = B.rmsnorm_bwd(x, gam, w, eps)
    num = fd.grad(lambda z: float(np.sum(w * F.rmsnorm(z, gam, eps))), x)
    assert fd.rel_err(an, num) < 1e-7


def test_rmsnorm_bwd_textbook_jacobian():
    # gamma = 1: dx = J^T dy with J = (I - x x^T / (n r^2)) / r (symmetric)
    r = rng(1)
    n, eps = 9, 1e-3
    x = r.standard_normal(n)
    dy = r.standard_normal(n)
    rr = np.sqrt(np.mean(x * x) + eps)
    J = (np.eye(n) - np.outer(x, x) / (n * rr * rr)) / rr
    np.testing.assert_allclose(B.rmsnorm_bwd(x[None], np.ones(n), dy[None], eps)[0],
                               J.T @ dy, rtol=1e-13, atol=1e-14)


def test_rmsnorm_bwd_scale_invariance_identity():
    # x . dx = eps * <dy*gamma, x> / r^3  (-> 0 as eps -> 0)
    r = rng(2)
    x = r.standard_normal((4, 33))
    gam = 1 + 0.1 * r.standard_normal(33)
    dy = r.standard_normal((4, 33))
    for eps in (1e-6, 0.3):
        dx = B.rmsnorm_bwd(x, gam, dy, eps)
        rr = np.sqrt(np.mean(x * x, -1) + eps)
        want = eps * np.sum(dy * gam * x, -1) / rr ** 3
        np.testing.assert_allclose(np.sum(x * dx, -1), want, rtol=1e-9, atol=1e-15)


# ---------------------------------------------------------------- RoPE
def test_rope_bwd_golden():
    g = load_golden("rope_bwd_example.txt")
    D = int(g["head_dim"])
    for tag in ("a", "b"):
        dx = B.rope_bwd(g["dy_" + tag][None], 1, D, [int(g["pos"])], g["base"])[0]
        np.testing.assert_allclose(dx, g["dx_" + tag], rtol=0, atol=1e-15)


def test_rope_theta_closed_form():
    th = B.rope_theta([0, 1, 3], 8, 10000.0)
    want = np.array([[p * 10000.0 ** (-2 * d / 8) for d in range(4)] for p in (0, 1, 3)])
    np.testing.assert_allclose(th, want, rtol=1e-15)
    assert th[2, 0] == 3.0 and th[1, 2] == pytest.approx(1e-2, rel=1e-14)


def test_rope_bwd_inverse_and_norm():
    r = rng(3)
    Hh, D = 3, 16
    y = r.standard_normal((40, Hh * D))
    pos = np.arange(40) + 1000
    x = B.rope_bwd(y, Hh, D, pos, 10000.0)
    np.testing.assert_allclose(F.rope(x, Hh, D, pos, 10000.0), y, rtol=0, atol=1e-12)
    nx = np.linalg.norm(x.reshape(40, Hh, D), axis=-1)
    ny = np.linalg.norm(y.reshape(40, Hh, D), axis=-1)
    np.testing.assert_allclose(nx, ny, rtol=1e-12)


def test_rope_bwd_pos0_identity_and_adjoint():
    r = rng(4)
    y = r.standard_normal((1, 2 * 8))
    assert np.array_equal(B.rope_bwd(y, 2, 8, [0], 10000.0), y)
    x = r.standard_normal((5, 2 * 8))
    y = r.standard_normal((5, 2 * 8))
    pos = np.arange(5) * 7
    lhs = np.sum(F.rope(x, 2, 8, pos, 500.0) * y)
    rhs = np.sum(x * B.rope_bwd(y, 2, 8, pos, 500.0))
    assert abs(lhs - rhs) < 1e-12 * max(1, abs(lhs))


# ---------------------------------------------------------------- activations
def test_relu2_golden():
    g = load_golden("relu2_mul_bwd_example.txt")
    dg, du = B.relu2_mul_bwd(g["gate"], g["up"], g["dh"])
    np.testing.assert_array_equal(dg, g["dgate"])
    np.testing.assert_array_equal(du, g["dup"])


def test_relu2_nonpositive_gate_zero_grad():
    r = rng(5)
    gate = -np.abs(r.standard_normal(100))
    gate[:10] = 0.0
    dg, du = B.relu2_mul_bwd(gate, r.standard_normal(100), r.standard_normal(100))
    assert np.all(dg == 0.0) and np.all(du == 0.0)


@pytest.mark.parametrize("act", ["relu2", "swiglu"])
def test_act_bwd_fd(act):
    r = rng(6)
    gate = r.standard_normal(50) * 2
    gate[0] = 0.0  # ReLU^2 is C^1 at 0, so FD is valid there too
    up = r.standard_normal(50)
    dh = r.standard_normal(50)
    dg, du = B.act_bwd(act, gate, up, dh)
    ng = fd.grad(lambda z: float(np.sum(dh * F.act_fwd(act, z, up))), gate)
    nu = fd.grad(lambda z: float(np.sum(dh * F.act_fwd(act, gate, z))), up)
    # (at gate = 0 the central difference of a C^1 kink carries an O(h) error)
    assert fd.rel_err(dg, ng) < 1e-7 and fd.rel_err(du, nu) < 1e-7


def test_swiglu_at_zero():
    # silu'(0) = 1/2 and silu(0) = 0 exactly
    dg, du = B.swiglu_bwd(np.array([0.0]), np.array([3.0]), np.array([2.0]))
    assert dg[0] == 3.0 and du[0] == 0.0


# ---------------------------------------------------------------- softmax / attention
def test_softmax_bwd_golden():
    g = load_golden("softmax_bwd_example.txt")
    np.testing.assert_array_equal(B.softmax_bwd(g["attn"], g["dattn"]), g["dscores"])


def test_softmax_bwd_rows_sum_zero_and_textbook():
    r = rng(7)
    z = r.standard_normal((3, 5, 11))
    e = np.exp(z - z.max(-1, keepdims=True))
    P = e / e.sum(-1, keepdims=True)
    dA = r.standard_normal(P.shape)
    dS = B.softmax_bwd(P, dA)
    assert np.max(np.abs(dS.sum(-1))) < 1e-12
    p = P[0, 0]
    J = np.diag(p) - np.outer(p, p)
    np.testing.assert_allclose(dS[0, 0], J @ dA[0, 0], rtol=1e-12, atol=1e-15)
    # FD of <w, softmax(z)>
    w = dA[1, 2]
    sm = lambda v: np.exp(v - v.max()) / np.exp(v - v.max()).sum()  # noqa: E731
    num = fd.grad(lambda v: float(np.sum(w * sm(v))), z[1, 2])
    assert fd.rel_err(B.softmax_bwd(sm(z[1, 2]), w), num) < 1e-8


def _attn_case(seed, s_q, s_kv, Hq, Hkv, D, causal):
    r = rng(seed)
    q = r.standard_normal((s_q, Hq * D))
    k = r.standard_normal((s_kv, Hkv * D))
    v = r.standard_normal((s_kv, Hkv * D))
    P, ctx = F.attention(q, k, v, Hq, Hkv, D, 1 / np.sqrt(D), causal)
    dctx = r.standard_normal(ctx.shape)
    return q, k, v, P, ctx, dctx


@pytest.mark.parametrize("s_q,s_kv,Hq,Hkv,D,causal", [
    (6, 6, 4, 2, 8, True), (1, 9, 4, 1, 8, True), (5, 5, 2, 2, 4, False), (3, 7, 3, 1, 6, True)])
def test_attention_bwd_fd(s_q, s_kv, Hq, Hkv, D, causal):
    q, k, v, P, ctx, dctx = _attn_case(11, s_q, s_kv, Hq, Hkv, D, causal)
    sc = 1 / np.sqrt(D)
    dq, dv = B.attention_bwd(dctx, P, k, v, Hq, Hkv, sc)
    nq = fd.grad(lambda z: float(np.sum(dctx * F.attention(z, k, v, Hq, Hkv, D, sc, causal)[1])), q)
    nv = fd.grad(lambda z: float(np.sum(dctx * F.attention(q, k, z, Hq, Hkv, D, sc, causal)[1])), v)
    assert fd.rel_err(dq, nq) < 1e-7
    assert fd.rel_err(dv, nv) < 1e-7
    # dK from the same product rule, against finite differences in K
    _, _, dk = B.attention_bwd(dctx, P, k, v, Hq, Hkv, sc, Q=q)
    nk = fd.grad(lambda z: float(np.sum(dctx * F.attention(q, z, v, Hq, Hkv, D, sc, causal)[1])), k)
    assert fd.rel_err(dk, nk) < 1e-7


def test_attention_delta_identity_and_row_sums():
    # rowsum(P o dA) = rowsum(dCtx o ctx) when ctx = P V; sum_j dS = 0
    q, k, v, P, ctx, dctx = _attn_case(12, 8, 8, 4, 2, 16, True)
    _, _, parts = B.attention_bwd(dctx, P, k, v, 4, 2, 0.25, return_parts=True)
    for h, (dA, dS) in enumerate(parts):
        d1 = np.sum(P[h] * dA, -1)
        d2 = np.sum(dctx[:, h * 16:(h + 1) * 16] * ctx[:, h * 16:(h + 1) * 16], -1)
        assert np.max(np.abs(d1 - d2)) < 1e-12
        assert np.max(np.abs(dS.sum(-1))) < 1e-12
        assert np.all(dS[np.triu_indices(8, 1)] == 0.0)  # masked pairs stay zero


def test_attention_bwd_brute_force_loops():
    # the attention backward as explicit scalar loops (per head, query, key, dim)
    q, k, v, P, ctx, dctx = _attn_case(13, 4, 5, 4, 2, 3, True)
    Hq, Hkv, D, sc = 4, 2, 3, 0.7
    dq, dv = B.attention_bwd(dctx, P, k, v, Hq, Hkv, sc)
    dq2 = np.zeros_like(dq)
    dv2 = np.zeros_like(dv)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        for i in range(4):
            gs = [sum(dctx[i, h * D + d] * v[j, g * D + d] for d in range(D)) for j in range(5)]
            dot = sum(P[h, i, j] * gs[j] for j in range(5))
            for j in range(5):
                gp = P[h, i, j] * (gs[j] - dot) * sc
                for d in range(D):
                    dq2[i, h * D + d] += gp * k[j, g * D + d]
                    dv2[j, g * D + d] += P[h, i, j] * dctx[i, h * D + d]
    np.testing.assert_allclose(dq, dq2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dv, dv2, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("s_q,s_kv,Hq,Hkv,causal", [
    (5, 5, 4, 2, True), (5, 5, 4, 2, False), (4, 7, 6, 2, True), (3, 6, 6, 2, False)])
def test_context_is_the_apply_step(s_q, s_kv, Hq, Hkv, causal):
    # ctx_h = P_h V_g with g = h // (Hq/Hkv) ([ENT] backward_through_layers,
    # kv_head = head / heads_per_kv), pinned three ways: scalar loops; the
    # forward's own attention output on the same P; and the delta identity
    # rowsum(P o (dCtx V^T)) = <dCtx, ctx> (the page form of delta against
    # the ctx form) on a P that is NOT a softmax of anything (random rows)
    D = 3
    r = rng(31 + Hq + s_kv)
    P = r.random((Hq, s_q, s_kv))
    if causal:
        P = np.where(F.causal_mask(s_q, s_kv)[None], P, 0.0)
    V = r.standard_normal((s_kv, Hkv * D))
    ctx = F.context(P, V, Hq, Hkv)
    assert ctx.shape == (s_q, Hq * D)
    loops = np.zeros_like(ctx)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        for i in range(s_q):
            for d in range(D):
                loops[i, h * D + d] = sum(P[h, i, j] * V[j, g * D + d] for j in range(s_kv))
    np.testing.assert_allclose(ctx, loops, rtol=1e-13, atol=1e-15)
    dctx = r.standard_normal(ctx.shape)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        dA = dctx[:, h * D:(h + 1) * D] @ V[:, g * D:(g + 1) * D].T
        page = np.sum(P[h] * dA, axis=-1)
        form = np.sum(dctx[:, h * D:(h + 1) * D] * ctx[:, h * D:(h + 1) * D], axis=-1)
        assert np.max(np.abs(page - form)) < 1e-12
    # the forward's attention (softmax of real scores) gives the same ctx
    q = r.standard_normal((s_q, Hq * D))
    k = r.standard_normal((s_kv, Hkv * D))
    P2, ctx2 = F.attention(q, k, V, Hq, Hkv, D, 0.5, causal)
    np.testing.assert_allclose(F.context(P2, V, Hq, Hkv), ctx2, rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- LoRA / AdamW
def test_lora_grads_fd_and_loops():
    r = rng(14)
    S, Hin, out, rk, alpha = 5, 7, 6, 3, 6.0
    x = r.standard_normal((S, Hin))
    A = r.standard_normal((rk, Hin)) * 0.1
    Bm = r.standard_normal((out, rk)) * 0.1
    dy = r.standard_normal((S, out))
    s = alpha / rk
    f = lambda A_, B_: float(np.sum(dy * (s * (x @ A_.T) @ B_.T)))  # noqa: E731
    dA, dB = B.lora_grads(dy, x @ A.T, x, Bm, alpha, rk)
    assert fd.rel_err(dA, fd.grad(lambda z: f(z, Bm), A)) < 1e-8
    assert fd.rel_err(dB, fd.grad(lambda z: f(A, z), Bm)) < 1e-8
    h = x @ A.T
    dB2 = np.array([[s * sum(dy[i, o] * h[i, c] for i in range(S)) for c in range(rk)] for o in range(out)])
    g = np.array([[s * sum(dy[i, o] * Bm[o, c] for o in range(out)) for c in range(rk)] for i in range(S)])
    dA2 = np.array([[sum(g[i, c] * x[i, k] for i in range(S)) for k in range(Hin)] for c in range(rk)])
    np.testing.assert_allclose(dB, dB2, rtol=1e-12)
    np.testing.assert_allclose(dA, dA2, rtol=1e-12)


def test_lora_zero_B_gives_zero_dA():
    r = rng(15)
    dA, dB = B.lora_grads(r.standard_normal((4, 6)), r.standard_normal((4, 2)),
                          r.standard_normal((4, 5)), np.zeros((6, 2)), 4.0, 2)
    assert np.all(dA == 0.0) and np.any(dB != 0.0)


def test_adamw_golden():
    g = load_golden("adamw_step1_example.txt")
    p, m, v = B.adamw(g["p"], g["g"], 0.0, 0.0, g["lr"], g["beta1"], g["beta2"], g["eps"],
                      g["wd"], int(g["step"]))
    assert p == pytest.approx(g["p_new"], abs=1e-15)
    assert m == pytest.approx(g["m_new"], abs=1e-17)
    assert v == pytest.approx(g["v_new"], abs=1e-18)


def test_adamw_step1_closed_forms():
    r = rng(16)
    p = r.standard_normal(50)
    g = r.standard_normal(50)
    g[:5] = 0.0
    lr, wd, eps = 1e-3, 0.01, 1e-8
    p1, _, _ = B.adamw(p, g, np.zeros(50), np.zeros(50), lr, 0.9, 0.999, eps, wd, 1)
    np.testing.assert_allclose(p1, p - lr * (g / (np.abs(g) + eps) + wd * p), rtol=1e-14)
    np.testing.assert_array_equal(p1[:5], p[:5] - lr * wd * p[:5])


@pytest.mark.parametrize("step", [2, 10, 1000])
def test_adamw_matches_torch_float64(step):
    torch = pytest.importorskip("torch")
    r = rng(17 + step)
    p = r.standard_normal(64)
    g = r.standard_normal(64)
    m = r.standard_normal(64) * 1e-2
    v = (r.standard_normal(64) * 1e-2) ** 2
    lr, b1, b2, eps, wd = 1e-3, 0.9, 0.999, 1e-8, 0.01
    ours, om, ov = B.adamw(p, g, m, v, lr, b1, b2, eps, wd, step)
    tp = torch.tensor(p, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.AdamW([tp], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd, foreach=False)
    tp.grad = torch.tensor(g, dtype=torch.float64)
    opt.state[tp] = {"step": torch.tensor(float(step - 1), dtype=torch.float64),
                     "exp_avg": torch.tensor(m, dtype=torch.float64),
                     "exp_avg_sq": torch.tensor(v, dtype=torch.float64)}
    opt.step()
    np.testing.assert_allclose(ours, tp.detach().numpy(), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(om, opt.state[tp]["exp_avg"].numpy(), rtol=1e-13)
    np.testing.assert_allclose(ov, opt.state[tp]["exp_avg_sq"].numpy(), rtol=1e-13)


# ---------------------------------------------------------------- packed ternary weights
def test_ternary_pack_golden():
    from oracle import bitlinear as BL
    g = load_golden("ternary_pack_example.txt")
    w = np.stack([g["w_row0"], g["w_row1"]])
    packed = BL.pack_ternary(w)
    assert packed.dtype == np.uint8 and packed.shape == (2, 2)
    np.testing.assert_array_equal(packed.reshape(-1), g["packed"].astype(np.uint8))
    np.testing.assert_array_equal(BL.unpack_ternary(packed, 8), np.sign(w))


def test_ternary_pack_round_trip_and_product():
    from oracle import bitlinear as BL
    r = rng(51)
    t = r.integers(-1, 2, size=(7, 24))
    w = 0.02 * t
    packed = BL.pack_ternary(w)
    # every byte holds only the codes 00, 01, 11 in each 2-bit field
    for j in range(4):
        assert not np.any(((packed >> (2 * j)) & 3) == 2)
    np.testing.assert_array_equal(BL.unpack_ternary(packed, 24), t)
    dy = r.standard_normal((3, 7))
    np.testing.assert_allclose(BL.bitlinear_t(dy, packed, 0.02, 24), dy @ w, rtol=1e-14, atol=1e-16)
    # the bit position of one column: a single +1 at column 4c + j sets code 01 at bits 2j
    for c in range(6):
        for j in range(4):
            e = np.zeros((1, 24))
            e[0, 4 * c + j] = 1.0
            p = BL.pack_ternary(e)
            assert p[0, c] == 1 << (2 * j) and p.sum() == 1 << (2 * j)


# ---------------------------------------------------------------- whole layer
def _layer_fd(cfg, seed_layer=0):
    d = synth.draw_layer(cfg, seed_layer)
    w, saved, lora = F.make_layer(cfg, d)
    res = B.layer_bwd(cfg, w, saved, d["d_out"], lora)
    x0 = d["x"]

    def L(**kw):
        out, _ = F.layer_forward(cfg, w, kw.pop("x", x0), x_attn=x0, **kw)
        return float(np.sum(d["d_out"] * out))
    return d, w, saved, lora, res, L


def test_layer_fd_tiny_swiglu_lora(tiny):
    d, w, saved, lora, res, L = _layer_fd(tiny)
    assert fd.rel_err(res["d_hidden"], fd.grad(lambda z: L(x=z, lora=lora), d["x"])) < 1e-5
    for k in ("A_q", "B_q", "A_v", "B_v"):
        def Lk(z, k=k):
            l2 = dict(lora)
            l2[k] = z
            return L(lora=l2)
        num = fd.grad(Lk, lora[k], rel_step=1e-5)
        assert fd.rel_err(res["d" + k], num) < 1e-5, k
    # the Q signal before RoPE and the value gradient
    nq = fd.grad(lambda z: L(lora=lora, q_pre=z), saved["q_pre"])
    assert fd.rel_err(res["dq_pre"], nq) < 1e-5
    nv = fd.grad(lambda z: L(lora=lora, v_in=z), saved["V"])
    assert fd.rel_err(res["dv"], nv) < 1e-5


def test_layer_fd_chunk_after_cached_prefix(tiny):
    # 5 tokens after a 6-row cached prefix (kv_len 11, positions 6..10): the
    # value adapter acts on the chunk's own values only, so its gradients come
    # from the last 5 rows of dV; finite differences of the forward decide
    cfg = tiny.with_(seq=5, kv_len=11, pos0=6)
    d, w, saved, lora, res, L = _layer_fd(cfg)
    assert saved["K"].shape[0] == 11 and res["dv"].shape[0] == 11
    assert fd.rel_err(res["d_hidden"], fd.grad(lambda z: L(x=z, lora=lora), d["x"])) < 1e-5
    for k in ("A_q", "B_q", "A_v", "B_v"):
        def Lk(z, k=k):
            l2 = dict(lora)
            l2[k] = z
            return L(lora=l2)
        assert fd.rel_err(res["d" + k], fd.grad(Lk, lora[k], rel_step=1e-5)) < 1e-5, k


def test_layer_fd_qk_norm(tiny):
    # QK-norm (per-head RMSNorm of the Q and K projections before RoPE, one
    # head_dim scale vector): finite differences of the forward with respect
    # to the Q projection output (before the norm) and the Q adapter, at late
    # positions and with GQA 4:2
    cfg = tiny.with_(qk_norm=True, pos0=37)
    d, w, saved, lora, res, L = _layer_fd(cfg)
    assert "q_raw" in saved and "k_raw" in saved
    num = fd.grad(lambda z: L(q_pre=z, lora=lora), saved["q_raw"])
    assert fd.rel_err(res["dq_pre"], num) < 1e-5
    for k in ("A_q", "B_q"):
        def Lk(z, k=k):
            l2 = dict(lora)
            l2[k] = z
            return L(lora=l2)
        assert fd.rel_err(res["d" + k], fd.grad(Lk, lora[k], rel_step=1e-5)) < 1e-5, k
    # and it differs from the layer without the norm (the step is not a no-op)
    res0 = B.layer_bwd(cfg.with_(qk_norm=False), w, saved, d["d_out"], lora)
    assert fd.rel_err(res0["dq_pre"], res["dq_pre"]) > 1e-2


def test_head_rmsnorm_bwd_per_head_loops():
    # the per-head norm backward equals the row norm backward on each head's
    # slice separately, with the shared scale vector
    r = rng(41)
    x = r.standard_normal((3, 4 * 6))
    dy = r.standard_normal(x.shape)
    g = 1 + 0.1 * r.standard_normal(6)
    dx = B.head_rmsnorm_bwd(x, 4, g, dy, 1e-6)
    for i in range(3):
        for h in range(4):
            sl = slice(6 * h, 6 * h + 6)
            np.testing.assert_allclose(dx[i, sl], B.rmsnorm_bwd(x[i, sl], g, dy[i, sl], 1e-6),
                                       rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("over", [
    {},                                                   # GQA 4:2, SwiGLU, both adapters
    {"qk_norm": True, "pos0": 23},                        # QK-norm on Q and K, late positions
    {"seq": 5, "kv_len": 11, "pos0": 6},                  # a chunk after a cached prefix
    {"n_kv_heads": 4, "causal": False, "rank": 0},        # MHA, no mask, no adapters
])
def test_layer_fd_input_gradient_without_stop_gradient(tiny, over):
    # the exact gradient of the layer with respect to its input x, through
    # the residual stream AND the attention branch (x feeds both): central
    # differences of <dOut, out(x)> with x_attn = x
    cfg = tiny.with_(input_grad=True, **over)
    d = synth.draw_layer(cfg)
    w, saved, lora = F.make_layer(cfg, d)
    res = B.layer_bwd(cfg, w, saved, d["d_out"], lora)

    def L(z):
        out, _ = F.layer_forward(cfg, w, z, lora=lora)
        return float(np.sum(d["d_out"] * out))
    assert fd.rel_err(res["d_hidden"], fd.grad(L, d["x"])) < 1e-5
    # the attention branch is not negligible: the stop-gradient answer differs
    assert fd.rel_err(res["dh1"], res["d_hidden"]) > 1e-3


def test_layer_fd_decode_like_relu2_subnorms():
    # the decode layer at a tiny size: one token at the last of 12 cache slots,
    # ReLU^2 x up FFN, both sub-norms, ternary weights, no adapters
    cfg = synth.get_config("decode").with_(hidden=32, ffn=48, n_heads=4, n_kv_heads=2,
                                          head_dim=8, kv_len=12, pos0=11)
    d, w, saved, lora, res, L = _layer_fd(cfg)
    assert lora is None
    assert fd.rel_err(res["d_hidden"], fd.grad(lambda z: L(x=z), d["x"])) < 1e-5
    assert fd.rel_err(res["dq_pre"], fd.grad(lambda z: L(q_pre=z), saved["q_pre"])) < 1e-5
    assert fd.rel_err(res["dv"], fd.grad(lambda z: L(v_in=z), saved["V"])) < 1e-5
    assert "gnorm_sq" in res and res["gnorm_sq"] == 0.0


def test_layer_adamw_uses_lora_plus_and_a_only_gnorm(tiny):
    d = synth.draw_layer(tiny)
    w, saved, lora = F.make_layer(tiny, d)
    res = B.layer_bwd(tiny, w, saved, d["d_out"], lora)
    gsq = float(np.sum(res["dA_q"] ** 2) + np.sum(res["dA_v"] ** 2))
    assert res["gnorm_sq"] == pytest.approx(gsq, rel=1e-15)
    g = res["dB_q"]
    b0 = np.asarray(lora["B_q"], np.float64)
    want = b0 - tiny.lr * 16 * (g / (np.abs(g) + tiny.adam_eps) + tiny.weight_decay * b0)
    np.testing.assert_allclose(res["B_q"], want, rtol=1e-13)


def test_two_layer_stack_fd(tiny):
    # a real two-layer composition: layer 1's saved activations come from
    # layer 0's output; the stack gradient must be the FD of <g, out1(out0(x))>
    # with each attention branch input held fixed
    d0 = synth.draw_layer(tiny, 0)
    d1 = synth.draw_layer(tiny, 1)
    w0, s0, l0 = F.make_layer(tiny, d0)
    out0, _ = F.layer_forward(tiny, w0, d0["x"], lora=l0)
    w1 = {k: v for k, v in d1.items() if k.startswith("W_") or k.startswith("gamma_")}
    l1 = {k: v for k, v in d1.items() if k[:2] in ("A_", "B_") or k[:4] in ("m_A_", "m_B_", "v_A_", "v_B_")}
    _, s1 = F.layer_forward(tiny, w1, out0, lora=l1)
    g = d1["d_out"]
    dx, res, gnorm = B.stack_bwd(tiny, [(w0, s0, l0), (w1, s1, l1)], g)

    def L(x):
        o0, _ = F.layer_forward(tiny, w0, x, x_attn=d0["x"], lora=l0)
        o1, _ = F.layer_forward(tiny, w1, o0, x_attn=out0, lora=l1)
        return float(np.sum(g * o1))
    assert fd.rel_err(dx, fd.grad(L, d0["x"])) < 1e-5
    assert gnorm == pytest.approx(np.sqrt(res[0]["gnorm_sq"] + res[1]["gnorm_sq"]), rel=1e-15)


def test_trainer_smoke_scenario_on_oracle():
    # the trainer test's scenario (entrenar wgpu_backward.rs,
    # test_backward_through_layers_gradient_flow): 2 layers, hidden 8, ffn 16,
    # 2 tokens, rank 4, 2/2 heads of 4, constant 0.01 weights, ramp/constant
    # activations, ramp gradient, lr 1e-3, alpha 32; A must change, the norm is
    # non-negative and the propagated gradient finite
    cfg = synth.get_config("tiny").with_(seq=2, kv_len=2, hidden=8, ffn=16, n_heads=2,
                                        n_kv_heads=2, head_dim=4, rank=4, alpha=32.0,
                                        lr=1e-3, causal=False)
    s, h, i = 2, 8, 16
    ramp = (np.arange(s * h) - 8.0) * 0.1
    layers = []
    for l in range(2):
        w = {"W_o": np.full((h, 8), 0.01), "W_gate": np.full((i, h), 0.01),
             "W_up": np.full((i, h), 0.01), "W_down": np.full((h, i), 0.01),
             "gamma_ffn": np.ones(h)}
        saved = {"attn_input": ramp.reshape(s, h), "resid1": ramp.reshape(s, h),
                 "gate": np.full((s, i), 0.5), "up": np.full((s, i), 0.3),
                 "K": np.full((s, 8), 0.1), "V": np.full((s, 8), 0.1),
                 "P": np.full((2, s, s), 0.5), "ctx": np.full((s, 8), 0.1),
                 "lora_q_h": np.full((s, 4), 0.01), "lora_v_h": np.full((s, 4), 0.01)}
        dr = synth.draw_layer(cfg, l)
        lora = {k: dr[k] for k in dr if k[:2] in ("A_", "B_") or k[:4] in ("m_A_", "m_B_", "v_A_", "v_B_")}
        layers.append((w, saved, lora))
    gh = (np.arange(s * h) - 8.0) * 0.01
    dx, res, gnorm = B.stack_bwd(cfg, layers, gh.reshape(s, h))
    assert not np.array_equal(res[0]["A_q"], layers[0][2]["A_q"])
    assert not np.array_equal(res[0]["A_v"], layers[0][2]["A_v"])
    assert gnorm >= 0.0 and np.all(np.isfinite(dx))


# ---------------------------------------------------------------- lm_head
def _lm_case(seed, S, H, V):
    r = rng(seed)
    h = r.standard_normal((S, H))
    W = 0.3 * r.standard_normal((V, H))
    labels = r.integers(0, V, size=S)
    return h, W, labels


def test_lm_head_fd_and_row_sums():
    from oracle import lmhead as LM
    h, W, labels = _lm_case(61, 3, 5, 7)
    res = LM.lm_head_bwd(h, h @ W.T, labels, W, np.zeros_like(W), np.zeros_like(W),
                         1e-3, 0.9, 0.999, 1e-8, 0.01, 1)
    loss = lambda h_, W_: LM.cross_entropy(h_ @ W_.T, labels)  # noqa: E731
    assert abs(res["loss"] - loss(h, W)) < 1e-15
    assert fd.rel_err(res["grad_hidden"], fd.grad(lambda z: loss(z, W), h)) < 1e-8
    assert fd.rel_err(res["dW"], fd.grad(lambda z: loss(h, z), W)) < 1e-8
    # each row of dlogits sums to zero; the label entry is (p - 1) / S
    assert np.max(np.abs(res["dlogits"].sum(-1))) < 1e-15
    p = LM.softmax_rows(h @ W.T)
    for s in range(3):
        assert abs(res["dlogits"][s, labels[s]] - (p[s, labels[s]] - 1.0) / 3) < 1e-15


def test_lm_head_closed_forms_and_torch():
    torch = pytest.importorskip("torch")
    from oracle import lmhead as LM
    # uniform logits: loss = log V and dlogits = (1/V - onehot) / S
    V, S = 32, 4
    labels = np.array([0, 5, 31, 5])
    z = np.zeros((S, V))
    assert abs(LM.cross_entropy(z, labels) - np.log(V)) < 1e-15
    W = np.zeros((V, 8))
    res = LM.lm_head_bwd(np.ones((S, 8)), z, labels, W, W, W, 1e-3, 0.9, 0.999, 1e-8, 0.0, 1)
    want = np.full((S, V), 1.0 / V)
    want[np.arange(S), labels] -= 1.0
    np.testing.assert_allclose(res["dlogits"], want / S, rtol=0, atol=1e-17)
    # torch.nn.functional.cross_entropy (mean) and autograd in float64
    h, W, labels = _lm_case(62, 6, 9, 40)
    th = torch.tensor(h, requires_grad=True)
    tW = torch.tensor(W, requires_grad=True)
    tl = torch.nn.functional.cross_entropy(th @ tW.T, torch.tensor(labels))
    tl.backward()
    res = LM.lm_head_bwd(h, h @ W.T, labels, W, np.zeros_like(W), np.zeros_like(W),
                         1e-3, 0.9, 0.999, 1e-8, 0.01, 1)
    assert abs(res["loss"] - tl.item()) < 1e-13
    np.testing.assert_allclose(res["grad_hidden"], th.grad.numpy(), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(res["dW"], tW.grad.numpy(), rtol=1e-12, atol=1e-15)


def test_lm_head_ignored_rows():
    """Labels outside the vocabulary mark rows to skip: against float64 torch
    cross_entropy with ignore_index (its mean is over the kept rows), and
    finite differences of the loss over the kept rows alone."""
    torch = pytest.importorskip("torch")
    from oracle import lmhead as LM
    h, W, labels = _lm_case(63, 7, 6, 11)
    labels[[1, 4]] = -100
    th = torch.tensor(h, requires_grad=True)
    tW = torch.tensor(W, requires_grad=True)
    tl = torch.nn.functional.cross_entropy(th @ tW.T, torch.tensor(labels), ignore_index=-100)
    tl.backward()
    res = LM.lm_head_bwd(h, h @ W.T, labels, W, np.zeros_like(W), np.zeros_like(W),
                         1e-3, 0.9, 0.999, 1e-8, 0.01, 1)
    assert abs(res["loss"] - tl.item()) < 1e-13
    np.testing.assert_allclose(res["grad_hidden"], th.grad.numpy(), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(res["dW"], tW.grad.numpy(), rtol=1e-12, atol=1e-15)
    assert not res["dlogits"][[1, 4]].any()
    # a label equal to the vocabulary size is out of range too
    labels[4] = 11
    keep = [0, 2, 3, 5, 6]
    loss = lambda h_: float(np.mean(  # noqa: E731
        np.log(np.exp(h_[keep] @ W.T).sum(-1)) - (h_[keep] @ W.T)[np.arange(5), labels[keep]]))
    res = LM.lm_head_bwd(h, h @ W.T, labels, W, np.zeros_like(W), np.zeros_like(W),
                         1e-3, 0.9, 0.999, 1e-8, 0.01, 1)
    assert abs(res["loss"] - loss(h)) < 1e-13
    assert fd.rel_err(res["grad_hidden"], fd.grad(loss, h)) < 1e-8
    # every row ignored: no loss, no gradient, and AdamW sees a zero gradient
    res = LM.lm_head_bwd(h, h @ W.T, np.full(7, -1), W, np.zeros_like(W), np.zeros_like(W),
                         1e-3, 0.9, 0.999, 1e-8, 0.01, 1)
    assert res["loss"] == 0.0 and not res["grad_hidden"].any() and not res["dW"].any()
    np.testing.assert_allclose(res["W"], W * (1 - 1e-3 * 0.01), rtol=1e-15)


def test_lm_head_sampled_matches_the_whole_computation():
    """The block-wise form used at full sizes keeps lm_head_bwd's values at
    the requested rows and columns (a small block size spans several blocks
    and a ragged last one)."""
    from oracle import lmhead as LM
    h, W, labels = _lm_case(64, 11, 6, 13)
    labels[3] = -100
    z = h @ W.T + 0.5
    full = LM.lm_head_bwd(h, z, labels, W, np.zeros_like(W), np.zeros_like(W),
                          1e-3, 0.9, 0.999, 1e-8, 0.01, 1)
    rows, cols = [0, 3, 10, 5], [12, 0, 7]
    smp = LM.lm_head_sampled(h, z, labels, W.astype(np.float32), rows, cols, chunk=4)
    assert abs(smp["loss"] - full["loss"]) < 1e-14
    np.testing.assert_allclose(smp["dW"], full["dW"][cols], rtol=0, atol=1e-15)
    ref = full["dlogits"][rows] @ W.astype(np.float32).astype(np.float64)
    np.testing.assert_allclose(smp["grad_hidden"], ref, rtol=0, atol=1e-15)
