"""GPU parity at the documented size limits: each entry point with one
dimension at its maximum (2^20 rows or features, 4096 query heads) and the
others small, against the float64 oracle.  The CPU tests check that one past
each limit is refused; these check that the limit itself is computed."""
import numpy as np
import pytest

import synth
from oracle import backward as OB
from tests import harness as Hn

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
DEV = "cuda:0"
F32 = torch.float32
BIG = 1 << 20
TOL = Hn.TOL["f32"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import layer_backward_pass_amd as lbp
    lbp.load_library()


def lbp():
    import layer_backward_pass_amd as m
    return m


def rnd(seed, shape, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


@pytest.mark.parametrize("rows,n", [(1, BIG), (BIG, 8)])
def test_rmsnorm_at_the_limits(rows, n):
    print("rmsnorm", rows, n, flush=True)
    x = Hn.dev(rnd(1, (rows, n)), F32, DEV)
    g = Hn.dev(1 + 0.1 * rnd(2, n), F32, DEV)
    dy = Hn.dev(rnd(3, (rows, n)), F32, DEV)
    dx = torch.empty_like(dy)
    lbp().lorabwd_rmsnorm_backward(x, g, dy, dx, eps=1e-6)
    torch.cuda.synchronize()
    want = OB.rmsnorm_bwd(Hn.host(x), Hn.host(g), Hn.host(dy), 1e-6)
    assert Hn.rel_err(Hn.host(dx), want) <= TOL


@pytest.mark.parametrize("rows,H,D", [(BIG, 1, 16), (2, 4096, 16)])
def test_rope_at_the_limits(rows, H, D):
    print("rope", rows, H, D, flush=True)
    dy = Hn.dev(rnd(5, (rows, H * D)), F32, DEV)
    dx = torch.empty_like(dy)
    lbp().lorabwd_rope_backward(dy, dx, H, D, pos0=0, base=10000.0)
    torch.cuda.synchronize()
    want = OB.rope_bwd(Hn.host(dy), H, D, np.arange(rows), 10000.0)
    assert Hn.rel_err(Hn.host(dx), want) <= TOL


@pytest.mark.parametrize("s_q,s_kv,Hq,Hkv,D,causal,use_ctx", [
    (1, BIG, 1, 1, 16, 1, 1),      # a one-token query over 2^20 cached keys
    (1, BIG, 2, 1, 16, 1, 0),      # the same without ctx (page-form delta)
    (16, BIG, 1, 1, 16, 1, 1),     # a short query block at the end of 2^20 keys
    (2, 2, 4096, 1024, 16, 0, 1),  # 4096 query heads
    (1, 8, 4096, 1024, 16, 0, 1),  # 4096 query heads, one token
])
def test_attention_at_the_limits(s_q, s_kv, Hq, Hkv, D, causal, use_ctx):
    print("attn", s_q, s_kv, Hq, Hkv, D, causal, use_ctx, flush=True)
    from oracle import forward as OF
    r = np.random.default_rng(9)
    q = r.standard_normal((s_q, Hq * D))
    k = r.standard_normal((s_kv, Hkv * D))
    v = r.standard_normal((s_kv, Hkv * D))
    P, ctx = OF.attention(q, k, v, Hq, Hkv, D, D ** -0.5, bool(causal))
    dctx = r.standard_normal((s_q, Hq * D))
    t = [Hn.dev(a, F32, DEV) for a in (dctx, P, k, v, ctx)]
    dq = torch.empty(s_q, Hq * D, device=DEV)
    dv = torch.empty(s_kv, Hkv * D, device=DEV)
    lbp().lorabwd_attn_backward(t[0], t[1], t[2], t[3], t[4] if use_ctx else None, dq, dv, Hq,
                                Hkv, D, causal=bool(causal))
    torch.cuda.synchronize()
    wq, wv = OB.attention_bwd(dctx, P, k, v, Hq, Hkv, D ** -0.5)
    assert Hn.rel_err(Hn.host(dq), wq) <= TOL
    assert Hn.rel_err(Hn.host(dv), wv) <= TOL


@pytest.mark.parametrize("rows,dim,ffn", [(2, 8, BIG), (1, 8, BIG), (BIG, 8, 16), (2, BIG, 8)])
def test_ffn_at_the_limits(rows, dim, ffn):
    print("ffn", rows, dim, ffn, flush=True)
    r = np.random.default_rng(11)
    t = lambda a: Hn.dev(a, F32, DEV)  # noqa: E731
    d_out = t(r.standard_normal((rows, dim)))
    w_down = t(r.standard_normal((dim, ffn)) * 0.02)
    w_gate = t(r.standard_normal((ffn, dim)) * 0.02)
    w_up = t(r.standard_normal((ffn, dim)) * 0.02)
    gate = t(r.standard_normal((rows, ffn)))
    up = t(r.standard_normal((rows, ffn)))
    resid1 = t(r.standard_normal((rows, dim)))
    gffn = t(1 + 0.1 * r.standard_normal(dim))
    d_resid = d_out.clone()
    m = lbp()
    m.lorabwd_ffn_backward(d_out, w_down, w_gate, w_up, gate, up, resid1, gffn, d_resid,
                           act=m.ACT_SWIGLU)
    torch.cuda.synchronize()
    H = Hn.host
    want = OB.ffn_bwd(H(d_out), H(w_down), H(w_gate), H(w_up), H(gate), H(up), H(resid1),
                      H(gffn), 1e-6, "swiglu")
    assert Hn.rel_err(H(d_resid), want) <= TOL


@pytest.mark.parametrize("rows,H,out", [(3, BIG, 16), (3, 16, BIG), (BIG, 8, 8)])
def test_lora_at_the_limits(rows, H, out):
    print("lora", rows, H, out, flush=True)
    rank = 4
    r = np.random.default_rng(12)
    x = r.standard_normal((rows, H))
    A = r.standard_normal((rank, H)) * 0.02
    Bm = r.standard_normal((out, rank)) * 0.02
    dy = r.standard_normal((rows, out))
    tx, th = Hn.dev(x, F32, DEV), Hn.dev(x @ A.T, F32, DEV)
    T = {k: Hn.dev(v, F32, DEV) for k, v in dict(A=A, B=Bm, m_a=0 * A, v_a=0 * A, m_b=0 * Bm,
                                                    v_b=0 * Bm).items()}
    ga = torch.empty(rank, H, device=DEV)
    gb = torch.empty(out, rank, device=DEV)
    gn = torch.zeros(1, device=DEV)
    alpha, lr, lr_b = 2.0 * rank, 1e-3, 1.6e-2
    lbp().lorabwd_lora_grad_adamw(Hn.dev(dy, F32, DEV), tx, th, T["A"], T["B"], T["m_a"],
                                  T["v_a"], T["m_b"], T["v_b"], alpha, lr, lr_b, grad_a=ga,
                                  grad_b=gb, gnorm_sq=gn)
    torch.cuda.synchronize()
    dA, dB = OB.lora_grads(dy, Hn.host(th), Hn.host(tx), Bm, alpha, rank)
    assert Hn.rel_err(Hn.host(ga), dA) <= TOL
    assert Hn.rel_err(Hn.host(gb), dB) <= TOL
    nA = OB.adamw(A, dA, 0 * A, 0 * A, lr, 0.9, 0.999, 1e-8, 0.01, 1)[0]
    nB = OB.adamw(Bm, dB, 0 * Bm, 0 * Bm, lr_b, 0.9, 0.999, 1e-8, 0.01, 1)[0]
    assert Hn.update_err(Hn.host(T["A"]), nA, dA, lr, TOL) <= TOL
    assert Hn.update_err(Hn.host(T["B"]), nB, dB, lr_b, TOL) <= TOL
    assert Hn.rel_err(Hn.host(gn), [np.sum(dA * dA)]) <= TOL


@pytest.mark.parametrize("rows,hidden,vocab", [(2, 8, BIG), (BIG, 8, 4), (2, BIG, 4)])
def test_lm_head_at_the_limits(rows, hidden, vocab):
    print("lm_head", rows, hidden, vocab, flush=True)
    cfg = synth.get_config("lmhead").with_(rows=rows, hidden=hidden, vocab=vocab)
    errs = Hn.lm_head_parity(cfg, DEV)
    bad = {k: v for k, v in errs.items() if not v <= TOL}
    assert not bad, bad
