"""GPU parity of each C-ABI entry point against the float64 oracle, at small
shapes that span several tiles and ragged tails, plus edge cases."""
import numpy as np
import pytest

import synth
from oracle import backward as OB
from tests import harness as Hn

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
DEV = "cuda:0"
F32 = torch.float32
BF16 = torch.bfloat16


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


def tol(dt):
    return 2e-2 if dt == BF16 else 1e-4


# ------------------------------------------------------------------ RMSNorm
@pytest.mark.parametrize("rows,n,acc,dt", [
    (1, 8, 0, F32), (3, 2560, 0, F32), (37, 1000, 1, F32), (5, 6912, 0, F32),
    (17, 2560, 1, BF16), (2, 9728, 0, BF16)])
def test_rmsnorm(rows, n, acc, dt):
    print("rmsnorm", rows, n, acc, dt, flush=True)
    x = Hn.dev(rnd(1, (rows, n)), dt, DEV)
    g = Hn.dev(1 + 0.1 * rnd(2, n), F32, DEV)
    dy = Hn.dev(rnd(3, (rows, n)), F32, DEV)
    dx0 = rnd(4, (rows, n))
    dx = Hn.dev(dx0, F32, DEV)
    lbp().lorabwd_rmsnorm_backward(x, g, dy, dx, eps=1e-6, accumulate=bool(acc))
    torch.cuda.synchronize()
    want = OB.rmsnorm_bwd(Hn.host(x), Hn.host(g), Hn.host(dy), 1e-6) + (dx0 if acc else 0)
    assert Hn.rel_err(Hn.host(dx), want) <= 1e-4


def test_rmsnorm_in_place():
    x = Hn.dev(rnd(1, (4, 64)), F32, DEV)
    g = Hn.dev(1 + 0.1 * rnd(2, 64), F32, DEV)
    dy = Hn.dev(rnd(3, (4, 64)), F32, DEV)
    want = OB.rmsnorm_bwd(Hn.host(x), Hn.host(g), Hn.host(dy), 1e-6)
    lbp().lorabwd_rmsnorm_backward(x, g, dy, dy)
    torch.cuda.synchronize()
    assert Hn.rel_err(Hn.host(dy), want) <= 1e-4


# ------------------------------------------------------------------ RoPE
@pytest.mark.parametrize("rows,H,D,pos0", [(1, 20, 128, 511), (33, 4, 16, 0), (2048, 2, 128, 0),
                                           (7, 3, 64, 100000), (5, 9, 32, 3)])
def test_rope(rows, H, D, pos0):
    print("rope", rows, H, D, pos0, flush=True)
    dy = Hn.dev(rnd(5, (rows, H * D)), F32, DEV)
    dx = torch.empty_like(dy)
    lbp().lorabwd_rope_backward(dy, dx, H, D, pos0=pos0, base=10000.0)
    torch.cuda.synchronize()
    want = OB.rope_bwd(Hn.host(dy), H, D, pos0 + np.arange(rows), 10000.0)
    assert Hn.rel_err(Hn.host(dx), want) <= 1e-4
    # in place
    lbp().lorabwd_rope_backward(dy, dy, H, D, pos0=pos0, base=10000.0)
    torch.cuda.synchronize()
    assert Hn.rel_err(Hn.host(dy), want) <= 1e-4


# ------------------------------------------------------------------ attention
def _attn_inputs(seed, s_q, s_kv, Hq, Hkv, D, causal, dt):
    from oracle import forward as OF
    r = np.random.default_rng(seed)
    q = r.standard_normal((s_q, Hq * D))
    k = r.standard_normal((s_kv, Hkv * D))
    v = r.standard_normal((s_kv, Hkv * D))
    P, ctx = OF.attention(q, k, v, Hq, Hkv, D, D ** -0.5, causal)
    dctx = r.standard_normal((s_q, Hq * D))
    return [Hn.dev(a, t, DEV) for a, t in ((dctx, F32), (P, dt), (k, dt), (v, dt), (ctx, dt))]


@pytest.mark.parametrize("s_q,s_kv,Hq,Hkv,D,causal,use_ctx,dt", [
    (16, 16, 4, 2, 16, 1, 1, F32),
    (100, 100, 4, 2, 64, 1, 1, F32),      # ragged: not a multiple of 64 or 32
    (130, 130, 4, 1, 128, 1, 0, F32),     # page-form delta (no ctx)
    (70, 70, 2, 2, 32, 0, 1, F32),        # non-causal
    (40, 97, 8, 2, 128, 1, 1, F32),       # fewer queries than keys
    (1, 512, 20, 5, 128, 1, 1, F32),      # decode
    (1, 77, 4, 2, 16, 1, 0, F32),         # decode, ragged cache
    (1, 77, 4, 2, 16, 1, 1, F32),         # decode, delta from ctx
    (1, 300, 8, 4, 64, 0, 1, BF16),
    (1, 1000, 32, 4, 32, 1, 1, F32),
    (96, 96, 8, 2, 128, 1, 1, BF16),
    (1, 300, 8, 4, 64, 0, 0, BF16),
    (200, 333, 6, 2, 32, 1, 1, F32),      # group of 3, key count not a multiple of 4
    (64, 64, 16, 2, 16, 0, 0, F32),       # group of 8, no mask, no ctx
    (257, 257, 4, 4, 128, 1, 1, F32),     # group of 1, one row past a tile
    (33, 1030, 8, 2, 64, 1, 1, F32),      # short query block at the end of a long cache
    (200, 200, 8, 2, 64, 1, 1, BF16),
    (130, 333, 6, 2, 32, 1, 0, BF16),     # bf16: group of 3, no ctx, keys not a multiple of 8
    (257, 257, 4, 4, 128, 0, 1, BF16),    # bf16: no mask, group of 1, odd block count
    (64, 64, 16, 2, 16, 1, 1, BF16),      # bf16: head dim 16
    (33, 1030, 8, 2, 128, 1, 1, BF16),    # bf16: short query block, long cache
    (640, 640, 8, 2, 128, 1, 1, BF16),    # bf16: several dv chunks
    (700, 900, 8, 2, 64, 1, 1, BF16),     # bf16: dv chunks over (head, block) steps, ragged
    (520, 520, 12, 4, 128, 0, 1, BF16),   # bf16: no mask, group of 3, ragged last block
])
def test_attention(s_q, s_kv, Hq, Hkv, D, causal, use_ctx, dt):
    print("attn", s_q, s_kv, Hq, Hkv, D, causal, use_ctx, dt, flush=True)
    dctx, P, K, V, ctx = _attn_inputs(7, s_q, s_kv, Hq, Hkv, D, bool(causal), dt)
    dq = torch.empty(s_q, Hq * D, device=DEV)
    dv = torch.empty(s_kv, Hkv * D, device=DEV)
    lbp().lorabwd_attn_backward(dctx, P, K, V, ctx if use_ctx else None, dq, dv, Hq, Hkv, D,
                                causal=bool(causal))
    torch.cuda.synchronize()
    wq, wv = OB.attention_bwd(Hn.host(dctx), Hn.host(P), Hn.host(K), Hn.host(V), Hq, Hkv,
                              D ** -0.5)
    assert Hn.rel_err(Hn.host(dq), wq) <= tol(dt)
    assert Hn.rel_err(Hn.host(dv), wv) <= tol(dt)


def test_attention_without_dv_and_empty_queries():
    dctx, P, K, V, ctx = _attn_inputs(8, 20, 20, 4, 2, 16, True, F32)
    dq = torch.empty(20, 64, device=DEV)
    lbp().lorabwd_attn_backward(dctx, P, K, V, ctx, dq, None, 4, 2, 16)
    torch.cuda.synchronize()
    wq, _ = OB.attention_bwd(Hn.host(dctx), Hn.host(P), Hn.host(K), Hn.host(V), 4, 2, 0.25)
    assert Hn.rel_err(Hn.host(dq), wq) <= 1e-4
    # zero query rows: dV is all zeros
    dv = torch.full((20, 32), 7.0, device=DEV)
    e = torch.empty(0, 64, device=DEV)
    lbp().lorabwd_attn_backward(e, torch.empty(4, 0, 20, device=DEV), K, V, None,
                                torch.empty(0, 64, device=DEV), dv, 4, 2, 16, causal=False)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dv).item() == 0


@pytest.mark.parametrize("s_q,s_kv,Hq,Hkv,D,dt", [
    (96, 96, 8, 2, 128, BF16),    # the bf16 MFMA kernels: only Kᵀ is transposed
    (130, 200, 8, 2, 64, BF16),
    (70, 70, 8, 2, 128, F32),     # fp32 MFMA kernels with the causal key split
])
def test_attention_dq_only(s_q, s_kv, Hq, Hkv, D, dt):
    """dQ without dV on the MFMA paths (no dV launches, no dCtx transpose)."""
    dctx, P, K, V, ctx = _attn_inputs(9, s_q, s_kv, Hq, Hkv, D, True, dt)
    dq = torch.empty(s_q, Hq * D, device=DEV)
    lbp().lorabwd_attn_backward(dctx, P, K, V, ctx, dq, None, Hq, Hkv, D)
    torch.cuda.synchronize()
    wq, _ = OB.attention_bwd(Hn.host(dctx), Hn.host(P), Hn.host(K), Hn.host(V), Hq, Hkv,
                             D ** -0.5)
    assert Hn.rel_err(Hn.host(dq), wq) <= tol(dt)


# ------------------------------------------------------------------ FFN
@pytest.mark.parametrize("rows,dim,ffn,act,sub,dt", [
    (16, 64, 256, "swiglu", False, F32),
    (1, 64, 96, "relu2", True, F32),        # decode GEMV path
    (133, 192, 320, "swiglu", False, F32),  # ragged tiles
    (1, 2560, 6912, "relu2", True, F32),    # decode layer shape
    (1, 128, 344, "swiglu", False, BF16),   # decode GEMV path, bf16, ragged chunk
    (1, 512, 1032, "swiglu", True, F32),
    (70, 256, 512, "relu2", True, BF16),
    (300, 128, 256, "swiglu", False, BF16),
    # 7 x 37 product tiles: 256 run whole, the last 3 (rows 512.. of the last
    # column panel) split in k and added after
    (833, 256, 9400, "swiglu", False, F32),
    (833, 512, 9400, "relu2", True, BF16),
    # without a sub-norm the dHid product applies the activation backward
    # in its store: bf16 whole tiles + a split tail reduced through it, and
    # fp32 whole tiles with ragged rows and columns
    (833, 512, 9400, "relu2", False, BF16),
    (700, 128, 520, "relu2", False, F32),
    # the gate/up product on the wide bf16 kernel (256 x 256 tiles): ragged
    # rows and columns, split in k
    (600, 520, 1024, "swiglu", False, BF16),
    (1100, 776, 1600, "relu2", True, BF16),
])
def test_ffn(rows, dim, ffn, act, sub, dt):
    print("ffn", rows, dim, ffn, act, sub, dt, flush=True)
    r = np.random.default_rng(11)
    t = lambda a, d=dt: Hn.dev(a, d, DEV)  # noqa: E731
    d_out = t(r.standard_normal((rows, dim)), F32)
    w_down = t(r.standard_normal((dim, ffn)) * 0.02)
    w_gate = t(r.standard_normal((ffn, dim)) * 0.02)
    w_up = t(r.standard_normal((ffn, dim)) * 0.02)
    gate = t(r.standard_normal((rows, ffn)))
    up = t(r.standard_normal((rows, ffn)))
    resid1 = t(r.standard_normal((rows, dim)))
    gffn = t(1 + 0.1 * r.standard_normal(dim), F32)
    hp = t(r.standard_normal((rows, ffn))) if sub else None
    gsub = t(1 + 0.1 * r.standard_normal(ffn), F32) if sub else None
    d_resid = d_out.clone()
    m = lbp()
    m.lorabwd_ffn_backward(d_out, w_down, w_gate, w_up, gate, up, resid1, gffn, d_resid,
                           act=m.ACT_SWIGLU if act == "swiglu" else m.ACT_RELU2,
                           hidden_pre=hp, gamma_sub=gsub)
    torch.cuda.synchronize()
    H = Hn.host
    want = OB.ffn_bwd(H(d_out), H(w_down), H(w_gate), H(w_up), H(gate), H(up), H(resid1),
                      H(gffn), 1e-6, act, hidden_pre=H(hp) if sub else None,
                      gamma_fsub=H(gsub) if sub else None)
    assert Hn.rel_err(H(d_resid), want) <= tol(dt)


# ------------------------------------------------------------------ LoRA
@pytest.mark.parametrize("rows,H,out,rank,step,dt", [
    (16, 64, 64, 4, 1, F32), (300, 256, 96, 16, 1, F32), (129, 64, 40, 7, 5, F32),
    (200, 128, 64, 16, 1, BF16), (0, 64, 32, 4, 2, F32), (77, 520, 37, 33, 1, F32),
    (45, 64, 130, 64, 2, BF16), (1000, 264, 300, 16, 3, F32), (513, 2560, 1024, 24, 1, F32),
    # a row slice whose g (80 rows x rank 64) exceeds the dA launch's LDS
    # slice: the B update runs as a launch of its own
    (600, 8192, 64, 64, 2, F32), (600, 8192, 48, 64, 1, BF16)])
def test_lora_adamw(rows, H, out, rank, step, dt):
    print("lora", rows, H, out, rank, step, dt, flush=True)
    r = np.random.default_rng(12)
    x = r.standard_normal((rows, H))
    A = r.standard_normal((rank, H)) * 0.02
    Bm = r.standard_normal((out, rank)) * 0.02
    dy = r.standard_normal((rows, out))
    cfg = synth.get_config("tiny")
    m_a, v_a = synth.gen.draw_adam_state(cfg, 0, A.shape, 0) if step > 1 else (0 * A, 0 * A)
    m_b, v_b = synth.gen.draw_adam_state(cfg, 0, Bm.shape, 1) if step > 1 else (0 * Bm, 0 * Bm)
    tx = Hn.dev(x, dt, DEV)
    th = Hn.dev(x @ A.T, dt, DEV)
    T = {k: Hn.dev(v, F32, DEV) for k, v in dict(A=A, B=Bm, m_a=m_a, v_a=v_a, m_b=m_b, v_b=v_b).items()}
    tdy = Hn.dev(dy, F32, DEV)
    ga = torch.empty(rank, H, device=DEV)
    gb = torch.empty(out, rank, device=DEV)
    gn = torch.full((1,), 0.5, device=DEV)
    alpha, lr, lr_b = 2.0 * rank, 1e-3, 1.6e-2
    lbp().lorabwd_lora_grad_adamw(tdy, tx, th, T["A"], T["B"], T["m_a"], T["v_a"], T["m_b"],
                                  T["v_b"], alpha, lr, lr_b, step=step, grad_a=ga, grad_b=gb,
                                  gnorm_sq=gn)
    torch.cuda.synchronize()
    hx, hh = Hn.host(tx), Hn.host(th)
    dA, dB = OB.lora_grads(dy if rows else np.zeros((0, out)), hh, hx, Bm, alpha, rank)
    tl = tol(dt)
    if rows:
        assert Hn.rel_err(Hn.host(ga), dA) <= tl
        assert Hn.rel_err(Hn.host(gb), dB) <= tl
    nA, mA, vA = OB.adamw(A, dA, m_a, v_a, lr, 0.9, 0.999, 1e-8, 0.01, step)
    nB, mB, vB = OB.adamw(Bm, dB, m_b, v_b, lr_b, 0.9, 0.999, 1e-8, 0.01, step)
    assert Hn.update_err(Hn.host(T["A"]), nA, dA, lr, tl) <= tl
    assert Hn.update_err(Hn.host(T["B"]), nB, dB, lr_b, tl) <= tl
    for k, w in (("m_a", mA), ("v_a", vA), ("m_b", mB), ("v_b", vB)):
        assert Hn.rel_err(Hn.host(T[k]), w) <= tl or np.max(np.abs(w)) == 0
    assert Hn.rel_err(Hn.host(gn), [0.5 + np.sum(dA * dA)]) <= tl


# ------------------------------------------------------------------ whole layer, small
@pytest.mark.parametrize("name,over", [
    ("tiny", {}),
    ("tiny", {"seq": 45, "kv_len": 45}),                          # ragged
    ("tiny", {"dtype": "bf16"}),
    ("decode", {"hidden": 128, "ffn": 256, "n_heads": 4, "n_kv_heads": 2, "head_dim": 32,
                "kv_len": 70, "pos0": 69}),
    # 19 key chunks, ragged
    ("decode", {"hidden": 256, "ffn": 512, "n_heads": 8, "n_kv_heads": 2, "head_dim": 64,
                "kv_len": 300, "pos0": 299}),
    # six heads per KV head (dV takes a second block of heads), W_o's second
    # column block ragged
    ("decode", {"hidden": 192, "ffn": 384, "n_heads": 12, "n_kv_heads": 2, "head_dim": 32,
                "kv_len": 40, "pos0": 39}),
    ("decode", {"hidden": 256, "ffn": 512, "n_heads": 8, "n_kv_heads": 2, "head_dim": 128,
                "kv_len": 130, "pos0": 129, "dtype": "bf16"}),
    ("decode", {"hidden": 256, "ffn": 512, "n_heads": 8, "n_kv_heads": 4, "head_dim": 64,
                "kv_len": 97, "pos0": 96, "sub_norms": 0, "act": "swiglu"}),
    ("seq512", {"seq": 80, "kv_len": 80, "hidden": 256, "ffn": 512, "n_heads": 4,
                "n_kv_heads": 1, "head_dim": 64, "rank": 8, "alpha": 16.0}),
    # bf16 sequence attention with the inverse RoPE in the dq kernel, late positions
    ("seq512", {"seq": 96, "kv_len": 96, "hidden": 256, "ffn": 512, "n_heads": 8,
                "n_kv_heads": 2, "head_dim": 64, "rank": 8, "alpha": 16.0, "dtype": "bf16",
                "pos0": 1900}),
    ("seq512", {"seq": 70, "kv_len": 70, "hidden": 256, "ffn": 512, "n_heads": 4,
                "n_kv_heads": 2, "head_dim": 128, "rank": 4, "alpha": 8.0, "pos0": 3000}),
    # bf16, whole 64-query blocks: the W_o product also writes dCtxᵀ for dV
    ("seq512", {"seq": 128, "kv_len": 128, "hidden": 256, "ffn": 512, "n_heads": 8,
                "n_kv_heads": 2, "head_dim": 128, "rank": 8, "alpha": 16.0, "dtype": "bf16"}),
    # a chunk of tokens after a cached prefix (kv_len > seq) with both
    # adapters: the value adapter takes the chunk's last rows of dV
    ("seq512", {"seq": 40, "kv_len": 100, "pos0": 60, "hidden": 256, "ffn": 512, "n_heads": 4,
                "n_kv_heads": 2, "head_dim": 64, "rank": 8, "alpha": 16.0}),
    ("seq512", {"seq": 64, "kv_len": 200, "pos0": 136, "hidden": 256, "ffn": 512,
                "n_heads": 8, "n_kv_heads": 2, "head_dim": 128, "rank": 8, "alpha": 16.0,
                "dtype": "bf16"}),
    # one token against a cache too long for the single-token attention
    # kernels' LDS: the general composition with one query row
    ("decode", {"hidden": 128, "ffn": 256, "n_heads": 4, "n_kv_heads": 2, "head_dim": 32,
                "kv_len": 16400, "pos0": 16399}),
    # QK-norm: the per-head norm backward after the inverse RoPE, fused into
    # the standalone RoPE launch (tiny, bf16), into the launch that adds the
    # dV chunk partials (fp32 sequence), and after the single-token attention
    ("tiny", {"qk_norm": True, "pos0": 9}),
    ("seq512", {"seq": 100, "kv_len": 100, "hidden": 256, "ffn": 512, "n_heads": 8,
                "n_kv_heads": 2, "head_dim": 128, "rank": 8, "alpha": 16.0, "qk_norm": True}),
    ("seq512", {"seq": 96, "kv_len": 96, "hidden": 256, "ffn": 512, "n_heads": 8,
                "n_kv_heads": 2, "head_dim": 64, "rank": 8, "alpha": 16.0, "dtype": "bf16",
                "qk_norm": True, "pos0": 700}),
    ("decode", {"hidden": 256, "ffn": 512, "n_heads": 8, "n_kv_heads": 2, "head_dim": 64,
                "kv_len": 130, "pos0": 129, "qk_norm": True}),
    # the exact input gradient through the attention branch (dK = scale dS^T Q
    # from the dQ kernels' stored dS, the transposed Q/K/V products, the
    # adapters' terms and the attention-norm backward): fp32 with ragged
    # tiles, with QK-norm, after a cached prefix, non-causal; bf16
    ("tiny", {"input_grad": True}),
    ("tiny", {"input_grad": True, "seq": 45, "kv_len": 45}),
    ("seq512", {"seq": 100, "kv_len": 100, "hidden": 256, "ffn": 512, "n_heads": 8,
                "n_kv_heads": 2, "head_dim": 128, "rank": 8, "alpha": 16.0, "input_grad": True,
                "qk_norm": True, "pos0": 33}),
    ("seq512", {"seq": 40, "kv_len": 100, "pos0": 60, "hidden": 256, "ffn": 512, "n_heads": 4,
                "n_kv_heads": 2, "head_dim": 64, "rank": 8, "alpha": 16.0, "input_grad": True}),
    ("seq512", {"seq": 70, "kv_len": 70, "hidden": 256, "ffn": 512, "n_heads": 4,
                "n_kv_heads": 4, "head_dim": 32, "rank": 0, "causal": False, "input_grad": True}),
    ("seq512", {"seq": 128, "kv_len": 128, "hidden": 256, "ffn": 512, "n_heads": 8,
                "n_kv_heads": 2, "head_dim": 128, "rank": 8, "alpha": 16.0, "dtype": "bf16",
                "input_grad": True}),
    ("seq512", {"seq": 96, "kv_len": 96, "hidden": 256, "ffn": 512, "n_heads": 8,
                "n_kv_heads": 2, "head_dim": 64, "rank": 8, "alpha": 16.0, "dtype": "bf16",
                "input_grad": True, "qk_norm": True, "pos0": 300}),
    # one token after a 39-row prefix: the general composition with one query
    # row (a single key would make the softmax constant and dQ identically 0)
    ("seq512", {"seq": 1, "kv_len": 40, "pos0": 39, "hidden": 256, "ffn": 512, "n_heads": 4,
                "n_kv_heads": 2, "head_dim": 64, "rank": 4, "alpha": 8.0, "input_grad": True}),
    # bf16 products on the wide 256 x 256 kernel inside the layer (gate/up,
    # W_down with its activation epilogue, the three transposed input-gradient
    # products), ragged rows
    ("seq512", {"seq": 520, "kv_len": 520, "hidden": 512, "ffn": 1024, "n_heads": 8,
                "n_kv_heads": 2, "head_dim": 64, "rank": 8, "alpha": 16.0, "dtype": "bf16",
                "input_grad": True}),
])
def test_layer_small(name, over):
    cfg = synth.get_config(name).with_(**over)
    print("layer", cfg, flush=True)
    errs = Hn.layer_parity(cfg, DEV)
    bad = {k: v for k, v in errs.items() if not v <= Hn.TOL[cfg.dtype]}
    assert not bad, bad


@pytest.mark.parametrize("name,over", [
    ("decode", {"hidden": 256, "ffn": 512, "n_heads": 8, "n_kv_heads": 2, "head_dim": 64,
                "kv_len": 300, "pos0": 299}),
    ("tiny", {"seq": 45, "kv_len": 45}),
    ("tiny", {"dtype": "bf16"}),
])
def test_layer_out_of_place(name, over):
    """A separate d_out gives bitwise the in-place results and is not written."""
    cfg = synth.get_config(name).with_(**over)
    outs = []
    for oop in (False, True):
        dl = Hn.DeviceLayer(cfg, 0, DEV)
        dq = torch.empty(cfg.seq, cfg.q_dim, device=DEV)
        dv = torch.empty(cfg.kv_len, cfg.kv_dim, device=DEV)
        g = torch.zeros(1, device=DEV)
        if oop:
            d_in = dl.d_out.clone()
            d = torch.full_like(d_in, float("nan"))
            dl.run_gpu(d, dq, dv, g, d_out=d_in)
            torch.cuda.synchronize()
            assert torch.equal(d_in, dl.d_out)
        else:
            d = dl.d_out.clone()
            dl.run_gpu(d, dq, dv, g)
        torch.cuda.synchronize()
        o = [d.cpu(), dq.cpu(), dv.cpu(), g.cpu()]
        if dl.lora:
            o += [dl.lora[t][k].cpu() for t in ("q", "v") for k in ("A", "B")]
        outs.append(o)
    for a, b in zip(*outs):
        assert torch.equal(a, b)


@pytest.mark.parametrize("name,over", [
    ("decode", {}),                                   # the benchmark's workload
    ("tiny", {"seq": 70, "kv_len": 70}),              # LoRA state advances each call
    ("tiny", {"dtype": "bf16", "seq": 96, "kv_len": 96}),
])
def test_layer_graph_replay(name, over):
    """The layer captured once in a HIP graph and replayed (as the benchmark
    times it) matches eager calls bitwise, replay after replay, with eager
    work and synchronisation between the replays."""
    cfg = synth.get_config(name).with_(**over)
    sides = []
    for _ in range(2):
        dl = Hn.DeviceLayer(cfg, 0, DEV)
        bufs = {"d_in": dl.d_out.clone(), "d": torch.empty_like(dl.d_out),
                "dq": torch.empty(cfg.seq, cfg.q_dim, device=DEV),
                "dv": torch.empty(cfg.kv_len, cfg.kv_dim, device=DEV),
                "g": torch.zeros(1, device=DEV)}
        sides.append((dl, bufs))

    def call(side):
        dl, b = side
        dl.run_gpu(b["d"], b["dq"], b["dv"], b["g"], d_out=b["d_in"])

    # one eager call each first (sizes the workspace before the capture)
    for side in sides:
        call(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(sides[1])
    torch.cuda.synchronize()

    def state(side):
        dl, b = side
        o = [b[k].cpu() for k in ("d", "dq", "dv", "g")]
        if dl.lora:
            o += [dl.lora[t][k].cpu() for t in ("q", "v") for k in ("A", "B", "m_a", "v_b")]
        return o

    for rep in range(3):
        for side in sides:
            side[1]["g"].zero_()
            side[1]["d"].fill_(float("nan"))
        torch.cuda.synchronize()
        call(sides[0])
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(state(sides[0]), state(sides[1])):
            assert torch.equal(a, b), rep


def test_layer_deterministic():
    cfg = synth.get_config("tiny").with_(seq=70, kv_len=70)
    outs = []
    for _ in range(2):
        dl = Hn.DeviceLayer(cfg, 0, DEV)
        d = dl.d_out.clone()
        g = torch.zeros(1, device=DEV)
        dl.run_gpu(d, gnorm=g)
        torch.cuda.synchronize()
        outs.append((d.cpu(), g.cpu(), dl.lora["q"]["A"].cpu(), dl.lora["v"]["B"].cpu()))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


# ------------------------------------------------------------------ packed ternary weights
@pytest.mark.parametrize("rows,cols,dt", [(7, 24, "f32"), (33, 64, "bf16"), (1, 8, "f32")])
def test_pack_ternary_bytes(rows, cols, dt):
    """lorabwd_pack_ternary equals the oracle's packing byte for byte."""
    import layer_backward_pass_amd as lbp
    from oracle import bitlinear as BL
    r = np.random.default_rng(rows + cols)
    w = 0.02 * r.integers(-1, 2, size=(rows, cols))
    wd = torch.tensor(w, dtype=torch.float32 if dt == "f32" else torch.bfloat16, device=DEV)
    pk = lbp.lorabwd_pack_ternary(wd)
    torch.cuda.synchronize()
    assert np.array_equal(pk.cpu().numpy(), BL.pack_ternary(Hn.host(wd)))


@pytest.mark.parametrize("over", [
    {"hidden": 256, "ffn": 512, "n_heads": 8, "n_kv_heads": 2, "head_dim": 64, "kv_len": 300,
     "pos0": 299},
    {"hidden": 192, "ffn": 384, "n_heads": 12, "n_kv_heads": 2, "head_dim": 32, "kv_len": 40,
     "pos0": 39},
    {"hidden": 256, "ffn": 512, "n_heads": 8, "n_kv_heads": 2, "head_dim": 128, "kv_len": 130,
     "pos0": 129, "dtype": "bf16"},
    {"hidden": 256, "ffn": 512, "n_heads": 8, "n_kv_heads": 4, "head_dim": 64, "kv_len": 97,
     "pos0": 96, "sub_norms": 0, "act": "swiglu"},
])
def test_layer_packed_ternary_small(over):
    """The single-token layer on packed ternary weights (the three GEMV
    streams decode 2-bit codes) against the oracle on the dense values."""
    cfg = synth.get_config("decode").with_(**over)
    print("packed layer", cfg, flush=True)
    errs = Hn.packed_layer_parity(cfg, DEV, check_bytes=True)
    bad = {k: v for k, v in errs.items() if not v <= Hn.TOL[cfg.dtype]}
    assert not bad, bad


# ------------------------------------------------------------------ lm_head
LM = synth.get_config("lmhead")


@pytest.mark.parametrize("over,kw", [
    # ragged everywhere: 37 rows (not a multiple of 4: the dW product's k
    # tail), 1000 vocabulary rows (7 whole 128-row tiles and a tail), hidden
    # below one column tile; every fifth row ignored, one label = vocab
    ({"rows": 37, "hidden": 64, "vocab": 1000, "ignore_every": 5}, {"labels": "with_vocab"}),
    # split-K grad_hidden, ragged column tiles (520 = 2 * 256 + 8), a later
    # AdamW step with non-zero moments
    ({"rows": 300, "hidden": 520, "vocab": 4100, "step": 3}, {"state": True}),
    # one row, the 32-entry vocabulary of the gradient-flow example
    ({"rows": 1, "hidden": 64, "vocab": 32}, {}),
    # vocabulary entries excluded from the softmax (-inf logits)
    ({"rows": 66, "hidden": 128, "vocab": 2048}, {"inf_cols": 100}),
    # every row ignored: loss and gradients 0, AdamW steps on a zero gradient
    ({"rows": 20, "hidden": 64, "vocab": 256}, {"labels": "none", "state": True}),
    # no rows at all
    ({"rows": 0, "hidden": 64, "vocab": 256}, {}),
    # the smallest shapes the boundary takes: hidden 8, vocabulary 4
    ({"rows": 3, "hidden": 8, "vocab": 4}, {"state": True}),
])
def test_lm_head(over, kw):
    cfg = LM.with_(**over)
    kw = dict(kw)
    if kw.get("labels") == "with_vocab":
        lab = synth.draw_lm_head(cfg)["labels"].copy()
        lab[1] = cfg.vocab
        lab[2] = -7
        kw["labels"] = lab
    elif kw.get("labels") == "none":
        kw["labels"] = np.full(cfg.rows, -100, np.int32)
    errs = Hn.lm_head_parity(cfg, DEV, **kw)
    bad = {k: v for k, v in errs.items() if not v <= Hn.TOL["f32"]}
    assert not bad, bad


def test_lm_head_deterministic():
    """Two calls on the same inputs give bitwise the same outputs."""
    import layer_backward_pass_amd as lbp
    cfg = LM.with_(rows=130, hidden=256, vocab=3000)
    d = synth.draw_lm_head(cfg)
    outs = []
    for _ in range(2):
        T = {k: torch.from_numpy(v).to(DEV) for k, v in d.items()}
        gh = torch.empty((cfg.rows, cfg.hidden), device=DEV)
        loss = torch.empty(1, device=DEV)
        lbp.lorabwd_lm_head_backward(T["h"], T["logits"], T["labels"], T["W"], T["m"], T["v"], gh,
                                     loss, lr=1e-3)
        torch.cuda.synchronize()
        outs.append((gh.cpu(), loss.cpu(), T["W"].cpu(), T["v"].cpu()))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_lm_head_graph_replay():
    """The lm_head backward captured once in a HIP graph and replayed matches
    eager calls bitwise, step after step (the AdamW state of each side
    advances in lockstep), with eager work and synchronisation between the
    replays; 300 rows so the cross-entropy workgroups take several rows."""
    import layer_backward_pass_amd as lbp
    cfg = LM.with_(rows=300, hidden=264, vocab=3000, ignore_every=7)
    d = synth.draw_lm_head(cfg)
    sides = []
    for _ in range(2):
        T = {k: torch.from_numpy(v).to(DEV) for k, v in d.items()}
        T["gh"] = torch.empty((cfg.rows, cfg.hidden), device=DEV)
        T["loss"] = torch.empty(1, device=DEV)
        T["gw"] = torch.empty((cfg.vocab, cfg.hidden), device=DEV)
        sides.append(T)

    def call(T, step):
        lbp.lorabwd_lm_head_backward(T["h"], T["logits"], T["labels"], T["W"], T["m"], T["v"],
                                     T["gh"], T["loss"], lr=1e-3, step=step, grad_w=T["gw"])

    # one eager call each first (sizes the workspace before the capture)
    for T in sides:
        call(T, 1)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(sides[1], 2)
    torch.cuda.synchronize()
    for rep in range(3):
        for T in sides:
            T["gh"].fill_(float("nan"))
            T["gw"].fill_(float("nan"))
        torch.cuda.synchronize()
        call(sides[0], 2)
        graph.replay()
        torch.cuda.synchronize()
        for k in ("gh", "loss", "gw", "W", "m", "v"):
            assert torch.equal(sides[0][k].cpu(), sides[1][k].cpu()), (rep, k)
