"""Shared helpers of the GPU parity tests and the smoke check.

Seeded draws (synth) go through the oracle's float64 forward to become
consistent saved activations; those are cast to the storage dtype on the
GPU, and the oracle then runs on exactly the values the GPU received (read
back and widened to float64).  GPU results come through the C-ABI binding.

Error measure, per output tensor: ||gpu - oracle||_inf / ||oracle||_inf.
Bound: 1e-4 for float32 inputs, 2e-2 for bf16 inputs.

AdamW after one step is p - lr (sign(g) + wd p) up to eps, which jumps where
g crosses zero; an element whose oracle gradient is within the gradient
tolerance (bound * ||g||_inf) of zero may take either sign.  Updated
parameters are therefore compared at the bound on elements with
|g| >= 2 * bound * ||g||_inf, and within 2 lr + bound elsewhere.  Moments
m, v (continuous in g) use the plain bound.
"""
import numpy as np

import synth
from oracle import backward as OB
from oracle import forward as OF

TOL = {"f32": 1e-4, "bf16": 2e-2}


def _torch():
    import torch
    return torch


def tdtype(cfg):
    torch = _torch()
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def dev(a, dtype, device):
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(a, np.float64)).to(device=device, dtype=dtype)


def host(t):
    """Device tensor -> float64 numpy (exactly the values the GPU holds)."""
    return t.detach().to(dtype=_torch().float64).cpu().numpy()


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = float(np.max(np.abs(b))) if b.size else 0.0
    num = float(np.max(np.abs(a - b))) if b.size else 0.0
    return num / den if den > 0 else num


def update_err(p_gpu, p_or, g_or, lr, tol):
    """Error of an AdamW-updated tensor, scaled so that <= tol passes (see
    the module docstring)."""
    p_gpu = np.asarray(p_gpu, np.float64)
    p_or = np.asarray(p_or, np.float64)
    g_or = np.asarray(g_or, np.float64)
    scale = max(float(np.max(np.abs(p_or))), 1e-30)
    gmax = float(np.max(np.abs(g_or))) if g_or.size else 0.0
    diff = np.abs(p_gpu - p_or)
    firm = np.abs(g_or) >= 2.0 * tol * gmax
    e1 = float(np.max(diff[firm])) / scale if firm.any() else 0.0
    loose = ~firm
    e2 = 0.0
    if loose.any():
        e2 = float(np.max(diff[loose])) / (2.0 * lr + tol * scale) * tol
    return max(e1, e2)


def f32_scalars(cfg):
    """The config with every scalar the C ABI takes as float rounded to
    float32, so the oracle sees the values the GPU receives."""
    r = lambda x: float(np.float32(x))  # noqa: E731
    c = cfg.with_(eps=r(cfg.eps), rope_base=r(cfg.rope_base), alpha=r(cfg.alpha), lr=r(cfg.lr),
                  beta1=r(cfg.beta1), beta2=r(cfg.beta2), adam_eps=r(cfg.adam_eps),
                  weight_decay=r(cfg.weight_decay), lr_b_ratio=1.0)
    object.__setattr__(c, "_lr_b", r(cfg.lr_b))
    object.__setattr__(c, "_scale", r(cfg.scale))
    return c


WEIGHTS = ("W_o", "W_gate", "W_up", "W_down")
SAVED = ("attn_input", "resid1", "gate", "up", "hidden_pre", "ctx", "P", "K", "V",
         "lora_q_h", "lora_v_h", "q_raw")
# the attention input gradient's extra weights and saved tensors
IG_WEIGHTS = ("W_q", "W_k", "W_v")
IG_SAVED = ("x", "q", "k_raw")


def desc_of(c):
    """The C-ABI layer descriptor of a workload config."""
    import layer_backward_pass_amd as lbp
    return lbp.make_desc(c.seq, c.kv_len, c.hidden, c.ffn, c.n_heads, c.n_kv_heads,
                         c.head_dim, act=lbp.ACT_SWIGLU if c.act == "swiglu" else lbp.ACT_RELU2,
                         sub_norms=c.sub_norms, causal=c.causal,
                         dtype=lbp.BF16 if c.dtype == "bf16" else lbp.F32, pos0=c.pos0,
                         eps=c.eps, rope_base=c.rope_base, attn_scale=c.scale,
                         lora_alpha=c.alpha, qk_norm=c.qk_norm, input_grad=c.input_grad,
                         weight_format=1 if c.packed else 0)


class DeviceLayer:
    """One layer's weights, saved activations and LoRA state on the GPU, plus
    the float64 copies the oracle reads."""

    def __init__(self, cfg, layer=0, device="cuda:0", host_dtype=np.float64):
        torch = _torch()
        self.cfg = cfg
        draws = synth.draw_layer(cfg, layer)
        w, saved, lora = OF.make_layer(cfg, draws)
        dt = tdtype(cfg)
        f32 = torch.float32
        ig = cfg.input_grad
        self.w = {k.lower(): dev(w[k], dt, device) for k in WEIGHTS + (IG_WEIGHTS if ig else ())}
        gammas = ("gamma_ffn", "gamma_fsub", "gamma_asub", "gamma_q")
        for k in gammas + (("gamma_attn", "gamma_k") if ig else ()):
            if k in w:
                self.w[k] = dev(w[k], f32, device)
        self.saved = {k: dev(saved[k], dt, device) for k in SAVED + (IG_SAVED if ig else ())
                      if k in saved}
        self.d_out = dev(draws["d_out"], f32, device)
        self.lora = None
        if lora is not None:
            self.lora = {}
            for tag in ("q", "v"):
                self.lora[tag] = {
                    "A": dev(lora["A_" + tag], f32, device), "B": dev(lora["B_" + tag], f32, device),
                    "m_a": dev(lora["m_A_" + tag], f32, device),
                    "v_a": dev(lora["v_A_" + tag], f32, device),
                    "m_b": dev(lora["m_B_" + tag], f32, device),
                    "v_b": dev(lora["v_B_" + tag], f32, device)}
        # oracle copies: exactly what the GPU holds (float32 host copies are
        # exact for float32 and bf16 device values; the oracle widens them)
        hc = lambda t: host(t).astype(host_dtype)  # noqa: E731
        self.o_w = {("W_" + k[2:] if k.startswith("w_") else k): hc(v)
                    for k, v in self.w.items()}
        self.o_saved = {k: hc(v) for k, v in self.saved.items()}
        self.o_dout = hc(self.d_out)
        self.o_lora = None
        if self.lora is not None:
            self.o_lora = {}
            for tag, st in self.lora.items():
                self.o_lora["A_" + tag] = hc(st["A"])
                self.o_lora["B_" + tag] = hc(st["B"])
                self.o_lora["m_A_" + tag] = hc(st["m_a"])
                self.o_lora["v_A_" + tag] = hc(st["v_a"])
                self.o_lora["m_B_" + tag] = hc(st["m_b"])
                self.o_lora["v_B_" + tag] = hc(st["v_b"])

    def desc(self):
        return desc_of(self.cfg)

    def adamw(self):
        import layer_backward_pass_amd as lbp
        c = self.cfg
        return lbp.AdamW(c.lr, c.lr_b, c.beta1, c.beta2, c.adam_eps, c.weight_decay, c.step)

    def run_gpu(self, d_hidden, dq_pre=None, dv=None, gnorm=None, d_out=None):
        import layer_backward_pass_amd as lbp
        return lbp.lorabwd_layer_backward(
            self.desc(), self.w, self.saved, d_hidden,
            q_state=self.lora["q"] if self.lora else None,
            v_state=self.lora["v"] if self.lora else None,
            adamw=self.adamw() if self.lora else None, dq_pre_out=dq_pre, dv_out=dv,
            gnorm_sq=gnorm, d_out=d_out)

    def run_oracle(self, d_out):
        return OB.layer_bwd(f32_scalars(self.cfg), self.o_w, self.o_saved, d_out, self.o_lora)


def compare_lora(cfg, dl, ref, tol):
    """Errors of the updated LoRA tensors of one layer against the oracle."""
    errs = {}
    for tag in ("q", "v"):
        st = dl.lora[tag]
        errs["A_" + tag] = update_err(host(st["A"]), ref["A_" + tag], ref["dA_" + tag], cfg.lr, tol)
        errs["B_" + tag] = update_err(host(st["B"]), ref["B_" + tag], ref["dB_" + tag], cfg.lr_b, tol)
        for k, rk in (("m_a", "m_A_"), ("v_a", "v_A_"), ("m_b", "m_B_"), ("v_b", "v_B_")):
            errs[k + "_" + tag] = rel_err(host(st[k]), ref[rk + tag])
    return errs


def layer_parity(cfg, device="cuda:0", layer=0):
    """Run one layer on the GPU and on the oracle; returns {output: rel err}."""
    torch = _torch()
    dl = DeviceLayer(cfg, layer, device)
    ref = dl.run_oracle(dl.o_dout)
    d_hidden = dl.d_out.clone()
    dq_pre = torch.empty(cfg.seq, cfg.q_dim, device=device)
    dv = torch.empty(cfg.kv_len, cfg.kv_dim, device=device)
    gnorm = torch.zeros(1, device=device)
    dl.run_gpu(d_hidden, dq_pre, dv, gnorm)
    torch.cuda.synchronize()
    errs = {"d_hidden": rel_err(host(d_hidden), ref["d_hidden"]),
            "dq_pre": rel_err(host(dq_pre), ref["dq_pre"]),
            "dv": rel_err(host(dv), ref["dv"])}
    if dl.lora is not None:
        errs.update(compare_lora(cfg, dl, ref, TOL[cfg.dtype]))
        errs["gnorm_sq"] = rel_err(host(gnorm), np.array([ref["gnorm_sq"]]))
    return errs


def _layer_call(cfg, d, d_hidden, gnorm):
    import layer_backward_pass_amd as lbp
    desc = lbp.make_desc(cfg.seq, cfg.kv_len, cfg.hidden, cfg.ffn, cfg.n_heads, cfg.n_kv_heads,
                         cfg.head_dim, act=lbp.ACT_SWIGLU if cfg.act == "swiglu" else lbp.ACT_RELU2,
                         sub_norms=cfg.sub_norms, causal=cfg.causal,
                         dtype=lbp.BF16 if cfg.dtype == "bf16" else lbp.F32, pos0=cfg.pos0,
                         eps=cfg.eps, rope_base=cfg.rope_base, attn_scale=cfg.scale,
                         lora_alpha=cfg.alpha)
    hp = lbp.AdamW(cfg.lr, cfg.lr_b, cfg.beta1, cfg.beta2, cfg.adam_eps, cfg.weight_decay, cfg.step)
    lbp.lorabwd_layer_backward(desc, d["weights"], d["saved"], d_hidden, q_state=d["lora"]["q"],
                               v_state=d["lora"]["v"], adamw=hp, gnorm_sq=gnorm)


def stack_parity(cfg, device="cuda:0", log=print):
    """The whole stack on the GPU (layers n-1 .. 0, d_hidden in place), in the
    benchmark's launch configuration, against the oracle's stack backward
    layer by layer in full: every layer's updated LoRA A/B/m/v, the gradient
    norm accumulated over all layers, and the final gradient handed below
    the stack.  The oracle follows its own float64 gradient chain, so errors
    would compound rather than be reset at each layer.
    Inputs are device-drawn (synth.device) except ctx, which the oracle forms
    as P V so that the saved attention tensors are consistent."""
    torch = _torch()
    from synth.device import draw_timing_layer_device
    n = cfg.n_layers
    layers, init_lora = [], []
    for l in range(n):
        d = draw_timing_layer_device(cfg, l, device)
        ctx = OF.context(host(d["saved"]["P"]), host(d["saved"]["V"]), cfg.n_heads,
                         cfg.n_kv_heads)
        d["saved"]["ctx"] = dev(ctx, tdtype(cfg), device)
        init_lora.append({tag: {k: host(v) for k, v in st.items()} for tag, st in d["lora"].items()})
        layers.append(d)
        if l % 6 == 5:
            log("stack: %d layers drawn" % (l + 1))
    grad = layers[-1]["d_out"].clone()
    d_hidden = grad.clone()
    gnorm = torch.zeros(1, device=device)
    for l in range(n - 1, -1, -1):
        _layer_call(cfg, layers[l], d_hidden, gnorm)
    torch.cuda.synchronize()
    log("stack: GPU done")
    tol = TOL[cfg.dtype]
    errs = {}
    oc = f32_scalars(cfg)
    dd = host(grad)
    gsq = 0.0
    for l in range(n - 1, -1, -1):
        d = layers[l]
        w = {("W_" + k[2:] if k.startswith("w_") else k): host(v) for k, v in d["weights"].items()}
        saved = {k: host(v) for k, v in d["saved"].items()}
        lo = {}
        for tag in ("q", "v"):
            st = init_lora[l][tag]
            lo.update({"A_" + tag: st["A"], "B_" + tag: st["B"], "m_A_" + tag: st["m_a"],
                       "v_A_" + tag: st["v_a"], "m_B_" + tag: st["m_b"], "v_B_" + tag: st["v_b"]})
        ref = OB.layer_bwd(oc, w, saved, dd, lo)
        del w, saved

        class _L:  # the GPU-updated state, shaped for compare_lora
            lora = d["lora"]
        for k, v in compare_lora(cfg, _L, ref, tol).items():
            errs["layer%d_%s" % (l, k)] = v
        gsq += ref["gnorm_sq"]
        dd = ref["d_hidden"]
        if l % 6 == 0:
            log("stack: oracle at layer %d" % l)
    errs["d_hidden"] = rel_err(host(d_hidden), dd)
    errs["gnorm_sq"] = rel_err(host(gnorm), np.array([gsq]))
    log("stack: %d layers compared" % n)
    return errs


PACKED = ("w_o", "w_gate", "w_up", "w_down")


def pack_layer_weights(dl, check_bytes):
    """The layer's ternary weights packed on the GPU (lorabwd_pack_ternary),
    with their scale (the magnitude of the stored nonzero values).  Every
    packed matrix is checked on the host: unpacked by the oracle it gives the
    signs of the dense matrix and holds no unused code; with check_bytes the
    bytes also equal the oracle's packing of the same matrix."""
    import layer_backward_pass_amd as lbp
    from oracle import bitlinear as BL
    out = {}
    for k in PACKED:
        wd = dl.w[k]
        pk = lbp.lorabwd_pack_ternary(wd)
        _torch().cuda.synchronize()
        hw = host(wd)
        hp = pk.cpu().numpy()
        assert np.array_equal(BL.unpack_ternary(hp, hw.shape[1]), np.sign(hw)), k
        for j in range(4):
            assert not np.any(((hp >> (2 * j)) & 3) == 2), k
        if check_bytes:
            assert np.array_equal(hp, BL.pack_ternary(hw)), k
        nz = np.abs(hw[hw != 0])
        assert nz.size and np.all(nz == nz[0]), k  # one scale per matrix
        out[k] = pk
        out["scale_" + k[2:]] = float(nz[0])
    return out


def packed_layer_parity(cfg, device="cuda:0", check_bytes=True):
    """The single-token layer with its ternary weights packed (weight_format
    1) against the float64 oracle on the dense values."""
    torch = _torch()
    dl = DeviceLayer(cfg.with_(packed=False), 0, device)
    ref = dl.run_oracle(dl.o_dout)
    pw = pack_layer_weights(dl, check_bytes)
    wts = dict(dl.w)
    wts.update(pw)
    import layer_backward_pass_amd as lbp
    d_hidden = torch.empty_like(dl.d_out)
    dq_pre = torch.empty(cfg.seq, cfg.q_dim, device=device)
    dv = torch.empty(cfg.kv_len, cfg.kv_dim, device=device)
    lbp.lorabwd_layer_backward(desc_of(cfg.with_(packed=True)), wts, dl.saved, d_hidden,
                               dq_pre_out=dq_pre, dv_out=dv, d_out=dl.d_out)
    torch.cuda.synchronize()
    return {"d_hidden": rel_err(host(d_hidden), ref["d_hidden"]),
            "dq_pre": rel_err(host(dq_pre), ref["dq_pre"]), "dv": rel_err(host(dv), ref["dv"])}


# ------------------------------------------------------------------ lm_head
def lm_head_parity(cfg, device="cuda:0", state=False, inf_cols=0, labels=None, full=False,
                   log=print):
    """lorabwd_lm_head_backward against the oracle.  Small shapes: every
    output against lm_head_bwd.  full=True (the workload's own size, drawn on
    the device): the loss, grad_hidden at sampled rows, and dW, W, m, v at
    sampled vocabulary rows, against the oracle's block-wise form.  state:
    non-zero AdamW moments (a later step); inf_cols: that many vocabulary
    entries excluded from the softmax (-inf logits, never a label)."""
    torch = _torch()
    import layer_backward_pass_amd as lbp
    from oracle import lmhead as LM
    S, H, V = cfg.rows, cfg.hidden, cfg.vocab
    if full:
        from synth.device import draw_lm_head_device
        T = draw_lm_head_device(cfg, 0, device)
    else:
        d = synth.draw_lm_head(cfg)
        T = {k: torch.from_numpy(np.ascontiguousarray(v)).to(device) for k, v in d.items()}
    if labels is not None:
        T["labels"] = torch.as_tensor(np.asarray(labels, np.int32), device=device)
    if state:
        m, v = synth.gen.draw_adam_state(cfg, 0, (V, H), 0)
        T["m"] = torch.from_numpy(m.astype(np.float32)).to(device)
        T["v"] = torch.from_numpy(v.astype(np.float32)).to(device)
    if inf_cols:
        lab = set(T["labels"].cpu().numpy().tolist())
        cols = [c for c in range(V - 1, -1, -3) if c not in lab][:inf_cols]
        T["logits"][:, cols] = float("-inf")
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    if full:
        rows = np.unique(np.concatenate([[0, S - 1], rng.integers(0, S, 14)]))
        lab_h = T["labels"].cpu().numpy()
        cols = np.unique(np.concatenate([[0, V - 1], lab_h[rows[:8]], rng.integers(0, V, 48)]))
        cols = cols[(cols >= 0) & (cols < V)]
        W0 = T["W"].cpu().numpy()  # float32, before the update
        m0 = host(T["m"][torch.as_tensor(cols, device=device)])
        v0 = host(T["v"][torch.as_tensor(cols, device=device)])
    else:
        pre = {k: host(T[k]) for k in ("h", "logits", "W", "m", "v")}
        pre["labels"] = T["labels"].cpu().numpy()
    gh = torch.empty((S, H), device=device)
    loss = torch.full((1,), 123.0, device=device)
    gw = None if full else torch.empty((V, H), device=device)
    hp = dict(lr=cfg.lr, beta1=cfg.beta1, beta2=cfg.beta2, eps=cfg.adam_eps,
              weight_decay=cfg.weight_decay, step=cfg.step)
    log("lm_head S=%d H=%d V=%d state=%s inf_cols=%d full=%s" % (S, H, V, state, inf_cols, full))
    lbp.lorabwd_lm_head_backward(T["h"], T["logits"], T["labels"], T["W"], T["m"], T["v"], gh,
                                 loss, grad_w=gw, **hp)
    torch.cuda.synchronize()
    f = lambda x: float(np.float32(x))  # noqa: E731  (the scalars the GPU received)
    adam = (f(cfg.lr), f(cfg.beta1), f(cfg.beta2), f(cfg.adam_eps), f(cfg.weight_decay), cfg.step)
    errs = {}
    if full:
        ref = LM.lm_head_sampled(host(T["h"]), T["logits"].cpu().numpy(), lab_h, W0, rows, cols)
        errs["loss"] = rel_err(host(loss), [ref["loss"]])
        errs["grad_hidden"] = rel_err(host(gh)[rows], ref["grad_hidden"])
        nW, nm, nv = OB.adamw(W0[cols], ref["dW"], m0, v0, *adam)
        ci = torch.as_tensor(cols, device=device)
        errs["W"] = update_err(host(T["W"][ci]), nW, ref["dW"], adam[0], TOL["f32"])
        errs["m"] = rel_err(host(T["m"][ci]), nm)
        errs["v"] = rel_err(host(T["v"][ci]), nv)
        return errs
    ref = LM.lm_head_bwd(pre["h"], pre["logits"], pre["labels"], pre["W"], pre["m"], pre["v"],
                         *adam)
    errs["loss"] = rel_err(host(loss), [ref["loss"]])
    errs["grad_hidden"] = rel_err(host(gh), ref["grad_hidden"])
    errs["grad_w"] = rel_err(host(gw), ref["dW"])
    errs["W"] = update_err(host(T["W"]), ref["W"], ref["dW"], adam[0], TOL["f32"])
    errs["m"] = rel_err(host(T["m"]), ref["m"])
    errs["v"] = rel_err(host(T["v"]), ref["v"])
    return errs
