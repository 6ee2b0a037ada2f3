"""Float64 forward of the layer whose backward the oracle computes.

TEST INFRASTRUCTURE ONLY.  It has two jobs: turn seeded draws into saved
activations that are consistent with one another (softmax rows that sum to
one, context = P V, h = x A^T, ...), and be the scalar function that the
finite-difference pins differentiate.

The layer (pre-norm; [FFN] "Forward" for the FFN half, [ATTN] "Gradient Flow"
read forwards for the attention half, [ENT] LayerActivations for what is
saved):

  x_a    = RMSNorm(x_attn; gamma_attn)            attn_input
  q_pre  = x_a W_q^T + s (x_a A_q^T) B_q^T        LoRA on the Q output, s = alpha/r
  k_pre  = x_a W_k^T
  v      = x_a W_v^T + s (x_a A_v^T) B_v^T        LoRA on the V output
  (qk_norm) q_pre, k_pre = HeadNorm(q_pre; gamma_q), HeadNorm(k_pre; gamma_k):
                   RMSNorm over each head's head_dim features, one scale
                   vector of head_dim shared by the heads (the trainer saves Q
                   and K "after QK-norm + RoPE")
  q, k   = RoPE(q_pre), RoPE(k_pre)               NeoX split-half, row i at pos0+i
  P_h    = softmax(scale q_h k_g^T + causal mask) scale = 1/sqrt(D)
  ctx    = P V                                    per head
  c      = RMSNorm(ctx; gamma_asub) or ctx        attention sub-norm (decode layer)
  h1     = x_res + c W_o^T                        residual1 (pre FFN-norm)
  n2     = RMSNorm(h1; gamma_ffn)
  gate, up = n2 W_gate^T, n2 W_up^T
  hid    = act(gate, up)                          silu(g)*u or max(0,g)^2*u
  f      = RMSNorm(hid; gamma_fsub) or hid        FFN sub-norm (decode layer)
  out    = h1 + f W_down^T

x_attn is x_res held fixed (the stop-gradient reading: the gradient passed to
the layer below flows through the residual stream only).  In the decode layer
the keys and values come from a cache whose last slot is the current token,
and there are no adapters.  A chunk of S tokens after a cached prefix
(K_prefix, V_prefix: the prefix's post-RoPE keys and its values, held fixed)
attends to the prefix rows followed by its own; the adapters act on the
chunk's own projections only.
"""
import numpy as np


def rmsnorm(x, gamma, eps):
    x = np.asarray(x, np.float64)
    r = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x / r * np.asarray(gamma, np.float64)


def rope(x, n_heads, head_dim, positions, base):
    """Forward NeoX rotation R(theta): y[d] = x[d]cos - x[d+half]sin,
    y[d+half] = x[d]sin + x[d+half]cos."""
    x = np.asarray(x, np.float64)
    rows = x.shape[0]
    half = head_dim // 2
    freq = np.array([float(base) ** (-(2.0 * d) / head_dim) for d in range(half)])
    th = np.outer(np.asarray(positions, np.float64), freq)
    c, s = np.cos(th)[:, None, :], np.sin(th)[:, None, :]
    y = x.reshape(rows, n_heads, head_dim)
    lo, hi = y[..., :half], y[..., half:]
    out = np.empty_like(y)
    out[..., :half] = lo * c - hi * s
    out[..., half:] = lo * s + hi * c
    return out.reshape(rows, n_heads * head_dim)


def head_rmsnorm(x, n_heads, gamma, eps):
    """RMSNorm over each head's slice of a [rows, n_heads*head_dim] tensor,
    with one scale vector gamma [head_dim] for every head."""
    x = np.asarray(x, np.float64)
    rows = x.shape[0]
    y = rmsnorm(x.reshape(rows, n_heads, -1), gamma, eps)
    return y.reshape(rows, -1)


def act_fwd(act, gate, up):
    if act == "swiglu":
        return gate / (1.0 + np.exp(-gate)) * up
    if act == "relu2":
        r = np.maximum(gate, 0.0)
        return r * r * up
    raise ValueError(act)


def causal_mask(s_q, s_kv):
    """True where query i may attend key j: j <= s_kv - s_q + i."""
    i = np.arange(s_q)[:, None]
    j = np.arange(s_kv)[None, :]
    return j <= (s_kv - s_q + i)


def attention(q, k, v, n_heads, n_kv_heads, head_dim, scale, causal):
    s_q, s_kv = q.shape[0], k.shape[0]
    D = head_dim
    grp = n_heads // n_kv_heads
    P = np.zeros((n_heads, s_q, s_kv))
    ctx = np.zeros((s_q, n_heads * D))
    mask = causal_mask(s_q, s_kv) if causal else np.ones((s_q, s_kv), bool)
    for h in range(n_heads):
        g = h // grp
        sc = scale * (q[:, h * D:(h + 1) * D] @ k[:, g * D:(g + 1) * D].T)
        sc = np.where(mask, sc, -np.inf)
        sc = sc - sc.max(axis=-1, keepdims=True)
        e = np.exp(sc)
        P[h] = e / e.sum(axis=-1, keepdims=True)
        ctx[:, h * D:(h + 1) * D] = P[h] @ v[:, g * D:(g + 1) * D]
    return P, ctx


def context(P, V, n_heads, n_kv_heads):
    """The attention output ctx_h = P_h V_g (the apply step of the forward),
    for saved softmax weights P [Hq, s_q, s_kv] and values V [s_kv, Hkv*D]."""
    P = np.asarray(P, np.float64)
    V = np.asarray(V, np.float64)
    D = V.shape[1] // n_kv_heads
    grp = n_heads // n_kv_heads
    ctx = np.zeros((P.shape[1], n_heads * D))
    for h in range(n_heads):
        g = h // grp
        ctx[:, h * D:(h + 1) * D] = P[h] @ V[:, g * D:(g + 1) * D]
    return ctx


def layer_forward(cfg, w, x_res, x_attn=None, lora=None, q_pre=None, v_in=None):
    """Returns (out, saved).  lora: dict with A_q, B_q, A_v, B_v (or None).
    q_pre / v_in override the Q projection output (pre-RoPE) and the value
    tensor, for finite differences with respect to them."""
    x_res = np.asarray(x_res, np.float64)
    x_attn = x_res if x_attn is None else np.asarray(x_attn, np.float64)
    S = x_res.shape[0]
    H, Hq, Hkv, D = cfg.hidden, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    pos = cfg.pos0 + np.arange(S)
    x_a = rmsnorm(x_attn, w["gamma_attn"], cfg.eps)
    saved = {"attn_input": x_a}
    if q_pre is None:
        q_pre = x_a @ w["W_q"].T
        if lora is not None:
            h_q = x_a @ lora["A_q"].T
            saved["lora_q_h"] = h_q
            q_pre = q_pre + (cfg.alpha / lora["A_q"].shape[0]) * (h_q @ lora["B_q"].T)
    elif lora is not None:
        saved["lora_q_h"] = x_a @ lora["A_q"].T
    qk_norm = getattr(cfg, "qk_norm", False)
    if qk_norm:
        saved["q_raw"] = q_pre
        q = rope(head_rmsnorm(q_pre, Hq, w["gamma_q"], cfg.eps), Hq, D, pos, cfg.rope_base)
    else:
        q = rope(q_pre, Hq, D, pos, cfg.rope_base)
    if "K_cache" in w:
        k = np.asarray(w["K_cache"], np.float64)
        v = np.asarray(w["V_cache"], np.float64) if v_in is None else v_in
    else:
        k_pre = x_a @ w["W_k"].T
        if qk_norm:
            saved["k_raw"] = k_pre
            k_pre = head_rmsnorm(k_pre, Hkv, w["gamma_k"], cfg.eps)
        k = rope(k_pre, Hkv, D, pos, cfg.rope_base)
        if "K_prefix" in w:
            k = np.concatenate([np.asarray(w["K_prefix"], np.float64), k])
        if v_in is None:
            v = x_a @ w["W_v"].T
            if lora is not None:
                h_v = x_a @ lora["A_v"].T
                saved["lora_v_h"] = h_v
                v = v + (cfg.alpha / lora["A_v"].shape[0]) * (h_v @ lora["B_v"].T)
            if "V_prefix" in w:
                v = np.concatenate([np.asarray(w["V_prefix"], np.float64), v])
        else:
            v = v_in
            if lora is not None:
                saved["lora_v_h"] = x_a @ lora["A_v"].T
    P, ctx = attention(q, k, v, Hq, Hkv, D, cfg.scale, cfg.causal)
    c = rmsnorm(ctx, w["gamma_asub"], cfg.eps) if cfg.sub_norms else ctx
    h1 = x_res + c @ w["W_o"].T
    n2 = rmsnorm(h1, w["gamma_ffn"], cfg.eps)
    gate = n2 @ w["W_gate"].T
    up = n2 @ w["W_up"].T
    hid = act_fwd(cfg.act, gate, up)
    f = rmsnorm(hid, w["gamma_fsub"], cfg.eps) if cfg.sub_norms else hid
    out = h1 + f @ w["W_down"].T
    saved.update(q_pre=q_pre, q=q, K=k, V=v, P=P, ctx=ctx, resid1=h1,
                 hidden_input=n2, gate=gate, up=up, x=x_attn)
    if cfg.sub_norms:
        saved["hidden_pre"] = hid
    return out, saved


def make_layer(cfg, draws):
    """Split seeded draws into (weights, saved activations, LoRA state) by
    running the forward once on the drawn layer input."""
    w = {k: v for k, v in draws.items()
         if k.startswith("W_") or k.startswith("gamma_")
         or k in ("K_cache", "V_cache", "K_prefix", "V_prefix")}
    lora = None
    if cfg.rank > 0:
        lora = {k: draws[k] for k in draws
                if k[:2] in ("A_", "B_") or k[:4] in ("m_A_", "m_B_", "v_A_", "v_B_")}
    _, saved = layer_forward(cfg, w, draws["x"], lora=lora)
    return w, saved, lora
