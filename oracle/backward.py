"""Float64 backward of one pre-norm transformer layer for LoRA fine-tuning.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Plain NumPy, formula
shaped, no blocking or fusion: each function is the definition it cites.

Conventions (readings of the pages, also listed in the design notes):
  * Weights are [out, in] row-major and a projection is y = x @ W.T, so the
    input gradient of a projection is dx = dy @ W.  ([FFN] "Forward" writes
    the per-token product W @ x; the entrenar trainer stores pre-transposed
    copies, which is the same product on another layout.)
  * Activations are token-major [rows, features]; head h owns the contiguous
    feature slice [h*D, (h+1)*D).  Saved softmax weights P are
    [n_heads, s_q, s_kv].
  * GQA: query head h reads KV head h // (n_heads // n_kv_heads)
    ([ENT] backward_through_layers, attention backward: kv_head = head /
    heads_per_kv).
  * RMSNorm: r = sqrt(mean(x^2) + eps) over the last axis, a separate frozen
    gamma per norm ([ATTN] "RMSNorm Backward" formula; [FFN] names two scales,
    ffnSubNormScale and ffnNormScale).
  * The residual skip and the FFN-norm backward are part of the path
    ([FFN] "Backward (reverse)" step 5); the gradient reaching the layer below
    is the residual-stream gradient dH1 ([ENT] passes grad_hidden down; neither
    page differentiates the attention input), i.e. a stop-gradient at the
    attention branch input.
  * The LoRA Q signal is the gradient of the pre-RoPE Q projection output
    ([ATTN] "Gradient Flow": dQpre after the inverse rotation).
"""
import numpy as np


# --------------------------------------------------------------------------
# RMSNorm backward
# --------------------------------------------------------------------------
def rmsnorm_bwd(x, gamma, dy, eps):
    """[ATTN] "RMSNorm Backward": per row of n features,
    dx = (1/r) * (dy*gamma - x * <dy*gamma, x> / (n * r^2)),
    with r = sqrt(mean(x^2) + eps)."""
    x = np.asarray(x, np.float64)
    dy = np.asarray(dy, np.float64)
    n = x.shape[-1]
    r = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    g = dy * np.asarray(gamma, np.float64)
    dot = np.sum(g * x, axis=-1, keepdims=True)
    return (g - x * dot / (n * r * r)) / r


def head_rmsnorm_bwd(x, n_heads, gamma, dy, eps):
    """QK-norm backward: the RMSNorm backward above applied to each head's
    head_dim slice of a [rows, n_heads*head_dim] tensor (x the norm's input,
    the projection output), with one scale vector gamma [head_dim] for every
    head.  The trainer's saved Q and K are "after QK-norm + RoPE" ([ENT]
    LayerActivations), so this step sits between the inverse RoPE and the
    LoRA Q signal."""
    x = np.asarray(x, np.float64)
    rows = x.shape[0]
    dx = rmsnorm_bwd(x.reshape(rows, n_heads, -1), gamma, np.asarray(dy, np.float64).reshape(rows, n_heads, -1), eps)
    return dx.reshape(rows, -1)


# --------------------------------------------------------------------------
# RoPE backward (NeoX split-half)
# --------------------------------------------------------------------------
def rope_theta(positions, head_dim, base):
    """[ATTN] "RoPE Backward": theta[p, d] = pos_p * base^(-2d/headDim) for d in
    the first half of the head; computed in float64."""
    half = head_dim // 2
    d = np.arange(half, dtype=np.float64)
    inv_freq = np.power(float(base), -2.0 * d / head_dim)
    return np.asarray(positions, np.float64)[:, None] * inv_freq[None, :]


def rope_bwd(dy, n_heads, head_dim, positions, base):
    """[ATTN] "RoPE Backward (inverse rotation)": per head, with half = D/2,
      dx[d]      =  dy[d] cos(theta) + dy[d+half] sin(theta)
      dx[d+half] = -dy[d] sin(theta) + dy[d+half] cos(theta)
    dy: [rows, n_heads*head_dim]; positions: one per row."""
    dy = np.asarray(dy, np.float64)
    rows = dy.shape[0]
    half = head_dim // 2
    th = rope_theta(positions, head_dim, base)          # [rows, half]
    c, s = np.cos(th)[:, None, :], np.sin(th)[:, None, :]
    y = dy.reshape(rows, n_heads, head_dim)
    lo, hi = y[..., :half], y[..., half:]
    dx = np.empty_like(y)
    dx[..., :half] = lo * c + hi * s
    dx[..., half:] = -lo * s + hi * c
    return dx.reshape(rows, n_heads * head_dim)


# --------------------------------------------------------------------------
# Gated activation backward
# --------------------------------------------------------------------------
def relu2_mul_bwd(gate, up, dh):
    """[FFN] "ReLU²×Mul Backward": h = max(0, gate)^2 * up, so
    dGate = dH * up * 2 * max(0, gate),  dUp = dH * max(0, gate)^2."""
    gate = np.asarray(gate, np.float64)
    up = np.asarray(up, np.float64)
    dh = np.asarray(dh, np.float64)
    r = np.maximum(gate, 0.0)
    return dh * up * 2.0 * r, dh * r * r


def swiglu_bwd(gate, up, dh):
    """[ENT] backward_through_layers, "SiLU backward": h = silu(gate) * up with
    sig = 1/(1+exp(-gate)), silu' = sig * (1 + gate - gate*sig);
    dGate = dH * up * silu',  dUp = dH * silu(gate).  silu(gate) is recomputed
    here in float64 (the trainer reads its saved copy; they agree when the
    saved activations come from the forward)."""
    gate = np.asarray(gate, np.float64)
    up = np.asarray(up, np.float64)
    dh = np.asarray(dh, np.float64)
    sig = 1.0 / (1.0 + np.exp(-gate))
    silu = gate * sig
    dsilu = sig * (1.0 + gate - silu)
    return dh * up * dsilu, dh * silu


def act_bwd(act, gate, up, dh):
    if act == "swiglu":
        return swiglu_bwd(gate, up, dh)
    if act == "relu2":
        return relu2_mul_bwd(gate, up, dh)
    raise ValueError(act)


# --------------------------------------------------------------------------
# Attention backward
# --------------------------------------------------------------------------
def softmax_bwd(P, dA):
    """[ATTN] "Softmax Backward": dScores[s] = attn[s] * (dAttn[s] - sum_s'
    attn[s'] dAttn[s']) along the last axis."""
    P = np.asarray(P, np.float64)
    dA = np.asarray(dA, np.float64)
    delta = np.sum(P * dA, axis=-1, keepdims=True)
    return P * (dA - delta)


def attention_bwd(dctx, P, K, V, n_heads, n_kv_heads, scale, return_parts=False, Q=None):
    """Attention backward from saved softmax weights, per query head h with
    KV head g = h // (n_heads // n_kv_heads):
      apply backward  dA  = dCtx_h @ V_g^T        [ATTN] "Attention Apply Backward"
      softmax bwd     dS  = softmax_bwd(P_h, dA)  [ATTN] "Softmax Backward"
      score bwd (Q)   dQ_h = scale * dS @ K_g     [ATTN] "Attention Score Backward"
      value grad      dV_g += P_h^T @ dCtx_h      [ENT] attention backward, grad_v
      score bwd (K)   dK_g += scale * dS^T @ Q_h  (scores = scale Q K^T, the
                      same product rule as dQ; only with Q given)
    dctx [s_q, Hq*D]; P [Hq, s_q, s_kv]; K, V [s_kv, Hkv*D] (K post-RoPE);
    Q [s_q, Hq*D] post-RoPE or None.
    Returns dQ [s_q, Hq*D] (post-RoPE domain) and dV [s_kv, Hkv*D], and dK
    [s_kv, Hkv*D] (post-RoPE domain) last when Q is given."""
    dctx = np.asarray(dctx, np.float64)
    P = np.asarray(P, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    s_q = dctx.shape[0]
    s_kv = K.shape[0]
    D = dctx.shape[1] // n_heads
    grp = n_heads // n_kv_heads
    dQ = np.zeros((s_q, n_heads * D))
    dV = np.zeros((s_kv, n_kv_heads * D))
    dK = None if Q is None else np.zeros((s_kv, n_kv_heads * D))
    parts = []
    for h in range(n_heads):
        g = h // grp
        dC = dctx[:, h * D:(h + 1) * D]
        Kg = K[:, g * D:(g + 1) * D]
        Vg = V[:, g * D:(g + 1) * D]
        dA = dC @ Vg.T
        dS = softmax_bwd(P[h], dA)
        dQ[:, h * D:(h + 1) * D] = scale * (dS @ Kg)
        dV[:, g * D:(g + 1) * D] += P[h].T @ dC
        if dK is not None:
            dK[:, g * D:(g + 1) * D] += scale * (dS.T @ np.asarray(Q, np.float64)[:, h * D:(h + 1) * D])
        if return_parts:
            parts.append((dA, dS))
    out = (dQ, dV) if dK is None else (dQ, dV, dK)
    if return_parts:
        return out + (parts,)
    return out


# --------------------------------------------------------------------------
# LoRA gradients and AdamW
# --------------------------------------------------------------------------
def lora_grads(dy, h, x, B, alpha, rank):
    """[ENT] backward_through_layers, "LoRA Q backward" (and the V block, same
    pattern).  Adapter output s * (x A^T) B^T with s = alpha/rank and saved
    h = x A^T:
      dB = s * dy^T @ h     [out, rank]
      g  = s * dy @ B       [rows, rank]   (B before its update)
      dA = g^T @ x          [rank, in]"""
    dy = np.asarray(dy, np.float64)
    h = np.asarray(h, np.float64)
    x = np.asarray(x, np.float64)
    B = np.asarray(B, np.float64)
    s = float(alpha) / float(rank)
    dB = s * (dy.T @ h)
    g = s * (dy @ B)
    dA = g.T @ x
    return dA, dB


def adamw(p, g, m, v, lr, beta1, beta2, eps, wd, step):
    """[ENT] cpu_adamw: bias corrections 1/(1 - beta^step); moments
    m = b1 m + (1-b1) g, v = b2 v + (1-b2) g^2; decoupled decay scaled by lr:
    p -= lr * (m_hat / (sqrt(v_hat) + eps) + wd * p).  Returns new (p, m, v)."""
    p = np.asarray(p, np.float64)
    g = np.asarray(g, np.float64)
    m = np.asarray(m, np.float64)
    v = np.asarray(v, np.float64)
    bc1 = 1.0 / (1.0 - beta1 ** step)
    bc2 = 1.0 / (1.0 - beta2 ** step)
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    p = p - lr * ((m * bc1) / (np.sqrt(v * bc2) + eps) + wd * p)
    return p, m, v


# --------------------------------------------------------------------------
# FFN backward, layer backward, stack
# --------------------------------------------------------------------------
def ffn_bwd(d_out, W_down, W_gate, W_up, gate, up, resid1, gamma_ffn, eps, act,
            hidden_pre=None, gamma_fsub=None, return_parts=False):
    """[FFN] "Backward (reverse)", five steps, with the SwiGLU variant of step 3
    from [ENT]:
      1. dHid = dOut @ W_down
      2. (sub-norm present) dHid = rmsnorm_bwd(hidden_pre, gamma_fsub, dHid)
      3. dGate, dUp = act_bwd(gate, up, dHid)
      4. dN2 = dGate @ W_gate + dUp @ W_up
      5. dH1 = dOut + rmsnorm_bwd(resid1, gamma_ffn, dN2)   (residual skip)"""
    d_out = np.asarray(d_out, np.float64)
    dhid = d_out @ np.asarray(W_down, np.float64)
    if hidden_pre is not None:
        dhid = rmsnorm_bwd(hidden_pre, gamma_fsub, dhid, eps)
    dgate, dup = act_bwd(act, gate, up, dhid)
    dn2 = dgate @ np.asarray(W_gate, np.float64) + dup @ np.asarray(W_up, np.float64)
    dh1 = d_out + rmsnorm_bwd(resid1, gamma_ffn, dn2, eps)
    if return_parts:
        return dh1, dict(dhid=dhid, dgate=dgate, dup=dup, dn2=dn2)
    return dh1


def layer_bwd(cfg, w, saved, d_out, lora=None):
    """Backward of one layer, in the order of [FFN] "Backward (reverse)" then
    [ATTN] "Gradient Flow", then the LoRA blocks of [ENT]
    backward_through_layers:

      dH1   = ffn_bwd(...)                               (to the layer below)
      dCtx  = dH1 @ W_o                 O-projection backward
      dCtx  = rmsnorm_bwd(ctx, gamma_asub, dCtx)   (only with sub-norms)
      dQ,dV = attention_bwd(dCtx, P, K, V)
      dQpre = rope_bwd(dQ), row i at position pos0 + i
      (qk_norm) dQpre = head_rmsnorm_bwd(q_raw, gamma_q, dQpre)
      for (Q: dQpre, lora_q_h), (V: dV[-S:], lora_v_h):
          dA, dB = lora_grads(...); gnorm_sq += ||dA||^2 (A only)
          A <- adamw(A, dA, lr), B <- adamw(B, dB, lr_b)

    cfg needs: n_heads, n_kv_heads, head_dim, act, sub_norms, eps, rope_base,
    pos0, scale, and for LoRA alpha, lr, lr_b, beta1, beta2, adam_eps,
    weight_decay, step.  w: weights and gammas; saved: attn_input, resid1,
    gate, up, hidden_pre (sub-norms), ctx, P, K, V, lora_q_h, lora_v_h.
    lora: dict with A_q, B_q, A_v, B_v and their m_/v_ moments, or None.
    The value adapter acts on the values of the S current tokens, which are
    the last S of the kv_len rows (all of them when kv_len == S); a cached
    prefix's rows receive dV but no adapter gradient."""
    sub = bool(cfg.sub_norms)
    dh1 = ffn_bwd(d_out, w["W_down"], w["W_gate"], w["W_up"], saved["gate"],
                  saved["up"], saved["resid1"], w["gamma_ffn"], cfg.eps, cfg.act,
                  hidden_pre=saved.get("hidden_pre") if sub else None,
                  gamma_fsub=w.get("gamma_fsub") if sub else None)
    dctx = dh1 @ np.asarray(w["W_o"], np.float64)
    if sub:
        dctx = rmsnorm_bwd(saved["ctx"], w["gamma_asub"], dctx, cfg.eps)
    input_grad = getattr(cfg, "input_grad", False)
    r_att = attention_bwd(dctx, saved["P"], saved["K"], saved["V"], cfg.n_heads,
                          cfg.n_kv_heads, cfg.scale, Q=saved["q"] if input_grad else None)
    dq, dv = r_att[0], r_att[1]
    rows = dq.shape[0]
    dq_pre = rope_bwd(dq, cfg.n_heads, cfg.head_dim, cfg.pos0 + np.arange(rows),
                      cfg.rope_base)
    if getattr(cfg, "qk_norm", False):
        dq_pre = head_rmsnorm_bwd(saved["q_raw"], cfg.n_heads, w["gamma_q"], dq_pre, cfg.eps)
    res = dict(d_hidden=dh1, dctx=dctx, dq=dq, dq_pre=dq_pre, dv=dv, gnorm_sq=0.0)
    if input_grad:
        res.update(attn_input_bwd(cfg, w, saved, dh1, dq_pre, r_att[2], dv, lora))
    if lora is not None:
        x_a = saved["attn_input"]
        for tag, dy, h in (("q", dq_pre, saved["lora_q_h"]),
                           ("v", dv[dv.shape[0] - rows:], saved["lora_v_h"])):
            A, B = lora["A_" + tag], lora["B_" + tag]
            rank = A.shape[0]
            dA, dB = lora_grads(dy, h, x_a, B, cfg.alpha, rank)
            res["gnorm_sq"] += float(np.sum(dA * dA))
            nA, mA, vA = adamw(A, dA, lora["m_A_" + tag], lora["v_A_" + tag], cfg.lr,
                               cfg.beta1, cfg.beta2, cfg.adam_eps, cfg.weight_decay,
                               cfg.step)
            nB, mB, vB = adamw(B, dB, lora["m_B_" + tag], lora["v_B_" + tag], cfg.lr_b,
                               cfg.beta1, cfg.beta2, cfg.adam_eps, cfg.weight_decay,
                               cfg.step)
            res.update({"dA_" + tag: dA, "dB_" + tag: dB,
                        "A_" + tag: nA, "m_A_" + tag: mA, "v_A_" + tag: vA,
                        "B_" + tag: nB, "m_B_" + tag: mB, "v_B_" + tag: vB})
    return res


def attn_input_bwd(cfg, w, saved, dh1, dq_pre, dk, dv, lora=None):
    """The attention branch's input gradient (no stop-gradient at the
    attention input), added to the residual-stream gradient dH1:
      dKpre = rope_bwd(dK), key row j at position pos0 - (kv_len - S) + j
      (qk_norm) dKpre = head_rmsnorm_bwd(k_raw, gamma_k, dKpre)
      dXa   = dQpre W_q + dKpre W_k + dV W_v       (the chunk's own S key and
              value rows; a cached prefix's rows are held fixed)
              + s (dQpre B_q) A_q + s (dV B_v) A_v  (adapters, before the update)
      dX    = dH1 + rmsnorm_bwd(x, gamma_attn, dXa)
    This is the gradient of the layer with respect to its input x through
    both the residual stream and the attention branch.  [ATTN] "Gradient
    Flow" stops at dQpre and [ENT] backward_through_layers passes only the
    residual-stream gradient down; this step completes the chain rule
    through the projections and the attention norm that both omit."""
    if "K_cache" in w:
        raise ValueError("the attention input gradient needs the K and V projections (a cache "
                         "drawn whole has no dependence on the layer input)")
    S = dh1.shape[0]
    L = dk.shape[0]
    Hkv, D = cfg.n_kv_heads, cfg.head_dim
    kpos = cfg.pos0 - (L - S) + np.arange(L)
    dk_pre = rope_bwd(dk, Hkv, D, kpos, cfg.rope_base)
    dk_cur = dk_pre[L - S:]
    if getattr(cfg, "qk_norm", False):
        dk_cur = head_rmsnorm_bwd(saved["k_raw"], Hkv, w["gamma_k"], dk_cur, cfg.eps)
    dv_cur = np.asarray(dv, np.float64)[L - S:]
    dxa = (dq_pre @ np.asarray(w["W_q"], np.float64) + dk_cur @ np.asarray(w["W_k"], np.float64)
           + dv_cur @ np.asarray(w["W_v"], np.float64))
    if lora is not None:
        for tag, dy in (("q", dq_pre), ("v", dv_cur)):
            A, Bm = np.asarray(lora["A_" + tag], np.float64), np.asarray(lora["B_" + tag], np.float64)
            dxa = dxa + (float(cfg.alpha) / A.shape[0]) * ((dy @ Bm) @ A)
    dx = dh1 + rmsnorm_bwd(saved["x"], w["gamma_attn"], dxa, cfg.eps)
    return dict(d_hidden=dx, dh1=dh1, dk=dk, dk_pre=dk_cur, dxa=dxa)


def stack_bwd(cfg, layers, grad_hidden):
    """[ENT] backward_through_layers: layers visited in reverse order, the
    hidden-state gradient handed from each layer to the one below; the
    returned LoRA gradient norm is sqrt of the sum over all layers of the
    squared A-gradient norms (Q and V).  layers: list of (w, saved, lora)."""
    d = np.asarray(grad_hidden, np.float64)
    out = [None] * len(layers)
    gsq = 0.0
    for l in range(len(layers) - 1, -1, -1):
        w, saved, lora = layers[l]
        r = layer_bwd(cfg, w, saved, d, lora)
        out[l] = r
        gsq += r["gnorm_sq"]
        d = r["d_hidden"]
    return d, out, float(np.sqrt(gsq))
