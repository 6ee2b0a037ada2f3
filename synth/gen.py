"""Seeded random draws for the layer-backward workloads.

Every tensor has its own PCG64 stream seeded from
SeedSequence([0, config index, layer index, tensor id]), so any tensor of any
layer can be regenerated on its own, in any order.  Large tensors are drawn as
float32 (N(0,1) ziggurat in single precision); casting to the storage dtype
is left to the caller.

Distributions (the workload recipe):
  * layer input x, upstream gradient d_out, decode K/V cache: N(0, 1)
  * base weights, LoRA A and B: N(0, 0.02); decode weights 0.02 * t with
    t uniform on {-1, 0, +1}
  * RMSNorm scales gamma (also the per-head QK-norm scales): 1 + 0.1 * N(0, 1)
  * AdamW moments m, v: zero (one step from a fresh optimizer)
  * lm_head: h ~ N(0, 1), W ~ N(0, 0.02), logits drawn on their own as
    N(0, logit_std^2) (the backward takes them as saved; 1.0 is the spread
    of h W^T at these scales), labels uniform over the vocabulary, every
    ignore_every-th row -100 (ignored) when that is set
"""
import numpy as np

TENSOR_IDS = {
    "x": 0, "d_out": 1, "W_q": 2, "W_k": 3, "W_v": 4, "W_o": 5, "W_gate": 6,
    "W_up": 7, "W_down": 8, "gamma_attn": 9, "gamma_ffn": 10, "gamma_fsub": 11,
    "gamma_asub": 12, "A_q": 13, "B_q": 14, "A_v": 15, "B_v": 16, "K_cache": 17,
    "V_cache": 18, "m_state": 19, "v_state": 20, "K_prefix": 21, "V_prefix": 22,
    "gamma_q": 23, "gamma_k": 24,
    "lm_h": 25, "lm_logits": 26, "lm_labels": 27, "lm_W": 28,
    # timing-only draws (stand-ins for saved activations)
    "t_attn_input": 40, "t_resid1": 41, "t_gate": 42, "t_up": 43,
    "t_hidden_pre": 44, "t_ctx": 45, "t_P": 46, "t_K": 47, "t_V": 48,
    "t_lora_q_h": 49, "t_lora_v_h": 50, "t_q_raw": 51, "t_x": 52, "t_q": 53, "t_k_raw": 54,
}


def stream(cfg_index, layer, tensor):
    tid = TENSOR_IDS[tensor] if isinstance(tensor, str) else int(tensor)
    ss = np.random.SeedSequence([0, int(cfg_index), int(layer), tid])
    return np.random.Generator(np.random.PCG64(ss))


def normal(cfg, layer, name, shape, std=1.0):
    """N(0, std^2) draws, generated in float32 (values widen exactly)."""
    a = stream(cfg.index, layer, name).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def ternary(cfg, layer, name, shape, scale=0.02):
    t = stream(cfg.index, layer, name).integers(-1, 2, size=shape)
    return t.astype(np.float64) * scale


def gamma(cfg, layer, name, n):
    return 1.0 + 0.1 * stream(cfg.index, layer, name).standard_normal(n)  # float64, small


def _weight(cfg, layer, name, shape):
    if cfg.ternary:
        return ternary(cfg, layer, name, shape)
    return normal(cfg, layer, name, shape, 0.02)


def draw_layer(cfg, layer=0):
    """Independent draws of one layer: input, upstream gradient, weights
    ([out, in] row-major), RMSNorm scales, LoRA adapters and optimizer state."""
    S, H, I = cfg.seq, cfg.hidden, cfg.ffn
    qd, kvd, r = cfg.q_dim, cfg.kv_dim, cfg.rank
    d = {
        "x": normal(cfg, layer, "x", (S, H)),
        "d_out": normal(cfg, layer, "d_out", (S, H)),
        "W_q": _weight(cfg, layer, "W_q", (qd, H)),
        "W_o": _weight(cfg, layer, "W_o", (H, qd)),
        "W_gate": _weight(cfg, layer, "W_gate", (I, H)),
        "W_up": _weight(cfg, layer, "W_up", (I, H)),
        "W_down": _weight(cfg, layer, "W_down", (H, I)),
        "gamma_attn": gamma(cfg, layer, "gamma_attn", H),
        "gamma_ffn": gamma(cfg, layer, "gamma_ffn", H),
    }
    if cfg.sub_norms:
        d["gamma_fsub"] = gamma(cfg, layer, "gamma_fsub", I)
        d["gamma_asub"] = gamma(cfg, layer, "gamma_asub", qd)
    if cfg.qk_norm:
        d["gamma_q"] = gamma(cfg, layer, "gamma_q", cfg.head_dim)
        d["gamma_k"] = gamma(cfg, layer, "gamma_k", cfg.head_dim)
    if cfg.seq == cfg.kv_len:
        d["W_k"] = _weight(cfg, layer, "W_k", (kvd, H))
        d["W_v"] = _weight(cfg, layer, "W_v", (kvd, H))
    elif cfg.seq == 1 and r == 0:
        # decode: the cache (post-RoPE keys, values) is drawn directly; the
        # last slot is the current token
        d["K_cache"] = normal(cfg, layer, "K_cache", (cfg.kv_len, kvd))
        d["V_cache"] = normal(cfg, layer, "V_cache", (cfg.kv_len, kvd))
    else:
        # a chunk of tokens after a cached prefix: the prefix's post-RoPE keys
        # and values are drawn directly, the chunk's come from its projections
        d["W_k"] = _weight(cfg, layer, "W_k", (kvd, H))
        d["W_v"] = _weight(cfg, layer, "W_v", (kvd, H))
        d["K_prefix"] = normal(cfg, layer, "K_prefix", (cfg.kv_len - S, kvd))
        d["V_prefix"] = normal(cfg, layer, "V_prefix", (cfg.kv_len - S, kvd))
    if r > 0:
        d["A_q"] = normal(cfg, layer, "A_q", (r, H), 0.02)
        d["B_q"] = normal(cfg, layer, "B_q", (qd, r), 0.02)
        d["A_v"] = normal(cfg, layer, "A_v", (r, H), 0.02)
        d["B_v"] = normal(cfg, layer, "B_v", (kvd, r), 0.02)
        for k in ("A_q", "B_q", "A_v", "B_v"):
            d["m_" + k] = np.zeros_like(d[k])
            d["v_" + k] = np.zeros_like(d[k])
    return d


def draw_lm_head(cfg, copy=0):
    """Inputs of one lm_head backward (float32, labels int32)."""
    S, H, V = cfg.rows, cfg.hidden, cfg.vocab
    d = {
        "h": normal(cfg, copy, "lm_h", (S, H)),
        "logits": normal(cfg, copy, "lm_logits", (S, V), cfg.logit_std),
        "labels": stream(cfg.index, copy, "lm_labels").integers(0, V, size=S).astype(np.int32),
        "W": normal(cfg, copy, "lm_W", (V, H), 0.02),
        "m": np.zeros((V, H), np.float32),
        "v": np.zeros((V, H), np.float32),
    }
    if cfg.ignore_every:
        d["labels"][::cfg.ignore_every] = -100
    return d


def draw_adam_state(cfg, layer, shape, salt):
    """Non-trivial optimizer moments for multi-step AdamW cases: m ~ N(0, 1e-3),
    v = (N(0, 1e-3))^2 (non-negative, as a second moment must be)."""
    m = stream(cfg.index, layer, 100 + 2 * salt).standard_normal(shape) * 1e-3
    v = (stream(cfg.index, layer, 101 + 2 * salt).standard_normal(shape) * 1e-3) ** 2
    return m, v


def causal_rows(rng, n_heads, s_q, s_kv, causal):
    """Random softmax-like rows: positive where key j <= s_kv - s_q + i (all
    keys when not causal), exactly zero elsewhere, each row normalised to 1."""
    P = rng.random((n_heads, s_q, s_kv), dtype=np.float32) + np.float32(1e-3)
    if causal:
        i = np.arange(s_q)[:, None]
        j = np.arange(s_kv)[None, :]
        P[:, j > (s_kv - s_q + i)] = 0.0
    P /= P.sum(axis=-1, keepdims=True)
    return P


def draw_timing_layer(cfg, layer=0):
    """Shape- and structure-faithful stand-ins for every saved tensor, drawn
    independently (float32).  Kernel cost does not depend on the values, so the
    throughput benchmark uses these instead of running a forward pass; parity
    tests never use them."""
    S, L, H, I = cfg.seq, cfg.kv_len, cfg.hidden, cfg.ffn
    qd, kvd, r = cfg.q_dim, cfg.kv_dim, cfg.rank
    f = np.float32

    def n(name, shape, std=1.0):
        return (stream(cfg.index, layer, name).standard_normal(shape, dtype=f) * f(std))

    wshapes = {"W_o": (H, qd), "W_gate": (I, H), "W_up": (I, H), "W_down": (H, I)}
    if cfg.ternary:
        weights = {k: ternary(cfg, layer, k, shp).astype(f) for k, shp in wshapes.items()}
    else:
        weights = {k: n(k, shp, 0.02) for k, shp in wshapes.items()}
    t = {
        "d_out": n("d_out", (S, H)), **weights,
        "gamma_ffn": (1 + n("gamma_ffn", (H,), 0.1)).astype(f),
        "attn_input": n("t_attn_input", (S, H)), "resid1": n("t_resid1", (S, H)),
        "gate": n("t_gate", (S, I)), "up": n("t_up", (S, I)),
        "ctx": n("t_ctx", (S, qd)),
        "P": causal_rows(stream(cfg.index, layer, "t_P"), cfg.n_heads, S, L, cfg.causal),
        "K": n("t_K", (L, kvd)), "V": n("t_V", (L, kvd)),
    }
    if cfg.sub_norms:
        t["hidden_pre"] = n("t_hidden_pre", (S, I))
        t["gamma_fsub"] = (1 + n("gamma_fsub", (I,), 0.1)).astype(f)
        t["gamma_asub"] = (1 + n("gamma_asub", (qd,), 0.1)).astype(f)
    if cfg.qk_norm:
        t["q_raw"] = n("t_q_raw", (S, qd))
        t["gamma_q"] = (1 + n("gamma_q", (cfg.head_dim,), 0.1)).astype(f)
    if cfg.input_grad:
        for k, shp in (("W_q", (qd, H)), ("W_k", (kvd, H)), ("W_v", (kvd, H))):
            t[k] = n(k, shp, 0.02)
        t["gamma_attn"] = (1 + n("gamma_attn", (H,), 0.1)).astype(f)
        t["x"] = n("t_x", (S, H))
        t["q"] = n("t_q", (S, qd))
        if cfg.qk_norm:
            t["k_raw"] = n("t_k_raw", (S, kvd))
            t["gamma_k"] = (1 + n("gamma_k", (cfg.head_dim,), 0.1)).astype(f)
    if r > 0:
        t["lora_q_h"] = n("t_lora_q_h", (S, r), 0.1)
        t["lora_v_h"] = n("t_lora_v_h", (S, r), 0.1)
        for k, shp in (("A_q", (r, H)), ("B_q", (qd, r)), ("A_v", (r, H)), ("B_v", (kvd, r))):
            t[k] = n(k, shp, 0.02)
            t["m_" + k] = np.zeros(shp, f)
            t["v_" + k] = np.zeros(shp, f)
    return t
