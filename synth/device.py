"""Seeded timing inputs generated on the GPU (torch RNG), for the benchmark.

Same shapes, dtypes and structure as synth.gen.draw_timing_layer (causal,
row-normalised P with exact zeros above the diagonal; ternary decode
weights; N(0, 0.02) weights; 1 + 0.1 N(0, 1) norm scales; zero AdamW
moments), but drawn on the device so multi-gigabyte workloads are ready in
seconds.  Kernel cost does not depend on the values; parity tests never use
these tensors.
"""
import torch


def _gen(cfg, layer, device):
    g = torch.Generator(device=device)
    g.manual_seed(1_000_003 * (cfg.index + 1) + 7919 * layer)
    return g


def draw_timing_layer_device(cfg, layer=0, device="cuda:0"):
    S, L, H, I = cfg.seq, cfg.kv_len, cfg.hidden, cfg.ffn
    qd, kvd, r = cfg.q_dim, cfg.kv_dim, cfg.rank
    g = _gen(cfg, layer, device)
    act = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    f32 = torch.float32

    def n(shape, std=1.0, dtype=act):
        return (torch.randn(shape, generator=g, device=device, dtype=f32) * std).to(dtype)

    def w(shape):
        if cfg.ternary:
            t = torch.randint(-1, 2, shape, generator=g, device=device).to(f32) * 0.02
            return t.to(act)
        return n(shape, 0.02)

    P = torch.rand((cfg.n_heads, S, L), generator=g, device=device, dtype=f32) + 1e-3
    if cfg.causal:
        i = torch.arange(S, device=device)[:, None]
        j = torch.arange(L, device=device)[None, :]
        P.masked_fill_(j > (L - S + i), 0.0)
    P /= P.sum(-1, keepdim=True)
    d = {
        "weights": {"w_o": w((H, qd)), "w_gate": w((I, H)), "w_up": w((I, H)),
                    "w_down": w((H, I)), "gamma_ffn": 1 + n((H,), 0.1, f32)},
        "saved": {"attn_input": n((S, H)), "resid1": n((S, H)), "gate": n((S, I)),
                  "up": n((S, I)), "ctx": n((S, qd)), "P": P.to(act), "K": n((L, kvd)),
                  "V": n((L, kvd))},
        "d_out": n((S, H), 1.0, f32),
        "lora": None,
    }
    del P
    if cfg.qk_norm:
        d["weights"]["gamma_q"] = 1 + n((cfg.head_dim,), 0.1, f32)
        d["saved"]["q_raw"] = n((S, qd))
    if cfg.input_grad:
        d["weights"].update(w_q=w((qd, H)), w_k=w((kvd, H)), w_v=w((kvd, H)),
                            gamma_attn=1 + n((H,), 0.1, f32))
        d["saved"].update(x=n((S, H)), q=n((S, qd)))
        if cfg.qk_norm:
            d["weights"]["gamma_k"] = 1 + n((cfg.head_dim,), 0.1, f32)
            d["saved"]["k_raw"] = n((S, kvd))
    if cfg.sub_norms:
        d["weights"]["gamma_fsub"] = 1 + n((I,), 0.1, f32)
        d["weights"]["gamma_asub"] = 1 + n((qd,), 0.1, f32)
        d["saved"]["hidden_pre"] = n((S, I))
    if r > 0:
        d["saved"]["lora_q_h"] = n((S, r), 0.1)
        d["saved"]["lora_v_h"] = n((S, r), 0.1)
        d["lora"] = {}
        for tag, out in (("q", qd), ("v", kvd)):
            d["lora"][tag] = {"A": n((r, H), 0.02, f32), "B": n((out, r), 0.02, f32),
                              "m_a": torch.zeros((r, H), device=device),
                              "v_a": torch.zeros((r, H), device=device),
                              "m_b": torch.zeros((out, r), device=device),
                              "v_b": torch.zeros((out, r), device=device)}
    return d


def draw_lm_head_device(cfg, copy=0, device="cuda:0"):
    """synth.gen.draw_lm_head's recipe drawn on the GPU (torch RNG)."""
    g = _gen(cfg, copy, device)
    S, H, V = cfg.rows, cfg.hidden, cfg.vocab
    f32 = torch.float32
    labels = torch.randint(0, V, (S,), generator=g, device=device, dtype=torch.int64).to(torch.int32)
    if cfg.ignore_every:
        labels[::cfg.ignore_every] = -100
    return {
        "h": torch.randn((S, H), generator=g, device=device, dtype=f32),
        "logits": torch.randn((S, V), generator=g, device=device, dtype=f32) * cfg.logit_std,
        "labels": labels,
        "W": torch.randn((V, H), generator=g, device=device, dtype=f32) * 0.02,
        "m": torch.zeros((V, H), device=device, dtype=f32),
        "v": torch.zeros((V, H), device=device, dtype=f32),
    }
