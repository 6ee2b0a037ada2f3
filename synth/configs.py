"""Workload shapes of the LoRA layer-backward path.

Five workloads, named by what they are:
  tiny        hidden 64, ffn 256, 4/2 heads of 16, 16 tokens, SwiGLU, LoRA r4
  decode      one token against a 512-slot K/V cache, hidden 2560, ffn 6912,
              20/5 heads of 128, ReLU^2 x up FFN with sub-norms, ternary weights
  seq512      hidden 2560, ffn 9728, 32/8 heads of 128, 512 tokens, SwiGLU,
              LoRA r16 on Q and V
  seq2048bf16 the seq512 layer at 2048 tokens with bf16 activations/weights
  stack36     36 seq512-shaped layers at 1024 tokens, fp32
  seq512qk    the seq512 layer with QK-norm (per-head RMSNorm of Q and K before
              RoPE, as Qwen3-style layers have)
  decode_packed
              the decode layer with its ternary weights packed 2 bits per value
              (BitLinear storage)
  seq512ig, seq2048bf16ig
              the seq512 / seq2048bf16 layers with the exact input gradient
              through the attention branch (dK, the transposed Q/K/V
              products, the adapters' terms, the attention-norm backward)

and the step upstream of the stack (LmHeadConfig):
  lmhead      the lm_head backward of the stack36 model: 1024 tokens, hidden
              2560, vocabulary 151936 (a Qwen-family vocabulary), fp32, with
              AdamW on the lm_head weight
"""
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class LayerConfig:
    name: str
    index: int           # seeds the per-tensor random streams
    seq: int             # query rows S
    kv_len: int          # key/value rows (= seq, or the cache length in decode)
    hidden: int
    ffn: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    act: str             # "swiglu" or "relu2"
    sub_norms: bool      # RMSNorm after attention context and after the FFN activation
    rank: int            # LoRA rank on Q and V (0 = no adapters)
    alpha: float
    dtype: str           # "f32" or "bf16": storage type of saved activations and base weights
    n_layers: int = 1
    pos0: int = 0        # RoPE position of query row 0
    causal: bool = True
    rope_base: float = 10000.0
    eps: float = 1e-6
    lr: float = 1e-4
    lr_b_ratio: float = 16.0   # LoRA+: lr_B = 16 * lr_A
    beta1: float = 0.9
    beta2: float = 0.999
    adam_eps: float = 1e-8
    weight_decay: float = 0.01
    step: int = 1
    ternary: bool = False      # weights are 0.02 * {-1, 0, +1}
    qk_norm: bool = False      # per-head RMSNorm of the Q and K projections before RoPE
    input_grad: bool = False   # differentiate the attention branch input too (no stop-gradient)
    packed: bool = False       # ternary weights stored packed (2 bits per value)

    @property
    def q_dim(self):
        return self.n_heads * self.head_dim

    @property
    def kv_dim(self):
        return self.n_kv_heads * self.head_dim

    @property
    def scale(self):
        s = self.__dict__.get("_scale")
        return s if s is not None else 1.0 / float(self.head_dim) ** 0.5

    @property
    def lr_b(self):
        s = self.__dict__.get("_lr_b")
        return s if s is not None else self.lr * self.lr_b_ratio

    def with_(self, **kw):
        return replace(self, **kw)


TINY = LayerConfig("tiny", 0, seq=16, kv_len=16, hidden=64, ffn=256, n_heads=4,
                   n_kv_heads=2, head_dim=16, act="swiglu", sub_norms=False,
                   rank=4, alpha=8.0, dtype="f32")
DECODE = LayerConfig("decode", 1, seq=1, kv_len=512, hidden=2560, ffn=6912,
                     n_heads=20, n_kv_heads=5, head_dim=128, act="relu2",
                     sub_norms=True, rank=0, alpha=0.0, dtype="f32", pos0=511,
                     ternary=True)
SEQ512 = LayerConfig("seq512", 2, seq=512, kv_len=512, hidden=2560, ffn=9728,
                     n_heads=32, n_kv_heads=8, head_dim=128, act="swiglu",
                     sub_norms=False, rank=16, alpha=32.0, dtype="f32")
SEQ2048BF16 = SEQ512.with_(name="seq2048bf16", index=3, seq=2048, kv_len=2048,
                           dtype="bf16")
STACK36 = SEQ512.with_(name="stack36", index=4, seq=1024, kv_len=1024, n_layers=36)
SEQ512QK = SEQ512.with_(name="seq512qk", index=5, qk_norm=True)
SEQ512IG = SEQ512.with_(name="seq512ig", index=6, input_grad=True)
SEQ2048BF16IG = SEQ2048BF16.with_(name="seq2048bf16ig", index=7, input_grad=True)
DECODE_PACKED = DECODE.with_(name="decode_packed", index=8, packed=True)



@dataclass(frozen=True)
class LmHeadConfig:
    """The lm_head backward: final hidden state h [rows, hidden], logits
    [rows, vocab] as saved by the forward, int32 labels, the weight
    [vocab, hidden] with AdamW moments."""
    name: str
    index: int
    rows: int
    hidden: int
    vocab: int
    logit_std: float = 1.0    # the spread of h W^T at these weight scales
    ignore_every: int = 0     # every k-th row gets label -100 (ignored); 0: none
    lr: float = 1e-4
    beta1: float = 0.9
    beta2: float = 0.999
    adam_eps: float = 1e-8
    weight_decay: float = 0.01
    step: int = 1

    @property
    def seq(self):
        return self.rows

    def with_(self, **kw):
        return replace(self, **kw)


LMHEAD = LmHeadConfig("lmhead", 9, rows=1024, hidden=2560, vocab=151936)

CONFIGS = {c.name: c for c in (TINY, DECODE, SEQ512, SEQ2048BF16, STACK36, SEQ512QK, SEQ512IG,
                               SEQ2048BF16IG, DECODE_PACKED, LMHEAD)}


def get_config(name):
    return CONFIGS[name]
