/*
 * lorabwd.h - per-layer transformer backward pass for LoRA fine-tuning on
 * AMD Instinct MI355X (gfx950).  C ABI.
 *
 * Sources (web pages, cited by title and section):
 *   [FFN]  Hesper API docs, "FFN Backward GPU Kernels"
 *   [ATTN] Hesper API docs, "Attention Backward GPU Kernels"
 *   [ENT]  entrenar train/transformer_trainer/wgpu_backward.rs
 *          (cpu_adamw, LayerActivations, backward_through_layers)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensor pointers are DEVICE pointers to dense row-major arrays, 16-byte
 *    aligned.  Activations are token-major [rows, features]; head h owns the
 *    feature slice [h*head_dim, (h+1)*head_dim).  Saved softmax weights P are
 *    [n_heads, s_q, s_kv].  Weights are [out, in] (a projection is
 *    y = x W^T), so each input gradient is dx = dy W.
 *  - "act" arguments (saved activations and base weights, typed const void*)
 *    are float32 (dtype LORABWD_F32) or bfloat16 (LORABWD_BF16).  Gradients,
 *    RMSNorm scales, LoRA A/B and the AdamW moments are always float32.
 *    bf16 inputs are multiplied on the matrix cores with float32
 *    accumulation; gradient operands of those products are rounded to bf16.
 *  - Feature sizes (hidden, ffn, n_heads*head_dim, n_kv_heads*head_dim) must
 *    be multiples of 8; head_dim must be 16, 32, 64 or 128; row counts may be
 *    any value >= 0 (0 is a no-op that returns LORABWD_OK).
 *  - Size limits: row counts (rows, seq, kv_len, s_q, s_kv) and feature sizes
 *    at most 2^20, at most 4096 query heads.  Within these, a shape that one
 *    of the kernels cannot take (a buffer range of 1 GiB or more, such as one
 *    chunk of weight rows of a one-token product or a one-token K/V cache,
 *    or the one-token attention's LDS) is refused with LORABWD_ERR_SHAPE by a
 *    checking pass of the whole call that runs before anything is enqueued.
 *  - GQA: query head h reads KV head h / (n_heads / n_kv_heads).
 *  - Every call validates all arguments before touching the GPU: a status
 *    other than LORABWD_OK and LORABWD_ERR_HIP means nothing was enqueued
 *    and no output was written.  LORABWD_ERR_HIP (a launch the runtime
 *    refused, e.g. no usable device) can leave the kernels before it
 *    enqueued.  A zero
 *    status means the work is enqueued on `stream`; results are valid once
 *    the stream is synchronised.  No call allocates or frees device memory,
 *    synchronises the device, or keeps state between calls: scratch memory
 *    is the caller's `workspace`, sized by the matching *_workspace_size
 *    function (the caller owns every buffer, as the [FFN]
 *    executeFFNBackward scratch buffers are).  Calls on different streams
 *    with different workspaces may run concurrently.
 *  - Non-finite inputs are not checked; NaN/Inf propagate ([ENT]
 *    backward_through_layers states finiteness of the incoming gradient as
 *    the caller's precondition).
 *  - Results are deterministic: no floating-point atomics; every reduction
 *    has a fixed order, so repeated calls give bitwise-identical results.
 */
#ifndef LORABWD_H
#define LORABWD_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum lorabwd_status {
  LORABWD_OK = 0,
  LORABWD_ERR_NULL = -1,      /* a required pointer is NULL */
  LORABWD_ERR_SHAPE = -2,     /* a size is negative, inconsistent or unsupported */
  LORABWD_ERR_ALIGN = -3,     /* a pointer is not 16-byte aligned */
  LORABWD_ERR_DTYPE = -4,     /* unknown dtype or activation code */
  LORABWD_ERR_WORKSPACE = -5, /* workspace NULL or smaller than required */
  LORABWD_ERR_STEP = -6,      /* AdamW step < 1 (bias correction divides by zero) */
  LORABWD_ERR_ALIAS = -7,     /* two buffers overlap where that is not allowed */
  LORABWD_ERR_HIP = -8,       /* a kernel launch failed */
  LORABWD_ERR_ARG = -9        /* a scalar argument is out of range */
} lorabwd_status;

enum { LORABWD_F32 = 0, LORABWD_BF16 = 1 };
enum { LORABWD_ACT_SWIGLU = 0, LORABWD_ACT_RELU2 = 1 };

/* Human-readable name of a status code (static storage, never NULL). */
const char* lorabwd_status_string(int status);

/* Version of the ABI described by this header. */
int lorabwd_abi_version(void);

/* ------------------------------------------------------------------------
 * RMSNorm backward.  [ATTN] "RMSNorm Backward": per row of n features,
 *   dx = (1/r) (dy*gamma - x <dy*gamma, x> / (n r^2)),  r = sqrt(mean(x^2) + eps)
 * x     act [rows, n]   the norm's input (pre-norm activations)
 * gamma f32 [n]         the norm's scale (frozen; no dgamma)
 * dy    f32 [rows, n]   gradient of the norm's output
 * dx    f32 [rows, n]   accumulate = 0: dx = result; 1: dx += result (the
 *                       residual skip of [FFN] "Backward (reverse)" step 5).
 *                       dx may equal dy (in place); no other overlap.
 * ---------------------------------------------------------------------- */
int lorabwd_rmsnorm_backward(int64_t rows, int64_t n, const void* x, const float* gamma,
                             const float* dy, float* dx, float eps, int accumulate,
                             int dtype, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Packed ternary (BitLinear) weights.  The decode layer's projections are
 * BitLinear layers ([FFN] executeFFNBackward takes W_down, W_gate, W_up as
 * BitLinear; [ATTN] "Gradient Flow": O projection backward, BitLinear
 * transpose), whose values are {-s, 0, +s} with one scale s per matrix.  The
 * pages give no storage format; this library's is 2 bits per value by sign
 * (0 -> 00, +s -> 01, -s -> 11), four consecutive columns of a row per byte
 * (column 4c + j in bits 2j .. 2j+1 of byte c), rows one after another: a
 * [rows, cols] matrix packs into uint8 [rows, cols / 4], 1/16 of its float32
 * bytes.
 * w      act [rows, cols] (float32 or bfloat16, `dtype`), coded by sign (the
 *        scale is the caller's: pass it with the packed matrix)
 * packed uint8 [rows, cols / 4]; cols a multiple of 8, rows <= 2^20.
 * ---------------------------------------------------------------------- */
size_t lorabwd_ternary_packed_bytes(int64_t rows, int64_t cols);
int lorabwd_pack_ternary(int64_t rows, int64_t cols, const void* w, int dtype, uint8_t* packed,
                         hipStream_t stream);

/* ------------------------------------------------------------------------
 * Inverse NeoX RoPE.  [ATTN] "RoPE Backward (inverse rotation)": per head,
 * with half = head_dim/2 and theta_d = pos * base^(-2d/head_dim), d < half,
 *   dx[d]      =  dy[d] cos(theta_d) + dy[d+half] sin(theta_d)
 *   dx[d+half] = -dy[d] sin(theta_d) + dy[d+half] cos(theta_d)
 * Row i is at position pos0 + i.  The angle is formed and rotated in float64
 * and rounded to float32 once.
 * dy, dx f32 [rows, n_heads*head_dim]; dx may equal dy (in place).
 * ---------------------------------------------------------------------- */
int lorabwd_rope_backward(int64_t rows, int64_t n_heads, int64_t head_dim, const float* dy,
                          float* dx, int64_t pos0, float base, hipStream_t stream);

/* ------------------------------------------------------------------------
 * GQA attention backward from saved softmax weights, per query head h
 * (KV head g = h / (n_heads/n_kv_heads)):
 *   dA  = dctx_h V_g^T               [ATTN] "Attention Apply Backward"
 *   dS  = P_h o (dA - delta)         [ATTN] "Softmax Backward",
 *         delta_i = sum_j P_h[i,j] dA[i,j]
 *   dq_h = scale dS K_g              [ATTN] "Attention Score Backward"
 *   dv_g += P_h^T dctx_h             [ENT] attention backward (grad_v)
 * When ctx (= P V, the forward attention output saved by the trainer) is
 * given, delta_i = <dctx_h[i], ctx_h[i]>, which equals the sum above when
 * ctx = P V and lets P be streamed once per output; with ctx NULL the sum
 * is formed from P and dA directly.
 * s_q, s_kv       query / key rows (s_q <= s_kv); query i sits at key
 *                 position s_kv - s_q + i.  causal = 1 lets the kernels skip
 *                 key blocks beyond that position (P must hold zeros there,
 *                 as a masked softmax does); causal = 0 reads all of P.
 * dctx  f32 [s_q, n_heads*head_dim]
 * P     act [n_heads, s_q, s_kv]
 * K, V  act [s_kv, n_kv_heads*head_dim]   (K after RoPE)
 * ctx   act [s_q, n_heads*head_dim] or NULL
 * dq    f32 [s_q, n_heads*head_dim]       (gradient of post-RoPE q)
 * dv    f32 [s_kv, n_kv_heads*head_dim] or NULL (not computed)
 * ---------------------------------------------------------------------- */
size_t lorabwd_attn_workspace_size(int64_t s_q, int64_t s_kv, int64_t n_heads,
                                   int64_t n_kv_heads, int64_t head_dim, int dtype);
int lorabwd_attn_backward(int64_t s_q, int64_t s_kv, int64_t n_heads, int64_t n_kv_heads,
                          int64_t head_dim, const float* dctx, const void* P, const void* K,
                          const void* V, const void* ctx, float* dq, float* dv, float scale,
                          int causal, int dtype, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/* ------------------------------------------------------------------------
 * Gated-FFN backward.  [FFN] "Backward (reverse)", with the SwiGLU form of
 * step 3 from [ENT] backward_through_layers ("SiLU backward"):
 *   1. dHid = d_out W_down
 *   2. dHid = rmsnorm_bwd(hidden_pre, gamma_sub, dHid)   (only if hidden_pre)
 *   3. act = SWIGLU: s = sigmoid(gate), dGate = dHid up s (1 + gate (1 - s)),
 *                    dUp = dHid gate s
 *      act = RELU2:  dGate = dHid up 2 max(0,gate), dUp = dHid max(0,gate)^2
 *                    ([FFN] "ReLU²×Mul Backward")
 *   4. dN2 = dGate W_gate + dUp W_up
 *   5. d_resid += rmsnorm_bwd(resid1, gamma_ffn, dN2)
 * d_out      f32 [rows, dim]
 * w_down     act [dim, ffn_dim];  w_gate, w_up act [ffn_dim, dim]
 * gate, up   act [rows, ffn_dim]  (projection outputs saved by the forward)
 * hidden_pre act [rows, ffn_dim] or NULL (no sub-norm); gamma_sub f32 [ffn_dim]
 * resid1     act [rows, dim]      (residual stream before the FFN norm)
 * gamma_ffn  f32 [dim]
 * d_resid    f32 [rows, dim] in/out.  Passing d_resid == d_out gives the
 *            full residual-stream gradient d_out + step 5 in place.
 * ---------------------------------------------------------------------- */
size_t lorabwd_ffn_workspace_size(int64_t rows, int64_t dim, int64_t ffn_dim, int dtype);
int lorabwd_ffn_backward(int64_t rows, int64_t dim, int64_t ffn_dim, int act,
                         const float* d_out, const void* w_down, const void* w_gate,
                         const void* w_up, const void* gate, const void* up,
                         const void* hidden_pre, const float* gamma_sub, const void* resid1,
                         const float* gamma_ffn, float* d_resid, float eps, int dtype,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * LoRA adapter gradients fused with AdamW (LoRA+ learning rate on B).
 * [ENT] backward_through_layers, LoRA Q and V blocks, and cpu_adamw.
 * Adapter output s (x A^T) B^T with s = alpha / rank and saved h = x A^T:
 *   g  = s dy B        [rows, rank]   (B before this call's update)
 *   dB = s dy^T h      [out, rank]
 *   dA = g^T x         [rank, in]
 *   gnorm_sq += ||dA||^2           (A only, before the update)
 *   for (P, dP, lr) in (A, dA, lr_a), (B, dB, lr_b):
 *     m = b1 m + (1-b1) dP;  v = b2 v + (1-b2) dP^2
 *     P -= lr (m/(1-b1^step) / (sqrt(v/(1-b2^step)) + eps) + weight_decay P)
 * dy f32 [rows, out]; x act [rows, in]; h act [rows, rank]
 * A, m_a, v_a f32 [rank, in]; B, m_b, v_b f32 [out, rank] (updated in place)
 * grad_a f32 [rank, in] or NULL; grad_b f32 [out, rank] or NULL (copies of
 * the gradients); gnorm_sq f32 device scalar or NULL (added to, once, after
 * a fixed-order reduction).  rank must be 1..64; step >= 1.
 * ---------------------------------------------------------------------- */
size_t lorabwd_lora_workspace_size(int64_t rows, int64_t in_dim, int64_t out_dim, int64_t rank);
int lorabwd_lora_grad_adamw(int64_t rows, int64_t in_dim, int64_t out_dim, int64_t rank,
                            const float* dy, const void* x, const void* h, float* A, float* B,
                            float* m_a, float* v_a, float* m_b, float* v_b, float* grad_a,
                            float* grad_b, float* gnorm_sq, float alpha, float lr_a,
                            float lr_b, float beta1, float beta2, float eps,
                            float weight_decay, int step, int dtype, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * The lm_head backward upstream of the layer stack, with AdamW on the
 * lm_head weight.  [ENT] wgpu_backward.rs, module doc (the gradient flows
 * from lm_head through the layers) and WgpuModelState (lm_head, lm_head_m,
 * lm_head_v).  With logits z = h W^T as saved by the forward and n the
 * number of rows whose label is in [0, vocab) (rows with any other label,
 * e.g. -100 for padding, are ignored: no loss, no gradient):
 *   loss        = (1/n) sum over labelled rows of logsumexp(z_s) - z_s[label_s]
 *   dlogits     = (softmax(z) - onehot(labels)) / n, zero on ignored rows
 *   grad_hidden = dlogits W            (W before this call's update)
 *   dW          = dlogits^T h
 *   m = b1 m + (1-b1) dW;  v = b2 v + (1-b2) dW^2
 *   W -= lr (m/(1-b1^step) / (sqrt(v/(1-b2^step)) + eps) + weight_decay W)
 * With no labelled row the loss and both gradients are 0 (AdamW still
 * steps, with a zero gradient).
 * h        f32 [rows, hidden]   the final hidden state (lm_head input)
 * logits   f32 [rows, vocab]    finite, or -inf for entries excluded from
 *                               the softmax (each labelled row needs one
 *                               finite entry)
 * labels   i32 [rows]           device memory
 * w, m, v  f32 [vocab, hidden]  updated in place
 * grad_hidden f32 [rows, hidden] out (the gradient handed to the top layer)
 * loss     f32 device scalar, out
 * grad_w   f32 [vocab, hidden] or NULL: a copy of dW
 * rows 0 .. 2^20; hidden a multiple of 8 up to 2^20; vocab a multiple of 4
 * up to 2^20 (vocabularies are commonly padded; give padding entries -inf
 * logits).  step >= 1.  Results are bitwise reproducible (no float atomics).
 * The workspace holds dlogits [rows, vocab] and the vocabulary-split partial
 * sums of grad_hidden.
 * ---------------------------------------------------------------------- */
size_t lorabwd_lm_head_workspace_size(int64_t rows, int64_t hidden, int64_t vocab);
int lorabwd_lm_head_backward(int64_t rows, int64_t hidden, int64_t vocab, const float* h,
                             const float* logits, const int32_t* labels, float* w, float* m,
                             float* v, float* grad_hidden, float* loss, float* grad_w, float lr,
                             float beta1, float beta2, float eps, float weight_decay, int step,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * One whole layer: [FFN] "Backward (reverse)" (lorabwd_ffn_backward with
 * d_resid == d_hidden), then [ATTN] "Gradient Flow": O-projection backward
 * dCtx = dH1 W_o, the attention sub-norm backward (sub_norms = 1),
 * lorabwd_attn_backward, lorabwd_rope_backward (positions pos0 + i), then
 * the LoRA Q and V updates of [ENT] backward_through_layers.
 *
 * With qk_norm = 1 the Q projection output went through a per-head RMSNorm
 * (one scale vector gamma_q of head_dim for every head) before RoPE, as the
 * trainer's saved Q is "after QK-norm + RoPE" ([ENT] LayerActivations): the
 * inverse RoPE is followed by that norm's backward on each head's slice,
 * from the saved projection output q_raw, and the LoRA Q signal is the
 * gradient of q_raw.  (On its own this step is lorabwd_rmsnorm_backward
 * with rows = seq * n_heads and n = head_dim.)
 *
 * With input_grad = 0 the gradient handed to the layer below is the
 * residual-stream gradient dH1 (the attention branch input is held fixed,
 * as [ATTN] "Gradient Flow" stops at dQpre and [ENT] passes only that
 * gradient down).  With input_grad = 1 it is the exact gradient of the
 * layer input x through both paths:
 *   dK    = scale dS^T Q (post-RoPE queries q), inverse RoPE at the key
 *           positions, (qk_norm) the per-head norm backward with gamma_k
 *           from the saved K projection output k_raw
 *   dXa   = dQpre W_q + dKpre W_k + dV W_v  over the chunk's own S rows
 *           + s (dQpre B_q) A_q + s (dV B_v) A_v  (adapters before the update)
 *   d_hidden = dH1 + rmsnorm_bwd(x, gamma_attn, dXa)
 * (needs w_q, w_k, w_v, gamma_attn, x and q; not for bf16 with head_dim 16;
 * one-token layers then run the general composition).
 * ---------------------------------------------------------------------- */
typedef struct lorabwd_layer_desc {
  int64_t seq;         /* query rows S */
  int64_t kv_len;      /* key/value rows (== seq, or the cache length in decode) */
  int64_t hidden;      /* H */
  int64_t ffn;         /* I */
  int64_t n_heads;     /* Hq */
  int64_t n_kv_heads;  /* Hkv */
  int64_t head_dim;    /* D */
  int64_t pos0;        /* RoPE position of query row 0 */
  int32_t act;         /* LORABWD_ACT_* */
  int32_t sub_norms;   /* 1: RMSNorm after the attention context and after the FFN activation */
  int32_t causal;      /* see lorabwd_attn_backward */
  int32_t dtype;       /* LORABWD_F32 / LORABWD_BF16: saved activations and base weights */
  float eps;           /* RMSNorm eps */
  float rope_base;
  float attn_scale;    /* usually 1/sqrt(head_dim) */
  float lora_alpha;    /* adapter scaling is lora_alpha / rank */
  int32_t qk_norm;     /* 1: per-head RMSNorm of the Q (and K) projection before RoPE */
  int32_t input_grad;  /* 1: differentiate the attention branch input too (see above) */
  int32_t weight_format; /* 0: w_o, w_gate, w_up, w_down in dtype; 1: packed ternary
                            (lorabwd_pack_ternary) with scales scale_o ... scale_down;
                            single-token layers only */
  int32_t reserved;    /* must be 0 */
} lorabwd_layer_desc;

typedef struct lorabwd_layer_weights {
  const void* w_o;          /* act [hidden, n_heads*head_dim] */
  const void* w_gate;       /* act [ffn, hidden] */
  const void* w_up;         /* act [ffn, hidden] */
  const void* w_down;       /* act [hidden, ffn] */
  const float* gamma_ffn;   /* [hidden] */
  const float* gamma_fsub;  /* [ffn]; sub_norms only */
  const float* gamma_asub;  /* [n_heads*head_dim]; sub_norms only */
  const float* gamma_q;     /* [head_dim]; qk_norm only */
  const void* w_q;          /* act [n_heads*head_dim, hidden]; input_grad only */
  const void* w_k;          /* act [n_kv_heads*head_dim, hidden]; input_grad only */
  const void* w_v;          /* act [n_kv_heads*head_dim, hidden]; input_grad only */
  const float* gamma_attn;  /* [hidden] the attention norm's scale; input_grad only */
  const float* gamma_k;     /* [head_dim]; qk_norm with input_grad */
  float scale_o, scale_gate, scale_up, scale_down;  /* packed ternary weights only */
} lorabwd_layer_weights;

typedef struct lorabwd_layer_saved {   /* all act type */
  const void* attn_input;  /* [seq, hidden]   normed attention input (LoRA x) */
  const void* resid1;      /* [seq, hidden]   residual stream before the FFN norm */
  const void* gate;        /* [seq, ffn] */
  const void* up;          /* [seq, ffn] */
  const void* hidden_pre;  /* [seq, ffn]      activation output before the sub-norm; sub_norms only */
  const void* ctx;         /* [seq, n_heads*head_dim]  P V before the attention sub-norm */
  const void* P;           /* [n_heads, seq, kv_len] */
  const void* K;           /* [kv_len, n_kv_heads*head_dim] after RoPE */
  const void* V;           /* [kv_len, n_kv_heads*head_dim] */
  const void* lora_q_h;    /* [seq, rank_q]   attn_input A_q^T */
  const void* lora_v_h;    /* [seq, rank_v]   attn_input A_v^T */
  const void* q_raw;       /* [seq, n_heads*head_dim]  Q projection output before QK-norm; qk_norm only */
  const void* x;           /* [seq, hidden]   layer input (before the attention norm); input_grad only */
  const void* q;           /* [seq, n_heads*head_dim]  Q after (QK-norm and) RoPE; input_grad only */
  const void* k_raw;       /* [seq, n_kv_heads*head_dim]  the chunk's K projection output before
                              QK-norm; qk_norm with input_grad */
} lorabwd_layer_saved;

typedef struct lorabwd_lora_state {
  int64_t rank;  /* 0 = no adapter (skipped, as the trainer skips rank 0) */
  float *A, *B, *m_a, *v_a, *m_b, *v_b;
} lorabwd_lora_state;

typedef struct lorabwd_adamw {
  float lr_a, lr_b, beta1, beta2, eps, weight_decay;
  int32_t step;
} lorabwd_adamw;

size_t lorabwd_layer_workspace_size(const lorabwd_layer_desc* d);
/* d_out     f32 [seq, hidden] or NULL: gradient of the layer output.  Read
 *           only; it must not overlap d_hidden.
 * d_hidden  f32 [seq, hidden]  out: dH1, the gradient at the layer input's
 *           residual stream.  With d_out NULL it is also the input (the
 *           gradient of the layer output, overwritten in place).
 * q_state / v_state: NULL (or rank 0) = no adapter on that projection.
 * dq_pre_out f32 [seq, n_heads*head_dim] or NULL: the LoRA Q signal (dL/d q_pre).
 * dv_out     f32 [kv_len, n_kv_heads*head_dim] or NULL: dL/dV.
 * gnorm_sq   f32 device scalar or NULL: += ||dA_q||^2 + ||dA_v||^2.
 * hp may be NULL only when both adapters are absent. */
int lorabwd_layer_backward(const lorabwd_layer_desc* d, const lorabwd_layer_weights* w,
                           const lorabwd_layer_saved* a, lorabwd_lora_state* q_state,
                           lorabwd_lora_state* v_state, const lorabwd_adamw* hp,
                           const float* d_out, float* d_hidden, float* dq_pre_out,
                           float* dv_out, float* gnorm_sq, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Measurement variant of lorabwd_layer_backward: the same work on the same
 * stream, and right after the i-th kernel it enqueues (i < capacity) it
 * records the caller-created HIP event events[i] on `stream` and fills
 * records[i] with the kernel's name, the algorithmic HBM bytes and
 * floating-point operations that kernel's step of the method has to move /
 * perform at this shape, and an estimate of the bytes it moves on top.
 * Algorithmic bytes are the method's single pass: every tensor at the step's
 * boundary read or written once at its storage type, masked attention pairs
 * excluded; a tensor that several launches of one step read (P in the dQ and
 * the dV launches, the partial sums of a split product) is counted once, at
 * one of them.  impl_bytes holds the rest: split-K and chunk partials,
 * transposed or rounded copies, second reads.  *n_kernels receives the
 * number of kernels enqueued.  With an event recorded just before the call,
 * consecutive events bracket each kernel.
 * ---------------------------------------------------------------------- */
typedef struct lorabwd_kernel_record {
  const char* name;  /* static string */
  double alg_bytes;
  double alg_flops;
  double impl_bytes;
} lorabwd_kernel_record;

int lorabwd_layer_backward_timed(const lorabwd_layer_desc* d, const lorabwd_layer_weights* w,
                                 const lorabwd_layer_saved* a, lorabwd_lora_state* q_state,
                                 lorabwd_lora_state* v_state, const lorabwd_adamw* hp,
                                 const float* d_out, float* d_hidden, float* dq_pre_out,
                                 float* dv_out, float* gnorm_sq, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream, hipEvent_t* events,
                                 lorabwd_kernel_record* records, int capacity, int* n_kernels);
/* The same measurement variant of lorabwd_lm_head_backward. */
int lorabwd_lm_head_backward_timed(int64_t rows, int64_t hidden, int64_t vocab, const float* h,
                                   const float* logits, const int32_t* labels, float* w,
                                   float* m, float* v, float* grad_hidden, float* loss,
                                   float* grad_w, float lr, float beta1, float beta2, float eps,
                                   float weight_decay, int step, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream, hipEvent_t* events,
                                   lorabwd_kernel_record* records, int capacity, int* n_kernels);

/* ------------------------------------------------------------------------
 * Allocation-free variant of lorabwd_layer_backward, for callers that cannot
 * allocate device memory or pass a workspace (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  Same arguments
 * and results as lorabwd_layer_backward, without workspace: the scratch is
 * a static device array of LORABWD_NOALLOC_SCRATCH_BYTES that every GPU the
 * library runs on holds until the process ends (found on the device that is
 * current at the call, once per device).  The single-token layer needs about
 * 3.6 MiB at hidden 2560 / ffn 6912 / 512 cached keys; a layer whose
 * lorabwd_layer_workspace_size exceeds the limit returns
 * LORABWD_ERR_WORKSPACE before anything is enqueued.  All calls on one GPU
 * share that scratch: calls that overlap in time on one GPU (different
 * streams, or graphs replayed concurrently) race and must not be issued.
 * ---------------------------------------------------------------------- */
#define LORABWD_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int lorabwd_layer_backward_noalloc(const lorabwd_layer_desc* d, const lorabwd_layer_weights* w,
                                   const lorabwd_layer_saved* a, lorabwd_lora_state* q_state,
                                   lorabwd_lora_state* v_state, const lorabwd_adamw* hp,
                                   const float* d_out, float* d_hidden, float* dq_pre_out,
                                   float* dv_out, float* gnorm_sq, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LORABWD_H */
