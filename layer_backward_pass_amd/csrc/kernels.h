// Internal launchers of the lorabwd kernels.  Each launcher only enqueues
// work on `stream`; arguments were validated by the C-ABI layer (api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lbp {

enum DType { F32 = 0, BF16 = 1, TERN2 = 2 };  // TERN2: packed ternary weights (GEMV only)

// Measurement hook: after each kernel launch a launcher calls mark() with the
// kernel's name, its algorithmic HBM bytes and flops (the method's single
// pass: every tensor at the step's boundary read or written once at its
// storage type, masked attention pairs excluded; a tensor read by several
// launches of one step is counted at one of them), and the implementation
// bytes it moves on top (split-K and chunk partials, transposed or rounded
// copies, second reads).  It does nothing unless the calling thread is inside
// lorabwd_layer_backward_timed, which then records a caller-owned event on
// the stream.
void mark(const char* name, double alg_bytes, double alg_flops, hipStream_t s,
          double impl_bytes = 0.0);

// Checking pass: while the calling thread runs a composition inside a dry
// run, every launcher only evaluates the shape limits of its kernels (buffer
// ranges, LDS sizes) and returns hipSuccess, or hipErrorInvalidValue for a
// shape its kernels cannot take, without any HIP call.  The C-ABI layer runs
// each composition this way before the real pass, so a shape the kernels
// reject is refused before anything is enqueued.  Outputs a launcher reports
// to its caller (split counts, which epilogue ran) are set as in a real pass.
bool dry_run();
enum ActKind { SWIGLU = 0, RELU2 = 1 };

// ---- row-wise kernels (rowwise.hip)
// dy may be `nparts` split-K partial sums [nparts][rows][n] (stride pstride),
// added in order; dx may alias dy when nparts == 1.  accumulate: dx = rin +
// result (rin NULL: dx += result).  dx16 (may be NULL): a bf16 copy of dx.
hipError_t launch_rmsnorm_bwd(int64_t rows, int64_t n, const void* x, int xdt, const float* gamma,
                              const float* dy, float* dx, float eps, int accumulate,
                              hipStream_t s, int nparts = 1, int64_t pstride = 0,
                              const float* rin = nullptr, uint16_t* dx16 = nullptr);
// The per-head RMSNorm backward that may follow the inverse RoPE (QK-norm):
// x [rows, n_heads * head_dim] (float, or bf16 when x_bf16), gamma
// [head_dim]; x NULL means no norm.
struct RopeNormArgs {
  const void* x;
  int x_bf16;
  const float* gamma;
  float eps;
};
// dy2 (may be NULL): a second term added to dy before the rotation; norm
// (may be NULL or have x NULL): the QK-norm backward after it
hipError_t launch_rope_bwd(int64_t rows, int64_t n_heads, int64_t head_dim, const float* dy,
                           float* dx, int64_t pos0, float base, hipStream_t s,
                           const float* dy2 = nullptr, const RopeNormArgs* norm = nullptr);
// threads of a row of the inverse RoPE: (pair, head group), at most 256
inline int rope_threads(int64_t n_heads, int64_t head_dim) {
  const int half = (int)head_dim / 2;
  int threads = 256 / half * half;
  if ((int64_t)(threads / half) > n_heads) threads = (int)n_heads * half;
  return threads;
}
// The inverse RoPE of the attention's dq rows into dx (positions pos0 ...),
// for launch_attn_bwd to run inside its last launch.
struct RopeArgs {
  float* dx;
  int64_t pos0;
  float base;
  RopeNormArgs norm;
};
// dgu[r, 0:I] = dGate, dgu[r, I:2I] = dUp; out_dt selects float or bf16 output;
// dhid may be `nparts` split-K partial sums (stride pstride), added in order.
hipError_t launch_act_bwd(int64_t rows, int64_t ffn, int act, const void* gate, const void* up,
                          int in_dt, const float* dhid, void* dgu, int out_dt, hipStream_t s,
                          int nparts = 1, int64_t pstride = 0);
// p[0:n] = 0 (a kernel, not a memset, so the call can sit in a captured graph)
hipError_t launch_fill_zero(int64_t n, float* p, hipStream_t s);

// ---- AdamW ([ENT] cpu_adamw): lr_a is the step size of every parameter but
// the LoRA B matrices, which take lr_b (LoRA+)
struct AdamHP {
  float lr_a, lr_b, beta1, beta2, eps, wd, bc1, bc2;
};
// One AdamW element step (bc1, bc2: the bias corrections 1/(1 - beta^step)).
__device__ __forceinline__ void adamw1(float& p, float gr, float& m, float& v, float lr,
                                       const AdamHP& hp) {
  m = hp.beta1 * m + (1.0f - hp.beta1) * gr;
  v = hp.beta2 * v + (1.0f - hp.beta2) * gr * gr;
  const float mh = m * hp.bc1, vh = v * hp.bc2;
  p -= lr * (mh / (sqrtf(vh) + hp.eps) + hp.wd * p);
}

// ---- products (gemm.hip)
// C[M,N] = A[M,K] B[K,N]; B rows k < K1 come from B1 (row k), rows k >= K1
// from B2 (row k - K1).  A is float or bf16 (a_dt), B is float or bf16
// (b_dt).  bf16 B runs on bf16 matrix cores (A rounded to bf16; an fp32 A
// is first rounded into `partials` after the split-K area).  split-K writes
// partial sums to `partials` ([splits, M, N]) and reduces them in order;
// `partials` must hold gemm_partial_bytes(M, N, K, a_dt, b_dt) bytes.
int gemm_splits(int64_t M, int64_t N, int64_t K, int b_dt);
size_t gemm_partial_bytes(int64_t M, int64_t N, int64_t K, int a_dt, int b_dt);
// With `deferred` non-null, a split-K product leaves its partial sums in
// `partials` ([splits][M][N], dense) for the consumer to add, and
// *deferred = splits (1: the result is in C).
// With `act` set, the product is dHid of a gated activation: where the plan
// allows (whole tiles, or a split tail that is reduced here) the store goes
// through the activation backward, out[r][0:N] = dGate, out[r][N:2N] = dUp
// from gate / up [M][N] (gdt, odt: F32 or BF16), C is not written and
// *act_done = true; otherwise C (or the deferred partials) as above.
struct ActEpi {
  const void* gate;
  const void* up;
  void* out;
  int act;  // ActKind
  int gdt, odt;
  int64_t ldt;  // (transposed copy) row stride of out
};
// With `tc` set (bf16 weights and A, no split), C is also written as a bf16
// copy transposed, tc->dst[n][m] with row stride tc->ld; *tc_done says so.
struct TCopy {
  uint16_t* dst;
  int64_t ld;
};
hipError_t launch_gemm(int64_t M, int64_t N, int64_t K, const void* A, int a_dt, int64_t lda,
                       const void* B1, const void* B2, int64_t K1, int b_dt, int64_t ldb,
                       float* C, int64_t ldc, float* partials, hipStream_t s,
                       int* deferred = nullptr, const ActEpi* act = nullptr,
                       bool* act_done = nullptr, const TCopy* tc = nullptr,
                       bool* tc_done = nullptr);
// A weight's gradient and its AdamW step in one launch: dW[M,N] = A^T[K,M]^T
// B[K,N] (fp32; A given transposed with row stride lda, B row stride ldb),
// never stored; W, m, v [M][N] (dense) are updated in place with step size
// lr, and dW is also copied to grad when that is set.  N % 8 == 0.
struct AdamEpi {
  float *w, *m, *v, *grad;
  AdamHP hp;
  float lr;
};
hipError_t launch_gemm_at_adamw(int64_t M, int64_t N, int64_t K, const float* At, int64_t lda,
                                const float* B, int64_t ldb, const AdamEpi& ad, hipStream_t s);

// ---- lm_head backward (lmhead.hip): softmax cross-entropy over the
// vocabulary, grad_hidden and AdamW on W (step size hp.lr_a); ws holds
// lm_head_ws_bytes.  vocab % 4 == 0, hidden % 8 == 0.
size_t lm_head_ws_bytes(int64_t rows, int64_t hidden, int64_t vocab);
hipError_t launch_lm_head_bwd(int64_t rows, int64_t hidden, int64_t vocab, const float* h,
                              const float* logits, const int32_t* labels, float* w, float* m,
                              float* v, float* grad_hidden, float* loss, float* grad_w,
                              const AdamHP& hp, void* ws, hipStream_t s);

// ---- single-token (decode) kernels (decode.hip)
// part[chunk, N] = x[K] W[K, N] over row chunks of kc rows (W rows k < K1
// from W1, the rest from W2).  With ng set, every workgroup also writes its
// share of the row sums of the RMSNorm that consumes y = sum of parts:
// scal[2*wg] = <y_part*ng, nx> over its columns and scal[2*wg+1] = sum nx^2
// over them (first row chunk only), wg = chunk * column_blocks + block.
// Prologue of a GEMV whose input x is the output of the previous one: every
// workgroup sums the producer's row-chunk partials for its own rows, takes
// the RMSNorm constants from the producer's shares, and applies the
// elementwise step on the way into LDS.
//   PRO_ACT    x = [dGate | dUp] of dHid = norm(sum of parts) (the norm only
//              when scal is set); x has 2 pn rows
//   PRO_RESID  x = resid + rmsnorm_bwd(nx, ngam, sum of parts); workgroups of
//              column block 0 also store x to xout
enum GemvProMode { PRO_COPY = 0, PRO_ACT = 1, PRO_RESID = 2 };
struct GemvPro {
  const float* part;
  int splits;
  int64_t pn;
  const float* scal;
  int64_t nscal;
  const void* nx;
  const float* ngam;
  float eps;
  const void* gate;
  const void* up;
  int act;
  const float* resid;
  float* xout;
};
// With packed ternary weights (w_dt TERN2), s1 / s2 are the scales of the
// rows k < K1 (W1) and k >= K1 (W2); dense weights ignore them.
struct GemvArgs {
  int64_t N, K, K1, kc;
  float s1, s2;
  const void* W1;
  const void* W2;
  const float* x;  // PRO_COPY input
  float* part;
  float* scal;
  const void* nx;
  const float* ng;
  int pro;  // GemvProMode
  GemvPro p;
};

// y = sum over `splits` chunks of part, then:
//   scal set: z = rmsnorm_bwd(nx, ngam, y) with row sums from the nscal
//             shares in scal; else z = y
//   RED_STORE  y_out[n] = z
//   RED_ACCUM  y_out[n] = (yin ? yin : y_out)[n] + z   (residual skip)
//   RED_ACT    y_out[n] = dGate(z), y_out[N + n] = dUp(z) from gate, up
enum RedMode { RED_STORE = 0, RED_ACCUM = 1, RED_ACT = 2 };
struct RedArgs {
  int64_t N;
  int splits;
  const float* part;
  float* y;
  const float* yin;  // RED_ACCUM: the residual term (NULL: y itself)
  const float* scal;
  int64_t nscal;
  const void* nx;
  const float* ngam;
  float eps;
  const void* gate;
  const void* up;
  int act;
  // optional plain copy done by the same launch: copy_dst[i] = copy_src[i]
  const float* copy_src;
  float* copy_dst;
  int64_t copy_n;
};

// rows per chunk, chunk count, partial bytes and norm-share count of the
// GEMV over K rows and N columns launched with prologue mode `pro`
int64_t dgemv_kc(int64_t N, int64_t K, int pro = PRO_COPY);
int64_t dgemv_splits(int64_t N, int64_t K, int pro = PRO_COPY);
size_t dgemv_part_bytes(int64_t N, int64_t K, int pro = PRO_COPY);
int64_t dgemv_nscal(int64_t N, int64_t K, int pro = PRO_COPY);
hipError_t launch_dgemv(int w_dt, int a_dt, GemvArgs a, hipStream_t s);
// Packed ternary weights: out [rows][cols / 4] bytes from w [rows][cols]
// (float or bf16, w_dt), each value coded by its sign (see tern2 in common.h).
hipError_t launch_pack_ternary(int64_t rows, int64_t cols, const void* w, int w_dt, uint8_t* out,
                               hipStream_t s);
hipError_t launch_dgemv_red(int mode, int a_dt, RedArgs a, hipStream_t s);

// One query row against s_kv keys.  With ctx: dec_attn1c (per key block:
// dA, dv, dS with delta = <dctx, ctx>, a share of dq) then dec_attn_dqc
// (sum of shares, scale, inverse RoPE when rope is set).  Without ctx:
// dec_attn1 (dA, dv) then dec_attn2 (delta = sum P dA, dS, dq, RoPE).
struct DecAttnArgs {
  int64_t s_kv;
  int Hq, grp;
  const float* dctx;
  const void* P;
  const void* K;
  const void* V;
  const void* ctx;  // P V (forward attention output) or NULL
  float* dA;        // scratch, dec_attn_ws_bytes (dA, or the dq shares when ctx is set)
  float* dq_part;   // same scratch as dA
  float* dv;
  float* dq;
  float scale;
  int rope;
  int64_t pos;
  double log2_base;
  // With part set (dec_attn_red_fits), dctx is not read: every workgroup
  // forms its KV group's dCtx columns from `splits` partial sums
  // part[splits][Hq D] and, with nsc set, applies the RMSNorm backward over
  // the concatenated heads (x = ctx, weight ngam, length Hq D) with the row
  // sums from the nscal share pairs nsc (<y ngam, x>, sum x^2).  copy_n
  // floats copy_src -> copy_dst are moved on the side.
  const float* part;
  int splits;
  const float* nsc;
  int64_t nscal;
  const float* ngam;
  float eps;
  const float* copy_src;
  float* copy_dst;
  int64_t copy_n;
};
bool dec_attn_red_fits(int64_t n_heads, int64_t n_kv_heads, int64_t head_dim, int splits);
bool dec_attn_fits(int64_t s_kv, int64_t n_heads, int64_t n_kv_heads, int64_t head_dim);
size_t dec_attn_ws_bytes(int64_t s_kv, int64_t n_heads, int64_t head_dim);
hipError_t launch_dec_attn(int dt, int head_dim, const DecAttnArgs& a, hipStream_t s);

// ---- attention (attn.hip)
// With rope set, the inverse RoPE of dq (plus the split second half) may run
// in the launch that adds the dV chunk partials; *rope_done says whether it
// did (else the caller runs it, with *dq_second as dy2).
// With dk set, also dK = scale dS^T Q [s_kv, n_kv_heads*head_dim] (after
// RoPE, like K) from the post-RoPE queries Q (act type): the dQ kernels store
// scale dS and the dV kernels run a second pass on (scale dS, Q).  The
// workspace must then be attn_ws_bytes(..., with_dk = true); not for bf16
// with head_dim 16 (hipErrorInvalidValue).
size_t attn_ws_bytes(int64_t s_q, int64_t s_kv, int64_t n_heads, int64_t n_kv_heads,
                     int64_t head_dim, int dt, bool with_dk = false);
hipError_t launch_attn_bwd(int64_t s_q, int64_t s_kv, int64_t n_heads, int64_t n_kv_heads,
                           int64_t head_dim, const float* dctx, const void* P, const void* K,
                           const void* V, const void* ctx, int dt, float* dq, float* dv,
                           float scale, int causal, void* ws, hipStream_t s,
                           const float** dq_second = nullptr, const RopeArgs* rope = nullptr,
                           bool* rope_done = nullptr, bool dct_ready = false,
                           const void* Q = nullptr, float* dk = nullptr);
// The bf16 attention's dCtxᵀ buffer inside its workspace (bf16 [Hq D][LQ],
// LQ = s_q rounded up to 64), or NULL where the path takes none.  A caller
// that fills it (dct_ready) spares the attention its transposition.
uint16_t* attn_dct_buffer(void* ws, int64_t s_q, int64_t s_kv, int64_t n_heads,
                          int64_t n_kv_heads, int64_t head_dim, int dt, int64_t* LQ);

// ---- LoRA + AdamW (lora.hip)
size_t lora_ws_bytes(int64_t rows, int64_t in_dim, int64_t out_dim, int64_t rank);
// One adapter's LoRA gradient + AdamW work (ws: its own lora_ws_bytes).
struct LoraJob {
  int64_t rows, in_dim, out_dim, rank;
  const float* dy;
  const void* x;
  const void* h;
  int dt;
  float *A, *B, *m_a, *v_a, *m_b, *v_b, *grad_a, *grad_b;
  float scaling;
  void* ws;
};
// Up to two adapters, in the same launches where their shapes allow;
// gnorm_sq += ||dA||^2 of each, in job order.  With dx set (jobs sharing
// rows and in_dim), also dx [rows][in_dim] = sum over the adapters of
// s (dy B) A with the B and A of before the update: their share of the
// gradient at the adapters' input.
hipError_t launch_lora_adamw_jobs(const LoraJob* jobs, int njobs, float* gnorm_sq,
                                  const AdamHP& hp, hipStream_t s, float* dx = nullptr);
hipError_t launch_lora_adamw(int64_t rows, int64_t in_dim, int64_t out_dim, int64_t rank,
                             const float* dy, const void* x, const void* h, int dt, float* A,
                             float* B, float* m_a, float* v_a, float* m_b, float* v_b,
                             float* grad_a, float* grad_b, float* gnorm_sq, float scaling,
                             const AdamHP& hp, void* ws, hipStream_t s);

}  // namespace lbp
