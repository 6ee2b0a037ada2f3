// C ABI of the lorabwd library: argument validation (always before any HIP
// call, so a rejected call enqueues nothing), workspace sizing, and the
// composition of the FFN and whole-layer backward from the kernels.
#include <math.h>
#include <string.h>

#include <mutex>

#include "../../include/lorabwd.h"
#include "kernels.h"

using namespace lbp;

namespace lbp {

struct Recorder {
  hipEvent_t* events;
  lorabwd_kernel_record* records;
  int capacity;
  int count;
};
static thread_local Recorder* tl_recorder = nullptr;
static thread_local bool tl_dry = false;

bool dry_run() { return tl_dry; }

void mark(const char* name, double alg_bytes, double alg_flops, hipStream_t s,
          double impl_bytes) {
  Recorder* r = tl_recorder;
  if (r == nullptr) return;
  if (r->count < r->capacity) {
    (void)hipEventRecord(r->events[r->count], s);
    r->records[r->count].name = name;
    r->records[r->count].alg_bytes = alg_bytes;
    r->records[r->count].alg_flops = alg_flops;
    r->records[r->count].impl_bytes = impl_bytes;
  }
  ++r->count;
}

}  // namespace lbp

namespace {

constexpr size_t kAlign = 256;

inline size_t up(size_t b) { return (b + kAlign - 1) / kAlign * kAlign; }
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline bool dtype_ok(int dt) { return dt == LORABWD_F32 || dt == LORABWD_BF16; }
inline size_t esize(int dt) { return dt == LORABWD_BF16 ? 2 : 4; }
// Size limits of every entry point (lorabwd.h): row counts and feature
// sizes up to 2^20, at most 4096 heads.  Within them all grid dimensions fit;
// the kernels' own limits (1 GiB buffer ranges, LDS) are checked by the
// checking pass below.
constexpr int64_t kMaxRows = int64_t(1) << 20;
constexpr int64_t kMaxFeat = int64_t(1) << 20;
constexpr int64_t kMaxHeads = 4096;
inline bool rows_ok(int64_t r) { return r >= 0 && r <= kMaxRows; }
inline bool feat_ok(int64_t n) { return n > 0 && n % 8 == 0 && n <= kMaxFeat; }
inline bool head_dim_ok(int64_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }
inline bool heads_ok(int64_t hq, int64_t hkv, int64_t d) {
  return hq >= 1 && hkv >= 1 && hq <= kMaxHeads && hq % hkv == 0 && head_dim_ok(d) &&
         hq * d <= kMaxFeat;
}
inline bool finite(float x) { return isfinite(x); }

// Byte ranges [a, a+na) and [b, b+nb) intersect.
inline bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// Carves aligned sub-buffers out of a workspace.
struct Carver {
  char* p;
  size_t used = 0;
  explicit Carver(void* base) : p((char*)base) {}
  template <typename T>
  T* take(size_t bytes) {
    T* r = (T*)(p ? p + used : nullptr);
    used += up(bytes);
    return r;
  }
};

#define LBP_CHECK(cond, code) \
  do {                        \
    if (!(cond)) return (code); \
  } while (0)

#define LBP_HIP(expr)                                   \
  do {                                                  \
    if ((expr) != hipSuccess) return LORABWD_ERR_HIP;   \
  } while (0)

// Runs a composition of launchers as a checking pass (no HIP call is made,
// see dry_run in kernels.h): LORABWD_OK, or LORABWD_ERR_SHAPE where some
// kernel cannot take the shape.  Every entry point passes this before its
// real pass, so a refused shape leaves nothing enqueued.
template <typename Fn>
int check_pass(Fn&& fn) {
  tl_dry = true;
  const hipError_t e = fn();
  tl_dry = false;
  return e == hipSuccess ? LORABWD_OK : LORABWD_ERR_SHAPE;
}

#define LBP_E(expr)                                \
  do {                                             \
    if ((e = (expr)) != hipSuccess) return e;      \
  } while (0)

#define LBP_RUN(expr)                                   \
  do {                                                  \
    const int st_ = check_pass([&] { return (expr); }); \
    if (st_ != LORABWD_OK) return st_;                  \
    LBP_HIP(expr);                                      \
  } while (0)

// ---------------------------------------------------------------- FFN
struct FfnPlan {
  float *dhid, *dn2, *partials;          // rows > 1
  void* dgu;
  float *part1, *part2, *scal1, *scal2;  // rows == 1
  size_t bytes;
};

// rows == 1 runs the single-token GEMV chain (decode.hip); more rows run
// the MFMA products with the elementwise kernels between them.
FfnPlan ffn_plan(void* ws, int64_t rows, int64_t dim, int64_t ffn, int dt) {
  Carver c(ws);
  FfnPlan p{};
  if (rows == 1) {
    p.part1 = c.take<float>(dgemv_part_bytes(ffn, dim));
    p.part2 = c.take<float>(dgemv_part_bytes(dim, 2 * ffn, PRO_ACT));
    p.scal1 = c.take<float>((size_t)2 * dgemv_nscal(ffn, dim) * 4);
    p.scal2 = c.take<float>((size_t)2 * dgemv_nscal(dim, 2 * ffn, PRO_ACT) * 4);
  } else {
    p.dhid = c.take<float>((size_t)rows * ffn * 4);
    p.dgu = c.take<void>((size_t)rows * 2 * ffn * esize(dt));
    p.dn2 = c.take<float>((size_t)rows * dim * 4);
    const size_t a = gemm_partial_bytes(rows, ffn, dim, F32, dt);
    const size_t b = gemm_partial_bytes(rows, dim, 2 * ffn, dt, dt);
    p.partials = c.take<float>(a > b ? a : b);
  }
  p.bytes = c.used;
  return p;
}

int ffn_validate(int64_t rows, int64_t dim, int64_t ffn, int act, const float* d_out,
                 const void* w_down, const void* w_gate, const void* w_up, const void* gate,
                 const void* up_, const void* hidden_pre, const float* gamma_sub,
                 const void* resid1, const float* gamma_ffn, float* d_resid, float eps, int dt,
                 bool packed_w = false) {
  LBP_CHECK(dtype_ok(dt), LORABWD_ERR_DTYPE);
  LBP_CHECK(act == LORABWD_ACT_SWIGLU || act == LORABWD_ACT_RELU2, LORABWD_ERR_DTYPE);
  LBP_CHECK(rows_ok(rows) && feat_ok(dim) && feat_ok(ffn), LORABWD_ERR_SHAPE);
  LBP_CHECK(finite(eps) && eps >= 0.f, LORABWD_ERR_ARG);
  if (rows == 0) return LORABWD_OK;
  LBP_CHECK(d_out && w_down && w_gate && w_up && gate && up_ && resid1 && gamma_ffn && d_resid,
            LORABWD_ERR_NULL);
  LBP_CHECK((hidden_pre == nullptr) == (gamma_sub == nullptr), LORABWD_ERR_NULL);
  const void* ptrs[] = {d_out, w_down, w_gate, w_up, gate, up_, resid1, gamma_ffn, d_resid,
                        hidden_pre, gamma_sub};
  for (const void* q : ptrs) LBP_CHECK(aligned16(q), LORABWD_ERR_ALIGN);
  const size_t nres = (size_t)rows * dim * 4;
  LBP_CHECK(d_resid == d_out || !overlap(d_resid, nres, d_out, nres), LORABWD_ERR_ALIAS);
  const size_t es = esize(dt);
  const size_t wn = packed_w ? (size_t)dim * ffn / 4 : (size_t)dim * ffn * es;  // weight bytes
  const void* ins[] = {w_down, w_gate, w_up, gate, up_, resid1, hidden_pre};
  const size_t ns[] = {wn, wn, wn,
                       (size_t)rows * ffn * es, (size_t)rows * ffn * es, (size_t)rows * dim * es,
                       (size_t)rows * ffn * es};
  for (int i = 0; i < 7; ++i) LBP_CHECK(!overlap(d_resid, nres, ins[i], ns[i]), LORABWD_ERR_ALIAS);
  LBP_CHECK(!overlap(d_resid, nres, gamma_ffn, (size_t)dim * 4), LORABWD_ERR_ALIAS);
  return LORABWD_OK;
}

hipError_t ffn_run(int64_t rows, int64_t dim, int64_t ffn, int act, const float* d_out,
                   const void* w_down, const void* w_gate, const void* w_up, const void* gate,
                   const void* up_, const void* hidden_pre, const float* gamma_sub,
                   const void* resid1, const float* gamma_ffn, float* d_resid, float eps, int dt,
                   void* ws, hipStream_t s, const float* resid_in = nullptr,
                   uint16_t* d_resid16 = nullptr) {
  if (rows == 0) return hipSuccess;
  FfnPlan p = ffn_plan(ws, rows, dim, ffn, dt);
  hipError_t e;
  if (rows == 1) {
    // 1. part1 = d_out W_down (+ the FFN sub-norm's row-sum shares)
    GemvArgs g{};
    g.N = ffn;
    g.K = dim;
    g.W1 = w_down;
    g.x = d_out;
    g.part = p.part1;
    if (hidden_pre) {
      g.ng = gamma_sub;
      g.nx = hidden_pre;
      g.scal = p.scal1;
    }
    if ((e = launch_dgemv(dt, dt, g, s)) != hipSuccess) return e;
    // 2-4. part2 = [dGate | dUp] [W_gate; W_up] (+ the FFN norm's row-sum
    // shares); the prologue forms each workgroup's slice of [dGate | dUp]
    // from part1: dHid, sub-norm backward, activation backward
    g = GemvArgs{};
    g.N = dim;
    g.K = 2 * ffn;
    g.K1 = ffn;
    g.W1 = w_gate;
    g.W2 = w_up;
    g.part = p.part2;
    g.ng = gamma_ffn;
    g.nx = resid1;
    g.scal = p.scal2;
    g.pro = PRO_ACT;
    g.p.part = p.part1;
    g.p.splits = (int)dgemv_splits(ffn, dim);
    g.p.pn = ffn;
    if (hidden_pre) {
      g.p.scal = p.scal1;
      g.p.nscal = dgemv_nscal(ffn, dim);
      g.p.nx = hidden_pre;
      g.p.ngam = gamma_sub;
      g.p.eps = eps;
    }
    g.p.gate = gate;
    g.p.up = up_;
    g.p.act = act;
    if ((e = launch_dgemv(dt, dt, g, s)) != hipSuccess) return e;
    // 5. d_resid = (resid_in or d_resid) + rmsnorm_bwd(resid1, gamma_ffn, dN2)
    RedArgs r{};
    r.N = dim;
    r.splits = (int)dgemv_splits(dim, 2 * ffn, PRO_ACT);
    r.part = p.part2;
    r.y = d_resid;
    r.yin = resid_in;
    r.scal = p.scal2;
    r.nscal = dgemv_nscal(dim, 2 * ffn, PRO_ACT);
    r.nx = resid1;
    r.ngam = gamma_ffn;
    r.eps = eps;
    return launch_dgemv_red(RED_ACCUM, dt, r, s);
  }
  // 1. dHid = d_out W_down (split-K partials are added by the next kernel);
  // without a sub-norm the product's store may apply step 3 itself
  int n1 = 1;
  const ActEpi ae{gate, up_, p.dgu, act, dt, dt};
  bool act_done = false;
  e = launch_gemm(rows, ffn, dim, d_out, F32, dim, w_down, nullptr, dim, dt, ffn, p.dhid, ffn,
                  p.partials, s, &n1, hidden_pre ? nullptr : &ae, &act_done);
  if (e != hipSuccess) return e;
  const float* dh = n1 > 1 ? p.partials : p.dhid;
  const int64_t dhs = n1 > 1 ? rows * ffn : 0;
  // 2. sub-norm backward
  if (hidden_pre) {
    e = launch_rmsnorm_bwd(rows, ffn, hidden_pre, dt, gamma_sub, dh, p.dhid, eps, 0, s, n1, dhs);
    if (e != hipSuccess) return e;
    dh = p.dhid;
    n1 = 1;
  }
  // 3. gated activation backward -> [dGate | dUp]
  if (!act_done) {
    e = launch_act_bwd(rows, ffn, act, gate, up_, dt, dh, p.dgu, dt, s, n1, dhs);
    if (e != hipSuccess) return e;
  }
  // 4. dN2 = [dGate | dUp] [W_gate; W_up] (the partials of W_down are dead);
  // split-K partials are left for the norm below, which reads its row once
  int n2 = 1;
  e = launch_gemm(rows, dim, 2 * ffn, p.dgu, dt, 2 * ffn, w_gate, w_up, ffn, dt, dim, p.dn2, dim,
                  p.partials, s, &n2);
  if (e != hipSuccess) return e;
  // 5. d_resid = (resid_in or d_resid) + rmsnorm_bwd(resid1, gamma_ffn, dN2),
  // with a bf16 copy in d_resid16 when asked for
  return launch_rmsnorm_bwd(rows, dim, resid1, dt, gamma_ffn, n2 > 1 ? p.partials : p.dn2, d_resid,
                            eps, 1, s, n2, n2 > 1 ? rows * dim : 0, resid_in, d_resid16);
}

// ---------------------------------------------------------------- LoRA
int lora_validate(int64_t rows, int64_t in_dim, int64_t out_dim, int64_t rank, const float* dy,
                  const void* x, const void* h, float* A, float* B, float* m_a, float* v_a,
                  float* m_b, float* v_b, float* grad_a, float* grad_b, float* gnorm_sq,
                  float alpha, float lr_a, float lr_b, float beta1, float beta2, float eps,
                  float wd, int step, int dt) {
  LBP_CHECK(dtype_ok(dt), LORABWD_ERR_DTYPE);
  LBP_CHECK(rows_ok(rows) && feat_ok(in_dim) && out_dim > 0 && out_dim <= kMaxFeat && rank >= 1 &&
                rank <= 64,
            LORABWD_ERR_SHAPE);
  LBP_CHECK(step >= 1, LORABWD_ERR_STEP);
  LBP_CHECK(finite(alpha) && finite(lr_a) && finite(lr_b) && finite(wd) && finite(eps) &&
                eps >= 0.f && beta1 >= 0.f && beta1 < 1.f && beta2 >= 0.f && beta2 < 1.f,
            LORABWD_ERR_ARG);
  LBP_CHECK(A && B && m_a && v_a && m_b && v_b, LORABWD_ERR_NULL);
  if (rows > 0) LBP_CHECK(dy && x && h, LORABWD_ERR_NULL);
  const void* ptrs[] = {dy, x, h, A, B, m_a, v_a, m_b, v_b, grad_a, grad_b};
  for (const void* q : ptrs) LBP_CHECK(aligned16(q), LORABWD_ERR_ALIGN);
  LBP_CHECK(((uintptr_t)gnorm_sq & 3u) == 0, LORABWD_ERR_ALIGN);
  const size_t na = (size_t)rank * in_dim * 4, nb = (size_t)out_dim * rank * 4;
  float* outs[] = {A, m_a, v_a, grad_a, B, m_b, v_b, grad_b};
  const size_t ns[] = {na, na, na, na, nb, nb, nb, nb};
  for (int i = 0; i < 8; ++i)
    for (int j = i + 1; j < 8; ++j)
      LBP_CHECK(!overlap(outs[i], ns[i], outs[j], ns[j]), LORABWD_ERR_ALIAS);
  for (int i = 0; i < 8; ++i) {
    LBP_CHECK(!overlap(outs[i], ns[i], dy, (size_t)rows * out_dim * 4), LORABWD_ERR_ALIAS);
    LBP_CHECK(!overlap(outs[i], ns[i], x, (size_t)rows * in_dim * esize(dt)), LORABWD_ERR_ALIAS);
    LBP_CHECK(!overlap(outs[i], ns[i], h, (size_t)rows * rank * esize(dt)), LORABWD_ERR_ALIAS);
    LBP_CHECK(!overlap(outs[i], ns[i], gnorm_sq, 4), LORABWD_ERR_ALIAS);
  }
  return LORABWD_OK;
}

AdamHP make_hp(float lr_a, float lr_b, float beta1, float beta2, float eps, float wd, int step) {
  AdamHP hp;
  hp.lr_a = lr_a;
  hp.lr_b = lr_b;
  hp.beta1 = beta1;
  hp.beta2 = beta2;
  hp.eps = eps;
  hp.wd = wd;
  // bias corrections 1/(1 - beta^step), formed in float64 once per call
  hp.bc1 = (float)(1.0 / (1.0 - pow((double)beta1, (double)step)));
  hp.bc2 = (float)(1.0 / (1.0 - pow((double)beta2, (double)step)));
  return hp;
}

// ---------------------------------------------------------------- attention
int attn_validate(int64_t s_q, int64_t s_kv, int64_t Hq, int64_t Hkv, int64_t D,
                  const float* dctx, const void* P, const void* K, const void* V,
                  const void* ctx, float* dq, float* dv, float scale, int causal, int dt) {
  LBP_CHECK(dtype_ok(dt), LORABWD_ERR_DTYPE);
  LBP_CHECK(rows_ok(s_q) && rows_ok(s_kv) && heads_ok(Hq, Hkv, D), LORABWD_ERR_SHAPE);
  LBP_CHECK(causal == 0 || causal == 1, LORABWD_ERR_ARG);
  LBP_CHECK(!causal || s_q <= s_kv, LORABWD_ERR_SHAPE);
  LBP_CHECK(s_q == 0 || s_kv >= 1, LORABWD_ERR_SHAPE);
  LBP_CHECK(finite(scale), LORABWD_ERR_ARG);
  if (s_q == 0 && (dv == nullptr || s_kv == 0)) return LORABWD_OK;
  if (s_q > 0) LBP_CHECK(dctx && P && K && V && dq, LORABWD_ERR_NULL);
  const void* ptrs[] = {dctx, P, K, V, ctx, dq, dv};
  for (const void* q : ptrs) LBP_CHECK(aligned16(q), LORABWD_ERR_ALIGN);
  const size_t es = esize(dt);
  const size_t nq = (size_t)s_q * Hq * D, nkv = (size_t)s_kv * Hkv * D;
  const void* ins[] = {dctx, P, K, V, ctx};
  const size_t ns[] = {nq * 4, (size_t)Hq * s_q * s_kv * es, nkv * es, nkv * es, nq * es};
  for (int i = 0; i < 5; ++i) {
    LBP_CHECK(!overlap(dq, nq * 4, ins[i], ns[i]), LORABWD_ERR_ALIAS);
    LBP_CHECK(!overlap(dv, nkv * 4, ins[i], ns[i]), LORABWD_ERR_ALIAS);
  }
  LBP_CHECK(!overlap(dq, nq * 4, dv, nkv * 4), LORABWD_ERR_ALIAS);
  return LORABWD_OK;
}

}  // namespace

// =========================================================================
extern "C" {

const char* lorabwd_status_string(int status) {
  switch (status) {
    case LORABWD_OK: return "ok";
    case LORABWD_ERR_NULL: return "required pointer is NULL";
    case LORABWD_ERR_SHAPE: return "unsupported or inconsistent shape";
    case LORABWD_ERR_ALIGN: return "pointer not 16-byte aligned";
    case LORABWD_ERR_DTYPE: return "unknown dtype or activation";
    case LORABWD_ERR_WORKSPACE: return "workspace missing or too small";
    case LORABWD_ERR_STEP: return "AdamW step must be >= 1";
    case LORABWD_ERR_ALIAS: return "buffers overlap where not allowed";
    case LORABWD_ERR_HIP: return "HIP launch failed";
    case LORABWD_ERR_ARG: return "scalar argument out of range";
    default: return "unknown status";
  }
}

int lorabwd_abi_version(void) { return 6; }

int lorabwd_rmsnorm_backward(int64_t rows, int64_t n, const void* x, const float* gamma,
                             const float* dy, float* dx, float eps, int accumulate, int dtype,
                             hipStream_t stream) {
  LBP_CHECK(dtype_ok(dtype), LORABWD_ERR_DTYPE);
  LBP_CHECK(rows_ok(rows) && feat_ok(n), LORABWD_ERR_SHAPE);
  LBP_CHECK(finite(eps) && eps >= 0.f && (accumulate == 0 || accumulate == 1), LORABWD_ERR_ARG);
  if (rows == 0) return LORABWD_OK;
  LBP_CHECK(x && gamma && dy && dx, LORABWD_ERR_NULL);
  LBP_CHECK(aligned16(x) && aligned16(gamma) && aligned16(dy) && aligned16(dx), LORABWD_ERR_ALIGN);
  const size_t nb = (size_t)rows * n * 4;
  LBP_CHECK(dx == dy || !overlap(dx, nb, dy, nb), LORABWD_ERR_ALIAS);
  LBP_CHECK(!overlap(dx, nb, x, (size_t)rows * n * esize(dtype)), LORABWD_ERR_ALIAS);
  LBP_CHECK(!overlap(dx, nb, gamma, (size_t)n * 4), LORABWD_ERR_ALIAS);
  LBP_RUN(launch_rmsnorm_bwd(rows, n, x, dtype, gamma, dy, dx, eps, accumulate, stream));
  return LORABWD_OK;
}

int lorabwd_rope_backward(int64_t rows, int64_t n_heads, int64_t head_dim, const float* dy,
                          float* dx, int64_t pos0, float base, hipStream_t stream) {
  LBP_CHECK(rows_ok(rows) && heads_ok(n_heads, 1, head_dim) && pos0 >= 0 && pos0 <= (int64_t(1) << 40),
            LORABWD_ERR_SHAPE);
  LBP_CHECK(finite(base) && base > 0.f, LORABWD_ERR_ARG);
  if (rows == 0) return LORABWD_OK;
  LBP_CHECK(dy && dx, LORABWD_ERR_NULL);
  LBP_CHECK(aligned16(dy) && aligned16(dx), LORABWD_ERR_ALIGN);
  const size_t nb = (size_t)rows * n_heads * head_dim * 4;
  LBP_CHECK(dx == dy || !overlap(dx, nb, dy, nb), LORABWD_ERR_ALIAS);
  LBP_RUN(launch_rope_bwd(rows, n_heads, head_dim, dy, dx, pos0, base, stream));
  return LORABWD_OK;
}

size_t lorabwd_ternary_packed_bytes(int64_t rows, int64_t cols) {
  if (!rows_ok(rows) || rows > kMaxFeat || !feat_ok(cols)) return 0;
  return (size_t)rows * (size_t)(cols / 4);
}

int lorabwd_pack_ternary(int64_t rows, int64_t cols, const void* w, int dtype, uint8_t* packed,
                         hipStream_t stream) {
  LBP_CHECK(dtype_ok(dtype), LORABWD_ERR_DTYPE);
  LBP_CHECK(rows_ok(rows) && feat_ok(cols), LORABWD_ERR_SHAPE);
  if (rows == 0) return LORABWD_OK;
  LBP_CHECK(w && packed, LORABWD_ERR_NULL);
  LBP_CHECK(aligned16(w) && aligned16(packed), LORABWD_ERR_ALIGN);
  LBP_CHECK(!overlap(w, (size_t)rows * cols * esize(dtype), packed, (size_t)rows * (cols / 4)),
            LORABWD_ERR_ALIAS);
  LBP_RUN(launch_pack_ternary(rows, cols, w, dtype, packed, stream));
  return LORABWD_OK;
}

size_t lorabwd_attn_workspace_size(int64_t s_q, int64_t s_kv, int64_t n_heads,
                                   int64_t n_kv_heads, int64_t head_dim, int dtype) {
  if (s_q < 0 || s_kv < 0 || n_heads < 1 || n_kv_heads < 1) return 0;
  return up(attn_ws_bytes(s_q, s_kv, n_heads, n_kv_heads, head_dim, dtype));
}

int lorabwd_attn_backward(int64_t s_q, int64_t s_kv, int64_t n_heads, int64_t n_kv_heads,
                          int64_t head_dim, const float* dctx, const void* P, const void* K,
                          const void* V, const void* ctx, float* dq, float* dv, float scale,
                          int causal, int dtype, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  int st = attn_validate(s_q, s_kv, n_heads, n_kv_heads, head_dim, dctx, P, K, V, ctx, dq, dv,
                         scale, causal, dtype);
  if (st != LORABWD_OK) return st;
  if (s_q == 0 && (dv == nullptr || s_kv == 0)) return LORABWD_OK;
  const size_t need = lorabwd_attn_workspace_size(s_q, s_kv, n_heads, n_kv_heads, head_dim, dtype);
  LBP_CHECK(workspace_bytes >= need && (need == 0 || workspace != nullptr), LORABWD_ERR_WORKSPACE);
  LBP_CHECK(aligned16(workspace), LORABWD_ERR_ALIGN);
  LBP_RUN(launch_attn_bwd(s_q, s_kv, n_heads, n_kv_heads, head_dim, dctx, P, K, V, ctx, dtype, dq,
                          dv, scale, causal, workspace, stream));
  return LORABWD_OK;
}

size_t lorabwd_ffn_workspace_size(int64_t rows, int64_t dim, int64_t ffn_dim, int dtype) {
  if (rows <= 0 || dim <= 0 || ffn_dim <= 0) return 0;
  return ffn_plan(nullptr, rows, dim, ffn_dim, dtype).bytes;
}

int lorabwd_ffn_backward(int64_t rows, int64_t dim, int64_t ffn_dim, int act, const float* d_out,
                         const void* w_down, const void* w_gate, const void* w_up,
                         const void* gate, const void* up_, const void* hidden_pre,
                         const float* gamma_sub, const void* resid1, const float* gamma_ffn,
                         float* d_resid, float eps, int dtype, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  int st = ffn_validate(rows, dim, ffn_dim, act, d_out, w_down, w_gate, w_up, gate, up_,
                        hidden_pre, gamma_sub, resid1, gamma_ffn, d_resid, eps, dtype);
  if (st != LORABWD_OK || rows == 0) return st;
  const size_t need = lorabwd_ffn_workspace_size(rows, dim, ffn_dim, dtype);
  LBP_CHECK(workspace && workspace_bytes >= need, LORABWD_ERR_WORKSPACE);
  LBP_CHECK(aligned16(workspace), LORABWD_ERR_ALIGN);
  LBP_RUN(ffn_run(rows, dim, ffn_dim, act, d_out, w_down, w_gate, w_up, gate, up_, hidden_pre,
                  gamma_sub, resid1, gamma_ffn, d_resid, eps, dtype, workspace, stream));
  return LORABWD_OK;
}

size_t lorabwd_lora_workspace_size(int64_t rows, int64_t in_dim, int64_t out_dim, int64_t rank) {
  if (rows < 0 || in_dim <= 0 || out_dim <= 0 || rank <= 0) return 0;
  return up(lora_ws_bytes(rows, in_dim, out_dim, rank));
}

int lorabwd_lora_grad_adamw(int64_t rows, int64_t in_dim, int64_t out_dim, int64_t rank,
                            const float* dy, const void* x, const void* h, float* A, float* B,
                            float* m_a, float* v_a, float* m_b, float* v_b, float* grad_a,
                            float* grad_b, float* gnorm_sq, float alpha, float lr_a, float lr_b,
                            float beta1, float beta2, float eps, float weight_decay, int step,
                            int dtype, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  int st = lora_validate(rows, in_dim, out_dim, rank, dy, x, h, A, B, m_a, v_a, m_b, v_b, grad_a,
                         grad_b, gnorm_sq, alpha, lr_a, lr_b, beta1, beta2, eps, weight_decay,
                         step, dtype);
  if (st != LORABWD_OK) return st;
  const size_t need = lorabwd_lora_workspace_size(rows, in_dim, out_dim, rank);
  LBP_CHECK(workspace && workspace_bytes >= need, LORABWD_ERR_WORKSPACE);
  LBP_CHECK(aligned16(workspace), LORABWD_ERR_ALIGN);
  const AdamHP hp = make_hp(lr_a, lr_b, beta1, beta2, eps, weight_decay, step);
  LBP_RUN(launch_lora_adamw(rows, in_dim, out_dim, rank, dy, x, h, dtype, A, B, m_a, v_a, m_b,
                            v_b, grad_a, grad_b, gnorm_sq, alpha / (float)rank, hp, workspace,
                            stream));
  return LORABWD_OK;
}

// ---------------------------------------------------------------- lm_head
size_t lorabwd_lm_head_workspace_size(int64_t rows, int64_t hidden, int64_t vocab) {
  if (!rows_ok(rows) || !feat_ok(hidden) || vocab <= 0 || vocab % 4 != 0 || vocab > kMaxFeat)
    return 0;
  return up(lm_head_ws_bytes(rows, hidden, vocab));
}

int lorabwd_lm_head_backward(int64_t rows, int64_t hidden, int64_t vocab, const float* h,
                             const float* logits, const int32_t* labels, float* w, float* m,
                             float* v, float* grad_hidden, float* loss, float* grad_w, float lr,
                             float beta1, float beta2, float eps, float weight_decay, int step,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  LBP_CHECK(rows_ok(rows) && feat_ok(hidden) && vocab > 0 && vocab % 4 == 0 && vocab <= kMaxFeat,
            LORABWD_ERR_SHAPE);
  LBP_CHECK(step >= 1, LORABWD_ERR_STEP);
  LBP_CHECK(finite(lr) && finite(weight_decay) && finite(eps) && eps >= 0.f && beta1 >= 0.f &&
                beta1 < 1.f && beta2 >= 0.f && beta2 < 1.f,
            LORABWD_ERR_ARG);
  LBP_CHECK(w && m && v && loss, LORABWD_ERR_NULL);
  if (rows > 0) LBP_CHECK(h && logits && labels && grad_hidden, LORABWD_ERR_NULL);
  const void* ptrs[] = {h, logits, w, m, v, grad_hidden, grad_w};
  for (const void* q : ptrs) LBP_CHECK(aligned16(q), LORABWD_ERR_ALIGN);
  LBP_CHECK(((uintptr_t)loss & 3u) == 0 && ((uintptr_t)labels & 3u) == 0, LORABWD_ERR_ALIGN);
  // outputs pairwise disjoint, and disjoint from every input
  const size_t nw = (size_t)vocab * hidden * 4, nh = (size_t)rows * hidden * 4;
  const void* outs[] = {w, m, v, grad_w, grad_hidden, loss};
  const size_t ns[] = {nw, nw, nw, nw, nh, 4};
  for (int i = 0; i < 6; ++i) {
    for (int j = i + 1; j < 6; ++j)
      LBP_CHECK(!overlap(outs[i], ns[i], outs[j], ns[j]), LORABWD_ERR_ALIAS);
    LBP_CHECK(!overlap(outs[i], ns[i], h, nh), LORABWD_ERR_ALIAS);
    LBP_CHECK(!overlap(outs[i], ns[i], logits, (size_t)rows * vocab * 4), LORABWD_ERR_ALIAS);
    LBP_CHECK(!overlap(outs[i], ns[i], labels, (size_t)rows * 4), LORABWD_ERR_ALIAS);
  }
  const size_t need = lorabwd_lm_head_workspace_size(rows, hidden, vocab);
  LBP_CHECK(need == 0 || (workspace && workspace_bytes >= need), LORABWD_ERR_WORKSPACE);
  LBP_CHECK(aligned16(workspace), LORABWD_ERR_ALIGN);
  const AdamHP hp = make_hp(lr, lr, beta1, beta2, eps, weight_decay, step);
  LBP_RUN(launch_lm_head_bwd(rows, hidden, vocab, h, logits, labels, w, m, v, grad_hidden, loss,
                             grad_w, hp, workspace, stream));
  return LORABWD_OK;
}

// ---------------------------------------------------------------- layer
namespace {

struct LayerPlan {
  float *dctx, *dq, *dv;
  float *dk, *dkp, *xa;  // input_grad: dK [kv_len, kvd], dKpre [seq, kvd], dXa parts [4, seq, hidden]
  uint16_t* h16;  // bf16 copy of dH1: the W_o product's operand (bf16 sequence layers)
  float *part2, *x2, *scal1, *scal2, *scal3, *dA;  // single-token chain only
  void* scratch;
  size_t lora_v_off;  // the V adapter's LoRA workspace: scratch + lora_v_off
  size_t bytes;
};

bool has_lora(const lorabwd_lora_state* s) { return s != nullptr && s->rank > 0; }

// One token whose attention fits the decode kernels runs the fused GEMV
// chain of decode.hip; everything else runs the general composition.
bool use_decode_chain(const lorabwd_layer_desc* d) {
  return d->seq == 1 && !d->input_grad &&
         dec_attn_fits(d->kv_len, d->n_heads, d->n_kv_heads, d->head_dim);
}

LayerPlan layer_plan(void* ws, const lorabwd_layer_desc* d, int64_t rq, int64_t rv) {
  const int64_t S = d->seq, L = d->kv_len, H = d->hidden, I = d->ffn;
  const int64_t qd = d->n_heads * d->head_dim, kvd = d->n_kv_heads * d->head_dim;
  Carver c(ws);
  LayerPlan p{};
  p.dctx = c.take<float>((size_t)S * qd * 4);
  p.dq = c.take<float>((size_t)S * qd * 4);
  p.dv = c.take<float>((size_t)L * kvd * 4);
  // the two adapters run in the same launches, each in its own region
  const size_t lq = rq > 0 ? up(lora_ws_bytes(S, H, qd, rq)) : 0;
  const size_t lv = rv > 0 ? up(lora_ws_bytes(S, H, kvd, rv)) : 0;
  size_t sc = lq + lv;
  p.lora_v_off = lq;
  if (use_decode_chain(d)) {
    p.part2 = c.take<float>(dgemv_part_bytes(H, 2 * I, PRO_ACT));
    p.x2 = c.take<float>((size_t)(2 * I > H ? 2 * I : H) * 4);
    p.scal1 = c.take<float>((size_t)2 * dgemv_nscal(I, H) * 4);
    p.scal2 = c.take<float>((size_t)2 * dgemv_nscal(H, 2 * I, PRO_ACT) * 4);
    p.scal3 = c.take<float>((size_t)2 * dgemv_nscal(qd, H, PRO_RESID) * 4);
    p.dA = c.take<float>(dec_attn_ws_bytes(L, d->n_heads, d->head_dim));
    // part1 and part3 share the scratch region (part1 is dead once the
    // second stream has reduced it), and so do the adapters afterwards
    for (size_t v : {dgemv_part_bytes(I, H), dgemv_part_bytes(qd, H, PRO_RESID)})
      if (v > sc) sc = v;
  } else {
    if (d->dtype == BF16 && S > 1) p.h16 = c.take<uint16_t>((size_t)S * H * 2);
    const bool ig = d->input_grad != 0;
    if (ig) {
      p.dk = c.take<float>((size_t)L * kvd * 4);
      p.dkp = c.take<float>((size_t)S * kvd * 4);
      p.xa = c.take<float>((size_t)4 * S * H * 4);
    }
    const size_t f = ffn_plan(nullptr, S, H, I, d->dtype).bytes;
    const size_t o = S == 1 ? dgemv_part_bytes(qd, H) : gemm_partial_bytes(S, qd, H, F32, d->dtype);
    const size_t a = up(attn_ws_bytes(S, L, d->n_heads, d->n_kv_heads, d->head_dim, d->dtype, ig));
    // the transposed Q, K and V products of the input gradient
    const size_t g1 = ig ? gemm_partial_bytes(S, H, qd, F32, d->dtype) : 0;
    const size_t g2 = ig ? gemm_partial_bytes(S, H, kvd, F32, d->dtype) : 0;
    for (size_t v : {f, o, a, g1, g2})
      if (v > sc) sc = v;
  }
  p.scratch = c.take<void>(sc);
  p.bytes = c.used;
  return p;
}

// The single-token layer: three weight streams, each followed by a light
// reduction that also applies the elementwise step after it (decode.hip).
hipError_t decode_chain(const lorabwd_layer_desc* d, const lorabwd_layer_weights* w,
                        const lorabwd_layer_saved* a, const LayerPlan& p, const float* d_in,
                        float* d_hidden, float* dqp, float* dv, hipStream_t s) {
  // d_in: the layer output's gradient; d_hidden receives dH1 (d_in == d_hidden
  // in place: then dH1 waits in x2 until W_o's prologue has read d_in)
  const bool inplace = d_in == d_hidden;
  const int64_t L = d->kv_len, H = d->hidden, I = d->ffn;
  const int64_t qd = d->n_heads * d->head_dim;
  const int dt = d->dtype;
  const bool sub = d->sub_norms != 0;
  // packed ternary weights (weight_format 1): each matrix's scale rides
  // with its GEMV
  const int wdt = d->weight_format ? TERN2 : dt;
  float* part13 = (float*)p.scratch;
  hipError_t e;
  // part1 = d_out W_down, with the FFN sub-norm's row-sum shares
  GemvArgs g{};
  g.N = I;
  g.K = H;
  g.W1 = w->w_down;
  g.x = d_in;
  g.part = part13;
  if (sub) {
    g.ng = w->gamma_fsub;
    g.nx = a->hidden_pre;
    g.scal = p.scal1;
  }
  g.s1 = g.s2 = w->scale_down;
  if ((e = launch_dgemv(wdt, dt, g, s)) != hipSuccess) return e;
  // part2 = [dGate | dUp] [W_gate; W_up], with the FFN norm's row-sum
  // shares; the prologue forms each workgroup's slice of [dGate | dUp] from
  // part1 (dHid, sub-norm backward, activation backward)
  g = GemvArgs{};
  g.N = H;
  g.K = 2 * I;
  g.K1 = I;
  g.W1 = w->w_gate;
  g.W2 = w->w_up;
  g.part = p.part2;
  g.ng = w->gamma_ffn;
  g.nx = a->resid1;
  g.scal = p.scal2;
  g.pro = PRO_ACT;
  g.p.part = part13;
  g.p.splits = (int)dgemv_splits(I, H);
  g.p.pn = I;
  if (sub) {
    g.p.scal = p.scal1;
    g.p.nscal = dgemv_nscal(I, H);
    g.p.nx = a->hidden_pre;
    g.p.ngam = w->gamma_fsub;
    g.p.eps = d->eps;
  }
  g.p.gate = a->gate;
  g.p.up = a->up;
  g.p.act = d->act;
  g.s1 = w->scale_gate;
  g.s2 = w->scale_up;
  if ((e = launch_dgemv(wdt, dt, g, s)) != hipSuccess) return e;
  // part3 = dH1 W_o, with the attention sub-norm's row-sum shares; the
  // prologue forms dH1 = d_out + rmsnorm_bwd(resid1, gamma_ffn, dN2) for its
  // rows from part2 (column block 0 also keeps it in x2)
  g = GemvArgs{};
  g.N = qd;
  g.K = H;
  g.W1 = w->w_o;
  g.part = part13;
  if (sub) {
    g.ng = w->gamma_asub;
    g.nx = a->ctx;
    g.scal = p.scal3;
  }
  g.pro = PRO_RESID;
  g.p.part = p.part2;
  g.p.splits = (int)dgemv_splits(H, 2 * I, PRO_ACT);
  g.p.pn = H;
  g.p.scal = p.scal2;
  g.p.nscal = dgemv_nscal(H, 2 * I, PRO_ACT);
  g.p.nx = a->resid1;
  g.p.ngam = w->gamma_ffn;
  g.p.eps = d->eps;
  g.p.resid = d_in;
  g.p.xout = inplace ? p.x2 : d_hidden;
  g.s1 = g.s2 = w->scale_o;
  if ((e = launch_dgemv(wdt, dt, g, s)) != hipSuccess) return e;
  // attention backward, inverse RoPE at the token's position
  DecAttnArgs at{};
  at.s_kv = L;
  at.Hq = (int)d->n_heads;
  at.grp = (int)(d->n_heads / d->n_kv_heads);
  at.dctx = p.dctx;
  at.P = a->P;
  at.K = a->K;
  at.V = a->V;
  at.ctx = a->ctx;
  at.dA = p.dA;
  at.dq_part = p.dA;
  at.dv = dv;
  at.dq = dqp;
  at.scale = d->attn_scale;
  at.rope = 1;
  at.pos = d->pos0;
  at.log2_base = log2((double)d->rope_base);
  const int wo_splits = (int)dgemv_splits(qd, H, PRO_RESID);
  if (a->ctx != nullptr && dec_attn_red_fits(d->n_heads, d->n_kv_heads, d->head_dim, wo_splits)) {
    // the attention launch adds the W_o partials (and applies the sub-norm
    // backward) itself; in place it also moves dH1 into d_hidden
    at.part = part13;
    at.splits = wo_splits;
    if (sub) {
      at.nsc = p.scal3;
      at.nscal = dgemv_nscal(qd, H, PRO_RESID);
      at.ngam = w->gamma_asub;
      at.eps = d->eps;
    }
    if (inplace) {
      at.copy_src = p.x2;
      at.copy_dst = d_hidden;
      at.copy_n = H;
    }
    return launch_dec_attn(dt, (int)d->head_dim, at, s);
  }
  // dCtx (sub-norm backward applied); in place, the same launch moves dH1
  // into the caller's d_hidden, whose old contents W_o's prologue has consumed
  RedArgs r{};
  r.N = qd;
  r.splits = (int)dgemv_splits(qd, H, PRO_RESID);
  r.part = part13;
  r.y = p.dctx;
  if (sub) {
    r.scal = p.scal3;
    r.nscal = dgemv_nscal(qd, H, PRO_RESID);
    r.nx = a->ctx;
    r.ngam = w->gamma_asub;
    r.eps = d->eps;
  }
  if (inplace) {
    r.copy_src = p.x2;
    r.copy_dst = d_hidden;
    r.copy_n = H;
  }
  if ((e = launch_dgemv_red(RED_STORE, dt, r, s)) != hipSuccess) return e;
  return launch_dec_attn(dt, (int)d->head_dim, at, s);
}

// Everything one layer enqueues (arguments already validated).
hipError_t layer_run(const lorabwd_layer_desc* d, const lorabwd_layer_weights* w,
                     const lorabwd_layer_saved* a, const lorabwd_lora_state* qs,
                     const lorabwd_lora_state* vs, const lorabwd_adamw* hp, const LayerPlan& plan,
                     const float* din, float* d_hidden, float* dqp, float* dv, float* gnorm_sq,
                     hipStream_t stream) {
  const int64_t S = d->seq, L = d->kv_len, H = d->hidden, I = d->ffn;
  const int64_t Hq = d->n_heads, Hkv = d->n_kv_heads, D = d->head_dim;
  const int64_t qd = Hq * D, kvd = Hkv * D;
  const int dt = d->dtype;
  const bool sub = d->sub_norms != 0;
  const bool lq = has_lora(qs), lv = has_lora(vs);
  const float lr_a = hp ? hp->lr_a : 0.f, lr_b = hp ? hp->lr_b : 0.f;
  const int step = hp ? hp->step : 1;
  hipError_t e;
  // QK-norm: the per-head RMSNorm backward after the inverse RoPE
  const RopeNormArgs qkn = d->qk_norm ? RopeNormArgs{a->q_raw, dt == BF16 ? 1 : 0, w->gamma_q, d->eps}
                                      : RopeNormArgs{nullptr, 0, nullptr, 0.f};
  if (use_decode_chain(d)) {
    LBP_E(decode_chain(d, w, a, plan, din, d_hidden, dqp, dv, stream));
    // the single-token attention applies the inverse RoPE as it stores dq;
    // the norm backward runs on each head's row (rows = heads, n = head_dim)
    if (d->qk_norm)
      LBP_E(launch_rmsnorm_bwd(S * Hq, D, a->q_raw, dt, w->gamma_q, dqp, dqp, d->eps, 0, stream));
  } else {
    // FFN half, residual-stream gradient: d_hidden <- dH1
    LBP_E(ffn_run(S, H, I, d->act, din, w->w_down, w->w_gate, w->w_up, a->gate, a->up,
                    sub ? a->hidden_pre : nullptr, sub ? w->gamma_fsub : nullptr, a->resid1,
                    w->gamma_ffn, d_hidden, d->eps, dt, plan.scratch, stream,
                    din == d_hidden ? nullptr : din, plan.h16));
    // O-projection backward: dCtx = dH1 W_o
    bool dct_ready = false;
    if (S == 1) {
      GemvArgs g{};
      g.N = qd;
      g.K = H;
      g.W1 = w->w_o;
      g.x = d_hidden;
      g.part = (float*)plan.scratch;
      LBP_E(launch_dgemv(dt, dt, g, stream));
      RedArgs r{};
      r.N = qd;
      r.splits = (int)dgemv_splits(qd, H);
      r.part = (float*)plan.scratch;
      r.y = plan.dctx;
      LBP_E(launch_dgemv_red(RED_STORE, dt, r, stream));
    } else {
      // bf16 weights take the bf16 copy the FFN norm wrote (no rounding
      // pass); without the sub-norm (which changes dCtx afterwards) the
      // product also writes dCtxᵀ for the attention's dV (whole row blocks
      // of 64 queries, so the attention finds no padding to clear)
      int64_t LQ = 0;
      uint16_t* dct = !sub && S % 64 == 0
                          ? attn_dct_buffer(plan.scratch, S, L, Hq, Hkv, D, dt, &LQ)
                          : nullptr;
      const TCopy tc{dct, LQ};
      LBP_E(launch_gemm(S, qd, H, plan.h16 ? (const void*)plan.h16 : (const void*)d_hidden,
                          plan.h16 ? BF16 : F32, H, w->w_o, nullptr, H, dt, qd, plan.dctx, qd,
                          (float*)plan.scratch, stream, nullptr, nullptr, nullptr,
                          dct ? &tc : nullptr, &dct_ready));
    }
    if (sub)
      LBP_E(launch_rmsnorm_bwd(S, qd, a->ctx, dt, w->gamma_asub, plan.dctx, plan.dctx, d->eps, 0,
                                 stream));
    // the inverse RoPE (which also adds a split dq's second key half) runs in
    // the attention's last launch where it can, else on its own
    const float* dq2 = nullptr;
    const RopeArgs rope{dqp, d->pos0, d->rope_base, qkn};
    bool rope_done = false;
    const bool ig = d->input_grad != 0;
    LBP_E(launch_attn_bwd(S, L, Hq, Hkv, D, plan.dctx, a->P, a->K, a->V, a->ctx, dt, plan.dq, dv,
                            d->attn_scale, d->causal, plan.scratch, stream, &dq2, &rope, &rope_done,
                            dct_ready, ig ? a->q : nullptr, ig ? plan.dk : nullptr));
    if (!rope_done)
      LBP_E(launch_rope_bwd(S, Hq, D, plan.dq, dqp, d->pos0, d->rope_base, stream, dq2, &qkn));
    if (ig) {
      // dKpre of the chunk's own key rows (positions pos0 ...): inverse RoPE,
      // and with QK-norm the per-head norm backward from the saved k_raw
      const RopeNormArgs kn = d->qk_norm
                                  ? RopeNormArgs{a->k_raw, dt == BF16 ? 1 : 0, w->gamma_k, d->eps}
                                  : RopeNormArgs{nullptr, 0, nullptr, 0.f};
      LBP_E(launch_rope_bwd(S, Hkv, D, plan.dk + (L - S) * kvd, plan.dkp, d->pos0, d->rope_base,
                            stream, nullptr, &kn));
      // the transposed Q, K and V products, one part of dXa each
      const int64_t SH = S * H;
      LBP_E(launch_gemm(S, H, qd, dqp, F32, qd, w->w_q, nullptr, qd, dt, H, plan.xa, H,
                        (float*)plan.scratch, stream));
      LBP_E(launch_gemm(S, H, kvd, plan.dkp, F32, kvd, w->w_k, nullptr, kvd, dt, H, plan.xa + SH,
                        H, (float*)plan.scratch, stream));
      LBP_E(launch_gemm(S, H, kvd, dv + (L - S) * kvd, F32, kvd, w->w_v, nullptr, kvd, dt, H,
                        plan.xa + 2 * SH, H, (float*)plan.scratch, stream));
    }
  }
  if (lq || lv) {
    // both adapters' gradient + AdamW passes in the same launches; the
    // value adapter sees the value rows of the current tokens: the last S of
    // the kv_len rows (all of them when kv_len == seq)
    const AdamHP h = make_hp(lr_a, lr_b, hp->beta1, hp->beta2, hp->eps, hp->weight_decay, step);
    LoraJob jobs[2];
    int nj = 0;
    if (lq)
      jobs[nj++] = LoraJob{S, H, qd, qs->rank, dqp, a->attn_input, a->lora_q_h, dt, qs->A, qs->B,
                           qs->m_a, qs->v_a, qs->m_b, qs->v_b, nullptr, nullptr,
                           d->lora_alpha / (float)qs->rank, plan.scratch};
    if (lv)
      jobs[nj++] = LoraJob{S, H, kvd, vs->rank, dv + (L - S) * kvd, a->attn_input, a->lora_v_h, dt,
                           vs->A, vs->B, vs->m_a, vs->v_a, vs->m_b, vs->v_b, nullptr, nullptr,
                           d->lora_alpha / (float)vs->rank,
                           (char*)plan.scratch + plan.lora_v_off};
    // with input_grad the adapters' share of dXa goes to its fourth part
    LBP_E(launch_lora_adamw_jobs(jobs, nj, gnorm_sq, h, stream,
                                 d->input_grad ? plan.xa + 3 * S * H : nullptr));
  }
  if (d->input_grad) {
    // d_hidden = dH1 + rmsnorm_bwd(x, gamma_attn, sum of the dXa parts)
    LBP_E(launch_rmsnorm_bwd(S, H, a->x, dt, w->gamma_attn, plan.xa, d_hidden, d->eps, 1, stream,
                             lq || lv ? 4 : 3, S * H));
  }
  return hipSuccess;
}


// Scratch of lorabwd_layer_backward_noalloc: a file-scope device array, so
// every GPU the library runs on holds its own copy until the process ends.
// Host code never uses the array's name as an address (on the host it is
// only a stand-in); it takes each device's address once from
// hipGetSymbolAddress and passes that pointer to the kernels.
constexpr size_t kNoAllocBytes = LORABWD_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kNoAllocBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The current device's scratch address (looked up once per device), or NULL
// if the runtime cannot give it.
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

int desc_validate(const lorabwd_layer_desc* d) {
  LBP_CHECK(d != nullptr, LORABWD_ERR_NULL);
  LBP_CHECK(dtype_ok(d->dtype), LORABWD_ERR_DTYPE);
  LBP_CHECK(d->act == LORABWD_ACT_SWIGLU || d->act == LORABWD_ACT_RELU2, LORABWD_ERR_DTYPE);
  LBP_CHECK(rows_ok(d->seq) && rows_ok(d->kv_len) && d->kv_len >= d->seq && d->kv_len >= 1 &&
                feat_ok(d->hidden) && feat_ok(d->ffn) &&
                heads_ok(d->n_heads, d->n_kv_heads, d->head_dim) && d->pos0 >= 0 &&
                d->pos0 <= (int64_t(1) << 40),
            LORABWD_ERR_SHAPE);
  LBP_CHECK((d->sub_norms == 0 || d->sub_norms == 1) && (d->causal == 0 || d->causal == 1) &&
                (d->qk_norm == 0 || d->qk_norm == 1) && (d->input_grad == 0 || d->input_grad == 1) &&
                (d->weight_format == 0 || d->weight_format == 1) && d->reserved == 0,
            LORABWD_ERR_ARG);
  // packed ternary weights run in the single-token chain only
  LBP_CHECK(!d->weight_format || use_decode_chain(d), LORABWD_ERR_SHAPE);
  // the attention input gradient's dK is not built for bf16 with head_dim 16
  LBP_CHECK(!d->input_grad || d->dtype != LORABWD_BF16 || d->head_dim >= 32, LORABWD_ERR_SHAPE);
  LBP_CHECK(finite(d->eps) && d->eps >= 0.f && finite(d->rope_base) && d->rope_base > 0.f &&
                finite(d->attn_scale) && finite(d->lora_alpha),
            LORABWD_ERR_ARG);
  return LORABWD_OK;
}

}  // namespace

size_t lorabwd_layer_workspace_size(const lorabwd_layer_desc* d) {
  if (desc_validate(d) != LORABWD_OK) return 0;
  if (d->seq == 0) return 0;
  // sized for the largest adapter rank the library accepts, so the size does
  // not depend on the adapter states
  return layer_plan(nullptr, d, 64, 64).bytes;
}

// lorabwd_layer_backward and, with noalloc, its allocation-free variant
// (the workspace is then this device's static scratch).
static int layer_entry(const lorabwd_layer_desc* d, const lorabwd_layer_weights* w,
                       const lorabwd_layer_saved* a, lorabwd_lora_state* qs,
                       lorabwd_lora_state* vs, const lorabwd_adamw* hp, const float* d_out,
                       float* d_hidden, float* dq_pre_out, float* dv_out, float* gnorm_sq,
                       void* workspace, size_t workspace_bytes, hipStream_t stream,
                       bool noalloc) {
  int st = desc_validate(d);
  if (st != LORABWD_OK) return st;
  LBP_CHECK(w && a, LORABWD_ERR_NULL);
  const int64_t S = d->seq, L = d->kv_len, H = d->hidden, I = d->ffn;
  const int64_t Hq = d->n_heads, Hkv = d->n_kv_heads, D = d->head_dim;
  const int64_t qd = Hq * D, kvd = Hkv * D;
  const int dt = d->dtype;
  const bool sub = d->sub_norms != 0;
  const bool lq = has_lora(qs), lv = has_lora(vs);
  LBP_CHECK(!(qs && qs->rank < 0) && !(vs && vs->rank < 0), LORABWD_ERR_SHAPE);
  if (lq || lv) {
    LBP_CHECK(hp != nullptr, LORABWD_ERR_NULL);
    LBP_CHECK(hp->step >= 1, LORABWD_ERR_STEP);
    LBP_CHECK(a->attn_input != nullptr, LORABWD_ERR_NULL);
  }
  if (lq) LBP_CHECK(a->lora_q_h != nullptr, LORABWD_ERR_NULL);
  if (lv) LBP_CHECK(a->lora_v_h != nullptr, LORABWD_ERR_NULL);
  if (sub) LBP_CHECK(w->gamma_fsub && w->gamma_asub && a->hidden_pre && a->ctx, LORABWD_ERR_NULL);
  if (d->qk_norm) LBP_CHECK(w->gamma_q && a->q_raw, LORABWD_ERR_NULL);
  if (d->input_grad) {
    LBP_CHECK(w->w_q && w->w_k && w->w_v && w->gamma_attn && a->x && a->q, LORABWD_ERR_NULL);
    if (d->qk_norm) LBP_CHECK(w->gamma_k && a->k_raw, LORABWD_ERR_NULL);
    const void* ps[] = {w->w_q, w->w_k, w->w_v, w->gamma_attn, w->gamma_k, a->x, a->q, a->k_raw};
    for (const void* q : ps) LBP_CHECK(aligned16(q), LORABWD_ERR_ALIGN);
  }
  if (S == 0) return LORABWD_OK;
  LBP_CHECK(d_hidden && w->w_o, LORABWD_ERR_NULL);
  const float* din = d_out ? d_out : d_hidden;
  LBP_CHECK(aligned16(din), LORABWD_ERR_ALIGN);
  LBP_CHECK(din == d_hidden || !overlap(din, (size_t)S * H * 4, d_hidden, (size_t)S * H * 4),
            LORABWD_ERR_ALIAS);
  st = ffn_validate(S, H, I, d->act, din, w->w_down, w->w_gate, w->w_up, a->gate, a->up,
                    sub ? a->hidden_pre : nullptr, sub ? w->gamma_fsub : nullptr, a->resid1,
                    w->gamma_ffn, d_hidden, d->eps, dt, d->weight_format == 1);
  if (st != LORABWD_OK) return st;
  if (d->weight_format)
    LBP_CHECK(finite(w->scale_o) && finite(w->scale_gate) && finite(w->scale_up) &&
                  finite(w->scale_down),
              LORABWD_ERR_ARG);
  if (st != LORABWD_OK) return st;
  LBP_CHECK(aligned16(w->w_o) && aligned16(w->gamma_asub) && aligned16(w->gamma_q) &&
                aligned16(a->q_raw) && aligned16(dq_pre_out) &&
                aligned16(dv_out) && aligned16(a->attn_input) && aligned16(a->lora_q_h) &&
                aligned16(a->lora_v_h),
            LORABWD_ERR_ALIGN);
  if (noalloc) {
    // the layer's workspace must fit the static scratch (nothing reads a
    // region of it before writing it: none has to start at zero)
    LBP_CHECK(lorabwd_layer_workspace_size(d) <= kNoAllocBytes, LORABWD_ERR_WORKSPACE);
    workspace = device_scratch();
    LBP_CHECK(workspace != nullptr, LORABWD_ERR_HIP);
    workspace_bytes = kNoAllocBytes;
  }
  const LayerPlan plan = layer_plan(workspace, d, lq ? qs->rank : 0, lv ? vs->rank : 0);
  LBP_CHECK(workspace && workspace_bytes >= lorabwd_layer_workspace_size(d),
            LORABWD_ERR_WORKSPACE);
  LBP_CHECK(aligned16(workspace), LORABWD_ERR_ALIGN);
  float* dv = dv_out ? dv_out : plan.dv;
  float* dqp = dq_pre_out ? dq_pre_out : plan.dq;
  st = attn_validate(S, L, Hq, Hkv, D, plan.dctx, a->P, a->K, a->V, a->ctx, plan.dq, dv,
                     d->attn_scale, d->causal, dt);
  if (st != LORABWD_OK) return st;
  LBP_CHECK(!overlap(dq_pre_out, (size_t)S * qd * 4, d_hidden, (size_t)S * H * 4) &&
                !overlap(dv_out, (size_t)L * kvd * 4, d_hidden, (size_t)S * H * 4) &&
                !overlap(dq_pre_out, (size_t)S * qd * 4, dv_out, (size_t)L * kvd * 4),
            LORABWD_ERR_ALIAS);
  const float lr_a = hp ? hp->lr_a : 0.f, lr_b = hp ? hp->lr_b : 0.f;
  const int step = hp ? hp->step : 1;
  if (lq) {
    st = lora_validate(S, H, qd, qs->rank, dqp, a->attn_input, a->lora_q_h, qs->A, qs->B,
                       qs->m_a, qs->v_a, qs->m_b, qs->v_b, nullptr, nullptr, gnorm_sq,
                       d->lora_alpha, lr_a, lr_b, hp->beta1, hp->beta2, hp->eps,
                       hp->weight_decay, step, dt);
    if (st != LORABWD_OK) return st;
  }
  if (lv) {
    st = lora_validate(S, H, kvd, vs->rank, dv + (L - S) * kvd, a->attn_input, a->lora_v_h,
                       vs->A, vs->B, vs->m_a, vs->v_a, vs->m_b, vs->v_b, nullptr, nullptr,
                       gnorm_sq, d->lora_alpha, lr_a, lr_b, hp->beta1, hp->beta2, hp->eps,
                       hp->weight_decay, step, dt);
    if (st != LORABWD_OK) return st;
  }

  // ---- all arguments valid: a checking pass of the whole composition,
  // then the real one
  st = check_pass([&] {
    return layer_run(d, w, a, qs, vs, hp, plan, din, d_hidden, dqp, dv, gnorm_sq, stream);
  });
  if (st != LORABWD_OK) return st;
  LBP_HIP(layer_run(d, w, a, qs, vs, hp, plan, din, d_hidden, dqp, dv, gnorm_sq, stream));
  return LORABWD_OK;
}

int lorabwd_layer_backward(const lorabwd_layer_desc* d, const lorabwd_layer_weights* w,
                           const lorabwd_layer_saved* a, lorabwd_lora_state* qs,
                           lorabwd_lora_state* vs, const lorabwd_adamw* hp, const float* d_out,
                           float* d_hidden, float* dq_pre_out, float* dv_out, float* gnorm_sq,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return layer_entry(d, w, a, qs, vs, hp, d_out, d_hidden, dq_pre_out, dv_out, gnorm_sq,
                     workspace, workspace_bytes, stream, false);
}

int lorabwd_layer_backward_noalloc(const lorabwd_layer_desc* d, const lorabwd_layer_weights* w,
                                   const lorabwd_layer_saved* a, lorabwd_lora_state* q_state,
                                   lorabwd_lora_state* v_state, const lorabwd_adamw* hp,
                                   const float* d_out, float* d_hidden, float* dq_pre_out,
                                   float* dv_out, float* gnorm_sq, hipStream_t stream) {
  return layer_entry(d, w, a, q_state, v_state, hp, d_out, d_hidden, dq_pre_out, dv_out, gnorm_sq,
                     nullptr, 0, stream, true);
}

int lorabwd_layer_backward_timed(const lorabwd_layer_desc* d, const lorabwd_layer_weights* w,
                                 const lorabwd_layer_saved* a, lorabwd_lora_state* q_state,
                                 lorabwd_lora_state* v_state, const lorabwd_adamw* hp,
                                 const float* d_out, float* d_hidden, float* dq_pre_out,
                                 float* dv_out, float* gnorm_sq, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream, hipEvent_t* events,
                                 lorabwd_kernel_record* records, int capacity, int* n_kernels) {
  LBP_CHECK(capacity >= 0, LORABWD_ERR_ARG);
  LBP_CHECK(capacity == 0 || (events != nullptr && records != nullptr), LORABWD_ERR_NULL);
  Recorder rec{events, records, capacity, 0};
  tl_recorder = &rec;
  const int st = lorabwd_layer_backward(d, w, a, q_state, v_state, hp, d_out, d_hidden,
                                        dq_pre_out, dv_out, gnorm_sq, workspace, workspace_bytes,
                                        stream);
  tl_recorder = nullptr;
  if (n_kernels) *n_kernels = rec.count;
  return st;
}

int lorabwd_lm_head_backward_timed(int64_t rows, int64_t hidden, int64_t vocab, const float* h,
                                   const float* logits, const int32_t* labels, float* w,
                                   float* m, float* v, float* grad_hidden, float* loss,
                                   float* grad_w, float lr, float beta1, float beta2, float eps,
                                   float weight_decay, int step, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream, hipEvent_t* events,
                                   lorabwd_kernel_record* records, int capacity, int* n_kernels) {
  LBP_CHECK(capacity >= 0, LORABWD_ERR_ARG);
  LBP_CHECK(capacity == 0 || (events != nullptr && records != nullptr), LORABWD_ERR_NULL);
  Recorder rec{events, records, capacity, 0};
  tl_recorder = &rec;
  const int st = lorabwd_lm_head_backward(rows, hidden, vocab, h, logits, labels, w, m, v,
                                          grad_hidden, loss, grad_w, lr, beta1, beta2, eps,
                                          weight_decay, step, workspace, workspace_bytes, stream);
  tl_recorder = nullptr;
  if (n_kernels) *n_kernels = rec.count;
  return st;
}

}  // extern "C"
