// Single-token (decode) backward.  Every transposed product is a GEMV over
// a weight matrix streamed from HBM once, so the layer is organised around
// the three weight streams (W_down, [W_gate; W_up], W_o) and everything
// elementwise rides along with them:
//
//   dgemv<PRO_COPY>   part1 = d_out W_down over row chunks; every workgroup
//                     also emits its share of <dHid*gamma_fsub, hidden_pre>
//                     (the FFN sub-norm's row sum is linear in dHid) and, for
//                     the first chunk, of sum hidden_pre^2
//   dgemv<PRO_ACT>    prologue: dHid for its rows from part1, sub-norm
//                     backward, ReLU^2 / SwiGLU backward; part2 =
//                     [dGate|dUp][W_gate;W_up] plus the FFN-norm shares over
//                     resid1
//   dgemv<PRO_RESID>  prologue: dN2 for its rows from part2, dH1 = d_out +
//                     rmsnorm_bwd(resid1, gamma_ffn, dN2); part3 = dH1 W_o
//                     plus the attention sub-norm shares over ctx
//   dec_attn_red      dCtx of the KV group = sum of part3, attention sub-norm
//                     backward applied (into LDS), then the dec_attn_mfma
//                     work below; dH1 copied to the caller's d_hidden when
//                     in place (dgemv_red + dec_attn_mfma where it does not
//                     fit: grp D > 1024, or no ctx)
//   dec_attn_mfma     per 16 keys of a KV head (one wave): dA = dCtx V^T,
//                     dS = P (dA - delta) with delta = dCtx . ctx (the row
//                     sum of P dA, as the output is P V), dV = P^T dCtx on
//                     the fp32 MFMA, and this block's share of dq = scale dS K
//   dec_attn_dqc      per head: the dq shares summed in order, then the
//                     inverse RoPE rotation at the token's position
//
// Hesper "FFN Backward GPU Kernels" (the five steps of "Backward
// (reverse)", "ReLU²×Mul Backward") and "Attention Backward GPU Kernels"
// ("Gradient Flow", "RMSNorm Backward", "Attention Apply Backward",
// "Softmax Backward", "Attention Score Backward", "RoPE Backward").
//
// GEMV layout: a workgroup owns 256 adjacent output columns (one float4 per
// lane) and a chunk of rows; its four waves split the rows and keep two
// stages of 8 rows of 16-byte loads in flight each, and add their results in
// a fixed order.  Loads are buffer loads whose bounds are offsets (out of
// range reads 0), so no branch interrupts the prefetch pipeline.  Every
// reduction has a fixed order, so results are bitwise reproducible.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace lbp {

constexpr int DG_COLS = 256;
constexpr int DG_U = 8;
constexpr int DR_COLS = 64;      // columns per reduce workgroup (16 lanes x float4)
constexpr int DG_STAGE = 8192;   // floats of LDS staging for the prologue reduction

static inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

__device__ __forceinline__ void fma4(float4& a, float x, const float4& w) {
  a.x += x * w.x;
  a.y += x * w.y;
  a.z += x * w.z;
  a.w += x * w.w;
}

// RMSNorm constants from per-workgroup shares sc[2*i] (dot), sc[2*i+1]
// (sum of squares), i < n: every thread gets inv_r = 1/sqrt(ss/len + eps)
// and c = dot / (len r^2).  Fixed order: strided per-thread sums (8 loads in
// flight), then the block tree.  All 256 threads must call it.
__device__ __forceinline__ void norm_consts_block(const float* sc, int64_t n, int64_t len,
                                                  float eps, float* red, float& inv_r,
                                                  float& c) {
  float dot = 0.f, ss = 0.f;
  for (int64_t i0 = threadIdx.x; i0 < n; i0 += 2048) {
    float2 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t i = i0 + 256 * u;
      v[u] = i < n ? *reinterpret_cast<const float2*>(sc + 2 * i) : make_float2(0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      dot += v[u].x;
      ss += v[u].y;
    }
  }
  dot = block_sum<4>(dot, red);
  ss = block_sum<4>(ss, red);
  const float nf = (float)len;
  const float r2 = ss / nf + eps;
  inv_r = 1.0f / sqrtf(r2);
  c = dot / (nf * r2);
}

// x[kb .. kb+R) for the PRO_ACT / PRO_RESID prologues (see GemvPro).  The
// producer's N is a multiple of 4 and so is R, so a thread takes 4 adjacent
// rows (one float4 per partial vector): row quad q = t % nq, and the
// S = 256 / nq threads of a quad split the producer's partials between them
// (8 loads in flight each, so one round covers 8 S partials).  issue() puts
// every load of the prologue in flight -- before the workgroup's first weight
// rows, so they do not queue behind them -- and finish() adds the partials
// (fixed order: per thread, then the S threads of a quad through LDS),
// applies the norm and elementwise step, and writes x to LDS.
template <typename TA, int PRO>
struct GemvPrologue {
  float4 v[8];
  float2 sv[8];
  typename BufVec<TA>::raw ex, e1, e2;
  float4 eg, r1;
  int nq, S, q, sub;
  int64_t rr, j;
  bool act, fin, norm;

  __device__ __forceinline__ void issue(const GemvPro& p, int64_t kb, int R) {
    const int t = threadIdx.x;
    nq = R >> 2;
    S = 256 / nq;
    q = t % nq;
    sub = t / nq;
    act = sub < S;
    fin = sub == 0;
    rr = kb + 4 * q;
    j = (PRO == PRO_ACT && rr >= p.pn) ? rr - p.pn : rr;
    norm = p.scal != nullptr;
    const brsrc_t rp = make_brsrc(p.part, (uint32_t)(p.splits * p.pn * 4));
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int sp = sub + u * S;
      const uint32_t off = (act && sp < p.splits) ? (uint32_t)((sp * p.pn + j) * 4) : BUF_OOB;
      v[u] = bload_f4(rp, off);
    }
    // absent inputs get an empty resource (every load reads 0)
    const brsrc_t rs = make_brsrc(norm ? (const void*)p.scal : p.part, norm ? (uint32_t)(p.nscal * 8) : 0u);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t i = t + 256 * u;
      sv[u] = bload_f2(rs, i < p.nscal ? (uint32_t)(i * 8) : BUF_OOB);
    }
    const uint32_t ae = sizeof(TA);
    const brsrc_t rx = make_brsrc(norm ? p.nx : (const void*)p.part, norm ? (uint32_t)(p.pn * ae) : 0u);
    const brsrc_t rg = make_brsrc(norm ? (const void*)p.ngam : (const void*)p.part, norm ? (uint32_t)(p.pn * 4) : 0u);
    ex = BufVec<TA>::load(rx, (uint32_t)(j * ae));
    eg = bload_f4(rg, (uint32_t)(j * 4));
    if (PRO == PRO_ACT) {
      e1 = BufVec<TA>::load(make_brsrc(p.gate, (uint32_t)(p.pn * ae)), (uint32_t)(j * ae));
      e2 = BufVec<TA>::load(make_brsrc(p.up, (uint32_t)(p.pn * ae)), (uint32_t)(j * ae));
    } else {
      r1 = bload_f4(make_brsrc(p.resid, (uint32_t)(p.pn * 4)), (uint32_t)(j * 4));
    }
  }

  __device__ __forceinline__ void finish(const GemvPro& p, float* xs, float* red, float4* lred) {
    const int t = threadIdx.x;
    float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      y.x += v[u].x;
      y.y += v[u].y;
      y.z += v[u].z;
      y.w += v[u].w;
    }
    for (int s0 = sub + 8 * S; s0 < p.splits; s0 += 8 * S) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int sp = s0 + u * S;
        v[u] = (act && sp < p.splits) ? *reinterpret_cast<const float4*>(p.part + (int64_t)sp * p.pn + j)
                                      : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        y.x += v[u].x;
        y.y += v[u].y;
        y.z += v[u].z;
        y.w += v[u].w;
      }
    }
    if (act) lred[t] = y;
    float inv_r = 1.f, cc = 0.f;
    if (norm) {
      float dot = 0.f, ss = 0.f;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        dot += sv[u].x;
        ss += sv[u].y;
      }
      for (int64_t i0 = t + 2048; i0 < p.nscal; i0 += 2048) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int64_t i = i0 + 256 * u;
          sv[u] = i < p.nscal ? *reinterpret_cast<const float2*>(p.scal + 2 * i) : make_float2(0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          dot += sv[u].x;
          ss += sv[u].y;
        }
      }
      dot = block_sum<4>(dot, red);  // its barriers also publish lred
      ss = block_sum<4>(ss, red);
      const float nf = (float)p.pn;
      const float r2 = ss / nf + p.eps;
      inv_r = 1.0f / sqrtf(r2);
      cc = dot / (nf * r2);
    } else {
      __syncthreads();
    }
    if (!fin) return;
    y = lred[q];
    for (int k = 1; k < S; ++k) {
      const float4 o = lred[k * nq + q];
      y.x += o.x;
      y.y += o.y;
      y.z += o.z;
      y.w += o.w;
    }
    float z[4] = {y.x, y.y, y.z, y.w};
    if (norm) {
      const float4 xv = BufVec<TA>::cvt(ex);
      const float xa[4] = {xv.x, xv.y, xv.z, xv.w}, ga[4] = {eg.x, eg.y, eg.z, eg.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) z[k] = (z[k] * ga[k] - xa[k] * cc) * inv_r;
    }
    float x[4];
    if (PRO == PRO_ACT) {
      const float4 gv = BufVec<TA>::cvt(e1), uv = BufVec<TA>::cvt(e2);
      const float ga[4] = {gv.x, gv.y, gv.z, gv.w}, ua[4] = {uv.x, uv.y, uv.z, uv.w};
      const bool is_gate = rr < p.pn;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float dg, du;
        if (p.act == SWIGLU) act_bwd1<SWIGLU>(ga[k], ua[k], z[k], dg, du);
        else act_bwd1<RELU2>(ga[k], ua[k], z[k], dg, du);
        x[k] = is_gate ? dg : du;
      }
    } else {
      x[0] = r1.x + z[0];
      x[1] = r1.y + z[1];
      x[2] = r1.z + z[2];
      x[3] = r1.w + z[3];
      if (blockIdx.x == 0) *reinterpret_cast<float4*>(p.xout + j) = make_float4(x[0], x[1], x[2], x[3]);
    }
    *reinterpret_cast<float4*>(xs + 4 * q) = make_float4(x[0], x[1], x[2], x[3]);
  }
};

template <typename TW, typename TA, int PRO>
__global__ __launch_bounds__(256) void dgemv_kernel(GemvArgs a) {
  extern __shared__ float xs[];  // [kc] the input vector of this chunk
  __shared__ float4 red4[3][64];
  __shared__ float nred[4];
  __shared__ float4 lred[PRO == PRO_COPY ? 1 : 256];
  typedef BufVec<TW> WB;
  typedef typename WB::raw WV;
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int64_t kb = (int64_t)blockIdx.y * a.kc;
  const int64_t ke = min(a.K, kb + a.kc);
  const int R = (int)(ke - kb);
  const int64_t n = (int64_t)blockIdx.x * DG_COLS + lane * 4;
  // rows [i0, i1) of the chunk belong to this wave (uniform across it)
  const int per = (R + 3) / 4;
  const int i0 = min(R, w * per), i1 = min(R, i0 + per);
  const bool nok = n < a.N;
  // the chunk's rows as two buffer ranges: rows of W1 (global row < K1) and
  // rows of W2; lanes past N and rows past the wave's share read 0
  const uint32_t rowb = (uint32_t)((a.N / 4) * ColBytes4<TW>::v);
  const int n1 = kb < a.K1 ? (int)(min(ke, a.K1) - kb) : 0;
  const int64_t kb2 = kb + n1 - a.K1;  // first row of the W2 part, within W2
  const brsrc_t rs1 = make_brsrc(n1 > 0 ? (const char*)a.W1 + kb * rowb : (const char*)a.W1, n1 * rowb);
  const brsrc_t rs2 = make_brsrc(n1 < R ? (const char*)a.W2 + kb2 * rowb : (const char*)a.W2,
                                 (uint32_t)(R - n1) * rowb);
  const uint32_t coff = nok ? (uint32_t)((n / 4) * ColBytes4<TW>::v) : BUF_OOB;
  // two named register stages (indices known at compile time): the next 8
  // rows are in flight while the current 8 are multiplied
  WV wa[DG_U], wb[DG_U];
  auto fetch = [&](WV (&wv)[DG_U], int i) {
#pragma unroll
    for (int u = 0; u < DG_U; ++u) {
      const int ii = i + u;
      const bool in1 = ii < n1;
      const uint32_t roff = ii < i1 ? (uint32_t)(in1 ? ii : ii - n1) * rowb : BUF_OOB;
      wv[u] = WB::load_stream(in1 ? rs1 : rs2, coff + roff);
    }
  };
  auto consume = [&](const WV (&wv)[DG_U], int i, float4& acc) {
#pragma unroll
    for (int u = 0; u < DG_U; ++u) {
      const int ii = i + u;
      float xv = xs[ii < R ? ii : R - 1];
      xv = ii < i1 ? xv : 0.f;
      fma4(acc, xv, WB::cvt(wv[u]));
    }
  };
  // the input vector's loads (or the prologue's) go out first, then two
  // stages of weight rows; the scheduling fences keep that order, since a
  // wait for a load also waits for every load issued before it
  GemvPrologue<TA, PRO> pro;
  float xr = 0.f;
  if (PRO == PRO_COPY) {
    // R <= 256 (kc <= 256): one element per thread
    xr = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
        make_brsrc(a.x + kb, (uint32_t)R * 4), t < R ? (int)(t * 4) : (int)BUF_OOB, 0, 0));
  } else {
    pro.issue(a.p, kb, R);
  }
  __builtin_amdgcn_sched_barrier(0);
  fetch(wa, i0);
  fetch(wb, i0 + DG_U);
  __builtin_amdgcn_sched_barrier(0);
  if (PRO == PRO_COPY) {
    if (t < R) xs[t] = xr;
  } else {
    pro.finish(a.p, xs, nred, lred);
  }
  __syncthreads();
  if constexpr (std::is_same<TW, tern2>::value) {
    // packed weights are {-1, 0, +1}: the rows' scales go into the input
    // vector (R <= 256 rows, one per thread)
    if (t < R) xs[t] *= kb + t < a.K1 ? a.s1 : a.s2;
    __syncthreads();
  }
  // every step refills both stages unconditionally (rows past the wave's
  // share read 0 and meet a 0 input), so no branch splits the pipeline
  float4 acc = make_float4(0, 0, 0, 0);
  for (int i = i0; i < i1; i += 2 * DG_U) {
    consume(wa, i, acc);
    fetch(wa, i + 2 * DG_U);
    consume(wb, i + DG_U, acc);
    fetch(wb, i + 3 * DG_U);
  }
  if (w > 0) red4[w - 1][lane] = acc;
  __syncthreads();
  if (w == 0) {
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      acc.x += red4[i][lane].x;
      acc.y += red4[i][lane].y;
      acc.z += red4[i][lane].z;
      acc.w += red4[i][lane].w;
    }
    if (nok) *reinterpret_cast<float4*>(a.part + (int64_t)blockIdx.y * a.N + n) = acc;
    if (a.ng != nullptr) {
      // this workgroup's share of the row sums of the norm that consumes y
      float dot = 0.f, ss = 0.f;
      if (nok) {
        const float4 x = Act<TA>::ld4((const TA*)a.nx, n);
        const float4 g = *reinterpret_cast<const float4*>(a.ng + n);
        dot = acc.x * g.x * x.x + acc.y * g.y * x.y + acc.z * g.z * x.z + acc.w * g.w * x.w;
        if (blockIdx.y == 0) ss = x.x * x.x + x.y * x.y + x.z * x.z + x.w * x.w;
      }
      dot = wave_sum(dot);
      ss = wave_sum(ss);
      if (lane == 0) {
        const int64_t wg = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
        a.scal[2 * wg] = dot;
        a.scal[2 * wg + 1] = ss;
      }
    }
  }
}

// y = sum over row chunks of part (a tile of up to 128 chunks in flight per
// 16-thread group; chunk order fixed), then the elementwise step of the
// path at that point (see RedMode), with RMSNorm constants from the
// producer's per-workgroup shares.  A workgroup owns 64 columns.
template <typename TA, int MODE>
__global__ __launch_bounds__(256) void dgemv_red_kernel(RedArgs a) {
  __shared__ float4 red[16][16];
  __shared__ float rs[2][4];
  const int t = threadIdx.x, c = t & 15, g = t >> 4;
  const int64_t n = (int64_t)blockIdx.x * DR_COLS + c * 4;
  const bool nok = n < a.N;
  const bool norm = a.scal != nullptr;
  // ---- every global load first (buffer loads, bounds as offsets): partial
  // sums, norm shares, elementwise inputs, the element this thread copies
  const uint32_t es = sizeof(TA);
  const uint32_t rowb = (uint32_t)(a.N * 4);
  const brsrc_t rp = make_brsrc(a.part, (uint32_t)a.splits * rowb);
  const uint32_t coff = nok ? (uint32_t)(n * 4) : BUF_OOB;
  float4 v[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int i = g + 16 * u;
    v[u] = bload_f4(rp, i < a.splits ? coff + (uint32_t)i * rowb : BUF_OOB);
  }
  float2 sv[8];
  const brsrc_t rsc = make_brsrc(norm ? (const void*)a.scal : (const void*)a.part,
                                 norm ? (uint32_t)(a.nscal * 8) : 0u);
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int64_t i = t + 256 * u;
    sv[u] = bload_f2(rsc, i < a.nscal ? (uint32_t)(i * 8) : BUF_OOB);
  }
  const bool ew = t < 16 && nok;
  const uint32_t eo = ew ? (uint32_t)(n * es) : BUF_OOB, eo4 = ew ? (uint32_t)(n * 4) : BUF_OOB;
  const typename BufVec<TA>::raw xin = BufVec<TA>::load(
      make_brsrc(norm ? a.nx : (const void*)a.part, norm ? (uint32_t)(a.N * es) : 0u), eo);
  const float4 gin = bload_f4(
      make_brsrc(norm ? (const void*)a.ngam : (const void*)a.part, norm ? rowb : 0u), eo4);
  typename BufVec<TA>::raw gt = BufVec<TA>::zero(), upv = gt;
  if (MODE == RED_ACT) {
    gt = BufVec<TA>::load(make_brsrc(a.gate, (uint32_t)(a.N * es)), eo);
    upv = BufVec<TA>::load(make_brsrc(a.up, (uint32_t)(a.N * es)), eo);
  }
  float4 prev = make_float4(0, 0, 0, 0);
  if (MODE == RED_ACCUM) prev = bload_f4(make_brsrc(a.yin ? a.yin : a.y, rowb), eo4);
  const int64_t ci = (int64_t)blockIdx.x * 256 + t;
  float cv = 0.f;
  if (a.copy_n > 0)
    cv = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
        make_brsrc(a.copy_src, (uint32_t)(a.copy_n * 4)), ci < a.copy_n ? (int)(ci * 4) : (int)BUF_OOB,
        0, 0));
  // ---- partial sums over row chunks (first tile in flight above)
  float4 s = make_float4(0, 0, 0, 0);
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    s.x += v[u].x;
    s.y += v[u].y;
    s.z += v[u].z;
    s.w += v[u].w;
  }
  for (int i0 = g + 128; i0 < a.splits; i0 += 128) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + 16 * u;
      v[u] = bload_f4(rp, i < a.splits ? coff + (uint32_t)i * rowb : BUF_OOB);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      s.x += v[u].x;
      s.y += v[u].y;
      s.z += v[u].z;
      s.w += v[u].w;
    }
  }
  red[g][c] = s;
  float inv_r = 1.f, cc = 0.f;
  if (norm) {
    float dot = 0.f, ss = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      dot += sv[u].x;
      ss += sv[u].y;
    }
    for (int64_t i0 = t + 2048; i0 < a.nscal; i0 += 2048) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t i = i0 + 256 * u;
        sv[u] = bload_f2(rsc, i < a.nscal ? (uint32_t)(i * 8) : BUF_OOB);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        dot += sv[u].x;
        ss += sv[u].y;
      }
    }
    dot = block_sum<4>(dot, rs[0]);
    ss = block_sum<4>(ss, rs[1]);
    const float nf = (float)a.N;
    const float r2 = ss / nf + a.eps;
    inv_r = 1.0f / sqrtf(r2);
    cc = dot / (nf * r2);
  } else {
    __syncthreads();
  }
  if (t < 16 && nok) {
    float4 y = red[0][t];
    for (int i = 1; i < 16; ++i) {
      y.x += red[i][t].x;
      y.y += red[i][t].y;
      y.z += red[i][t].z;
      y.w += red[i][t].w;
    }
    float o[4] = {y.x, y.y, y.z, y.w};
    if (norm) {
      const float4 xf = BufVec<TA>::cvt(xin);
      const float xv[4] = {xf.x, xf.y, xf.z, xf.w}, gv[4] = {gin.x, gin.y, gin.z, gin.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = (o[q] * gv[q] - xv[q] * cc) * inv_r;
    }
    if (MODE == RED_ACT) {
      // o = dHid: gated activation backward -> y[n] = dGate, y[N + n] = dUp
      const float4 gf = BufVec<TA>::cvt(gt), uf = BufVec<TA>::cvt(upv);
      const float gv[4] = {gf.x, gf.y, gf.z, gf.w}, uv[4] = {uf.x, uf.y, uf.z, uf.w};
      float dg[4], du[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (a.act == SWIGLU) act_bwd1<SWIGLU>(gv[q], uv[q], o[q], dg[q], du[q]);
        else act_bwd1<RELU2>(gv[q], uv[q], o[q], dg[q], du[q]);
      }
      *reinterpret_cast<float4*>(a.y + n) = make_float4(dg[0], dg[1], dg[2], dg[3]);
      *reinterpret_cast<float4*>(a.y + a.N + n) = make_float4(du[0], du[1], du[2], du[3]);
    } else {
      if (MODE == RED_ACCUM) {
        o[0] += prev.x;
        o[1] += prev.y;
        o[2] += prev.z;
        o[3] += prev.w;
      }
      *reinterpret_cast<float4*>(a.y + n) = make_float4(o[0], o[1], o[2], o[3]);
    }
  }
  if (ci < a.copy_n) a.copy_dst[ci] = cv;
  for (int64_t i = ci + (int64_t)gridDim.x * 256; i < a.copy_n; i += (int64_t)gridDim.x * 256)
    a.copy_dst[i] = a.copy_src[i];
}

// Rows per chunk (a multiple of 32, 64..256), from a target workgroup count
// measured on the decode layer's three weight streams: a plain GEMV takes
// about 512 workgroups (two per CU, every wave streaming 40 or more rows, so
// the per-workgroup start -- input vector, final cross-wave sum -- is paid
// rarely); one whose prologue reduces the producer's partials takes about 768,
// three per CU and all resident at once (the prologue's latency is exposed
// once per generation of workgroups on a CU); the residual prologue, whose
// GEMV is short, keeps small chunks (~400 workgroups for a 2560 x 2560 W_o).
int64_t dgemv_kc(int64_t N, int64_t K, int pro) {
  const int64_t cb = cdiv(N, DG_COLS);
  int64_t splits = cdiv(pro == PRO_ACT ? 768 : pro == PRO_RESID ? 1536 : 512, cb);
  if (splits < 1) splits = 1;
  int64_t kc = cdiv(cdiv(K, splits), 32) * 32;
  if (kc < 64) kc = 64;
  if (kc > 256) kc = 256;
  return kc;
}

int64_t dgemv_splits(int64_t N, int64_t K, int pro) { return cdiv(K, dgemv_kc(N, K, pro)); }

size_t dgemv_part_bytes(int64_t N, int64_t K, int pro) {
  return (size_t)dgemv_splits(N, K, pro) * N * sizeof(float);
}

int64_t dgemv_nscal(int64_t N, int64_t K, int pro) {
  return dgemv_splits(N, K, pro) * cdiv(N, DG_COLS);
}

hipError_t launch_dgemv(int w_dt, int a_dt, GemvArgs a, hipStream_t s) {
  a.kc = dgemv_kc(a.N, a.K, a.pro);
  // the prologues take rows in quads of a float4 partial (at most 64 quads
  // per chunk, kc <= 256, so every quad has at least 4 threads)
  if (a.pro != PRO_COPY && (a.p.pn % 4 != 0 || a.K % 4 != 0 || a.kc > 256 ||
                            a.K != (a.pro == PRO_ACT ? 2 * a.p.pn : a.p.pn) ||
                            (double)a.p.splits * a.p.pn * 4 >= BUF_MAX_BYTES ||
                            (double)a.p.nscal * 8 >= BUF_MAX_BYTES))
    return hipErrorInvalidValue;
  // buffer ranges: one chunk of weight rows, the input vector
  const double wes = w_dt == F32 ? 4 : w_dt == BF16 ? 2 : 0.25;
  if ((double)a.kc * a.N * wes >= BUF_MAX_BYTES || (double)a.K * 4 >= BUF_MAX_BYTES ||
      (w_dt == TERN2 && a.kc > 256))
    return hipErrorInvalidValue;
  if (dry_run()) return hipSuccess;
  if (a.W2 == nullptr) {
    a.W2 = a.W1;
    a.K1 = a.K;
  }
  dim3 grid((unsigned)cdiv(a.N, DG_COLS), (unsigned)cdiv(a.K, a.kc)), block(256);
  const size_t sm = (size_t)a.kc * sizeof(float);
#define LBP_DGEMV(TW, TA)                                                            \
  do {                                                                               \
    if (a.pro == PRO_ACT) dgemv_kernel<TW, TA, PRO_ACT><<<grid, block, sm, s>>>(a);     \
    else if (a.pro == PRO_RESID) dgemv_kernel<TW, TA, PRO_RESID><<<grid, block, sm, s>>>(a); \
    else dgemv_kernel<TW, TA, PRO_COPY><<<grid, block, sm, s>>>(a);                    \
  } while (0)
  if (w_dt == F32) {
    if (a_dt == F32) LBP_DGEMV(float, float);
    else LBP_DGEMV(float, bf16);
  } else if (w_dt == BF16) {
    if (a_dt == F32) LBP_DGEMV(bf16, float);
    else LBP_DGEMV(bf16, bf16);
  } else {
    if (a_dt == F32) LBP_DGEMV(tern2, float);
    else LBP_DGEMV(tern2, bf16);
  }
#undef LBP_DGEMV
  const double es = wes;
  // algorithmic bytes: the weights, the input vector and the result vector;
  // a prologue reads, in place of the input vector, the reduced producer
  // output and the elementwise inputs that form it (split partials are
  // implementation traffic and not counted)
  double xin = a.K * 4.0;
  if (a.pro != PRO_COPY) {
    const double ae = a_dt == F32 ? 4 : 2;
    xin = a.p.pn * 4.0;
    if (a.p.scal) xin += a.p.pn * (ae + 4);
    xin += a.pro == PRO_ACT ? a.p.pn * 2 * ae : a.p.pn * 8.0;
  }
  // implementation traffic: this launch's row-chunk partials beyond one
  // result vector, and the producer partials every column block re-reads
  const double nsp = (double)cdiv(a.K, a.kc);
  const double reread = a.pro != PRO_COPY ? (double)cdiv(a.N, DG_COLS) * a.p.splits * a.p.pn * 4.0 - a.p.pn * 4.0 : 0.0;
  mark("dgemv", (double)a.K * a.N * es + xin + a.N * 4.0, 2.0 * a.K * a.N, s,
       (nsp - 1) * a.N * 4.0 + reread);
  return hipGetLastError();
}

hipError_t launch_dgemv_red(int mode, int a_dt, RedArgs a, hipStream_t s) {
  if ((double)a.splits * a.N * 4 >= BUF_MAX_BYTES || (double)a.nscal * 8 >= BUF_MAX_BYTES ||
      (double)a.copy_n * 4 >= BUF_MAX_BYTES || (double)a.N * 4 >= BUF_MAX_BYTES)
    return hipErrorInvalidValue;
  if (dry_run()) return hipSuccess;
  dim3 grid((unsigned)cdiv(a.N, DR_COLS)), block(256);
#define LBP_RED(TA)                                                        \
  do {                                                                     \
    if (mode == RED_ACT) dgemv_red_kernel<TA, RED_ACT><<<grid, block, 0, s>>>(a);     \
    else if (mode == RED_ACCUM) dgemv_red_kernel<TA, RED_ACCUM><<<grid, block, 0, s>>>(a); \
    else dgemv_red_kernel<TA, RED_STORE><<<grid, block, 0, s>>>(a);                 \
  } while (0)
  if (a_dt == F32) LBP_RED(float);
  else LBP_RED(bf16);
#undef LBP_RED
  const double es = a_dt == F32 ? 4 : 2;
  double bytes = (double)a.N * 4;  // the result
  if (a.scal) bytes += (double)a.N * (es + 4);
  if (mode == RED_ACT) bytes += (double)a.N * (2 * es + 4);
  if (mode == RED_ACCUM) bytes += (double)a.N * 4;
  bytes += (double)a.copy_n * 8;
  mark(mode == RED_ACT ? "dgemv_red_act" : mode == RED_ACCUM ? "dgemv_red_resid" : "dgemv_red",
       bytes, 0, s);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Decode attention (one query row), two kernels with no serial chains:
//   dec_attn1  workgroup = (32 keys, KV head g): V rows staged in LDS;
//              dA[h, j] = dCtx_h . V_g[j] as 8 partial dots per (h, j)
//              summed across waves in a fixed order; dV[j] = sum_h P dCtx_h.
//   dec_attn2  workgroup = head, 16 waves: delta = sum_j P dA, dS = P (dA -
//              delta), dq = scale sum_j dS[j] K_g[j] with the waves taking
//              interleaved keys (partials added in order), then optionally
//              the inverse RoPE rotation.
constexpr int DA_KC = 32;   // keys per dec_attn1 workgroup

template <typename T, int D>
__global__ __launch_bounds__(256) void dec_attn1_kernel(DecAttnArgs a) {
  constexpr int NP = 8;            // partial dots per (head, key)
  constexpr int DP = D / NP;       // head dims per partial
  extern __shared__ float sm[];
  const int grp = a.grp;
  float* Vs = sm;                          // [DA_KC][D + 1]
  float* dC = Vs + DA_KC * (D + 1);        // [grp][D]
  float* Ps = dC + grp * D;                // [grp][DA_KC]
  float* red = Ps + grp * DA_KC;           // [NP][grp][DA_KC]
  const int t = threadIdx.x;
  const int g = blockIdx.y;
  const int64_t k0 = (int64_t)blockIdx.x * DA_KC;
  const int64_t ldk = (int64_t)(a.Hq / grp) * D;
  {
    // all global loads of the block first, then the LDS stores
    constexpr int NV = DA_KC * D / 1024;  // float4 of V per thread (>= 1 for D >= 32)
    float4 v[NV > 0 ? NV : 1];
#pragma unroll
    for (int u = 0; u < (NV > 0 ? NV : 1); ++u) {
      const int e = t * 4 + 1024 * u;
      const int kr = e / D, d = e - kr * D;
      const int64_t key = k0 + kr;
      v[u] = (e < DA_KC * D && key < a.s_kv) ? Act<T>::ld4((const T*)a.V, key * ldk + g * D + d)
                                             : make_float4(0, 0, 0, 0);
    }
    for (int e = t; e < grp * D; e += 256) dC[e] = a.dctx[(int64_t)g * grp * D + e];
    for (int e = t; e < grp * DA_KC; e += 256) {
      const int hh = e / DA_KC, kr = e - hh * DA_KC;
      const int64_t key = k0 + kr;
      Ps[e] = key < a.s_kv ? Act<T>::ld((const T*)a.P, (int64_t)(g * grp + hh) * a.s_kv + key) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < (NV > 0 ? NV : 1); ++u) {
      const int e = t * 4 + 1024 * u;
      if (e < DA_KC * D) {
        const int kr = e / D, d = e - kr * D;
        float* vr = Vs + kr * (D + 1) + d;
        vr[0] = v[u].x;
        vr[1] = v[u].y;
        vr[2] = v[u].z;
        vr[3] = v[u].w;
      }
    }
  }
  __syncthreads();
  {
    // thread (key kr = t % 32, part p = t / 32) over dims [p*DP, p*DP+DP)
    const int kr = t % DA_KC, p = t / DA_KC;
    for (int hh = 0; hh < grp; ++hh) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < DP; ++i) acc += dC[hh * D + p * DP + i] * Vs[kr * (D + 1) + p * DP + i];
      red[(p * grp + hh) * DA_KC + kr] = acc;
    }
  }
  __syncthreads();
  for (int e = t; e < grp * DA_KC; e += 256) {
    const int hh = e / DA_KC, kr = e - hh * DA_KC;
    const int64_t key = k0 + kr;
    float o = 0.f;
#pragma unroll
    for (int p = 0; p < NP; ++p) o += red[(p * grp + hh) * DA_KC + kr];
    if (key < a.s_kv) a.dA[(int64_t)(g * grp + hh) * a.s_kv + key] = o;
  }
  if (a.dv != nullptr) {
    for (int e = t; e < DA_KC * D; e += 256) {
      const int kr = e / D, d = e - kr * D;
      const int64_t key = k0 + kr;
      if (key >= a.s_kv) break;
      float o = 0.f;
      for (int hh = 0; hh < grp; ++hh) o += Ps[hh * DA_KC + kr] * dC[hh * D + d];
      a.dv[key * ldk + g * D + d] = o;
    }
  }
}

template <typename T, int VPL>
__device__ __forceinline__ void ldv(const T* p, int64_t i, float (&v)[VPL]) {
  if constexpr (VPL == 2 && sizeof(T) == 4) {
    const float2 x = *reinterpret_cast<const float2*>((const float*)p + i);
    v[0] = x.x;
    v[1] = x.y;
  } else {
#pragma unroll
    for (int j = 0; j < VPL; ++j) v[j] = Act<T>::ld(p, i + j);
  }
}

constexpr int DQ_W = 16;   // waves per dec_attn2 workgroup

template <typename T, int D>
__global__ __launch_bounds__(1024) void dec_attn2_kernel(DecAttnArgs a) {
  constexpr int VPL = D >= 64 ? D / 64 : 1;
  constexpr int NL = D / VPL;
  extern __shared__ float sm[];
  float* dS = sm;                  // [s_kv]
  float* accs = sm + a.s_kv;       // [DQ_W][D]
  float* o = accs + DQ_W * D;      // [D]
  __shared__ float rs[DQ_W];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int h = blockIdx.x, g = h / a.grp;
  const int64_t ldk = (int64_t)(a.Hq / a.grp) * D;
  const T* Ph = (const T*)a.P + (int64_t)h * a.s_kv;
  const float* dAh = a.dA + (int64_t)h * a.s_kv;
  const bool lok = lane < NL;
  const int d0 = lane * VPL;
  constexpr int UK = 16;  // keys in flight per wave
  // the first UK keys of this wave are fetched before delta is known
  float k[UK][VPL];
  auto fetch = [&](int64_t j0) {
#pragma unroll
    for (int u = 0; u < UK; ++u) {
      const int64_t j = j0 + DQ_W * u;
      if (lok && j < a.s_kv) {
        ldv<T, VPL>((const T*)a.K, j * ldk + g * D + d0, k[u]);
      } else {
#pragma unroll
        for (int q = 0; q < VPL; ++q) k[u][q] = 0.f;
      }
    }
  };
  fetch(w);
  float s = 0.f;
  for (int64_t j = t; j < a.s_kv; j += 1024) s += Act<T>::ld(Ph, j) * dAh[j];
  const float delta = block_sum<DQ_W>(s, rs);
  for (int64_t j = t; j < a.s_kv; j += 1024) dS[j] = Act<T>::ld(Ph, j) * (dAh[j] - delta);
  __syncthreads();
  float acc[VPL];
#pragma unroll
  for (int q = 0; q < VPL; ++q) acc[q] = 0.f;
  for (int64_t j0 = w; j0 < a.s_kv; j0 += UK * DQ_W) {
    if (j0 != w) fetch(j0);
#pragma unroll
    for (int u = 0; u < UK; ++u) {
      const int64_t j = j0 + DQ_W * u;
      const float ds = j < a.s_kv ? dS[j] : 0.f;
#pragma unroll
      for (int q = 0; q < VPL; ++q) acc[q] += ds * k[u][q];
    }
  }
  if (lok) {
#pragma unroll
    for (int q = 0; q < VPL; ++q) accs[w * D + d0 + q] = acc[q];
  }
  __syncthreads();
  if (t < D) {
    float v = accs[t];
    for (int i = 1; i < DQ_W; ++i) v += accs[i * D + t];
    o[t] = a.scale * v;
  }
  __syncthreads();
  constexpr int HALF = D / 2;
  if (!a.rope) {
    if (t < D) a.dq[(int64_t)h * D + t] = o[t];
  } else if (t < HALF) {
    const double inv_freq = exp2(-(2.0 * t / D) * a.log2_base);
    double sn, cs;
    sincos((double)a.pos * inv_freq, &sn, &cs);
    const float cf = (float)cs, sf = (float)sn;
    const float lo = o[t], hi = o[t + HALF];
    a.dq[(int64_t)h * D + t] = lo * cf + hi * sf;
    a.dq[(int64_t)h * D + t + HALF] = -lo * sf + hi * cf;
  }
}

// With ctx (= P V, the forward attention output) available, delta_h =
// <dCtx_h, ctx_h> is known up front, so one pass over each key block does
// everything: dA, dV, dS = P (dA - delta) and this block's share of dq.
//   dec_attn1c   workgroup = (32 keys, KV head g); K and V rows staged in LDS
//   dec_attn_dqc workgroup = head: dq = scale * sum of the block shares (in
//                order), then optionally the inverse RoPE rotation
template <typename T, int D>
__global__ __launch_bounds__(256) void dec_attn1c_kernel(DecAttnArgs a) {
  constexpr int NP = 8;            // partial dots per (head, key)
  constexpr int DP = D / NP;
  constexpr int NKG = 256 / D;     // key groups in the dq share
  constexpr int KPG = DA_KC / NKG; // keys per key group
  extern __shared__ float sm[];
  const int grp = a.grp;
  float* Vs = sm;                          // [DA_KC][D + 1]
  float* Ks = Vs + DA_KC * (D + 1);        // [DA_KC][D + 1]
  float* dC = Ks + DA_KC * (D + 1);        // [grp][D]
  float* Ps = dC + grp * D;                // [grp][DA_KC]
  float* red = Ps + grp * DA_KC;           // [NP][grp][DA_KC]
  float* dS = red + NP * grp * DA_KC;      // [grp][DA_KC]
  float* prod = dS + grp * DA_KC;          // [grp][D]
  float* dqs = prod + grp * D;             // [NKG][grp][D]
  __shared__ float delta[64];
  const int t = threadIdx.x;
  const int g = blockIdx.y;
  const int64_t k0 = (int64_t)blockIdx.x * DA_KC;
  const int64_t ldk = (int64_t)(a.Hq / grp) * D;
  {
    constexpr int NV = DA_KC * D / 1024 > 0 ? DA_KC * D / 1024 : 1;
    float4 v[NV], k[NV];
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int e = t * 4 + 1024 * u;
      const int kr = e / D, d = e - kr * D;
      const int64_t key = k0 + kr;
      const bool ok = e < DA_KC * D && key < a.s_kv;
      v[u] = ok ? Act<T>::ld4((const T*)a.V, key * ldk + g * D + d) : make_float4(0, 0, 0, 0);
      k[u] = ok ? Act<T>::ld4((const T*)a.K, key * ldk + g * D + d) : make_float4(0, 0, 0, 0);
    }
    for (int e = t; e < grp * D; e += 256) {
      const int64_t qi = (int64_t)g * grp * D + e;
      const float dc = a.dctx[qi];
      dC[e] = dc;
      prod[e] = dc * Act<T>::ld((const T*)a.ctx, qi);
    }
    for (int e = t; e < grp * DA_KC; e += 256) {
      const int hh = e / DA_KC, kr = e - hh * DA_KC;
      const int64_t key = k0 + kr;
      Ps[e] = key < a.s_kv ? Act<T>::ld((const T*)a.P, (int64_t)(g * grp + hh) * a.s_kv + key) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int e = t * 4 + 1024 * u;
      if (e < DA_KC * D) {
        const int kr = e / D, d = e - kr * D;
        float* vr = Vs + kr * (D + 1) + d;
        float* kq = Ks + kr * (D + 1) + d;
        vr[0] = v[u].x;
        vr[1] = v[u].y;
        vr[2] = v[u].z;
        vr[3] = v[u].w;
        kq[0] = k[u].x;
        kq[1] = k[u].y;
        kq[2] = k[u].z;
        kq[3] = k[u].w;
      }
    }
  }
  __syncthreads();
  // delta_h = <dCtx_h, ctx_h>: wave w reduces heads w, w+4, ... (fixed
  // lane order, then the butterfly); partial dots for dA
  {
    const int lane = t & 63, w = t >> 6;
    for (int hh = w; hh < grp; hh += 4) {
      float s = 0.f;
      for (int d = lane; d < D; d += 64) s += prod[hh * D + d];
      s = wave_sum(s);
      if (lane == 0) delta[hh] = s;
    }
  }
  {
    const int kr = t % DA_KC, p = t / DA_KC;
    for (int hh = 0; hh < grp; ++hh) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < DP; ++i) acc += dC[hh * D + p * DP + i] * Vs[kr * (D + 1) + p * DP + i];
      red[(p * grp + hh) * DA_KC + kr] = acc;
    }
  }
  __syncthreads();
  for (int e = t; e < grp * DA_KC; e += 256) {
    const int hh = e / DA_KC, kr = e - hh * DA_KC;
    float o = 0.f;
#pragma unroll
    for (int p = 0; p < NP; ++p) o += red[(p * grp + hh) * DA_KC + kr];
    dS[e] = Ps[e] * (o - delta[hh]);
  }
  if (a.dv != nullptr) {
    for (int e = t; e < DA_KC * D; e += 256) {
      const int kr = e / D, d = e - kr * D;
      const int64_t key = k0 + kr;
      if (key >= a.s_kv) break;
      float o = 0.f;
      for (int hh = 0; hh < grp; ++hh) o += Ps[hh * DA_KC + kr] * dC[hh * D + d];
      a.dv[key * ldk + g * D + d] = o;
    }
  }
  __syncthreads();
  {
    // this block's share of dq: thread (d, key group kg)
    const int d = t % D, kg = t / D;
    for (int hh = 0; hh < grp; ++hh) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < KPG; ++i) {
        const int kr = kg * KPG + i;
        acc += dS[hh * DA_KC + kr] * Ks[kr * (D + 1) + d];
      }
      dqs[(kg * grp + hh) * D + d] = acc;
    }
  }
  __syncthreads();
  for (int e = t; e < grp * D; e += 256) {
    const int hh = e / D, d = e - hh * D;
    float o = 0.f;
#pragma unroll
    for (int kg = 0; kg < NKG; ++kg) o += dqs[(kg * grp + hh) * D + d];
    a.dq_part[((int64_t)(g * grp + hh) * gridDim.x + blockIdx.x) * D + d] = o;
  }
}

// One query row with ctx given, on the fp32 MFMA (16x16x4): workgroup =
// one wave = 16 keys of one KV head (many small workgroups spread the
// cache reads over the CUs), the group's heads padded to the 16 MFMA
// columns (grp <= 16).
//   dA^T [key x head] = V dCtx^T       k = head dim (lane group c owns
//                                       dims DK c .. DK c + DK - 1)
//   dS^T = P^T o (dA^T - delta)         delta_h = <dCtx_h, ctx_h>
//   dq share [head x dim] = dS K        k = key (slot c of step v: key 4c + v)
//   dV [key x dim] = P^T dCtx           k = head (4 heads per MFMA)
// Every wave stores its dq share (chunk = workgroup) straight from the
// accumulators; dec_attn_dqc adds the chunks in order.  (Staging the
// shares through LDS was miscompiled by the ROCm 7.2 compiler: two of the
// merged ds_write2_b32 stores of the 128-wide case got wrong offsets.)
constexpr int DM_KB = 16;  // keys per workgroup (one wave)

template <typename T, int D>
__global__ __launch_bounds__(64) void dec_attn_mfma_kernel(DecAttnArgs a) {
  constexpr int DK = D / 4, ND = D / 16;
  const int lane = threadIdx.x;
  const int l16 = lane & 15, c = lane >> 4;
  const int g = blockIdx.y, grp = a.grp;
  const int64_t ldk = (int64_t)(a.Hq / grp) * D;
  const int64_t kb = (int64_t)blockIdx.x * DM_KB;
  const bool hok = l16 < grp;
  const int64_t hrow = (int64_t)(g * grp + (hok ? l16 : 0)) * D;
  const int64_t kr = kb + l16;
  const bool kok = kr < a.s_kv;
  const bool dvh = c < grp;  // first block of four heads for dV
  // ---- every independent global load first (one memory round trip)
  float4 xv[DK / 4], yv[DK / 4], vv[DK / 4];
#pragma unroll
  for (int i = 0; i < DK / 4; ++i) {
    xv[i] = yv[i] = vv[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (hok) {
      xv[i] = *reinterpret_cast<const float4*>(a.dctx + hrow + DK * c + 4 * i);
      yv[i] = Act<T>::ld4((const T*)a.ctx, hrow + DK * c + 4 * i);
    }
    if (kok) vv[i] = Act<T>::ld4((const T*)a.V, kr * ldk + g * D + DK * c + 4 * i);
  }
  float pd[4], kv[4][ND], pa = 0.f, bd[ND];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int64_t key = kb + 4 * c + v;
    const bool ok = key < a.s_kv;
    pd[v] = (hok && ok) ? Act<T>::ld((const T*)a.P, (int64_t)(g * grp + l16) * a.s_kv + key) : 0.f;
#pragma unroll
    for (int f = 0; f < ND; ++f)
      kv[v][f] = ok ? Act<T>::ld((const T*)a.K, key * ldk + g * D + 16 * f + l16) : 0.f;
  }
  if (a.dv != nullptr) {
    pa = (dvh && kok) ? Act<T>::ld((const T*)a.P, (int64_t)(g * grp + c) * a.s_kv + kr) : 0.f;
#pragma unroll
    for (int f = 0; f < ND; ++f)
      bd[f] = dvh ? a.dctx[(int64_t)(g * grp + c) * D + 16 * f + l16] : 0.f;
  }
  // ---- delta_h = <dCtx_h, ctx_h> (head l16; the four lane groups add up)
  float dl = 0.f;
#pragma unroll
  for (int i = 0; i < DK / 4; ++i)
    dl += xv[i].x * yv[i].x + xv[i].y * yv[i].y + xv[i].z * yv[i].z + xv[i].w * yv[i].w;
  dl += __shfl_xor(dl, 16, 64);
  dl += __shfl_xor(dl, 32, 64);
  // ---- dA^T: rows = keys kb + l16, four chains for the MFMA pipe
  floatx4 da[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) da[j] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < DK / 4; ++i) {
    da[0] = mfma16x16x4(vv[i].x, xv[i].x, da[0]);
    da[1] = mfma16x16x4(vv[i].y, xv[i].y, da[1]);
    da[2] = mfma16x16x4(vv[i].z, xv[i].z, da[2]);
    da[3] = mfma16x16x4(vv[i].w, xv[i].w, da[3]);
  }
  // ---- dS^T: lane (head l16, c) holds keys kb + 4c + v
  float ds[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) ds[v] = pd[v] * (((da[0][v] + da[1][v]) + (da[2][v] + da[3][v])) - dl);
  // ---- dq share: rows = heads, k = keys, columns = head dims
  floatx4 aq[ND];
#pragma unroll
  for (int f = 0; f < ND; ++f) aq[f] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int v = 0; v < 4; ++v)
#pragma unroll
    for (int f = 0; f < ND; ++f) aq[f] = mfma16x16x4(ds[v], kv[v][f], aq[f]);
  const int64_t nch = gridDim.x, chunk = blockIdx.x;
#pragma unroll
  for (int f = 0; f < ND; ++f)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int hh = 4 * c + v;
      if (hh < grp) a.dq_part[((int64_t)(g * grp + hh) * nch + chunk) * D + 16 * f + l16] = aq[f][v];
    }
  // ---- dV: rows = keys, k = heads (slot c of block j: head 4j + c), cols = dims
  if (a.dv != nullptr) {
#pragma unroll
    for (int f = 0; f < ND; ++f) {
      floatx4 av = mfma16x16x4(pa, bd[f], floatx4{0.f, 0.f, 0.f, 0.f});
      for (int j = 1; 4 * j < grp; ++j) {
        const int hh = 4 * j + c;
        const bool ok = hh < grp;
        const float p2 =
            (ok && kok) ? Act<T>::ld((const T*)a.P, (int64_t)(g * grp + hh) * a.s_kv + kr) : 0.f;
        const float b2 = ok ? a.dctx[(int64_t)(g * grp + hh) * D + 16 * f + l16] : 0.f;
        av = mfma16x16x4(p2, b2, av);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t key = kb + 4 * c + v;
        if (key < a.s_kv) a.dv[key * ldk + g * D + 16 * f + l16] = av[v];
      }
    }
  }
}

// The W_o reduction and the attention in one launch: workgroup = 16 DR_NA
// keys of one KV group.  All four waves first add the group's dCtx columns
// from the W_o partials (fixed split order per thread, then the threads of a
// column quad in order) and apply the attention sub-norm backward with the
// row sums from the W_o launch's shares; the columns go to LDS.  Then the
// first DR_NA waves do the dec_attn_mfma work of 16 keys each; their
// key/value/P loads, which do not depend on dCtx, are issued right after the
// partials' loads, so the two latencies overlap.  Replaces dgemv_red and a
// launch boundary (decode step 65.1 -> 64.2 us); every workgroup re-reads
// its group's partials, so small workgroups (many CUs) pay off.
constexpr int DR_SPL = 20;  // partials in flight per thread (splits / (256 / quads))
constexpr int DR_NA = 1;    // waves of a dec_attn_red workgroup that do attention (16 keys each; 1 measured fastest)

// One element of type T at byte offset off (0 when out of range), kept raw
// until it is converted, so that every load is issued before the first wait.
template <typename T> struct Buf1;
template <> struct Buf1<float> {
  typedef uint32_t raw;
  static __device__ __forceinline__ raw load(brsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
  }
  static __device__ __forceinline__ float cvt(raw v) { return __uint_as_float(v); }
};
template <> struct Buf1<bf16> {
  typedef uint16_t raw;
  static __device__ __forceinline__ raw load(brsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
  }
  static __device__ __forceinline__ float cvt(raw v) { return bf2f(v); }
};

bool dec_attn_red_fits(int64_t n_heads, int64_t n_kv_heads, int64_t head_dim, int splits) {
  const int64_t nq = n_heads / n_kv_heads * head_dim / 4;  // column quads of a group
  return n_heads / n_kv_heads <= 16 && nq <= 256 && 256 % nq == 0 &&
         splits <= DR_SPL * (256 / nq);
}

template <typename T, int D>
__global__ __launch_bounds__(256) void dec_attn_red_kernel(DecAttnArgs a) {
  constexpr int DK = D / 4, ND = D / 16;
  extern __shared__ float4 smem4[];
  __shared__ float nred[4];
  const int t = threadIdx.x;
  const int lane = t & 63, w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int l16 = lane & 15, c = lane >> 4;
  const int g = blockIdx.y, grp = a.grp;
  const int GC = grp * D, nq = GC / 4, S = 256 / nq;
  const int64_t qn = (int64_t)a.Hq * D;  // one query row, all heads
  const int64_t ldk = (int64_t)(a.Hq / grp) * D;
  float4* red4 = smem4;                         // [256]
  float* dC = reinterpret_cast<float*>(smem4 + 256);  // [GC]
  // ---- the group's dCtx partials first: thread (quad q, sub) takes splits
  // sub, sub + S, ... (one round of DR_SPL loads)
  const int q = t % nq, sub = t / nq;
  const brsrc_t rp = make_brsrc(a.part + (int64_t)g * GC, (uint32_t)(((a.splits - 1) * qn + GC) * 4));
  float4 pv[DR_SPL];
#pragma unroll
  for (int u = 0; u < DR_SPL; ++u) {
    const int sp = sub + S * u;
    pv[u] = bload_f4(rp, sp < a.splits ? (uint32_t)((sp * qn + 4 * q) * 4) : BUF_OOB);
  }
  const bool norm = a.nsc != nullptr;
  const brsrc_t rn = make_brsrc(norm ? (const void*)a.nsc : (const void*)a.part,
                                norm ? (uint32_t)(a.nscal * 8) : 0u);
  float2 sv[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t i = t + 256 * u;
    sv[u] = bload_f2(rn, i < a.nscal ? (uint32_t)(i * 8) : BUF_OOB);
  }
  // (buffer loads throughout: a load under a branch would make the compiler
  // wait for the partials at the join)
  constexpr uint32_t ES = sizeof(T);
  typedef typename BufVec<T>::raw R4;
  typedef typename Buf1<T>::raw R1;
  const bool nok = norm && t < nq;
  const R4 nxr = BufVec<T>::load(make_brsrc(norm ? a.ctx : (const void*)a.part, norm ? (uint32_t)(qn * ES) : 0u),
                                 nok ? (uint32_t)(((int64_t)g * GC + 4 * t) * ES) : BUF_OOB);
  const float4 ng = bload_f4(make_brsrc(norm ? (const void*)a.ngam : (const void*)a.part, norm ? (uint32_t)(qn * 4) : 0u),
                             nok ? (uint32_t)(((int64_t)g * GC + 4 * t) * 4) : BUF_OOB);
  // ---- the workgroup's 16 keys (wave 0): every load that does not need dCtx
  // (the other waves take out-of-range offsets: no memory is touched)
  const bool w0 = w < DR_NA;
  const int64_t kb = ((int64_t)blockIdx.x * DR_NA + w) * DM_KB;
  const bool hok = w0 && l16 < grp;
  const int64_t hrow = (int64_t)(g * grp + (hok ? l16 : 0)) * D;
  const int64_t kr = kb + l16;
  const bool kok = w0 && kr < a.s_kv;
  const bool dvh = w0 && c < grp;
  const brsrc_t rc = make_brsrc(a.ctx, (uint32_t)(qn * ES));
  const brsrc_t rv = make_brsrc(a.V, (uint32_t)(a.s_kv * ldk * ES));
  const brsrc_t rk = make_brsrc(a.K, (uint32_t)(a.s_kv * ldk * ES));
  const brsrc_t rpp = make_brsrc(a.P, (uint32_t)(a.Hq * a.s_kv * ES));
  R4 yr[DK / 4], vr[DK / 4];
#pragma unroll
  for (int i = 0; i < DK / 4; ++i) {
    yr[i] = BufVec<T>::load(rc, hok ? (uint32_t)((hrow + DK * c + 4 * i) * ES) : BUF_OOB);
    vr[i] = BufVec<T>::load(rv, kok ? (uint32_t)((kr * ldk + g * D + DK * c + 4 * i) * ES) : BUF_OOB);
  }
  R1 pdr[4], kvr[4][ND], par;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int64_t key = kb + 4 * c + v;
    const bool ok = w0 && key < a.s_kv;
    pdr[v] = Buf1<T>::load(rpp, (hok && ok) ? (uint32_t)(((int64_t)(g * grp + l16) * a.s_kv + key) * ES) : BUF_OOB);
#pragma unroll
    for (int f = 0; f < ND; ++f)
      kvr[v][f] = Buf1<T>::load(rk, ok ? (uint32_t)((key * ldk + g * D + 16 * f + l16) * ES) : BUF_OOB);
  }
  par = Buf1<T>::load(rpp, (a.dv != nullptr && dvh && kok)
                               ? (uint32_t)(((int64_t)(g * grp + c) * a.s_kv + kr) * ES)
                               : BUF_OOB);
  __builtin_amdgcn_sched_barrier(0);
  // ---- dCtx columns: partial sums, then the sub-norm backward
  float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int u = 0; u < DR_SPL; ++u) {
    y.x += pv[u].x;
    y.y += pv[u].y;
    y.z += pv[u].z;
    y.w += pv[u].w;
  }
  red4[t] = y;
  float inv_r = 1.f, cc = 0.f;
  if (norm) {
    float dot = 0.f, ss = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      dot += sv[u].x;
      ss += sv[u].y;
    }
    for (int64_t i0 = t + 1024; i0 < a.nscal; i0 += 256) {
      const float2 e = *reinterpret_cast<const float2*>(a.nsc + 2 * i0);
      dot += e.x;
      ss += e.y;
    }
    dot = block_sum<4>(dot, nred);  // its barriers also publish red4
    ss = block_sum<4>(ss, nred);
    const float nf = (float)qn;
    const float r2 = ss / nf + a.eps;
    inv_r = 1.0f / sqrtf(r2);
    cc = dot / (nf * r2);
  } else {
    __syncthreads();
  }
  if (t < nq) {
    float4 z = red4[t];
    for (int j = 1; j < S; ++j) {
      const float4 o = red4[j * nq + t];
      z.x += o.x;
      z.y += o.y;
      z.z += o.z;
      z.w += o.w;
    }
    if (norm) {
      const float4 xf = BufVec<T>::cvt(nxr);
      z.x = (z.x * ng.x - xf.x * cc) * inv_r;
      z.y = (z.y * ng.y - xf.y * cc) * inv_r;
      z.z = (z.z * ng.z - xf.z * cc) * inv_r;
      z.w = (z.w * ng.w - xf.w * cc) * inv_r;
    }
    *reinterpret_cast<float4*>(dC + 4 * t) = z;
  }
  __syncthreads();
  if (a.copy_n > 0) {
    const int64_t nwg = (int64_t)gridDim.x * gridDim.y;
    for (int64_t i = ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * 256 + t; i < a.copy_n; i += nwg * 256)
      a.copy_dst[i] = a.copy_src[i];
  }
  if (!w0) return;
  // ---- the dec_attn_mfma work, dCtx from LDS
  float4 xv[DK / 4], yv[DK / 4], vv[DK / 4];
  float bd[ND], pd[4], kv[4][ND];
#pragma unroll
  for (int i = 0; i < DK / 4; ++i) {
    yv[i] = BufVec<T>::cvt(yr[i]);
    vv[i] = BufVec<T>::cvt(vr[i]);
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    pd[v] = Buf1<T>::cvt(pdr[v]);
#pragma unroll
    for (int f = 0; f < ND; ++f) kv[v][f] = Buf1<T>::cvt(kvr[v][f]);
  }
  const float pa = Buf1<T>::cvt(par);
#pragma unroll
  for (int i = 0; i < DK / 4; ++i)
    xv[i] = hok ? *reinterpret_cast<const float4*>(dC + l16 * D + DK * c + 4 * i)
                : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int f = 0; f < ND; ++f) bd[f] = dvh ? dC[c * D + 16 * f + l16] : 0.f;
  float dl = 0.f;
#pragma unroll
  for (int i = 0; i < DK / 4; ++i)
    dl += xv[i].x * yv[i].x + xv[i].y * yv[i].y + xv[i].z * yv[i].z + xv[i].w * yv[i].w;
  dl += __shfl_xor(dl, 16, 64);
  dl += __shfl_xor(dl, 32, 64);
  floatx4 da[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) da[j] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < DK / 4; ++i) {
    da[0] = mfma16x16x4(vv[i].x, xv[i].x, da[0]);
    da[1] = mfma16x16x4(vv[i].y, xv[i].y, da[1]);
    da[2] = mfma16x16x4(vv[i].z, xv[i].z, da[2]);
    da[3] = mfma16x16x4(vv[i].w, xv[i].w, da[3]);
  }
  float ds[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) ds[v] = pd[v] * (((da[0][v] + da[1][v]) + (da[2][v] + da[3][v])) - dl);
  floatx4 aq[ND];
#pragma unroll
  for (int f = 0; f < ND; ++f) aq[f] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int v = 0; v < 4; ++v)
#pragma unroll
    for (int f = 0; f < ND; ++f) aq[f] = mfma16x16x4(ds[v], kv[v][f], aq[f]);
  const int64_t nch = (a.s_kv + DM_KB - 1) / DM_KB, chunk = (int64_t)blockIdx.x * DR_NA + w;
  if (chunk < nch) {
#pragma unroll
    for (int f = 0; f < ND; ++f)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int hh = 4 * c + v;
        if (hh < grp) a.dq_part[((int64_t)(g * grp + hh) * nch + chunk) * D + 16 * f + l16] = aq[f][v];
      }
  }
  if (a.dv != nullptr) {
#pragma unroll
    for (int f = 0; f < ND; ++f) {
      floatx4 av = mfma16x16x4(pa, bd[f], floatx4{0.f, 0.f, 0.f, 0.f});
      for (int j = 1; 4 * j < grp; ++j) {
        const int hh = 4 * j + c;
        const bool ok = hh < grp;
        const float p2 =
            (ok && kok) ? Act<T>::ld((const T*)a.P, (int64_t)(g * grp + hh) * a.s_kv + kr) : 0.f;
        const float b2 = ok ? dC[hh * D + 16 * f + l16] : 0.f;
        av = mfma16x16x4(p2, b2, av);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t key = kb + 4 * c + v;
        if (key < a.s_kv) a.dv[key * ldk + g * D + 16 * f + l16] = av[v];
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(D) void dec_attn_dqc_kernel(DecAttnArgs a, int nchunks) {
  __shared__ float o[D];
  const int t = threadIdx.x, h = blockIdx.x;
  const float* src = a.dq_part + (int64_t)h * nchunks * D + t;
  float v = 0.f;
  for (int c0 = 0; c0 < nchunks; c0 += 16) {
    float x[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) x[u] = c0 + u < nchunks ? src[(int64_t)(c0 + u) * D] : 0.f;
#pragma unroll
    for (int u = 0; u < 16; ++u) v += x[u];
  }
  o[t] = a.scale * v;
  __syncthreads();
  constexpr int HALF = D / 2;
  if (!a.rope) {
    a.dq[(int64_t)h * D + t] = o[t];
  } else if (t < HALF) {
    const double inv_freq = exp2(-(2.0 * t / D) * a.log2_base);
    double sn, cs;
    sincos((double)a.pos * inv_freq, &sn, &cs);
    const float cf = (float)cs, sf = (float)sn;
    const float lo = o[t], hi = o[t + HALF];
    a.dq[(int64_t)h * D + t] = lo * cf + hi * sf;
    a.dq[(int64_t)h * D + t + HALF] = -lo * sf + hi * cf;
  }
}

static size_t dec_attn1c_smem(int64_t grp, int64_t D) {
  return ((size_t)2 * DA_KC * (D + 1) + 2 * grp * D + 10 * grp * DA_KC + (256 / D) * grp * D) *
         sizeof(float);
}

static size_t dec_attn1_smem(int64_t grp, int64_t D) {
  return ((size_t)DA_KC * (D + 1) + grp * D + grp * DA_KC + 8 * grp * DA_KC) * sizeof(float);
}

static size_t dec_attn2_smem(int64_t s_kv, int64_t D) {
  return ((size_t)s_kv + (DQ_W + 1) * D) * sizeof(float);
}

template <typename T, int D>
static hipError_t dec_attn_launch(const DecAttnArgs& a, hipStream_t s) {
  const int Hkv = a.Hq / a.grp;
  const double es = sizeof(T);
  const int nch = (int)cdiv(a.s_kv, DA_KC);
  hipError_t e;
  // buffer ranges: the whole cache (K, V), P and the query row; the
  // two-pass path keeps a row of scores per head in LDS
  if ((double)a.s_kv * Hkv * D * es >= BUF_MAX_BYTES || (double)a.Hq * a.s_kv * es >= BUF_MAX_BYTES ||
      !dec_attn_fits(a.s_kv, a.Hq, Hkv, D))
    return hipErrorInvalidValue;
  if (a.part != nullptr) {
    // the caller checked dec_attn_red_fits and passes ctx
    if (a.ctx == nullptr || !dec_attn_red_fits(a.Hq, Hkv, D, a.splits) ||
        (double)a.splits * a.Hq * D * 4 >= BUF_MAX_BYTES || (double)a.nscal * 8 >= BUF_MAX_BYTES)
      return hipErrorInvalidValue;
  }
  if (dry_run()) return hipSuccess;
  if (a.part != nullptr) {
    const int nb = (int)cdiv(a.s_kv, DM_KB);
    const size_t sm = 256 * sizeof(float4) + (size_t)a.grp * D * sizeof(float);
    dec_attn_red_kernel<T, D><<<dim3((unsigned)cdiv(nb, DR_NA), (unsigned)Hkv), dim3(256), sm, s>>>(a);
    mark("dec_attn_red",
         2.0 * a.s_kv * Hkv * D * es + (double)a.Hq * a.s_kv * es + (double)a.Hq * D * (4 + es) +
             (a.dv ? (double)a.s_kv * Hkv * D * 4 : 0.0) + (double)a.copy_n * 8,
         6.0 * D * a.Hq * a.s_kv, s, (double)a.Hq * nb * D * 4);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    dec_attn_dqc_kernel<D><<<dim3((unsigned)a.Hq), dim3(D), 0, s>>>(a, nb);
    mark("dec_attn_dqc", (double)a.Hq * D * 4, 0, s, (double)a.Hq * nb * D * 4);
    return hipGetLastError();
  }
  if (a.ctx != nullptr && a.grp <= 16) {
    const int nb = (int)cdiv(a.s_kv, DM_KB);
    dec_attn_mfma_kernel<T, D><<<dim3((unsigned)nb, (unsigned)Hkv), dim3(64), 0, s>>>(a);
    mark("dec_attn_mfma",
         2.0 * a.s_kv * Hkv * D * es + (double)a.Hq * a.s_kv * es + (double)a.Hq * D * (4 + es) +
             (a.dv ? (double)a.s_kv * Hkv * D * 4 : 0.0),
         6.0 * D * a.Hq * a.s_kv, s, (double)a.Hq * nb * D * 4);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    dec_attn_dqc_kernel<D><<<dim3((unsigned)a.Hq), dim3(D), 0, s>>>(a, nb);
    mark("dec_attn_dqc", (double)a.Hq * D * 4, 0, s, (double)a.Hq * nb * D * 4);
    return hipGetLastError();
  }
  if (a.ctx != nullptr && a.grp <= 64 && dec_attn1c_smem(a.grp, D) <= 64 * 1024) {
    dec_attn1c_kernel<T, D><<<dim3((unsigned)nch, (unsigned)Hkv), dim3(256),
                              dec_attn1c_smem(a.grp, D), s>>>(a);
    mark("dec_attn1c",
         2.0 * a.s_kv * Hkv * D * es + (double)a.Hq * a.s_kv * es + (double)a.Hq * D * (4 + es) +
             (a.dv ? (double)a.s_kv * Hkv * D * 4 : 0.0),
         6.0 * D * a.Hq * a.s_kv, s, (double)a.Hq * nch * D * 4);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    dec_attn_dqc_kernel<D><<<dim3((unsigned)a.Hq), dim3(D), 0, s>>>(a, nch);
    mark("dec_attn_dqc", (double)a.Hq * D * 4, 0, s, (double)a.Hq * nch * D * 4);
    return hipGetLastError();
  }
  dec_attn1_kernel<T, D><<<dim3((unsigned)nch, (unsigned)Hkv), dim3(256),
                           dec_attn1_smem(a.grp, D), s>>>(a);
  // P, V, dCtx and K (second launch) once, dV and dq written; dA is an
  // intermediate written here and read by the second launch
  mark("dec_attn1",
       (double)a.s_kv * Hkv * D * es + (double)a.Hq * a.s_kv * es + (double)a.Hq * D * 4 +
           (a.dv ? (double)a.s_kv * Hkv * D * 4 : 0.0),
       4.0 * D * a.Hq * a.s_kv, s, (double)a.Hq * a.s_kv * 4);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  dec_attn2_kernel<T, D><<<dim3((unsigned)a.Hq), dim3(1024), dec_attn2_smem(a.s_kv, D), s>>>(a);
  mark("dec_attn2", (double)a.s_kv * Hkv * D * es + (double)a.Hq * D * 4, 2.0 * D * a.Hq * a.s_kv, s,
       (double)a.Hq * a.s_kv * (es + 4));
  return hipGetLastError();
}

bool dec_attn_fits(int64_t s_kv, int64_t n_heads, int64_t n_kv_heads, int64_t head_dim) {
  return dec_attn1_smem(n_heads / n_kv_heads, head_dim) <= 64 * 1024 &&
         dec_attn2_smem(s_kv, head_dim) <= 64 * 1024;
}

size_t dec_attn_ws_bytes(int64_t s_kv, int64_t n_heads, int64_t head_dim) {
  // dA [Hq, s_kv] for the two-pass path, or the dq shares [Hq, chunks, D]
  // (one per 16 keys for the MFMA kernel, one per DA_KC keys for the LDS one)
  const size_t a = (size_t)n_heads * s_kv, b = (size_t)n_heads * cdiv(s_kv, 16) * head_dim;
  return (a > b ? a : b) * sizeof(float);
}

hipError_t launch_dec_attn(int dt, int head_dim, const DecAttnArgs& a, hipStream_t s) {
#define LBP_DA(DD)                                                                 \
  case DD:                                                                         \
    return dt == F32 ? dec_attn_launch<float, DD>(a, s) : dec_attn_launch<bf16, DD>(a, s);
  switch (head_dim) {
    LBP_DA(16)
    LBP_DA(32)
    LBP_DA(64)
    LBP_DA(128)
    default:
      return hipErrorInvalidValue;
  }
#undef LBP_DA
}

// ---------------------------------------------------------------------------
// Packing of ternary weights (tern2 in common.h): one byte, four columns, per
// thread; each value coded by its sign.
template <typename T>
__global__ __launch_bounds__(256) void pack_ternary_kernel(int64_t rows, int64_t cols,
                                                           const T* __restrict__ w,
                                                           uint8_t* __restrict__ out) {
  const int64_t q = cols / 4, nb = rows * q;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nb; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / q, c = i - r * q;
    const float4 v = Act<T>::ld4(w, r * cols + 4 * c);
    const float e[4] = {v.x, v.y, v.z, v.w};
    uint32_t b = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) b |= (e[j] > 0.f ? 1u : e[j] < 0.f ? 3u : 0u) << (2 * j);
    out[i] = (uint8_t)b;
  }
}

hipError_t launch_pack_ternary(int64_t rows, int64_t cols, const void* w, int w_dt, uint8_t* out,
                               hipStream_t s) {
  const int64_t nb = rows * (cols / 4);
  if (nb == 0) return hipSuccess;
  if (dry_run()) return hipSuccess;
  int64_t blocks = cdiv(nb, 256);
  if (blocks > 8192) blocks = 8192;
  if (w_dt == F32)
    pack_ternary_kernel<float><<<dim3((unsigned)blocks), 256, 0, s>>>(rows, cols, (const float*)w, out);
  else
    pack_ternary_kernel<bf16><<<dim3((unsigned)blocks), 256, 0, s>>>(rows, cols, (const bf16*)w, out);
  mark("pack_ternary", (double)rows * cols * (w_dt == F32 ? 4 : 2) + (double)nb, 0, s);
  return hipGetLastError();
}

}  // namespace lbp
