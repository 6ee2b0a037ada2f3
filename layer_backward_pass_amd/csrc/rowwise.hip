// Row-wise and elementwise backward kernels: RMSNorm backward, inverse NeoX
// RoPE, and the gated-activation (SwiGLU, ReLU^2 x up) backward.  All are
// HBM-bound: each element is read once and written once, with float4 /
// 8-byte bf16 vector accesses.
#include "common.h"
#include "kernels.h"

namespace lbp {

static inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------------------
// RMSNorm backward, one 256-thread workgroup per row.  Hesper "Attention
// Backward GPU Kernels", section "RMSNorm Backward":
//   dx = (1/r) (dy*gamma - x <dy*gamma, x> / (n r^2)),  r = sqrt(mean(x^2)+eps)
// Pass 1 reduces sum(x^2) and <dy*gamma, x> over the row; pass 2 writes dx
// (or adds it to dx, or to a separate residual input rin).  Each thread re-reads only the elements it read in pass
// 1, so dx may alias dy.  dy may arrive as `nparts` split-K partial sums
// (stride pstride), added here in split order.
__device__ __forceinline__ float4 sum_parts4(const float* p, int nparts, int64_t pstride) {
  if (nparts == 1) return *reinterpret_cast<const float4*>(p);
  // up to 8 partials in flight (an index past the last re-reads part 0 and
  // its term is dropped), added in order
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int i0 = 0; i0 < nparts; i0 += 8) {
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = *reinterpret_cast<const float4*>(p + (i0 + u < nparts ? i0 + u : 0) * pstride);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bool take = i0 + u < nparts;
      s.x += take ? v[u].x : 0.f;
      s.y += take ? v[u].y : 0.f;
      s.z += take ? v[u].z : 0.f;
      s.w += take ? v[u].w : 0.f;
    }
  }
  return s;
}

template <typename T, int ACC>
__global__ __launch_bounds__(256) void rmsnorm_bwd_kernel(int64_t n, const T* __restrict__ x,
                                                          const float* __restrict__ gamma,
                                                          const float* dy, float* dx,
                                                          float eps, int nparts, int64_t pstride,
                                                          const float* rin, uint16_t* dx16) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const T* xr = x + row * n;
  const float* dyr = dy + row * n;
  float* dxr = dx + row * n;
  float ss = 0.f, dot = 0.f;
  for (int64_t i = (int64_t)threadIdx.x * 4; i < n; i += 1024) {
    float4 xv = Act<T>::ld4(xr, i);
    float4 gv = *reinterpret_cast<const float4*>(gamma + i);
    float4 dv = sum_parts4(dyr + i, nparts, pstride);
    ss += xv.x * xv.x + xv.y * xv.y + xv.z * xv.z + xv.w * xv.w;
    dot += dv.x * gv.x * xv.x + dv.y * gv.y * xv.y + dv.z * gv.z * xv.z + dv.w * gv.w * xv.w;
  }
  ss = block_sum<4>(ss, red);
  dot = block_sum<4>(dot, red);
  const float nf = (float)n;
  const float r2 = ss / nf + eps;
  const float inv_r = 1.0f / sqrtf(r2);
  const float c = dot / (nf * r2);
  for (int64_t i = (int64_t)threadIdx.x * 4; i < n; i += 1024) {
    float4 xv = Act<T>::ld4(xr, i);
    float4 gv = *reinterpret_cast<const float4*>(gamma + i);
    float4 dv = sum_parts4(dyr + i, nparts, pstride);
    float4 o;
    o.x = (dv.x * gv.x - xv.x * c) * inv_r;
    o.y = (dv.y * gv.y - xv.y * c) * inv_r;
    o.z = (dv.z * gv.z - xv.z * c) * inv_r;
    o.w = (dv.w * gv.w - xv.w * c) * inv_r;
    float4* dp = reinterpret_cast<float4*>(dxr + i);
    if (ACC) {
      // the residual term: dx itself, or the separate input rin
      const float4 p = *reinterpret_cast<const float4*>((rin ? rin + row * n : dxr) + i);
      o.x += p.x;
      o.y += p.y;
      o.z += p.z;
      o.w += p.w;
    }
    *dp = o;
    if (dx16 != nullptr)
      *reinterpret_cast<uint2*>(dx16 + row * n + i) = make_uint2(pk_bf16(o.x, o.y), pk_bf16(o.z, o.w));
  }
}

// The same with the row held in registers (n <= 1024 Q): x, gamma and dy
// (the sum of its nparts partials, in split order, PB partials in flight)
// are read once, so split-K partials cost one pass instead of two.
template <typename T, int ACC, int Q>
__global__ __launch_bounds__(256) void rmsnorm_bwd_reg_kernel(int64_t n, const T* __restrict__ x,
                                                              const float* __restrict__ gamma,
                                                              const float* dy, float* dx,
                                                              float eps, int nparts,
                                                              int64_t pstride, const float* rin,
                                                              uint16_t* dx16) {
  constexpr int PB = Q <= 4 ? 4 : 2;
  __shared__ float red[4];
  const int t = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int64_t n4 = n / 4;
  const uint32_t ES = sizeof(T);
  const brsrc_t rx = make_brsrc(x + row * n, (uint32_t)(n * ES));
  const brsrc_t rgm = make_brsrc(gamma, (uint32_t)(n * 4));
  const brsrc_t rdy = make_brsrc(dy + row * n, (uint32_t)(((nparts - 1) * pstride + n) * 4));
  typename BufVec<T>::raw xr[Q];
  float4 gm[Q], y[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int64_t i4 = t + 256 * q;
    const bool ok = i4 < n4;
    xr[q] = BufVec<T>::load(rx, ok ? (uint32_t)(i4 * 4 * ES) : BUF_OOB);
    gm[q] = bload_f4(rgm, ok ? (uint32_t)(i4 * 16) : BUF_OOB);
    y[q] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  for (int p0 = 0; p0 < nparts; p0 += PB) {
    float4 v[PB][Q];
#pragma unroll
    for (int u = 0; u < PB; ++u)
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const int64_t i4 = t + 256 * q;
        const int p = p0 + u;
        v[u][q] = bload_f4(rdy, (p < nparts && i4 < n4) ? (uint32_t)((p * pstride + 4 * i4) * 4) : BUF_OOB);
      }
#pragma unroll
    for (int u = 0; u < PB; ++u)
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        y[q].x += v[u][q].x;
        y[q].y += v[u][q].y;
        y[q].z += v[u][q].z;
        y[q].w += v[u][q].w;
      }
  }
  float4 xv[Q];
  float ss = 0.f, dot = 0.f;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    xv[q] = BufVec<T>::cvt(xr[q]);
    ss += xv[q].x * xv[q].x + xv[q].y * xv[q].y + xv[q].z * xv[q].z + xv[q].w * xv[q].w;
    dot += y[q].x * gm[q].x * xv[q].x + y[q].y * gm[q].y * xv[q].y + y[q].z * gm[q].z * xv[q].z +
           y[q].w * gm[q].w * xv[q].w;
  }
  ss = block_sum<4>(ss, red);
  dot = block_sum<4>(dot, red);
  const float nf = (float)n;
  const float r2 = ss / nf + eps;
  const float inv_r = 1.0f / sqrtf(r2);
  const float c = dot / (nf * r2);
  float* dxr = dx + row * n;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int64_t i4 = t + 256 * q;
    if (i4 >= n4) continue;
    float4 o;
    o.x = (y[q].x * gm[q].x - xv[q].x * c) * inv_r;
    o.y = (y[q].y * gm[q].y - xv[q].y * c) * inv_r;
    o.z = (y[q].z * gm[q].z - xv[q].z * c) * inv_r;
    o.w = (y[q].w * gm[q].w - xv[q].w * c) * inv_r;
    float4* dp = reinterpret_cast<float4*>(dxr + 4 * i4);
    if (ACC) {
      const float4 pr = *reinterpret_cast<const float4*>((rin ? rin + row * n : dxr) + 4 * i4);
      o.x += pr.x;
      o.y += pr.y;
      o.z += pr.z;
      o.w += pr.w;
    }
    *dp = o;
    if (dx16 != nullptr)
      *reinterpret_cast<uint2*>(dx16 + row * n + 4 * i4) =
          make_uint2(pk_bf16(o.x, o.y), pk_bf16(o.z, o.w));
  }
}

hipError_t launch_rmsnorm_bwd(int64_t rows, int64_t n, const void* x, int xdt, const float* gamma,
                              const float* dy, float* dx, float eps, int accumulate,
                              hipStream_t s, int nparts, int64_t pstride, const float* rin,
                              uint16_t* dx16) {
  if (rows == 0) return hipSuccess;
  if (dry_run()) return hipSuccess;
  dim3 grid((unsigned)rows), block(256);
  const int64_t Q = cdiv(n / 4, 256);
  if (Q <= 8 && ((double)(nparts - 1) * pstride + n) * 4 < BUF_MAX_BYTES) {
#define LBP_RN(T, QV)                                                                           \
  case QV:                                                                                      \
    if (accumulate)                                                                             \
      rmsnorm_bwd_reg_kernel<T, 1, QV><<<grid, block, 0, s>>>(n, (const T*)x, gamma, dy, dx,    \
                                                             eps, nparts, pstride, rin, dx16);        \
    else                                                                                        \
      rmsnorm_bwd_reg_kernel<T, 0, QV><<<grid, block, 0, s>>>(n, (const T*)x, gamma, dy, dx,    \
                                                             eps, nparts, pstride, rin, dx16);        \
    break;
    if (xdt == F32) {
      switch (Q) { LBP_RN(float, 1) LBP_RN(float, 2) LBP_RN(float, 3) LBP_RN(float, 4)
                   LBP_RN(float, 5) LBP_RN(float, 6) LBP_RN(float, 7) default: LBP_RN(float, 8) }
    } else {
      switch (Q) { LBP_RN(bf16, 1) LBP_RN(bf16, 2) LBP_RN(bf16, 3) LBP_RN(bf16, 4)
                   LBP_RN(bf16, 5) LBP_RN(bf16, 6) LBP_RN(bf16, 7) default: LBP_RN(bf16, 8) }
    }
#undef LBP_RN
  } else if (xdt == F32) {
    if (accumulate)
      rmsnorm_bwd_kernel<float, 1><<<grid, block, 0, s>>>(n, (const float*)x, gamma, dy, dx, eps, nparts, pstride, rin, dx16);
    else
      rmsnorm_bwd_kernel<float, 0><<<grid, block, 0, s>>>(n, (const float*)x, gamma, dy, dx, eps, nparts, pstride, rin, dx16);
  } else {
    if (accumulate)
      rmsnorm_bwd_kernel<bf16, 1><<<grid, block, 0, s>>>(n, (const bf16*)x, gamma, dy, dx, eps, nparts, pstride, rin, dx16);
    else
      rmsnorm_bwd_kernel<bf16, 0><<<grid, block, 0, s>>>(n, (const bf16*)x, gamma, dy, dx, eps, nparts, pstride, rin, dx16);
  }
  mark("rmsnorm_bwd",
       (double)rows * n * ((xdt == F32 ? 4 : 2) + 4 + 4 + (accumulate ? 4 : 0)) + n * 4.0,
       (double)rows * n * 8, s, (double)rows * n * (4.0 * (nparts - 1) + (dx16 ? 2 : 0)));
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Inverse NeoX RoPE (rope_bwd_row in common.h): one workgroup per row.
__global__ __launch_bounds__(256) void rope_bwd_kernel(int64_t n_heads, int head_dim,
                                                       const float* dy, const float* dy2,
                                                       float* dx, int64_t pos0,
                                                       double log2_base, RopeNorm nm) {
  rope_bwd_row(blockIdx.x, threadIdx.x, blockDim.x, n_heads, head_dim, dy, dy2, dx, pos0,
               log2_base, nm);
}

hipError_t launch_rope_bwd(int64_t rows, int64_t n_heads, int64_t head_dim, const float* dy,
                           float* dx, int64_t pos0, float base, hipStream_t s, const float* dy2,
                           const RopeNormArgs* norm) {
  if (rows == 0) return hipSuccess;
  if (dry_run()) return hipSuccess;
  const int threads = rope_threads(n_heads, head_dim);
  const RopeNorm nm = norm != nullptr && norm->x != nullptr
                          ? RopeNorm{norm->x, norm->x_bf16, norm->gamma, norm->eps}
                          : RopeNorm{nullptr, 0, nullptr, 0.f};
  rope_bwd_kernel<<<dim3((unsigned)rows), dim3(threads), 0, s>>>(n_heads, (int)head_dim, dy, dy2,
                                                                   dx, pos0, log2((double)base), nm);
  const double qe = (double)rows * n_heads * head_dim;
  mark("rope_bwd", qe * (8 + (nm.x ? (nm.x_bf16 ? 2 : 4) : 0)), qe * (nm.x ? 9 : 3), s,
       dy2 ? qe * 4 : 0.0);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Gated activation backward, 4 elements per thread.
//   SwiGLU (entrenar wgpu_backward.rs, "SiLU backward"): s = sigmoid(g),
//     dGate = dH up s (1 + g (1 - s)),  dUp = dH g s
//   ReLU^2 x up (Hesper "FFN Backward GPU Kernels", "ReLU²×Mul Backward"):
//     dGate = dH up 2 max(0,g),  dUp = dH max(0,g)^2
// Output row r is [dGate(0:I) | dUp(0:I)] so the next product runs over
// K = 2I against the stacked [W_gate; W_up].
template <typename T, int ACT, int OUT_BF16>
__global__ __launch_bounds__(256) void act_bwd_kernel(int64_t rows, int64_t ffn,
                                                      const T* __restrict__ gate,
                                                      const T* __restrict__ up,
                                                      const float* __restrict__ dhid, void* dgu,
                                                      int nparts, int64_t pstride) {
  const int64_t q = ffn / 4;
  const int64_t total = rows * q;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = t / q;
    const int64_t c = (t - r * q) * 4;
    const int64_t i = r * ffn + c;
    const float4 g = Act<T>::ld4(gate, i);
    const float4 u = Act<T>::ld4(up, i);
    const float4 dh = sum_parts4(dhid + i, nparts, pstride);
    float4 dg, du;
    act_bwd1<ACT>(g.x, u.x, dh.x, dg.x, du.x);
    act_bwd1<ACT>(g.y, u.y, dh.y, dg.y, du.y);
    act_bwd1<ACT>(g.z, u.z, dh.z, dg.z, du.z);
    act_bwd1<ACT>(g.w, u.w, dh.w, dg.w, du.w);
    const int64_t og = r * 2 * ffn + c, ou = og + ffn;
    if (OUT_BF16) {
      uint16_t* o = (uint16_t*)dgu;
      uint2 a, b;
      a.x = pk_bf16(dg.x, dg.y);
      a.y = pk_bf16(dg.z, dg.w);
      b.x = pk_bf16(du.x, du.y);
      b.y = pk_bf16(du.z, du.w);
      *reinterpret_cast<uint2*>(o + og) = a;
      *reinterpret_cast<uint2*>(o + ou) = b;
    } else {
      float* o = (float*)dgu;
      *reinterpret_cast<float4*>(o + og) = dg;
      *reinterpret_cast<float4*>(o + ou) = du;
    }
  }
}

template <typename T, int ACT>
static void act_launch(int64_t rows, int64_t ffn, const void* gate, const void* up,
                       const float* dhid, void* dgu, int out_dt, hipStream_t s, int nparts,
                       int64_t pstride) {
  const int64_t total = rows * (ffn / 4);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (out_dt == BF16)
    act_bwd_kernel<T, ACT, 1><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(
        rows, ffn, (const T*)gate, (const T*)up, dhid, dgu, nparts, pstride);
  else
    act_bwd_kernel<T, ACT, 0><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(
        rows, ffn, (const T*)gate, (const T*)up, dhid, dgu, nparts, pstride);
}

hipError_t launch_act_bwd(int64_t rows, int64_t ffn, int act, const void* gate, const void* up,
                          int in_dt, const float* dhid, void* dgu, int out_dt, hipStream_t s,
                          int nparts, int64_t pstride) {
  if (rows == 0) return hipSuccess;
  if (dry_run()) return hipSuccess;
  if (in_dt == F32) {
    if (act == SWIGLU) act_launch<float, SWIGLU>(rows, ffn, gate, up, dhid, dgu, out_dt, s, nparts, pstride);
    else act_launch<float, RELU2>(rows, ffn, gate, up, dhid, dgu, out_dt, s, nparts, pstride);
  } else {
    if (act == SWIGLU) act_launch<bf16, SWIGLU>(rows, ffn, gate, up, dhid, dgu, out_dt, s, nparts, pstride);
    else act_launch<bf16, RELU2>(rows, ffn, gate, up, dhid, dgu, out_dt, s, nparts, pstride);
  }
  mark("act_bwd", (double)rows * ffn * (2 * (in_dt == F32 ? 4 : 2) + 4 + 2 * (out_dt == F32 ? 4 : 2)),
       (double)rows * ffn * 12, s, (double)rows * ffn * 4 * (nparts - 1));
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void fill_zero_kernel(int64_t n, float* __restrict__ p) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.f;
}

hipError_t launch_fill_zero(int64_t n, float* p, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (dry_run()) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  fill_zero_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(n, p);
  mark("fill_zero", (double)n * 4, 0, s);  // dV of no queries: the output itself
  return hipGetLastError();
}

}  // namespace lbp
