// GQA attention backward from saved softmax weights.
//
// Hesper "Attention Backward GPU Kernels": "Attention Apply Backward"
// (dA = dCtx V^T), "Softmax Backward" (dS = P o (dA - delta)), "Attention
// Score Backward" (dQ = scale dS K); entrenar wgpu_backward.rs attention
// backward for dV = P^T dCtx.  Query head h reads KV head h / grp.
//
// Sequence path (s_q > 1), v_mfma_f32_16x16x4_f32 throughout:
//   attn_dq_kernel  one workgroup per (64 query rows, head); each wave owns
//                   16 rows, keeps its dCtx rows in registers, and walks the
//                   key blocks up to the causal limit: dA on the matrix
//                   cores, P read straight into the accumulator layout, dS
//                   formed in registers, transposed through LDS and
//                   multiplied by the K block.  delta comes from
//                   <dCtx, ctx> (ctx = P V), so P is streamed once.
//   attn_dv_kernel  one workgroup per (32 keys, KV head); sums P^T dCtx over
//                   the heads of the group and the query blocks that can
//                   see those keys.
//   attn_delta_kernel  delta = rowsum(P o dA) formed from P directly, for
//                   callers that do not pass ctx.
// One query row (decode) goes to the kernels in decode.hip.
#include "common.h"
#include "kernels.h"

namespace lbp {

constexpr int AQ = 64;  // query rows per dq workgroup (16 per wave)
constexpr int AK = 32;  // keys per dq inner block

template <typename T, int D, int HAS_CTX>
__global__ __launch_bounds__(256) void attn_dq_kernel(int64_t s_q, int64_t s_kv, int Hq, int grp,
                                                      const float* __restrict__ dctx,
                                                      const T* __restrict__ P,
                                                      const T* __restrict__ K,
                                                      const T* __restrict__ V,
                                                      const T* __restrict__ ctx,
                                                      const float* __restrict__ delta_ws,
                                                      float* __restrict__ dq, float scale,
                                                      int causal) {
  constexpr int DK = D / 4;   // MFMA k-steps over the head dimension
  constexpr int NF = D / 16;  // output column tiles of dQ
  __shared__ float Ks[AK][D + 4];
  __shared__ float Vs[AK][D + 4];
  __shared__ float dSs[4][16][AK + 1];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int r16 = lane & 15, c4 = lane >> 4;
  const int h = blockIdx.y, g = h / grp;
  const int64_t ldq = (int64_t)Hq * D, ldk = (int64_t)(Hq / grp) * D;
  const int64_t qb0 = (int64_t)blockIdx.x * AQ;
  const int64_t q0 = qb0 + 16 * w;

  // dCtx operand: lane holds row q0 + r16, head dims DK*c4 .. DK*c4+DK-1
  // (the k index of MFMA step ks in lane group c4 is d = DK*c4 + ks)
  float a_dc[DK];
  const int64_t qrow = q0 + r16;
  const bool qok = qrow < s_q;
#pragma unroll
  for (int i = 0; i < DK; i += 4) {
    float4 v = make_float4(0, 0, 0, 0);
    if (qok) v = *reinterpret_cast<const float4*>(dctx + qrow * ldq + h * D + DK * c4 + i);
    a_dc[i] = v.x;
    a_dc[i + 1] = v.y;
    a_dc[i + 2] = v.z;
    a_dc[i + 3] = v.w;
  }
  float dl = 0.f;
  if (HAS_CTX) {
#pragma unroll
    for (int i = 0; i < DK; i += 4) {
      float4 c = make_float4(0, 0, 0, 0);
      if (qok) c = Act<T>::ld4(ctx, qrow * ldq + h * D + DK * c4 + i);
      dl += a_dc[i] * c.x + a_dc[i + 1] * c.y + a_dc[i + 2] * c.z + a_dc[i + 3] * c.w;
    }
    dl += __shfl_xor(dl, 16, 64);
    dl += __shfl_xor(dl, 32, 64);
  } else {
    if (qok) dl = delta_ws[(int64_t)h * s_q + qrow];
  }
  float dlv[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) dlv[v] = __shfl(dl, 4 * c4 + v, 64);

  floatx4 acc[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) acc[f] = floatx4{0, 0, 0, 0};

  const int64_t off = s_kv - s_q;
  const int64_t qlast = min(s_q, qb0 + AQ) - 1;
  const int64_t kend = causal ? min(s_kv, off + qlast + 1) : s_kv;
  const T* Ph = P + (int64_t)h * s_q * s_kv;

  for (int64_t k0 = 0; k0 < kend; k0 += AK) {
    __syncthreads();
    for (int e = t * 4; e < AK * D; e += 1024) {
      const int kr = e / D, dc = e - kr * D;
      const int64_t key = k0 + kr;
      float4 kv = make_float4(0, 0, 0, 0), vv = kv;
      if (key < s_kv) {
        kv = Act<T>::ld4(K, key * ldk + g * D + dc);
        vv = Act<T>::ld4(V, key * ldk + g * D + dc);
      }
      *reinterpret_cast<float4*>(&Ks[kr][dc]) = kv;
      *reinterpret_cast<float4*>(&Vs[kr][dc]) = vv;
    }
    __syncthreads();
    floatx4 dA[2] = {floatx4{0, 0, 0, 0}, floatx4{0, 0, 0, 0}};
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) {
      dA[0] = mfma16x16x4(a_dc[ks], Vs[r16][DK * c4 + ks], dA[0]);
      dA[1] = mfma16x16x4(a_dc[ks], Vs[16 + r16][DK * c4 + ks], dA[1]);
    }
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int64_t key = k0 + 16 * f + r16;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t row = q0 + 4 * c4 + v;
        const float p = (row < s_q && key < s_kv) ? Act<T>::ld(Ph, row * s_kv + key) : 0.f;
        dSs[w][4 * c4 + v][16 * f + r16] = p * (dA[f][v] - dlv[v]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < AK / 4; ++ks) {
      const float a = dSs[w][r16][(AK / 4) * c4 + ks];
#pragma unroll
      for (int f = 0; f < NF; ++f) acc[f] = mfma16x16x4(a, Ks[(AK / 4) * c4 + ks][16 * f + r16], acc[f]);
    }
  }
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t row = q0 + 4 * c4 + v;
      if (row < s_q) dq[row * ldq + h * D + 16 * f + r16] = scale * acc[f][v];
    }
}

// dV.  Workgroup = (block of 16*NKW keys, KV head); wave w covers key
// sub-block w % NKW and head-dim slice w / NKW.  MFMA m = key, n = head
// dim, k = query row (row 16*c4 + ks of the current 64-row block).
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_dv_kernel(int64_t s_q, int64_t s_kv, int Hq, int grp,
                                                      const float* __restrict__ dctx,
                                                      const T* __restrict__ P,
                                                      float* __restrict__ dv, int causal) {
  constexpr int NKW = D >= 32 ? 2 : 4;  // key sub-blocks of 16 per workgroup
  constexpr int NDW = 4 / NKW;          // head-dim slices per workgroup
  constexpr int NF = D / 16 / NDW;      // 16-wide output tiles per wave
  constexpr int KB = 16 * NKW;
  __shared__ float dCs[64][D + 4];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int r16 = lane & 15, c4 = lane >> 4;
  const int g = blockIdx.y;
  const int64_t ldq = (int64_t)Hq * D, ldk = (int64_t)(Hq / grp) * D;
  const int64_t kb0 = (int64_t)blockIdx.x * KB;
  const int64_t key0 = kb0 + 16 * (w % NKW);
  const int d0 = (w / NKW) * (D / NDW);
  const int64_t off = s_kv - s_q;
  int64_t qstart = causal ? kb0 - off : 0;
  if (qstart < 0) qstart = 0;
  qstart = qstart / 64 * 64;

  floatx4 acc[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) acc[f] = floatx4{0, 0, 0, 0};
  const int64_t key = key0 + r16;
  for (int hh = 0; hh < grp; ++hh) {
    const int h = g * grp + hh;
    const T* Ph = P + (int64_t)h * s_q * s_kv;
    for (int64_t q0 = qstart; q0 < s_q; q0 += 64) {
      __syncthreads();
      for (int e = t * 4; e < 64 * D; e += 1024) {
        const int rr = e / D, dc = e - rr * D;
        const int64_t row = q0 + rr;
        float4 v = make_float4(0, 0, 0, 0);
        if (row < s_q) v = *reinterpret_cast<const float4*>(dctx + row * ldq + h * D + dc);
        *reinterpret_cast<float4*>(&dCs[rr][dc]) = v;
      }
      __syncthreads();
#pragma unroll 4
      for (int ks = 0; ks < 16; ++ks) {
        const int rr = 16 * c4 + ks;
        const int64_t row = q0 + rr;
        const float a = (row < s_q && key < s_kv) ? Act<T>::ld(Ph, row * s_kv + key) : 0.f;
#pragma unroll
        for (int f = 0; f < NF; ++f) acc[f] = mfma16x16x4(a, dCs[rr][d0 + 16 * f + r16], acc[f]);
      }
    }
  }
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t k = key0 + 4 * c4 + v;
      if (k < s_kv) dv[k * ldk + g * D + d0 + 16 * f + r16] = acc[f][v];
    }
}

// delta[h, i] = sum_j P[h,i,j] (dCtx_h[i] . V_g[j]), one wave per (row, head).
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_delta_kernel(int64_t s_q, int64_t s_kv, int Hq,
                                                         int grp, const float* __restrict__ dctx,
                                                         const T* __restrict__ P,
                                                         const T* __restrict__ V,
                                                         float* __restrict__ delta, int causal) {
  __shared__ float dc[4][D];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int h = blockIdx.y, g = h / grp;
  const int64_t i = (int64_t)blockIdx.x * 4 + w;
  const int64_t ldq = (int64_t)Hq * D, ldk = (int64_t)(Hq / grp) * D;
  for (int d = lane; d < D; d += 64) dc[w][d] = i < s_q ? dctx[i * ldq + h * D + d] : 0.f;
  __syncthreads();
  if (i >= s_q) return;
  const int64_t jend = causal ? min(s_kv, s_kv - s_q + i + 1) : s_kv;
  const T* Pr = P + ((int64_t)h * s_q + i) * s_kv;
  float s = 0.f;
  for (int64_t j = lane; j < jend; j += 64) {
    float a = 0.f;
    for (int d = 0; d < D; d += 4) {
      const float4 v = Act<T>::ld4(V, j * ldk + g * D + d);
      a += dc[w][d] * v.x + dc[w][d + 1] * v.y + dc[w][d + 2] * v.z + dc[w][d + 3] * v.w;
    }
    s += Act<T>::ld(Pr, j) * a;
  }
  s = wave_sum(s);
  if (lane == 0) delta[(int64_t)h * s_q + i] = s;
}

size_t attn_ws_bytes(int64_t s_q, int64_t s_kv, int64_t n_heads, int64_t n_kv_heads,
                     int64_t head_dim) {
  (void)n_kv_heads;
  if (s_q == 1) return dec_attn_ws_bytes(s_kv, n_heads, head_dim);
  return (size_t)n_heads * s_q * sizeof(float);
}

template <typename T, int D>
static hipError_t attn_launch(int64_t s_q, int64_t s_kv, int Hq, int Hkv, const float* dctx,
                              const T* P, const T* K, const T* V, const T* ctx, float* dq,
                              float* dv, float scale, int causal, float* ws, hipStream_t s) {
  const int grp = Hq / Hkv;
  const double es = sizeof(T);
  dim3 block(256);
  // unmasked (query, key) pairs per head: the work the method must do
  const double pairs = causal ? (double)s_q * (s_kv - s_q) + 0.5 * (double)s_q * (s_q + 1)
                              : (double)s_q * s_kv;
  const double pbytes = pairs * Hq * es, qbytes = (double)s_q * Hq * D;
  const double kvbytes = (double)s_kv * Hkv * D;
  dim3 gq((unsigned)((s_q + AQ - 1) / AQ), (unsigned)Hq);
  if (ctx != nullptr) {
    attn_dq_kernel<T, D, 1><<<gq, block, 0, s>>>(s_q, s_kv, Hq, grp, dctx, P, K, V, ctx, nullptr,
                                                  dq, scale, causal);
    mark("attn_dq_mfma", pbytes + qbytes * (8 + es) + 2 * kvbytes * es, 4.0 * D * pairs * Hq, s);
  } else {
    attn_delta_kernel<T, D><<<dim3((unsigned)((s_q + 3) / 4), (unsigned)Hq), block, 0, s>>>(
        s_q, s_kv, Hq, grp, dctx, P, V, ws, causal);
    mark("attn_delta", pbytes + qbytes * 4 + kvbytes * es + (double)Hq * s_q * 4,
         2.0 * D * pairs * Hq, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    attn_dq_kernel<T, D, 0><<<gq, block, 0, s>>>(s_q, s_kv, Hq, grp, dctx, P, K, V, nullptr, ws,
                                                  dq, scale, causal);
    mark("attn_dq_mfma", pbytes + qbytes * 8 + 2 * kvbytes * es + (double)Hq * s_q * 4,
         4.0 * D * pairs * Hq, s);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || dv == nullptr) return e;
  constexpr int KB = 16 * (D >= 32 ? 2 : 4);
  attn_dv_kernel<T, D><<<dim3((unsigned)((s_kv + KB - 1) / KB), (unsigned)Hkv), block, 0, s>>>(
      s_q, s_kv, Hq, grp, dctx, P, dv, causal);
  mark("attn_dv_mfma", pbytes + qbytes * 4 + kvbytes * 4, 2.0 * D * pairs * Hq, s);
  return hipGetLastError();
}

template <typename T>
static hipError_t attn_dispatch_d(int64_t s_q, int64_t s_kv, int Hq, int Hkv, int D,
                                  const float* dctx, const void* P, const void* K, const void* V,
                                  const void* ctx, float* dq, float* dv, float scale, int causal,
                                  float* ws, hipStream_t s) {
#define LBP_ATTN_D(DD)                                                                        \
  case DD:                                                                                    \
    return attn_launch<T, DD>(s_q, s_kv, Hq, Hkv, dctx, (const T*)P, (const T*)K, (const T*)V, \
                              (const T*)ctx, dq, dv, scale, causal, ws, s);
  switch (D) {
    LBP_ATTN_D(16)
    LBP_ATTN_D(32)
    LBP_ATTN_D(64)
    LBP_ATTN_D(128)
    default:
      return hipErrorInvalidValue;
  }
#undef LBP_ATTN_D
}

hipError_t launch_attn_bwd(int64_t s_q, int64_t s_kv, int64_t n_heads, int64_t n_kv_heads,
                           int64_t head_dim, const float* dctx, const void* P, const void* K,
                           const void* V, const void* ctx, int dt, float* dq, float* dv,
                           float scale, int causal, void* ws, hipStream_t s) {
  if (s_q == 0) {
    if (dv != nullptr) return launch_fill_zero(s_kv * n_kv_heads * head_dim, dv, s);
    return hipSuccess;
  }
  if (s_q == 1 && dec_attn_fits(s_kv, n_heads, n_kv_heads, head_dim)) {
    DecAttnArgs a{};
    a.s_kv = s_kv;
    a.Hq = (int)n_heads;
    a.grp = (int)(n_heads / n_kv_heads);
    a.dctx = dctx;
    a.P = P;
    a.K = K;
    a.V = V;
    a.ctx = ctx;
    a.dA = (float*)ws;
    a.dq_part = (float*)ws;
    a.dv = dv;
    a.dq = dq;
    a.scale = scale;
    return launch_dec_attn(dt, (int)head_dim, a, s);
  }
  if (dt == F32)
    return attn_dispatch_d<float>(s_q, s_kv, (int)n_heads, (int)n_kv_heads, (int)head_dim, dctx,
                                  P, K, V, ctx, dq, dv, scale, causal, (float*)ws, s);
  return attn_dispatch_d<bf16>(s_q, s_kv, (int)n_heads, (int)n_kv_heads, (int)head_dim, dctx, P,
                               K, V, ctx, dq, dv, scale, causal, (float*)ws, s);
}

}  // namespace lbp
