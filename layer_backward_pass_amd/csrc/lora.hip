// LoRA adapter gradients fused with the AdamW (LoRA+) update.
//
// entrenar wgpu_backward.rs, backward_through_layers, LoRA Q and V blocks,
// and cpu_adamw.  With s = alpha/rank and saved h = x A^T:
//   g  = s dy B       (lora_g_kernel; reads B before it is updated)
//   dB = s dy^T h     -> AdamW on B with lr_b   (lora_db_kernel)
//   dA = g^T x        -> AdamW on A with lr_a   (lora_da_kernel)
//   gnorm_sq += ||dA||^2, per-workgroup partials summed in a fixed order
// The three reductions run over the token rows (dB, dA) or the output
// features (g); all are deterministic.  The rows are split over several
// workgroups and the partial sums reduced in order before the update.
#include "common.h"
#include "kernels.h"

namespace lbp {

constexpr int LR_MAX = 64;   // largest supported rank
constexpr int L_ROWS = 128;  // token rows per partial-sum chunk

// g[i, r] = s sum_o dy[i, o] B[o, r]; one workgroup per token row.
__global__ __launch_bounds__(256) void lora_g_kernel(int64_t out_dim, int rank,
                                                     const float* __restrict__ dy,
                                                     const float* __restrict__ B, float s,
                                                     float* __restrict__ g) {
  __shared__ float red[4][LR_MAX];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int64_t i = blockIdx.x;
  float acc[LR_MAX];
#pragma unroll
  for (int r = 0; r < LR_MAX; ++r) acc[r] = 0.f;
  const float* dyr = dy + i * out_dim;
  for (int64_t o = t; o < out_dim; o += 256) {
    const float d = dyr[o];
    const float* br = B + o * rank;
#pragma unroll
    for (int r = 0; r < LR_MAX; ++r)
      if (r < rank) acc[r] += d * br[r];
  }
#pragma unroll
  for (int r = 0; r < LR_MAX; ++r) {
    if (r < rank) {
      const float v = wave_sum(acc[r]);
      if (lane == 0) red[w][r] = v;
    }
  }
  __syncthreads();
  if (t < rank) g[i * rank + t] = s * (((red[0][t] + red[1][t]) + red[2][t]) + red[3][t]);
}

__device__ __forceinline__ float adamw1(float& p, float gr, float& m, float& v, float lr,
                                        const AdamHP& hp) {
  m = hp.beta1 * m + (1.0f - hp.beta1) * gr;
  v = hp.beta2 * v + (1.0f - hp.beta2) * gr * gr;
  const float mh = m * hp.bc1, vh = v * hp.bc2;
  p -= lr * (mh / (sqrtf(vh) + hp.eps) + hp.wd * p);
  return p;
}

// Partial dB over one chunk of L_ROWS token rows: thread (o, r-group) owns
// outputs (o, r) for r = rg, rg+4, ...  part[chunk][o][r].
__global__ __launch_bounds__(256) void lora_db_part_kernel(int64_t rows, int64_t out_dim,
                                                           int rank,
                                                           const float* __restrict__ dy,
                                                           const void* __restrict__ hv, int hdt,
                                                           float* __restrict__ part) {
  const int t = threadIdx.x;
  const int64_t o = (int64_t)blockIdx.x * 64 + (t & 63);
  const int rg = t >> 6;
  const int64_t i0 = (int64_t)blockIdx.y * L_ROWS;
  const int64_t i1 = min(rows, i0 + L_ROWS);
  float acc[LR_MAX / 4];
#pragma unroll
  for (int j = 0; j < LR_MAX / 4; ++j) acc[j] = 0.f;
  if (o < out_dim) {
    for (int64_t i = i0; i < i1; ++i) {
      const float d = dy[i * out_dim + o];
#pragma unroll
      for (int j = 0; j < LR_MAX / 4; ++j) {
        const int r = rg + 4 * j;
        if (r < rank) {
          const float hh = hdt == F32 ? ((const float*)hv)[i * rank + r]
                                      : bf2f(((const uint16_t*)hv)[i * rank + r]);
          acc[j] += d * hh;
        }
      }
    }
    float* pp = part + ((int64_t)blockIdx.y * out_dim + o) * rank;
#pragma unroll
    for (int j = 0; j < LR_MAX / 4; ++j) {
      const int r = rg + 4 * j;
      if (r < rank) pp[r] = acc[j];
    }
  }
}

// dB = s sum_chunks part, then AdamW on B (lr_b).
__global__ __launch_bounds__(256) void lora_db_update_kernel(int64_t n, int chunks,
                                                             const float* __restrict__ part,
                                                             float s, float* B, float* m,
                                                             float* v, float* grad_b, AdamHP hp) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= n) return;
  float d = 0.f;
  for (int c = 0; c < chunks; ++c) d += part[(int64_t)c * n + e];
  d *= s;
  if (grad_b) grad_b[e] = d;
  float p = B[e], mm = m[e], vv = v[e];
  adamw1(p, d, mm, vv, hp.lr_b, hp);
  B[e] = p;
  m[e] = mm;
  v[e] = vv;
}

// Partial dA over one chunk of token rows: thread (k, r-group) owns (r, k).
template <typename T>
__global__ __launch_bounds__(256) void lora_da_part_kernel(int64_t rows, int64_t in_dim,
                                                           int rank, const float* __restrict__ g,
                                                           const T* __restrict__ x,
                                                           float* __restrict__ part) {
  const int t = threadIdx.x;
  const int64_t k = (int64_t)blockIdx.x * 64 + (t & 63);
  const int rg = t >> 6;
  const int64_t i0 = (int64_t)blockIdx.y * L_ROWS;
  const int64_t i1 = min(rows, i0 + L_ROWS);
  float acc[LR_MAX / 4];
#pragma unroll
  for (int j = 0; j < LR_MAX / 4; ++j) acc[j] = 0.f;
  if (k < in_dim) {
    for (int64_t i = i0; i < i1; ++i) {
      const float xv = Act<T>::ld(x, i * in_dim + k);
#pragma unroll
      for (int j = 0; j < LR_MAX / 4; ++j) {
        const int r = rg + 4 * j;
        if (r < rank) acc[j] += g[i * rank + r] * xv;
      }
    }
#pragma unroll
    for (int j = 0; j < LR_MAX / 4; ++j) {
      const int r = rg + 4 * j;
      if (r < rank) part[((int64_t)blockIdx.y * rank + r) * in_dim + k] = acc[j];
    }
  }
}

// dA = sum_chunks part, AdamW on A (lr_a), per-workgroup sum of dA^2.
__global__ __launch_bounds__(256) void lora_da_update_kernel(int64_t n, int chunks,
                                                             const float* __restrict__ part,
                                                             float* A, float* m, float* v,
                                                             float* grad_a,
                                                             float* __restrict__ sq_part,
                                                             AdamHP hp) {
  __shared__ float red[4];
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  float sq = 0.f;
  if (e < n) {
    float d = 0.f;
    for (int c = 0; c < chunks; ++c) d += part[(int64_t)c * n + e];
    if (grad_a) grad_a[e] = d;
    sq = d * d;
    float p = A[e], mm = m[e], vv = v[e];
    adamw1(p, d, mm, vv, hp.lr_a, hp);
    A[e] = p;
    m[e] = mm;
    v[e] = vv;
  }
  sq = block_sum<4>(sq, red);
  if (threadIdx.x == 0) sq_part[blockIdx.x] = sq;
}

__global__ void lora_gnorm_kernel(int nparts, const float* __restrict__ sq_part,
                                  float* gnorm_sq) {
  if (threadIdx.x != 0) return;
  float s = 0.f;
  for (int i = 0; i < nparts; ++i) s += sq_part[i];
  *gnorm_sq += s;
}

static inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

size_t lora_ws_bytes(int64_t rows, int64_t in_dim, int64_t out_dim, int64_t rank) {
  const int64_t chunks = cdiv(rows, L_ROWS);
  const int64_t g = rows * rank;
  const int64_t pb = chunks * out_dim * rank;
  const int64_t pa = chunks * rank * in_dim;
  const int64_t sq = cdiv(rank * in_dim, 256);
  const int64_t n = g + (pb > pa ? pb : pa) + sq + 64;
  return (size_t)n * sizeof(float);
}

hipError_t launch_lora_adamw(int64_t rows, int64_t in_dim, int64_t out_dim, int64_t rank,
                             const float* dy, const void* x, const void* h, int dt, float* A,
                             float* B, float* m_a, float* v_a, float* m_b, float* v_b,
                             float* grad_a, float* grad_b, float* gnorm_sq, float scaling,
                             const AdamHP& hp, void* ws, hipStream_t s) {
  const int64_t chunks = cdiv(rows, L_ROWS);
  float* g = (float*)ws;
  float* part = g + rows * rank;
  const int64_t pb = chunks * out_dim * rank, pa = chunks * rank * in_dim;
  float* sq = part + (pb > pa ? pb : pa);
  const int r = (int)rank;
  dim3 block(256);
  hipError_t e;
  if (rows > 0) {
    lora_g_kernel<<<dim3((unsigned)rows), block, 0, s>>>(out_dim, r, dy, B, scaling, g);
    mark("lora_g", (double)rows * out_dim * 4 + (double)out_dim * rank * 4 + (double)rows * rank * 4,
         2.0 * rows * out_dim * rank, s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    lora_db_part_kernel<<<dim3((unsigned)cdiv(out_dim, 64), (unsigned)chunks), block, 0, s>>>(
        rows, out_dim, r, dy, h, dt, part);
    mark("lora_db_part", (double)rows * out_dim * 4 + (double)rows * rank * (dt == F32 ? 4 : 2),
         2.0 * rows * out_dim * rank, s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // with no token rows the gradients are zero: a single zero "chunk"
  const int nb = (int)(rows > 0 ? chunks : 0);
  lora_db_update_kernel<<<dim3((unsigned)cdiv(out_dim * rank, 256)), block, 0, s>>>(
      out_dim * rank, nb, part, scaling, B, m_b, v_b, grad_b, hp);
  mark("lora_adamw_b", (double)out_dim * rank * 4 * (6 + (grad_b ? 1 : 0)), 12.0 * out_dim * rank, s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (rows > 0) {
    if (dt == F32)
      lora_da_part_kernel<float><<<dim3((unsigned)cdiv(in_dim, 64), (unsigned)chunks), block, 0,
                                   s>>>(rows, in_dim, r, g, (const float*)x, part);
    else
      lora_da_part_kernel<bf16><<<dim3((unsigned)cdiv(in_dim, 64), (unsigned)chunks), block, 0,
                                  s>>>(rows, in_dim, r, g, (const bf16*)x, part);
    mark("lora_da_part", (double)rows * in_dim * (dt == F32 ? 4 : 2) + (double)rows * rank * 4,
         2.0 * rows * in_dim * rank, s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int nsq = (int)cdiv(rank * in_dim, 256);
  lora_da_update_kernel<<<dim3((unsigned)nsq), block, 0, s>>>(rank * in_dim, nb, part, A, m_a,
                                                              v_a, grad_a, sq, hp);
  mark("lora_adamw_a", (double)rank * in_dim * 4 * (6 + (grad_a ? 1 : 0)), 14.0 * rank * in_dim, s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (gnorm_sq != nullptr) {
    lora_gnorm_kernel<<<dim3(1), dim3(64), 0, s>>>(nsq, sq, gnorm_sq);
    mark("lora_gnorm", 8, (double)nsq, s);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace lbp
