// Transposed products of the backward pass, dX = dY W with W [out, in]
// row-major: C[M,N] = A[M,K] B[K,N], A = gradient rows, B = weight.
//   * fp32 weights: v_mfma_f32_16x16x4_f32, 128x128x16 workgroup tiles
//   * bf16 weights: v_mfma_f32_16x16x32_bf16, 128x128x32 tiles, the
//     gradient operand rounded to bf16 when staged in LDS
// Split-K partial sums go to caller scratch and are reduced in a fixed
// order (no float atomics), so results are bitwise reproducible.
#include "common.h"
#include "kernels.h"

namespace lbp {

constexpr int GBM = 128, GBN = 128;

// Output tile of the 16x16 MFMA accumulators: lane l holds rows 4*(l/16)+v
// (v = 0..3) of column l%16.
__device__ __forceinline__ void store_tile(float* C, int64_t ldc, int64_t M, int64_t N,
                                           int64_t row0, int64_t col0, const floatx4 (&acc)[4][4]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int fi = 0; fi < 4; ++fi)
#pragma unroll
    for (int fj = 0; fj < 4; ++fj) {
      const int64_t c = col0 + fj * 16 + (lane & 15);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t r = row0 + fi * 16 + 4 * (lane >> 4) + v;
        if (r < M && c < N) C[r * ldc + c] = acc[fi][fj][v];
      }
    }
}

// ---------------------------------------------------------------------------
// fp32 GEMM.  4 waves in a 2x2 grid, each wave 64x64 = 4x4 MFMA tiles.
// LDS holds the A tile k-major (As[k][m]) and the B tile as stored
// (Bs[k][n]); row stride 144 floats puts lane groups 16 banks apart.
constexpr int F_BK = 16, F_LD = GBM + 16;

template <typename TA>
__global__ __launch_bounds__(256) void gemm_f32_kernel(int64_t M, int64_t N, int64_t K,
                                                       const TA* __restrict__ A, int64_t lda,
                                                       const float* __restrict__ B1,
                                                       const float* __restrict__ B2, int64_t K1,
                                                       int64_t ldb, float* __restrict__ C,
                                                       int64_t ldc, int64_t kps,
                                                       int64_t split_stride) {
  __shared__ float As[F_BK][F_LD];
  __shared__ float Bs[F_BK][F_LD];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int64_t bm = (int64_t)blockIdx.y * GBM, bn = (int64_t)blockIdx.x * GBN;
  const int64_t kbeg = (int64_t)blockIdx.z * kps;
  const int64_t kend = min(K, kbeg + kps);
  C += (int64_t)blockIdx.z * split_stride;
  const int wm = (w >> 1) * 64, wn = (w & 1) * 64;

  // global->register staging: A 2 x float4 (rows t/4 and t/4+64, k (t%4)*4),
  // B 2 x float4 (k rows t/32 and t/32+8, n (t%32)*4)
  float4 ra[2], rb[2];
  auto load = [&](int64_t k0) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int64_t m = bm + (t >> 2) + 64 * r;
      const int64_t k = k0 + (t & 3) * 4;
      ra[r] = (m < M && k < kend) ? Act<TA>::ld4(A, m * lda + k) : make_float4(0, 0, 0, 0);
      const int64_t kb = k0 + (t >> 5) + 8 * r;
      const int64_t n = bn + (t & 31) * 4;
      if (kb < kend && n < N) {
        const float* bp = kb < K1 ? B1 + kb * ldb : B2 + (kb - K1) * ldb;
        rb[r] = *reinterpret_cast<const float4*>(bp + n);
      } else {
        rb[r] = make_float4(0, 0, 0, 0);
      }
    }
  };
  floatx4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0, 0, 0, 0};

  if (kbeg < kend) load(kbeg);
  for (int64_t k0 = kbeg; k0 < kend; k0 += F_BK) {
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int m = (t >> 2) + 64 * r, k = (t & 3) * 4;
      As[k + 0][m] = ra[r].x;
      As[k + 1][m] = ra[r].y;
      As[k + 2][m] = ra[r].z;
      As[k + 3][m] = ra[r].w;
      *reinterpret_cast<float4*>(&Bs[(t >> 5) + 8 * r][(t & 31) * 4]) = rb[r];
    }
    __syncthreads();
    if (k0 + F_BK < kend) load(k0 + F_BK);
#pragma unroll
    for (int kk = 0; kk < F_BK; kk += 4) {
      float a[4], b[4];
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        a[f] = As[kk + (lane >> 4)][wm + f * 16 + (lane & 15)];
        b[f] = Bs[kk + (lane >> 4)][wn + f * 16 + (lane & 15)];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x4(a[i], b[j], acc[i][j]);
    }
  }
  store_tile(C, ldc, M, N, bm + wm, bn + wn, acc);
}

// ---------------------------------------------------------------------------
// bf16 GEMM.  Same wave layout; BK = 32.  A tile stored As[m][k] (bf16, k
// contiguous: one 16-byte read per MFMA operand); the B tile is transposed
// on its way into LDS (Bs[n][k]) by pairing consecutive k rows into 32-bit
// words.  Row stride 40 bf16 (80 bytes) keeps 16-byte alignment.
constexpr int H_BK = 32, H_LD = H_BK + 8;

template <typename TA>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(int64_t M, int64_t N, int64_t K,
                                                        const TA* __restrict__ A, int64_t lda,
                                                        const uint16_t* __restrict__ B1,
                                                        const uint16_t* __restrict__ B2,
                                                        int64_t K1, int64_t ldb,
                                                        float* __restrict__ C, int64_t ldc,
                                                        int64_t kps, int64_t split_stride) {
  __shared__ __attribute__((aligned(16))) uint16_t As[GBM][H_LD];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[GBN][H_LD];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int64_t bm = (int64_t)blockIdx.y * GBM, bn = (int64_t)blockIdx.x * GBN;
  const int64_t kbeg = (int64_t)blockIdx.z * kps;
  const int64_t kend = min(K, kbeg + kps);
  C += (int64_t)blockIdx.z * split_stride;
  const int wm = (w >> 1) * 64, wn = (w & 1) * 64;

  // A: rows t/4 and t/4+64, 8 consecutive k at (t%4)*8 -> one uint4 of bf16
  // B: k rows 2*(t/16), 2*(t/16)+1, 8 consecutive n at (t%16)*8
  uint4 ra[2];
  uint4 rb0, rb1;
  auto load = [&](int64_t k0) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int64_t m = bm + (t >> 2) + 64 * r;
      const int64_t k = k0 + (t & 3) * 8;
      if (m < M && k < kend) {
        if constexpr (sizeof(TA) == 4) {
          const float4 x = *reinterpret_cast<const float4*>((const float*)A + m * lda + k);
          const float4 y = *reinterpret_cast<const float4*>((const float*)A + m * lda + k + 4);
          ra[r].x = (uint32_t)f2bf(x.x) | ((uint32_t)f2bf(x.y) << 16);
          ra[r].y = (uint32_t)f2bf(x.z) | ((uint32_t)f2bf(x.w) << 16);
          ra[r].z = (uint32_t)f2bf(y.x) | ((uint32_t)f2bf(y.y) << 16);
          ra[r].w = (uint32_t)f2bf(y.z) | ((uint32_t)f2bf(y.w) << 16);
        } else {
          ra[r] = *reinterpret_cast<const uint4*>((const uint16_t*)A + m * lda + k);
        }
      } else {
        ra[r] = make_uint4(0, 0, 0, 0);
      }
    }
    const int64_t kb = k0 + 2 * (t >> 4);
    const int64_t n = bn + (t & 15) * 8;
    auto brow = [&](int64_t k) -> uint4 {
      if (k < kend && n < N) {
        const uint16_t* bp = k < K1 ? B1 + k * ldb : B2 + (k - K1) * ldb;
        return *reinterpret_cast<const uint4*>(bp + n);
      }
      return make_uint4(0, 0, 0, 0);
    };
    rb0 = brow(kb);
    rb1 = brow(kb + 1);
  };
  floatx4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0, 0, 0, 0};

  if (kbeg < kend) load(kbeg);
  for (int64_t k0 = kbeg; k0 < kend; k0 += H_BK) {
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 2; ++r)
      *reinterpret_cast<uint4*>(&As[(t >> 2) + 64 * r][(t & 3) * 8]) = ra[r];
    {
      const int kp = 2 * (t >> 4);
      const int n0 = (t & 15) * 8;
      const uint32_t a[4] = {rb0.x, rb0.y, rb0.z, rb0.w};
      const uint32_t b[4] = {rb1.x, rb1.y, rb1.z, rb1.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t lo = (a[i] & 0xffffu) | (b[i] << 16);
        const uint32_t hi = (a[i] >> 16) | (b[i] & 0xffff0000u);
        *reinterpret_cast<uint32_t*>(&Bs[n0 + 2 * i][kp]) = lo;
        *reinterpret_cast<uint32_t*>(&Bs[n0 + 2 * i + 1][kp]) = hi;
      }
    }
    __syncthreads();
    if (k0 + H_BK < kend) load(k0 + H_BK);
    ushortx8 a[4], b[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      a[f] = *reinterpret_cast<const ushortx8*>(&As[wm + f * 16 + (lane & 15)][8 * (lane >> 4)]);
      b[f] = *reinterpret_cast<const ushortx8*>(&Bs[wn + f * 16 + (lane & 15)][8 * (lane >> 4)]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32bf16(a[i], b[j], acc[i][j]);
  }
  store_tile(C, ldc, M, N, bm + wm, bn + wn, acc);
}

// ---------------------------------------------------------------------------
// Fixed-order reduction of split-K partials: C[m, n] = sum_s P[s, m, n].
__global__ __launch_bounds__(256) void splitk_reduce_kernel(int64_t M, int64_t N, int splits,
                                                            const float* __restrict__ P,
                                                            float* __restrict__ C, int64_t ldc) {
  const int64_t q = N / 4;
  const int64_t total = M * q;
  const int64_t stride = M * N;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = t / q, n = (t - m * q) * 4;
    const float* p = P + m * N + n;
    float4 s = *reinterpret_cast<const float4*>(p);
    for (int i = 1; i < splits; ++i) {
      const float4 v = *reinterpret_cast<const float4*>(p + i * stride);
      s.x += v.x;
      s.y += v.y;
      s.z += v.z;
      s.w += v.w;
    }
    *reinterpret_cast<float4*>(C + m * ldc + n) = s;
  }
}

static inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

int gemm_splits(int64_t M, int64_t N, int64_t K, int b_dt) {
  const int64_t tiles = cdiv(M, GBM) * cdiv(N, GBN);
  int s = 1;
  while (tiles * s < 256 && K / (2 * s) >= 256 && s < 16) s *= 2;
  (void)b_dt;
  return s;
}

size_t gemm_partial_bytes(int64_t M, int64_t N, int64_t K, int b_dt) {
  const int s = gemm_splits(M, N, K, b_dt);
  return s > 1 ? (size_t)s * M * N * sizeof(float) : 0;
}

hipError_t launch_gemm(int64_t M, int64_t N, int64_t K, const void* A, int a_dt, int64_t lda,
                       const void* B1, const void* B2, int64_t K1, int b_dt, int64_t ldb,
                       float* C, int64_t ldc, float* partials, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  const int splits = gemm_splits(M, N, K, b_dt);
  const int64_t kps = cdiv(cdiv(K, splits), 64) * 64;
  const int nsp = (int)cdiv(K, kps);
  float* out = nsp > 1 ? partials : C;
  const int64_t ldo = nsp > 1 ? N : ldc;
  const int64_t sstride = nsp > 1 ? M * N : 0;
  if (B2 == nullptr) {
    B2 = B1;
    K1 = K;
  }
  dim3 grid((unsigned)cdiv(N, GBN), (unsigned)cdiv(M, GBM), (unsigned)nsp), block(256);
  if (b_dt == F32) {
    gemm_f32_kernel<float><<<grid, block, 0, s>>>(M, N, K, (const float*)A, lda,
                                                  (const float*)B1, (const float*)B2, K1, ldb,
                                                  out, ldo, kps, sstride);
  } else if (a_dt == F32) {
    gemm_bf16_kernel<float><<<grid, block, 0, s>>>(M, N, K, (const float*)A, lda,
                                                   (const uint16_t*)B1, (const uint16_t*)B2, K1,
                                                   ldb, out, ldo, kps, sstride);
  } else {
    gemm_bf16_kernel<uint16_t><<<grid, block, 0, s>>>(M, N, K, (const uint16_t*)A, lda,
                                                      (const uint16_t*)B1, (const uint16_t*)B2,
                                                      K1, ldb, out, ldo, kps, sstride);
  }
  hipError_t e = hipGetLastError();
  mark(b_dt == F32 ? "gemm_f32_mfma" : "gemm_bf16_mfma",
       (double)M * K * (a_dt == F32 ? 4 : 2) + (double)K * N * (b_dt == F32 ? 4 : 2) +
           (double)M * N * 4,
       2.0 * M * N * K, s);
  if (e != hipSuccess || nsp == 1) return e;
  int64_t blocks = cdiv(M * (N / 4), 256);
  if (blocks > 4096) blocks = 4096;
  splitk_reduce_kernel<<<dim3((unsigned)blocks), block, 0, s>>>(M, N, nsp, partials, C, ldc);
  mark("splitk_reduce", 0, 0, s);
  return hipGetLastError();
}

}  // namespace lbp
