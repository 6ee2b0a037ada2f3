// The lm_head backward that feeds the layer stack its upstream gradient
// ([ENT] wgpu_backward.rs: gradients flow from lm_head through the layers;
// WgpuModelState keeps the lm_head weight [vocab, hidden] with AdamW moments).
// With logits z = h W^T saved by the forward and n the rows whose label is a
// vocabulary index (other rows are ignored):
//   loss        = (1/n) sum_s (logsumexp(z_s) - z_s[label_s])
//   dlogits     = (softmax(z) - onehot(labels)) / n        [rows, vocab]
//   grad_hidden = dlogits W          (W before the update)  [rows, hidden]
//   dW          = dlogits^T h, then AdamW on W              [vocab, hidden]
// Kernels, in stream order:
//   xent_count_kernel n, the labelled rows (one workgroup)
//   xent_bwd_kernel   a row at a time per workgroup (1024 threads, one
//                     workgroup per CU, rows in turn): row max and sum of
//                     exponentials in one pass (rescaled as the max grows),
//                     then dlogits and the row's loss term; bandwidth-bound
//                     (logits read twice from the fabric, the two reads of a
//                     row close together: 256 rows in flight, 155 MB at
//                     vocabulary 151936)
//   xent_loss_kernel  the row terms summed in a fixed order, divided by n
//   grad_hidden       launch_gemm (fp32 MFMA, split-K over the vocabulary)
//   dW + AdamW        launch_gemm_at_adamw: dlogits read transposed in place,
//                     W, m, v updated as each tile is stored
// No float atomics anywhere: the results are bitwise reproducible.
#include "common.h"
#include "kernels.h"

namespace lbp {

namespace {

constexpr int XT = 256;   // threads of the label count and the loss reduction
constexpr int XB = 1024;  // threads per row of xent_bwd_kernel
constexpr int XB_WG = 256;  // its workgroups (rows beyond run in turn)

// Merge of two (max, sum of exp(z - max)) pairs.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float n = fmaxf(m, m2);
  if (n == -INFINITY) return;  // both empty
  s = s * expf(m - n) + s2 * expf(m2 - n);
  m = n;
}

// Number of labels in [0, vocab) among labels[0, rows), by every thread of
// a workgroup of NT threads (the same value everywhere).
template <int NT>
__device__ int count_labelled(int64_t rows, int64_t vocab, const int32_t* __restrict__ labels,
                              int* red) {
  int c = 0;
  for (int64_t i = threadIdx.x; i < rows; i += NT) {
    const int32_t l = labels[i];
    c += (l >= 0 && l < vocab) ? 1 : 0;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) c += __shfl_xor(c, o);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = c;
  __syncthreads();
  int n = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) n += red[i];
  return n;
}

}  // namespace

__global__ __launch_bounds__(XB) void xent_bwd_kernel(int64_t rows, int64_t vocab,
                                                      const float* __restrict__ logits,
                                                      const int32_t* __restrict__ labels,
                                                      const int* __restrict__ nlab,
                                                      float* __restrict__ dlogits,
                                                      float* __restrict__ rowloss) {
  constexpr int NW = XB / 64;
  __shared__ float rm[NW], rs[NW];
  const int t = threadIdx.x;
  const int n = *nlab;
  const int64_t q = vocab / 4;
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    const int32_t lab = labels[row];
    const bool ok = lab >= 0 && lab < vocab;
    const float4* z4 = reinterpret_cast<const float4*>(logits + row * vocab);
    float4* d4 = reinterpret_cast<float4*>(dlogits + row * vocab);
    // pass 1: running max and sum of exp(z - max), four float4 loads in flight
    float m = -INFINITY, s = 0.f;
    auto take = [&](const float4& z) {
      const float zm = fmaxf(fmaxf(z.x, z.y), fmaxf(z.z, z.w));
      const float nm = fmaxf(m, zm);
      if (nm == -INFINITY) return;  // nothing finite yet
      s = s * expf(m - nm) + (expf(z.x - nm) + expf(z.y - nm)) +
          (expf(z.z - nm) + expf(z.w - nm));
      m = nm;
    };
    int64_t i = t;
    for (; i + 3 * XB < q; i += 4 * XB) {
      const float4 a = z4[i], b = z4[i + XB], c = z4[i + 2 * XB], d = z4[i + 3 * XB];
      take(a);
      take(b);
      take(c);
      take(d);
    }
    for (; i < q; i += XB) take(z4[i]);
    // the workgroup's pairs merged in a fixed pattern
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float m2 = __shfl_xor(m, o), s2 = __shfl_xor(s, o);
      lse_merge(m, s, m2, s2);
    }
    __syncthreads();  // the previous row's merge has read rm, rs
    if ((t & 63) == 0) {
      rm[t >> 6] = m;
      rs[t >> 6] = s;
    }
    __syncthreads();
    m = rm[0];
    s = rs[0];
#pragma unroll
    for (int wv = 1; wv < NW; ++wv) lse_merge(m, s, rm[wv], rs[wv]);
    const float lse = m + logf(s);
    // pass 2: dlogits = (exp(z - lse) - [v == label]) / n, zero for an ignored row
    const float scale = ok ? 1.0f / (float)n : 0.f;
    auto grad = [&](const float4& z, int64_t j) {
      float4 g;
      g.x = (expf(z.x - lse) - (4 * j == lab ? 1.f : 0.f)) * scale;
      g.y = (expf(z.y - lse) - (4 * j + 1 == lab ? 1.f : 0.f)) * scale;
      g.z = (expf(z.z - lse) - (4 * j + 2 == lab ? 1.f : 0.f)) * scale;
      g.w = (expf(z.w - lse) - (4 * j + 3 == lab ? 1.f : 0.f)) * scale;
      d4[j] = g;
    };
    for (i = t; i + 3 * XB < q; i += 4 * XB) {
      const float4 a = z4[i], b = z4[i + XB], c = z4[i + 2 * XB], d = z4[i + 3 * XB];
      grad(a, i);
      grad(b, i + XB);
      grad(c, i + 2 * XB);
      grad(d, i + 3 * XB);
    }
    for (; i < q; i += XB) grad(z4[i], i);
    if (t == 0) rowloss[row] = ok ? lse - logits[row * vocab + lab] : 0.f;
  }
}

// n = the number of rows whose label is a vocabulary index, counted once.
__global__ __launch_bounds__(XT) void xent_count_kernel(int64_t rows, int64_t vocab,
                                                        const int32_t* __restrict__ labels,
                                                        int* __restrict__ nlab) {
  __shared__ int rc[XT / 64];
  const int n = count_labelled<XT>(rows, vocab, labels, rc);
  if (threadIdx.x == 0) *nlab = n;
}

// loss = (sum of the row terms in a fixed order) / n; 0 when no row is labelled.
__global__ __launch_bounds__(XT) void xent_loss_kernel(int64_t rows,
                                                       const int* __restrict__ nlab,
                                                       const float* __restrict__ rowloss,
                                                       float* __restrict__ loss) {
  __shared__ float rf[4];
  const int t = threadIdx.x;
  const int n = *nlab;
  float a = 0.f;
  for (int64_t i = t; i < rows; i += XT) a += rowloss[i];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) a += __shfl_xor(a, o);
  if ((t & 63) == 0) rf[t >> 6] = a;
  __syncthreads();
  if (t == 0) loss[0] = n > 0 ? ((rf[0] + rf[1]) + (rf[2] + rf[3])) / (float)n : 0.f;
}

size_t lm_head_ws_bytes(int64_t rows, int64_t hidden, int64_t vocab) {
  auto up = [](size_t b) { return (b + 255) / 256 * 256; };
  return up((size_t)rows * vocab * 4) + up((size_t)rows * 4) + 256 +
         up(gemm_partial_bytes(rows, hidden, vocab, F32, F32));
}

hipError_t launch_lm_head_bwd(int64_t rows, int64_t hidden, int64_t vocab, const float* h,
                              const float* logits, const int32_t* labels, float* w, float* m,
                              float* v, float* grad_hidden, float* loss, float* grad_w,
                              const AdamHP& hp, void* ws, hipStream_t s) {
  if (vocab % 4 != 0 || hidden % 8 != 0) return hipErrorInvalidValue;
  char* p = (char*)ws;
  float* dlogits = (float*)p;
  p += ((size_t)rows * vocab * 4 + 255) / 256 * 256;
  float* rowloss = (float*)p;
  p += ((size_t)rows * 4 + 255) / 256 * 256;
  int* nlab = (int*)p;
  p += 256;
  float* partials = (float*)p;
  hipError_t e;
  if (!dry_run()) {
    xent_count_kernel<<<dim3(1), dim3(XT), 0, s>>>(rows, vocab, labels, nlab);
    mark("xent_count", rows * 4.0, 0, s);
    if (rows > 0) {
      const int64_t wg = rows < XB_WG ? rows : XB_WG;
      xent_bwd_kernel<<<dim3((unsigned)wg), dim3(XB), 0, s>>>(rows, vocab, logits, labels,
                                                              nlab, dlogits, rowloss);
      // logits read and dlogits written once; the second read of the
      // logits, the labels read again and the row terms are the kernel's own
      mark("xent_bwd", (double)rows * vocab * 8, 0, s, (double)rows * vocab * 4 + rows * 8.0);
    }
    xent_loss_kernel<<<dim3(1), dim3(XT), 0, s>>>(rows, nlab, rowloss, loss);
    mark("xent_loss", 4, 0, s, rows * 4.0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // grad_hidden = dlogits W (W as the forward used it: before the update)
  if ((e = launch_gemm(rows, hidden, vocab, dlogits, F32, vocab, w, nullptr, vocab, F32, hidden,
                       grad_hidden, hidden, partials, s)) != hipSuccess)
    return e;
  // dW = dlogits^T h and AdamW on W
  AdamEpi ad;
  ad.w = w;
  ad.m = m;
  ad.v = v;
  ad.grad = grad_w;
  ad.hp = hp;
  ad.lr = hp.lr_a;
  return launch_gemm_at_adamw(vocab, hidden, rows, dlogits, vocab, h, hidden, ad, s);
}

}  // namespace lbp
