// LoRA adapter gradients fused with the AdamW (LoRA+) update.
//
// entrenar wgpu_backward.rs, backward_through_layers, LoRA Q and V blocks,
// and cpu_adamw.  With s = alpha/rank and saved h = x A^T:
//   g  = s dy B       [rows, rank]  (B read before it is updated)
//   dB = s dy^T h     [out, rank]   -> AdamW on B with lr_b
//   dA = g^T x        [rank, in]    -> AdamW on A with lr_a
//   gnorm_sq += ||dA||^2
//
// Two MFMA passes carry the work.  lora_dy_kernel reads each element of dy
// once from HBM and forms both g (contraction over the output features) and
// dB (contraction over the token rows); lora_da_kernel reads x once for dA.
// Each workgroup owns 256 columns (4 waves x 64) and one slice of the rows;
// the per-slice partial sums are reduced in a fixed order by the update
// kernels, so every result is deterministic.  Ranks are padded to a multiple
// of 16 (the MFMA tile width) with zeros.
#include "common.h"
#include "kernels.h"

namespace lbp {

constexpr int LW_COLS = 64;    // columns per wave
constexpr int LG_COLS = 256;   // columns per workgroup
constexpr int L_TARGET = 256;  // workgroups aimed for per pass

static inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Four consecutive floats of row `row` starting at column `c`, zero outside
// [0, rows) x [0, ncol).  VEC: ncol % 4 == 0 and c % 4 == 0, one 16-byte load.
template <bool VEC>
__device__ __forceinline__ float4 ld4f(const float* p, int64_t row, int64_t rows, int64_t c,
                                       int64_t ncol) {
  float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
  if (row >= rows) return r;
  const float* q = p + row * ncol + c;
  if (VEC) {
    if (c < ncol) r = *reinterpret_cast<const float4*>(q);
  } else {
    if (c < ncol) r.x = q[0];
    if (c + 1 < ncol) r.y = q[1];
    if (c + 2 < ncol) r.z = q[2];
    if (c + 3 < ncol) r.w = q[3];
  }
  return r;
}

__device__ __forceinline__ float f4get(const float4& v, int j) {
  return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
}

__device__ __forceinline__ float ld_h(const void* h, int hdt, int64_t e) {
  return hdt == F32 ? ((const float*)h)[e] : bf2f(((const uint16_t*)h)[e]);
}

// One pass over dy [rows, out].  Wave w of workgroup (bx, by) owns the output
// features o0 .. o0+63 (o0 = 256 bx + 64 w) and the row slice by.
//   g part:  gpart[bx][i][r]  = sum_{o in workgroup} dy[i,o] B[o,r]
//   dB part: dbpart[by][o][r] = sum_{i in slice} dy[i,o] h[i,r]
// MFMA 16x16x4 f32 layouts: operand lane l holds (row l%16, k l/16); result
// lane l, register v holds (row 4(l/16)+v, col l%16).
// g:  rows = 16 tokens, k = features; lane loads dy[i0+l%16][o0+16c+4(l/16)+j]
// dB: rows = 16 features (tile j: o0 + 4m + j), k = tokens; lane loads
//     dy[i0+4q+l/16][o0+4(l%16)+j].
template <int RB, bool VEC, typename TH>
__global__ __launch_bounds__(256) void lora_dy_kernel(int64_t rows, int64_t out_dim, int rank,
                                                      int64_t rs, const float* __restrict__ dy,
                                                      const TH* __restrict__ h,
                                                      const float* __restrict__ Bm,
                                                      float* __restrict__ gpart,
                                                      float* __restrict__ dbpart) {
  constexpr int RP = 16 * RB;
  __shared__ float gs[4][16][RP + 1];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int l16 = lane & 15, l4 = lane >> 4;
  const int64_t o0 = (int64_t)blockIdx.x * LG_COLS + w * LW_COLS;
  const int64_t i_beg = (int64_t)blockIdx.y * rs;
  const int64_t i_end = min(rows, i_beg + rs);

  float bv[4][4][RB];  // B operand of g: B[o0+16c+4 l4+j][16b+l16]
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        const int64_t o = o0 + 16 * c + 4 * l4 + j;
        const int r = 16 * b + l16;
        bv[c][j][b] = (o < out_dim && r < rank) ? Bm[o * rank + r] : 0.f;
      }
  floatx4 accb[4][RB];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int b = 0; b < RB; ++b) accb[j][b] = floatx4{0.f, 0.f, 0.f, 0.f};

  // The slice's rows of dy and h as buffer ranges (bounds are offsets; rows
  // past the slice read 0), and two 16-row steps in flight: the next step's
  // loads are issued before the current one is multiplied.
  const int64_t nrow = i_end - i_beg;
  const brsrc_t rdy = make_brsrc(dy + i_beg * out_dim, nrow > 0 ? (uint32_t)(nrow * out_dim * 4) : 0u);
  const brsrc_t rh = make_brsrc(h + i_beg * rank, nrow > 0 ? (uint32_t)(nrow * rank * sizeof(TH)) : 0u);
  struct Step {
    float4 ga[4], da[4];
    float hv[4][RB];
  };
  auto ld4 = [&](int64_t row, int64_t c) -> float4 {
    const bool rok = row < i_end;
    const int64_t e = (row - i_beg) * out_dim + c;
    if (VEC) return bload_f4(rdy, (rok && c < out_dim) ? (uint32_t)(e * 4) : BUF_OOB);
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      v[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
          rdy, (rok && c + j < out_dim) ? (int)((e + j) * 4) : (int)BUF_OOB, 0, 0));
    return make_float4(v[0], v[1], v[2], v[3]);
  };
  auto fetch = [&](Step& S, int64_t i0) {
#pragma unroll
    for (int c = 0; c < 4; ++c) S.ga[c] = ld4(i0 + l16, o0 + 16 * c + 4 * l4);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t i = i0 + 4 * q + l4;
      S.da[q] = ld4(i, o0 + 4 * l16);
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        const int r = 16 * b + l16;
        const uint32_t off = (i < i_end && r < rank) ? (uint32_t)(((i - i_beg) * rank + r) * sizeof(TH))
                                                     : BUF_OOB;
        if (sizeof(TH) == 4)
          S.hv[q][b] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rh, (int)off, 0, 0));
        else
          S.hv[q][b] = bf2f(__builtin_amdgcn_raw_buffer_load_b16(rh, (int)off, 0, 0));
      }
    }
  };
  auto step = [&](const Step& S, int64_t i0) {
    floatx4 accg[RB];
#pragma unroll
    for (int b = 0; b < RB; ++b) accg[b] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int b = 0; b < RB; ++b) accg[b] = mfma16x16x4(f4get(S.ga[c], j), bv[c][j][b], accg[b]);
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int b = 0; b < RB; ++b) accb[j][b] = mfma16x16x4(f4get(S.da[q], j), S.hv[q][b], accb[j][b]);
    // sum the four waves' g tiles in a fixed order
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v) gs[w][4 * l4 + v][16 * b + l16] = accg[b][v];
    __syncthreads();
    for (int e = t; e < 16 * RP; e += 256) {
      const int row = e / RP, col = e % RP;
      if (i0 + row < i_end)
        gpart[((int64_t)blockIdx.x * rows + i0 + row) * RP + col] =
            ((gs[0][row][col] + gs[1][row][col]) + gs[2][row][col]) + gs[3][row][col];
    }
    __syncthreads();
  };
  // (an odd step count ends with a step of zeros, whose rows are not stored)
  Step s0, s1;
  fetch(s0, i_beg);
  fetch(s1, i_beg + 16);
  for (int64_t i0 = i_beg; i0 < i_end; i0 += 32) {
    step(s0, i0);
    fetch(s0, i0 + 32);
    step(s1, i0 + 16);
    fetch(s1, i0 + 48);
  }
  // dB tile j, register v: feature o0 + 4(4 l4 + v) + j, rank 16b + l16
  float* dp = dbpart + (int64_t)blockIdx.y * out_dim * rank;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t o = o0 + 4 * (4 * l4 + v) + j;
        const int r = 16 * b + l16;
        if (o < out_dim && r < rank) dp[o * rank + r] = accb[j][b][v];
      }
}

// One pass over x [rows, in]: dapart[by][r][k] = sum_{i in slice} g[i,r] x[i,k].
// Result rows = rank (16 per block b), cols = features (tile j: k0 + 4n + j),
// k = tokens.  g is [rows, 16 RB], already scaled and zero-padded.  Two
// 16-row steps in flight, loads through buffer ranges (in_dim % 8 == 0, so
// a 4-feature chunk is whole).
template <int RB, typename T>
__global__ __launch_bounds__(256) void lora_da_kernel(int64_t rows, int64_t in_dim, int rank,
                                                      int64_t rs, const float* __restrict__ g,
                                                      const T* __restrict__ x,
                                                      float* __restrict__ dapart) {
  constexpr int RP = 16 * RB;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int l16 = lane & 15, l4 = lane >> 4;
  const int64_t k0 = (int64_t)blockIdx.x * LG_COLS + w * LW_COLS;
  const int64_t i_beg = (int64_t)blockIdx.y * rs;
  const int64_t i_end = min(rows, i_beg + rs);
  const int64_t nrow = i_end - i_beg;
  const brsrc_t rx = make_brsrc(x + i_beg * in_dim, nrow > 0 ? (uint32_t)(nrow * in_dim * sizeof(T)) : 0u);
  const brsrc_t rg = make_brsrc(g + i_beg * RP, nrow > 0 ? (uint32_t)(nrow * RP * 4) : 0u);
  floatx4 acc[4][RB];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int b = 0; b < RB; ++b) acc[j][b] = floatx4{0.f, 0.f, 0.f, 0.f};
  struct Step {
    typename BufVec<T>::raw xa[4];
    float gv[4][RB];
  };
  auto fetch = [&](Step& S, int64_t i0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t i = i0 + 4 * q + l4;
      const int64_t c = k0 + 4 * l16;
      const bool ok = i < i_end;
      S.xa[q] = BufVec<T>::load(rx, (ok && c < in_dim) ? (uint32_t)(((i - i_beg) * in_dim + c) * sizeof(T)) : BUF_OOB);
#pragma unroll
      for (int b = 0; b < RB; ++b)
        S.gv[q][b] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            rg, ok ? (int)(((i - i_beg) * RP + 16 * b + l16) * 4) : (int)BUF_OOB, 0, 0));
    }
  };
  auto step = [&](const Step& S) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 xf = BufVec<T>::cvt(S.xa[q]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int b = 0; b < RB; ++b) acc[j][b] = mfma16x16x4(S.gv[q][b], f4get(xf, j), acc[j][b]);
    }
  };
  Step s0, s1;
  fetch(s0, i_beg);
  fetch(s1, i_beg + 16);
  for (int64_t i0 = i_beg; i0 < i_end; i0 += 32) {
    step(s0);
    fetch(s0, i0 + 32);
    step(s1);
    fetch(s1, i0 + 48);
  }
  // tile j, register v: rank 16b + 4 l4 + v, feature k0 + 4 l16 + j
  float* dp = dapart + (int64_t)blockIdx.y * rank * in_dim;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = 16 * b + 4 * l4 + v;
        const int64_t k = k0 + 4 * l16 + j;
        if (r < rank && k < in_dim) dp[(int64_t)r * in_dim + k] = acc[j][b][v];
      }
}

__device__ __forceinline__ void adamw1(float& p, float gr, float& m, float& v, float lr,
                                       const AdamHP& hp) {
  m = hp.beta1 * m + (1.0f - hp.beta1) * gr;
  v = hp.beta2 * v + (1.0f - hp.beta2) * gr * gr;
  const float mh = m * hp.bc1, vh = v * hp.bc2;
  p -= lr * (mh / (sqrtf(vh) + hp.eps) + hp.wd * p);
}

// Elements [0, nb): dB = s sum_slices dbpart, then AdamW on B (lr_b).
// Elements [nb, nb + ng): g = s sum_groups gpart (ng = rows * 16 RB).
// sum_{c < n} p[c * stride] in index order, 16 loads in flight at a time
__device__ __forceinline__ float sum_strided(const float* __restrict__ p, int n, int64_t stride) {
  float d = 0.f;
  int c = 0;
  for (; c + 16 <= n; c += 16) {
    float v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = p[(int64_t)(c + u) * stride];
#pragma unroll
    for (int u = 0; u < 16; ++u) d += v[u];
  }
  for (; c < n; ++c) d += p[(int64_t)c * stride];
  return d;
}

__global__ __launch_bounds__(256) void lora_b_update_kernel(int64_t nb, int slices,
                                                            const float* __restrict__ dbpart,
                                                            int64_t ng, int groups,
                                                            const float* __restrict__ gpart,
                                                            float* __restrict__ g, float s,
                                                            float* B, float* m, float* v,
                                                            float* grad_b, AdamHP hp) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e < nb) {
    float d = sum_strided(dbpart + e, slices, nb);
    d *= s;
    if (grad_b) grad_b[e] = d;
    float p = B[e], mm = m[e], vv = v[e];
    adamw1(p, d, mm, vv, hp.lr_b, hp);
    B[e] = p;
    m[e] = mm;
    v[e] = vv;
  } else if (e < nb + ng) {
    const int64_t f = e - nb;
    g[f] = s * sum_strided(gpart + f, groups, ng);
  }
}

// dA = sum_slices dapart, AdamW on A (lr_a), per-workgroup sum of dA^2.
__global__ __launch_bounds__(256) void lora_a_update_kernel(int64_t n, int slices,
                                                            const float* __restrict__ dapart,
                                                            float* A, float* m, float* v,
                                                            float* grad_a,
                                                            float* __restrict__ sq_part,
                                                            AdamHP hp) {
  __shared__ float red[4];
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  float sq = 0.f;
  if (e < n) {
    const float d = sum_strided(dapart + e, slices, n);
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

// gnorm_sq += sum of the per-workgroup partials, in index order.
__global__ __launch_bounds__(64) void lora_gnorm_kernel(int nparts,
                                                        const float* __restrict__ sq_part,
                                                        float* gnorm_sq) {
  const int lane = threadIdx.x;
  float s = 0.f;
  for (int i = lane; i < nparts; i += 64) s += sq_part[i];
  s = wave_sum(s);
  if (lane == 0) *gnorm_sq += s;
}

namespace {

// Row slicing of one pass: `cols` columns in groups of 256, rows cut into
// slices of a multiple of 16 rows so that about L_TARGET workgroups run.
struct Slicing {
  int64_t groups, rs, slices;
};
Slicing slicing(int64_t rows, int64_t cols) {
  Slicing s;
  s.groups = cdiv(cols, LG_COLS);
  if (rows <= 0) {
    s.rs = 16;
    s.slices = 0;
    return s;
  }
  int64_t want = cdiv(L_TARGET, s.groups);
  want = want < 1 ? 1 : want;
  s.rs = cdiv(cdiv(rows, want), 16) * 16;
  s.slices = cdiv(rows, s.rs);
  return s;
}

// Workspace carve-up, in floats: g | gpart | part (dB, then dA) | sq.
struct LoraWs {
  int64_t g, gpart, part, sq, end;
};
LoraWs lora_ws(int64_t rows, int64_t in_dim, int64_t out_dim, int64_t rank) {
  const int64_t rp = cdiv(rank, 16) * 16;
  const Slicing sy = slicing(rows, out_dim), sa = slicing(rows, in_dim);
  const int64_t pb = sy.slices * out_dim * rank, pa = sa.slices * rank * in_dim;
  LoraWs w;
  w.g = 0;
  w.gpart = w.g + cdiv(rows * rp, 64) * 64;
  w.part = w.gpart + cdiv(sy.groups * rows * rp, 64) * 64;
  w.sq = w.part + cdiv(pb > pa ? pb : pa, 64) * 64;
  w.end = w.sq + cdiv(cdiv(rank * in_dim, 256), 64) * 64;
  return w;
}

template <int RB>
void launch_dy(int64_t rows, int64_t out_dim, int rank, const Slicing& sl, const float* dy,
               const void* h, int hdt, const float* B, float* gpart, float* dbpart,
               hipStream_t s) {
  const dim3 grid((unsigned)sl.groups, (unsigned)sl.slices);
#define LBP_DY(VEC, TH)                                                                    \
  lora_dy_kernel<RB, VEC, TH><<<grid, 256, 0, s>>>(rows, out_dim, rank, sl.rs, dy,         \
                                                   (const TH*)h, B, gpart, dbpart)
  if (out_dim % 4 == 0) {
    if (hdt == F32) LBP_DY(true, float);
    else LBP_DY(true, uint16_t);
  } else {
    if (hdt == F32) LBP_DY(false, float);
    else LBP_DY(false, uint16_t);
  }
#undef LBP_DY
}

template <int RB>
void launch_da(int64_t rows, int64_t in_dim, int rank, const Slicing& sl, const float* g,
               const void* x, int dt, float* dapart, hipStream_t s) {
  const dim3 grid((unsigned)sl.groups, (unsigned)sl.slices);
  if (dt == F32)
    lora_da_kernel<RB, float><<<grid, 256, 0, s>>>(rows, in_dim, rank, sl.rs, g,
                                                   (const float*)x, dapart);
  else
    lora_da_kernel<RB, bf16><<<grid, 256, 0, s>>>(rows, in_dim, rank, sl.rs, g,
                                                  (const bf16*)x, dapart);
}

}  // namespace

size_t lora_ws_bytes(int64_t rows, int64_t in_dim, int64_t out_dim, int64_t rank) {
  return (size_t)lora_ws(rows, in_dim, out_dim, rank).end * sizeof(float);
}

hipError_t launch_lora_adamw(int64_t rows, int64_t in_dim, int64_t out_dim, int64_t rank,
                             const float* dy, const void* x, const void* h, int dt, float* A,
                             float* B, float* m_a, float* v_a, float* m_b, float* v_b,
                             float* grad_a, float* grad_b, float* gnorm_sq, float scaling,
                             const AdamHP& hp, void* ws, hipStream_t s) {
  const LoraWs o = lora_ws(rows, in_dim, out_dim, rank);
  float* const base = (float*)ws;
  struct {
    float *g, *gpart, *part, *sq;
  } w = {base + o.g, base + o.gpart, base + o.part, base + o.sq};
  const Slicing sy = slicing(rows, out_dim), sa = slicing(rows, in_dim);
  const int r = (int)rank, rb = (int)cdiv(rank, 16);
  const int64_t rp = 16 * rb;
  const double esz = dt == F32 ? 4.0 : 2.0;
  hipError_t e;
  if (rows > 0) {
    switch (rb) {
      case 1: launch_dy<1>(rows, out_dim, r, sy, dy, h, dt, B, w.gpart, w.part, s); break;
      case 2: launch_dy<2>(rows, out_dim, r, sy, dy, h, dt, B, w.gpart, w.part, s); break;
      case 3: launch_dy<3>(rows, out_dim, r, sy, dy, h, dt, B, w.gpart, w.part, s); break;
      default: launch_dy<4>(rows, out_dim, r, sy, dy, h, dt, B, w.gpart, w.part, s); break;
    }
    mark("lora_dy", (double)rows * out_dim * 4 + (double)rows * rank * esz + (double)out_dim * rank * 4,
         4.0 * rows * out_dim * rank, s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // with no token rows the gradients are zero: no slices, no groups
  const int64_t nb = out_dim * rank, ng = rows > 0 ? rows * rp : 0;
  lora_b_update_kernel<<<dim3((unsigned)cdiv(nb + ng, 256)), 256, 0, s>>>(
      nb, (int)sy.slices, w.part, ng, (int)sy.groups, w.gpart, w.g, scaling, B, m_b, v_b, grad_b,
      hp);
  mark("lora_adamw_b", (double)nb * 4 * (6 + (grad_b ? 1 : 0)) + (double)ng * 4, 12.0 * nb, s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (rows > 0) {
    switch (rb) {
      case 1: launch_da<1>(rows, in_dim, r, sa, w.g, x, dt, w.part, s); break;
      case 2: launch_da<2>(rows, in_dim, r, sa, w.g, x, dt, w.part, s); break;
      case 3: launch_da<3>(rows, in_dim, r, sa, w.g, x, dt, w.part, s); break;
      default: launch_da<4>(rows, in_dim, r, sa, w.g, x, dt, w.part, s); break;
    }
    mark("lora_da", (double)rows * in_dim * esz + (double)rows * rank * 4,
         2.0 * rows * in_dim * rank, s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int nsq = (int)cdiv(rank * in_dim, 256);
  lora_a_update_kernel<<<dim3((unsigned)nsq), 256, 0, s>>>(rank * in_dim, (int)sa.slices, w.part,
                                                            A, m_a, v_a, grad_a, w.sq, hp);
  mark("lora_adamw_a", (double)rank * in_dim * 4 * (6 + (grad_a ? 1 : 0)), 14.0 * rank * in_dim, s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (gnorm_sq != nullptr) {
    lora_gnorm_kernel<<<dim3(1), dim3(64), 0, s>>>(nsq, w.sq, gnorm_sq);
    mark("lora_gnorm", 4.0 * nsq + 8, (double)nsq, s);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace lbp
