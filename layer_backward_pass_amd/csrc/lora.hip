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
//
// A layer's two adapters (Q and V) run in the same launches: every kernel
// takes a pair of argument sets: the two passes over the data walk one flat
// list of both adapters' workgroups, the update kernels take blockIdx.z as
// the adapter (the grid covers the larger of the two and the other's
// surplus workgroups return).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace lbp {

constexpr int LW_COLS = 64;    // columns per wave
constexpr int LG_COLS = 256;   // columns per workgroup
constexpr int L_TARGET = 256;  // workgroups aimed for per pass

static inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Per-adapter arguments of each pass (gx, gy: that adapter's own grid).
struct DyArgs {
  int64_t rows, out_dim, rs;
  int rank, gx, gy;
  const float* dy;
  const void* h;
  const float* B;
  float* gpart;
  float* dbpart;
};
struct DaArgs {
  int64_t rows, in_dim, rs;
  int rank, gx, gy;
  const float* g;
  const void* x;
  float* dapart;
  // GRED: g reduced in the kernel from the dy pass's partials (groups of
  // them, scaled by s), and written to gout by the items of column group 0
  // when gout is set
  const float* gpart;
  int groups;
  float s;
  float* gout;
};
struct BUpdArgs {
  int64_t nb, ng;
  int slices, groups, nblk;
  const float* dbpart;
  const float* gpart;
  float* g;
  float s, lr;
  float *B, *m, *v, *grad_b;
};
struct AUpdArgs {
  int64_t n;
  int slices, nblk;
  const float* dapart;
  float *A, *m, *v, *grad_a;
  float* sq_part;
};
template <typename A>
struct Pair {
  A a[2];
  // the adapter of this workgroup (a select, not an indexed copy of the
  // kernel arguments)
  __device__ __forceinline__ const A& pick() const { return blockIdx.z == 0 ? a[0] : a[1]; }
  // Flat 1-D grid of the two adapters' (column group, row slice) items:
  // adapter 0's gx x gy first, then adapter 1's, column group fastest, so
  // consecutive workgroups (which the hardware deals out to the XCDs in
  // turn) spread each adapter over every XCD.
  __device__ __forceinline__ const A& item(int& bx, int& by) const {
    const int64_t L = blockIdx.x, n0 = (int64_t)a[0].gx * a[0].gy;
    const bool second = L >= n0;
    const A& r = second ? a[1] : a[0];
    const int64_t loc = second ? L - n0 : L;
    bx = (int)(loc % r.gx);
    by = (int)(loc / r.gx);
    return r;
  }
};

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
__global__ __launch_bounds__(256) void lora_dy_kernel(Pair<DyArgs> pa) {
  int bx, by;
  const DyArgs& A = pa.item(bx, by);
  const int64_t rows = A.rows, out_dim = A.out_dim, rs = A.rs;
  const int rank = A.rank;
  const float* __restrict__ dy = A.dy;
  const TH* __restrict__ h = (const TH*)A.h;
  const float* __restrict__ Bm = A.B;
  float* __restrict__ gpart = A.gpart;
  float* __restrict__ dbpart = A.dbpart;
  constexpr int RP = 16 * RB;
  __shared__ float gs[4][16][RP + 1];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int l16 = lane & 15, l4 = lane >> 4;
  const int64_t o0 = (int64_t)bx * LG_COLS + w * LW_COLS;
  const int64_t i_beg = (int64_t)by * rs;
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
        gpart[((int64_t)bx * rows + i0 + row) * RP + col] =
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
  float* dp = dbpart + (int64_t)by * out_dim * rank;
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

// dB = s sum_slices dbpart, then AdamW on B (lr_b), for element e of one
// adapter's B.
__device__ __forceinline__ void b_update_at(const BUpdArgs& A, int64_t e, const AdamHP& hp);

// g rows of one row slice held in LDS by lora_da_kernel (GRED), in floats
constexpr int DA_GSLICE = 4096;

// One pass over x [rows, in]: dapart[by][r][k] = sum_{i in slice} g[i,r] x[i,k].
// Result rows = rank (16 per block b), cols = features (tile j: k0 + 4n + j),
// k = tokens.  g is [rows, 16 RB], scaled and zero-padded: read from memory,
// or (GRED) first summed for the item's row slice from the dy pass's
// per-column-group partials, in group order, into LDS.  Two 16-row steps in
// flight, loads through buffer ranges (in_dim % 8 == 0, so a 4-feature chunk
// is whole).  With GRED the launch also carries the B updates: workgroups
// from nd on each update 256 elements of dB (adapter 0's, then adapter 1's),
// which need only the dy pass.
template <int RB, typename T, bool GRED>
__global__ __launch_bounds__(256) void lora_da_kernel(Pair<DaArgs> pa, Pair<BUpdArgs> pb,
                                                      int64_t nd, AdamHP hp) {
  __shared__ float gsl[GRED ? DA_GSLICE : 1];
  if (GRED && (int64_t)blockIdx.x >= nd) {
    const int64_t j = (int64_t)blockIdx.x - nd;
    const bool second = j >= pb.a[0].nblk;
    const BUpdArgs& B = second ? pb.a[1] : pb.a[0];
    b_update_at(B, (second ? j - pb.a[0].nblk : j) * 256 + threadIdx.x, hp);
    return;
  }
  int bx, by;
  const DaArgs& A = pa.item(bx, by);
  const int64_t rows = A.rows, in_dim = A.in_dim, rs = A.rs;
  const int rank = A.rank;
  const float* __restrict__ g = A.g;
  const T* __restrict__ x = (const T*)A.x;
  float* __restrict__ dapart = A.dapart;
  constexpr int RP = 16 * RB;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int l16 = lane & 15, l4 = lane >> 4;
  const int64_t k0 = (int64_t)bx * LG_COLS + w * LW_COLS;
  const int64_t i_beg = (int64_t)by * rs;
  const int64_t i_end = min(rows, i_beg + rs);
  const int64_t nrow = i_end - i_beg;
  const brsrc_t rx = make_brsrc(x + i_beg * in_dim, nrow > 0 ? (uint32_t)(nrow * in_dim * sizeof(T)) : 0u);
  const brsrc_t rg = make_brsrc(g + i_beg * RP, nrow > 0 && !GRED ? (uint32_t)(nrow * RP * 4) : 0u);
  if (GRED) {
    // g of the slice's rows, eight partial loads in flight per element
    const int ng = A.groups;
    for (int64_t e = t; e < nrow * RP; e += 256) {
      const float* src = A.gpart + i_beg * RP + e;
      const int64_t gst = rows * RP;
      float s = 0.f;
      for (int c0 = 0; c0 < ng; c0 += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = c0 + u < ng ? src[(int64_t)(c0 + u) * gst] : 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u) s += v[u];
      }
      s *= A.s;
      gsl[e] = s;
      if (A.gout != nullptr && bx == 0) A.gout[i_beg * RP + e] = s;
    }
    __syncthreads();
  }
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
      for (int b = 0; b < RB; ++b) {
        if (GRED)
          S.gv[q][b] = ok ? gsl[(i - i_beg) * RP + 16 * b + l16] : 0.f;
        else
          S.gv[q][b] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
              rg, ok ? (int)(((i - i_beg) * RP + 16 * b + l16) * 4) : (int)BUF_OOB, 0, 0));
      }
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
  float* dp = dapart + (int64_t)by * rank * in_dim;
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

__device__ __forceinline__ void b_update_at(const BUpdArgs& A, int64_t e, const AdamHP& hp) {
  if (e >= A.nb) return;
  float d = sum_strided(A.dbpart + e, A.slices, A.nb);
  d *= A.s;
  if (A.grad_b) A.grad_b[e] = d;
  float p = A.B[e], mm = A.m[e], vv = A.v[e];
  adamw1(p, d, mm, vv, A.lr, hp);
  A.B[e] = p;
  A.m[e] = mm;
  A.v[e] = vv;
}

__global__ __launch_bounds__(256) void lora_b_update_kernel(Pair<BUpdArgs> pa, AdamHP hp) {
  const BUpdArgs& A = pa.pick();
  if ((int)blockIdx.x >= A.nblk) return;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e < A.nb) {
    b_update_at(A, e, hp);
  } else if (e < A.nb + A.ng) {
    const int64_t f = e - A.nb;
    A.g[f] = A.s * sum_strided(A.gpart + f, A.groups, A.ng);
  }
}

// dA = sum_slices dapart, AdamW on A (lr_a), per-workgroup sum of dA^2.
__global__ __launch_bounds__(256) void lora_a_update_kernel(Pair<AUpdArgs> pa, AdamHP hp) {
  __shared__ float red[4];
  const AUpdArgs& A = pa.pick();
  if ((int)blockIdx.x >= A.nblk) return;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  float sq = 0.f;
  if (e < A.n) {
    const float d = sum_strided(A.dapart + e, A.slices, A.n);
    if (A.grad_a) A.grad_a[e] = d;
    sq = d * d;
    float p = A.A[e], mm = A.m[e], vv = A.v[e];
    adamw1(p, d, mm, vv, hp.lr_a, hp);
    A.A[e] = p;
    A.m[e] = mm;
    A.v[e] = vv;
  }
  sq = block_sum<4>(sq, red);
  if (threadIdx.x == 0) A.sq_part[blockIdx.x] = sq;
}

// The adapters' share of the gradient at their input x (the attention
// input gradient): out[i][n] (+)= sum over adapters of sum_{r < rank}
// g[i][r] A[r][n], with g = s dy B as the B update reduced it and A before
// its update.  Workgroup = 256 columns x 16 rows; the rows' g values are
// staged in LDS, each thread walks A's rank rows for its column.
struct DxArgs {
  const float* g;  // [rows][rp]
  int64_t rp;
  const float* A;  // [rank][n]
  int rank;
};
__global__ __launch_bounds__(256) void lora_dx_kernel(int64_t rows, int64_t n, DxArgs a0, DxArgs a1,
                                                      int nadp, float* __restrict__ out,
                                                      int accumulate) {
  __shared__ float gs[2][16][64];
  const int64_t col = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.y * 16;
  for (int z = 0; z < 2; ++z) {
    const DxArgs& a = z == 0 ? a0 : a1;
    for (int e = threadIdx.x; e < 16 * 64; e += 256) {
      const int i = e >> 6, r = e & 63;
      gs[z][i][r] = (z < nadp && r0 + i < rows && r < a.rank) ? a.g[(r0 + i) * a.rp + r] : 0.f;
    }
  }
  __syncthreads();
  if (col >= n) return;
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  for (int z = 0; z < nadp; ++z) {
    const DxArgs& a = z == 0 ? a0 : a1;
    for (int r = 0; r < a.rank; ++r) {
      const float av = a.A[(int64_t)r * n + col];
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] += gs[z][i][r] * av;
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t row = r0 + i;
    if (row < rows) {
      float* o = out + row * n + col;
      *o = accumulate ? *o + acc[i] : acc[i];
    }
  }
}

// gnorm_sq += the per-workgroup partials of adapter 0, then of adapter 1
// (n1 = 0: none), each summed in index order.
__global__ __launch_bounds__(64) void lora_gnorm_kernel(int n0, const float* __restrict__ sq0,
                                                        int n1, const float* __restrict__ sq1,
                                                        float* gnorm_sq) {
  const int lane = threadIdx.x;
  float s0 = 0.f, s1 = 0.f;
  for (int i = lane; i < n0; i += 64) s0 += sq0[i];
  for (int i = lane; i < n1; i += 64) s1 += sq1[i];
  s0 = wave_sum(s0);
  s1 = wave_sum(s1);
  if (lane == 0) *gnorm_sq = (*gnorm_sq + s0) + s1;
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

// Workspace carve-up, in floats: g | gpart | dB partials | dA partials | sq
// (the dA launch also runs the B updates, so the two partial sets coexist).
struct LoraWs {
  int64_t g, gpart, part, parta, sq, end;
};
LoraWs lora_ws(int64_t rows, int64_t in_dim, int64_t out_dim, int64_t rank) {
  const int64_t rp = cdiv(rank, 16) * 16;
  const Slicing sy = slicing(rows, out_dim), sa = slicing(rows, in_dim);
  const int64_t pb = sy.slices * out_dim * rank, pa = sa.slices * rank * in_dim;
  LoraWs w;
  w.g = 0;
  w.gpart = w.g + cdiv(rows * rp, 64) * 64;
  w.part = w.gpart + cdiv(sy.groups * rows * rp, 64) * 64;
  w.parta = w.part + cdiv(pb, 64) * 64;
  w.sq = w.parta + cdiv(pa, 64) * 64;
  w.end = w.sq + cdiv(cdiv(rank * in_dim, 256), 64) * 64;
  return w;
}

}  // namespace

size_t lora_ws_bytes(int64_t rows, int64_t in_dim, int64_t out_dim, int64_t rank) {
  return (size_t)lora_ws(rows, in_dim, out_dim, rank).end * sizeof(float);
}

// One launch group: one adapter, or two whose passes share template
// arguments (rank blocks, dtype, vector path), run in the same launches.
template <int RB, bool VEC, typename TH>
static hipError_t lora_group(const LoraJob* const* jobs, int nz, float* gnorm_sq,
                             const AdamHP& hp, hipStream_t s, float* dx, int dx_acc) {
  Pair<DyArgs> dy{};
  Pair<BUpdArgs> bu{};
  Pair<DaArgs> da{};
  Pair<AUpdArgs> au{};
  int64_t ny = 0, nd = 0;  // items of the dy and dA passes
  int bx = 0, ax = 0;
  double by_dy = 0, fl_dy = 0, by_b = 0, fl_b = 0, by_da = 0, fl_da = 0, by_a = 0, fl_a = 0;
  const int64_t rows = jobs[0]->rows;
  for (int z = 0; z < 2; ++z) {
    const LoraJob& j = *jobs[z < nz ? z : 0];
    const LoraWs o = lora_ws(j.rows, j.in_dim, j.out_dim, j.rank);
    float* const base = (float*)j.ws;
    const Slicing sy = slicing(j.rows, j.out_dim), sa = slicing(j.rows, j.in_dim);
    const int64_t rp = 16 * RB;
    dy.a[z] = DyArgs{j.rows, j.out_dim, sy.rs, (int)j.rank, (int)sy.groups, (int)sy.slices,
                     j.dy, j.h, j.B, base + o.gpart, base + o.part};
    const int64_t nb = j.out_dim * j.rank, ng = j.rows > 0 ? j.rows * rp : 0;
    bu.a[z] = BUpdArgs{nb, ng, (int)sy.slices, (int)sy.groups, (int)cdiv(nb + ng, 256),
                       base + o.part, base + o.gpart, base + o.g, j.scaling, hp.lr_b,
                       j.B, j.m_b, j.v_b, j.grad_b};
    da.a[z] = DaArgs{j.rows, j.in_dim, sa.rs, (int)j.rank, (int)sa.groups, (int)sa.slices,
                     base + o.g, j.x, base + o.parta, base + o.gpart, (int)sy.groups, j.scaling,
                     dx != nullptr ? base + o.g : nullptr};
    au.a[z] = AUpdArgs{j.rank * j.in_dim, (int)sa.slices, (int)cdiv(j.rank * j.in_dim, 256),
                       base + o.parta, j.A, j.m_a, j.v_a, j.grad_a, base + o.sq};
    if (z >= nz) continue;
    ny += sy.groups * sy.slices;
    nd += sa.groups * sa.slices;
    bx = max(bx, bu.a[z].nblk);
    ax = max(ax, au.a[z].nblk);
    const double esz = j.dt == F32 ? 4.0 : 2.0;
    by_dy += (double)j.rows * j.out_dim * 4 + (double)j.rows * j.rank * esz + (double)nb * 4;
    fl_dy += 4.0 * j.rows * j.out_dim * j.rank;
    by_b += (double)nb * 4 * (6 + (j.grad_b ? 1 : 0));
    fl_b += 12.0 * nb;
    by_da += (double)j.rows * j.in_dim * esz + (double)j.rows * j.rank * 4;
    fl_da += 2.0 * j.rows * j.in_dim * j.rank;
    by_a += (double)j.rank * j.in_dim * 4 * (6 + (j.grad_a ? 1 : 0));
    fl_a += 14.0 * j.rank * j.in_dim;
  }
  // buffer ranges: one row slice of dy, h, x and g
  for (int z = 0; z < nz; ++z) {
    const LoraJob& j = *jobs[z];
    const Slicing sy = slicing(j.rows, j.out_dim), sa = slicing(j.rows, j.in_dim);
    const double esz = j.dt == F32 ? 4.0 : 2.0;
    if ((double)sy.rs * j.out_dim * 4 >= BUF_MAX_BYTES || (double)sy.rs * j.rank * esz >= BUF_MAX_BYTES ||
        (double)sa.rs * j.in_dim * esz >= BUF_MAX_BYTES || (double)sa.rs * 16 * RB * 4 >= BUF_MAX_BYTES)
      return hipErrorInvalidValue;
  }
  // the dA launch reduces g itself when a row slice's g fits its LDS
  bool gred = true;
  for (int z = 0; z < nz; ++z) gred = gred && da.a[z].rs * 16 * RB <= DA_GSLICE;
  if (dry_run()) return hipSuccess;
  hipError_t e;
  typedef typename std::conditional<sizeof(TH) == 4, float, bf16>::type TX;
  if (rows > 0) {
    lora_dy_kernel<RB, VEC, TH><<<dim3((unsigned)ny), 256, 0, s>>>(dy);
    mark("lora_dy", by_dy, fl_dy, s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (gred) {
    // one launch: dA partials (g reduced per row slice) and the B updates
    // (with no token rows the gradients are zero: no slices, no groups)
    int64_t nbb = 0;
    for (int z = 0; z < 2; ++z) bu.a[z].nblk = z < nz ? (int)cdiv(bu.a[z].nb, 256) : 0;
    for (int z = 0; z < nz; ++z) nbb += bu.a[z].nblk;
    lora_da_kernel<RB, TX, true><<<dim3((unsigned)(nd + nbb)), 256, 0, s>>>(da, bu, nd, hp);
    mark("lora_da_adamw_b", by_da + by_b, fl_da + fl_b, s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  } else {
    lora_b_update_kernel<<<dim3((unsigned)bx, 1, (unsigned)nz), 256, 0, s>>>(bu, hp);
    mark("lora_adamw_b", by_b, fl_b, s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (dx != nullptr && rows > 0) {
    // the adapters' input-gradient term, while A is still the pre-update A
    DxArgs xa[2];
    for (int z = 0; z < 2; ++z) {
      const LoraJob& j = *jobs[z < nz ? z : 0];
      const LoraWs o = lora_ws(j.rows, j.in_dim, j.out_dim, j.rank);
      xa[z] = DxArgs{(const float*)j.ws + o.g, 16 * RB, j.A, (int)j.rank};
    }
    const int64_t n = jobs[0]->in_dim;
    lora_dx_kernel<<<dim3((unsigned)cdiv(n, 256), (unsigned)cdiv(rows, 16)), 256, 0, s>>>(
        rows, n, xa[0], xa[1], nz, dx, dx_acc);
    double rk = 0;
    for (int z = 0; z < nz; ++z) rk += (double)jobs[z]->rank;
    mark("lora_dx", (double)rows * n * 4 * (dx_acc ? 2 : 1) + rk * (n + rows) * 4, 2.0 * rows * n * rk, s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (rows > 0 && !gred) {
    lora_da_kernel<RB, TX, false><<<dim3((unsigned)nd), 256, 0, s>>>(da, bu, nd, hp);
    mark("lora_da", by_da, fl_da, s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  lora_a_update_kernel<<<dim3((unsigned)ax, 1, (unsigned)nz), 256, 0, s>>>(au, hp);
  mark("lora_adamw_a", by_a, fl_a, s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (gnorm_sq != nullptr) {
    lora_gnorm_kernel<<<dim3(1), dim3(64), 0, s>>>(au.a[0].nblk, au.a[0].sq_part,
                                                  nz > 1 ? au.a[1].nblk : 0, au.a[1].sq_part,
                                                  gnorm_sq);
    mark("lora_gnorm", 4.0 * (ax * nz) + 8, (double)(ax * nz), s);
    e = hipGetLastError();
  }
  return e;
}

static hipError_t lora_dispatch(const LoraJob* const* jobs, int nz, float* gnorm_sq,
                                const AdamHP& hp, hipStream_t s, float* dx, int dx_acc) {
  const LoraJob& j = *jobs[0];
  const int rb = (int)cdiv(j.rank, 16);
  const bool vec = j.out_dim % 4 == 0;
#define LBP_LG(RBV)                                                                    \
  case RBV:                                                                            \
    if (vec) {                                                                         \
      if (j.dt == F32) return lora_group<RBV, true, float>(jobs, nz, gnorm_sq, hp, s, dx, dx_acc);  \
      return lora_group<RBV, true, uint16_t>(jobs, nz, gnorm_sq, hp, s, dx, dx_acc);               \
    }                                                                                  \
    if (j.dt == F32) return lora_group<RBV, false, float>(jobs, nz, gnorm_sq, hp, s, dx, dx_acc);   \
    return lora_group<RBV, false, uint16_t>(jobs, nz, gnorm_sq, hp, s, dx, dx_acc);
  switch (rb) {
    LBP_LG(1)
    LBP_LG(2)
    LBP_LG(3)
    default:
      LBP_LG(4)
  }
#undef LBP_LG
}

hipError_t launch_lora_adamw_jobs(const LoraJob* jobs, int njobs, float* gnorm_sq,
                                  const AdamHP& hp, hipStream_t s, float* dx) {
  if (njobs <= 0) return hipSuccess;
  const LoraJob* p[2] = {&jobs[0], njobs > 1 ? &jobs[1] : &jobs[0]};
  if (njobs == 2) {
    const LoraJob &a = jobs[0], &b = jobs[1];
    const bool same = cdiv(a.rank, 16) == cdiv(b.rank, 16) && a.dt == b.dt &&
                      (a.out_dim % 4 == 0) == (b.out_dim % 4 == 0) && a.rows == b.rows;
    if (same) return lora_dispatch(p, 2, gnorm_sq, hp, s, dx, 0);
    hipError_t e = lora_dispatch(p, 1, gnorm_sq, hp, s, dx, 0);
    if (e != hipSuccess) return e;
    p[0] = &jobs[1];
    return lora_dispatch(p, 1, gnorm_sq, hp, s, dx, 1);
  }
  return lora_dispatch(p, 1, gnorm_sq, hp, s, dx, 0);
}

hipError_t launch_lora_adamw(int64_t rows, int64_t in_dim, int64_t out_dim, int64_t rank,
                             const float* dy, const void* x, const void* h, int dt, float* A,
                             float* B, float* m_a, float* v_a, float* m_b, float* v_b,
                             float* grad_a, float* grad_b, float* gnorm_sq, float scaling,
                             const AdamHP& hp, void* ws, hipStream_t s) {
  const LoraJob j{rows, in_dim, out_dim, rank, dy, x, h, dt, A, B, m_a, v_a, m_b, v_b,
                  grad_a, grad_b, scaling, ws};
  return launch_lora_adamw_jobs(&j, 1, gnorm_sq, hp, s, nullptr);
}

}  // namespace lbp
