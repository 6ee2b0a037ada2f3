// Transposed products of the backward pass, dX = dY W with W [out, in]
// row-major: C[M,N] = A[M,K] B[K,N], A = gradient rows, B = weight.
//   * fp32 weights: v_mfma_f32_16x16x4_f32, 128x256 workgroup tiles, BK 32
//   * bf16 weights: v_mfma_f32_16x16x32_bf16, 128x256 tiles, BK 64; an fp32
//     gradient operand is rounded to bf16 first (cvt_a_bf16_kernel)
// Split-K partial sums go to caller scratch and are reduced in a fixed
// order (no float atomics), so results are bitwise reproducible.  The W_down
// product can apply the gated-activation backward to its output as it is
// stored (ActEpi), so dHid never goes to memory; the W_o product can also
// store its output transposed in bf16 (TCopy) for the attention's dV.  The
// lm_head weight gradient dW = dlogits^T h reads its A operand transposed
// (dlogits as stored, [K][M]) and applies AdamW to the weight as each tile
// is stored (AdamEpi), so dW never goes to memory either.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace lbp {

// Output tile of the 16x16 MFMA accumulators: lane l holds rows 4*(l/16)+v
// (v = 0..3) of column l%16.
template <int FM, int FN>
__device__ __forceinline__ void store_tile(float* C, int64_t ldc, int64_t M, int64_t N,
                                           int64_t row0, int64_t col0,
                                           const floatx4 (&acc)[FM][FN]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int fi = 0; fi < FM; ++fi)
#pragma unroll
    for (int fj = 0; fj < FN; ++fj) {
      const int64_t c = col0 + fj * 16 + (lane & 15);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t r = row0 + fi * 16 + 4 * (lane >> 4) + v;
        if (r < M && c < N) C[r * ldc + c] = acc[fi][fj][v];
      }
    }
}

// A whole tile of dHid (C[r][c] = dHid of feature c; 32 FM rows x 256, the
// waves' FM x 4 accumulators at rows wm + 16 i) through the gated-activation
// backward: [dGate | dUp] go to e.out[r][c], e.out[r][N + c] (TO: float or
// bf16), from gate / up [M][N] (TG).  The accumulators pass through LDS
// (`stage`: 64 x EPI_LD floats, free once the k-loop is done) 64 rows at a
// time, so that each thread then takes eight consecutive features of a row
// with 16-byte loads and stores; a pass's gate/up loads are in flight while
// its accumulators are written.  N % 8 == 0.
constexpr int EPI_LD = 260;
template <typename TG, typename TO, int ACT, int FM = 4>
__device__ __forceinline__ void act_tile_epilogue(const ActEpi& e, int64_t M, int64_t N,
                                                  int64_t bm, int64_t bn, int wm, int wn,
                                                  const floatx4 (&acc)[FM][4], float* stage) {
  constexpr int GV = sizeof(TG) == 2 ? 1 : 2;  // 16-byte chunks per eight features
  constexpr int TR = 32 * FM;                  // tile rows
  const int t = threadIdx.x, lane = t & 63;
  const int64_t mrows = min((int64_t)TR, M - bm);
  const uint32_t bytes = (uint32_t)(mrows * N * sizeof(TG));
  const brsrc_t rg = make_brsrc((const TG*)e.gate + bm * N, bytes);
  const brsrc_t ru = make_brsrc((const TG*)e.up + bm * N, bytes);
  const int cl = 8 * (t & 31), rl = t >> 5;  // eight features of row rl (+16 p)
  const int64_t gc = bn + cl;
  __syncthreads();  // every wave is past its last LDS read of the k-loop
#pragma unroll
  for (int h = 0; h < TR / 64; ++h) {
    uint4 g[4][GV], u[4][GV];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int r = 64 * h + 16 * p + rl;
      const bool ok = r < mrows && gc < N;
#pragma unroll
      for (int q = 0; q < GV; ++q) {
        const uint32_t off = ok ? (uint32_t)((r * N + gc) * sizeof(TG) + 16 * q) : BUF_OOB;
        g[p][q] = bload_u4(rg, off);
        u[p][q] = bload_u4(ru, off);
      }
    }
    // the accumulator blocks whose rows fall in this pass (wave-uniform)
#pragma unroll
    for (int fi = 0; fi < FM; ++fi) {
      if ((wm + 16 * fi) / 64 != h) continue;
#pragma unroll
      for (int fj = 0; fj < 4; ++fj)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          stage[((wm + 16 * fi) % 64 + 4 * (lane >> 4) + v) * EPI_LD + wn + fj * 16 +
                (lane & 15)] = acc[fi][fj][v];
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int r = 64 * h + 16 * p + rl;
      const float4 d0 = *reinterpret_cast<const float4*>(&stage[(16 * p + rl) * EPI_LD + cl]);
      const float4 d1 = *reinterpret_cast<const float4*>(&stage[(16 * p + rl) * EPI_LD + cl + 4]);
      const float dh[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
      float gv[8], uv[8];
      if constexpr (GV == 1) {
        const uint32_t gw[4] = {g[p][0].x, g[p][0].y, g[p][0].z, g[p][0].w};
        const uint32_t uw[4] = {u[p][0].x, u[p][0].y, u[p][0].z, u[p][0].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          gv[2 * i] = __uint_as_float(gw[i] << 16);
          gv[2 * i + 1] = __uint_as_float(gw[i] & 0xffff0000u);
          uv[2 * i] = __uint_as_float(uw[i] << 16);
          uv[2 * i + 1] = __uint_as_float(uw[i] & 0xffff0000u);
        }
      } else {
        const uint32_t gw[8] = {g[p][0].x, g[p][0].y, g[p][0].z, g[p][0].w,
                                g[p][1].x, g[p][1].y, g[p][1].z, g[p][1].w};
        const uint32_t uw[8] = {u[p][0].x, u[p][0].y, u[p][0].z, u[p][0].w,
                                u[p][1].x, u[p][1].y, u[p][1].z, u[p][1].w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          gv[i] = __uint_as_float(gw[i]);
          uv[i] = __uint_as_float(uw[i]);
        }
      }
      float dg[8], du[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) act_bwd1<ACT>(gv[i], uv[i], dh[i], dg[i], du[i]);
      if (r < mrows && gc < N) {
        TO* o = (TO*)e.out + (bm + r) * 2 * N + gc;
        if constexpr (sizeof(TO) == 2) {
          *reinterpret_cast<uint4*>(o) = make_uint4(pk_bf16(dg[0], dg[1]), pk_bf16(dg[2], dg[3]),
                                                    pk_bf16(dg[4], dg[5]), pk_bf16(dg[6], dg[7]));
          *reinterpret_cast<uint4*>(o + N) =
              make_uint4(pk_bf16(du[0], du[1]), pk_bf16(du[2], du[3]), pk_bf16(du[4], du[5]),
                         pk_bf16(du[6], du[7]));
        } else {
          float* of = (float*)o;
          *reinterpret_cast<float4*>(of) = make_float4(dg[0], dg[1], dg[2], dg[3]);
          *reinterpret_cast<float4*>(of + 4) = make_float4(dg[4], dg[5], dg[6], dg[7]);
          *reinterpret_cast<float4*>(of + N) = make_float4(du[0], du[1], du[2], du[3]);
          *reinterpret_cast<float4*>(of + N + 4) = make_float4(du[4], du[5], du[6], du[7]);
        }
      }
    }
    if (h + 1 < TR / 64) __syncthreads();  // the next pass overwrites the stage
  }
}

// A whole 128 x 256 tile of a weight gradient (C[r][c] = dW[r][c], W dense
// [M][N]) through AdamW: W, m, v updated in place (and the gradient copied
// to e.grad when set).  As in the activation epilogue, the accumulators pass
// through LDS in two halves of 64 rows so that each thread then takes eight
// consecutive columns of a row with 16-byte accesses; a half's W, m, v loads
// are in flight while its accumulators are written.  N % 8 == 0.
__device__ __forceinline__ void adam_tile_epilogue(const AdamEpi& e, int64_t M, int64_t N,
                                                   int64_t bm, int64_t bn, int wm, int wn,
                                                   const floatx4 (&acc)[4][4], float* stage) {
  const int t = threadIdx.x, lane = t & 63;
  const int64_t mrows = min((int64_t)128, M - bm);
  const uint32_t bytes = (uint32_t)(mrows * N * 4);
  const brsrc_t rw = make_brsrc(e.w + bm * N, bytes);
  const brsrc_t rm = make_brsrc(e.m + bm * N, bytes);
  const brsrc_t rv = make_brsrc(e.v + bm * N, bytes);
  const int cl = 8 * (t & 31), rl = t >> 5;  // eight columns of row rl (+16 p)
  const int64_t gc = bn + cl;
  __syncthreads();  // every wave is past its last LDS read of the k-loop
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float4 pw[4][2], pm[4][2], pv[4][2];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int r = 64 * h + 16 * p + rl;
      const bool ok = r < mrows && gc < N;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint32_t off = ok ? (uint32_t)((r * N + gc) * 4 + 16 * q) : BUF_OOB;
        pw[p][q] = bload_f4(rw, off);
        pm[p][q] = bload_f4(rm, off);
        pv[p][q] = bload_f4(rv, off);
      }
    }
    if (wm == 64 * h) {
#pragma unroll
      for (int fi = 0; fi < 4; ++fi)
#pragma unroll
        for (int fj = 0; fj < 4; ++fj)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            stage[(fi * 16 + 4 * (lane >> 4) + v) * EPI_LD + wn + fj * 16 + (lane & 15)] =
                acc[fi][fj][v];
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int r = 64 * h + 16 * p + rl;
      if (r < mrows && gc < N) {
        const int64_t o = (bm + r) * N + gc;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const float4 d = *reinterpret_cast<const float4*>(&stage[(16 * p + rl) * EPI_LD + cl + 4 * q]);
          float4 w = pw[p][q], m = pm[p][q], v = pv[p][q];
          adamw1(w.x, d.x, m.x, v.x, e.lr, e.hp);
          adamw1(w.y, d.y, m.y, v.y, e.lr, e.hp);
          adamw1(w.z, d.z, m.z, v.z, e.lr, e.hp);
          adamw1(w.w, d.w, m.w, v.w, e.lr, e.hp);
          *reinterpret_cast<float4*>(e.w + o + 4 * q) = w;
          *reinterpret_cast<float4*>(e.m + o + 4 * q) = m;
          *reinterpret_cast<float4*>(e.v + o + 4 * q) = v;
          if (e.grad) *reinterpret_cast<float4*>(e.grad + o + 4 * q) = d;
        }
      }
    }
    if (h == 0) __syncthreads();  // the second half overwrites the stage
  }
}

// ---------------------------------------------------------------------------
// fp32 GEMM: workgroup of 8 waves (512 threads), tile 128 x 256, BK = 32; the
// waves form a 2 x 4 grid of 64 x 64 wave tiles (4 x 4 MFMA accumulators).
// Both LDS tiles are k-contiguous, As[m][k] and Bs[n][k], row stride 36
// floats: one 16-byte read gives a lane four consecutive k, which feed four
// MFMA steps (k slot c of step j is 16 kb + 4c + j for A and B alike).  A is
// read from HBM as 16-byte row segments; B, stored [k][n], is read as 4-byte
// columns that are coalesced across the lanes (n), so each thread gathers
// four k of one n and writes them with one 16-byte LDS store.  The LDS tiles
// are double-buffered: the next k-tile's global loads are in flight while
// the current one is used, one barrier per k-tile.  A wide workgroup tile
// keeps the HBM/L2 bytes per MFMA low; with one workgroup per CU the MFMA
// pipe then stays about three quarters busy.  AT: A is given transposed,
// A^T [K][lda] (m contiguous), and is gathered like B (four k of one m per
// thread, one 16-byte LDS store); the tiles are then numbered n-fastest.
// EPI 32 (with AT) is the AdamW epilogue.
constexpr int F_BK = 32, F_LD = F_BK + 4, F_BM = 128, F_BN = 256, F_NT = 512;
static_assert(2 * F_BN * F_LD >= 64 * EPI_LD, "activation stage fits in Bs");

// Work item of a product launch.  Tiles are numbered m-fastest over the
// nm x nn grid.  Items u < nfull are whole tiles written to C; the other
// tiles are split in k-chunks of kps, item nfull + j -> chunk z = j / ntail
// of tile nfull + j % ntail (chunk-major, so neighbouring items still share
// weight panels), written to partial slot z ([z][M][N], dense).  nfull = 0
// is plain split-K; nfull = all tiles is no split.  NFAST numbers the tiles
// n-fastest instead (the column tiles of one row panel together: they share
// the A panel, for a product whose A is the large operand).
struct GemmWork {
  int64_t bm, bn, kbeg, kend, ldo;
  float* out;
  bool whole;
};
template <int BM, int BN, bool NFAST = false>
__device__ __forceinline__ GemmWork gemm_work(int64_t M, int64_t N, int64_t K, int64_t kps,
                                              int64_t nfull, float* C, int64_t ldc, float* P) {
  const int64_t nm = (M + BM - 1) / BM, nn = (N + BN - 1) / BN, T = nm * nn;
  // Workgroups start in launch order, so the whole tiles (the long items)
  // take the first launch slots; each part is spread over the XCDs on its own.
  const int64_t b = blockIdx.x, G = gridDim.x;
  const int64_t u = b < nfull ? xcd_remap(b, nfull) : nfull + xcd_remap(b - nfull, G - nfull);
  int64_t tile, z;
  if (u < nfull) {
    tile = u;
    z = -1;
  } else {
    const int64_t j = u - nfull, nt = T - nfull;
    z = j / nt;
    tile = nfull + (j - z * nt);
  }
  GemmWork w;
  w.bm = (NFAST ? tile / nn : tile % nm) * BM;
  w.bn = (NFAST ? tile % nn : tile / nm) * BN;
  w.whole = z < 0;
  if (z < 0) {
    w.kbeg = 0;
    w.kend = K;
    w.out = C;
    w.ldo = ldc;
  } else {
    w.kbeg = z * kps;
    w.kend = min(K, w.kbeg + kps);
    w.out = P + z * M * N;
    w.ldo = N;
  }
  return w;
}


__device__ __forceinline__ float f4at(const float4& v, int j) {
  return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
}

// A whole 128 x 256 tile also stored as a bf16 copy transposed, T[c][r]
// (row stride e.ldt) for its columns c and rows r.  The accumulators pass
// through LDS as bf16 [256 columns][128 rows + 8] (the B staging area), so
// each thread then writes 16-byte chunks of 8 rows of one column.  M % 8 == 0.
constexpr int TC_LD = 136;
__device__ __forceinline__ void tcopy_tile_epilogue(const ActEpi& e, int64_t M, int64_t N,
                                                    int64_t bm, int64_t bn, int wm, int wn,
                                                    const floatx4 (&acc)[4][4],
                                                    uint16_t* stage) {
  const int t = threadIdx.x, lane = t & 63;
  uint16_t* T = (uint16_t*)e.out;
  __syncthreads();  // every wave is past its last LDS read of the k-loop
#pragma unroll
  for (int fi = 0; fi < 4; ++fi)
#pragma unroll
    for (int fj = 0; fj < 4; ++fj)
#pragma unroll
      for (int v = 0; v < 4; v += 2) {
        const int row = wm + fi * 16 + 4 * (lane >> 4) + v, col = wn + fj * 16 + (lane & 15);
        *reinterpret_cast<uint32_t*>(&stage[col * TC_LD + row]) =
            pk_bf16(acc[fi][fj][v], acc[fi][fj][v + 1]);
      }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int ch = t + 512 * i, col = ch >> 4, r8 = 8 * (ch & 15);
    const int64_t gc = bn + col, gr = bm + r8;
    if (gc < N && gr < M)
      *reinterpret_cast<uint4*>(T + gc * e.ldt + gr) =
          *reinterpret_cast<const uint4*>(&stage[col * TC_LD + r8]);
  }
}

// The store of a product's 128 x 256 tile: through the activation backward
// for a whole tile of an ACT-epilogue launch, else plain (C, or a partial
// slot), for EPI 16 plus the transposed bf16 copy.  EPI: 0 plain, 16
// transposed copy, else 1 + act + 2 (gate/up bf16) + 4 (out bf16).
template <int EPI>
__device__ __forceinline__ void store_out(const ActEpi& e, const GemmWork& wk, int64_t M,
                                          int64_t N, int wm, int wn, const floatx4 (&acc)[4][4],
                                          float* stage) {
  if constexpr (EPI == 16) {
    store_tile<4, 4>(wk.out, wk.ldo, M, N, wk.bm + wm, wk.bn + wn, acc);
    if (wk.whole)
      tcopy_tile_epilogue(e, M, N, wk.bm, wk.bn, wm, wn, acc, reinterpret_cast<uint16_t*>(stage));
    return;
  } else if constexpr (EPI != 0) {
    if (wk.whole) {
      constexpr int ACT = (EPI - 1) & 1;
      constexpr bool GB = ((EPI - 1) & 2) != 0, OB = ((EPI - 1) & 4) != 0;
      typedef typename std::conditional<GB, bf16, float>::type TG;
      typedef typename std::conditional<OB, bf16, float>::type TO;
      act_tile_epilogue<TG, TO, ACT>(e, M, N, wk.bm, wk.bn, wm, wn, acc, stage);
      return;
    }
  }
  store_tile<4, 4>(wk.out, wk.ldo, M, N, wk.bm + wm, wk.bn + wn, acc);
}

template <int EPI, bool AT>
__global__ __launch_bounds__(F_NT) void gemm_f32_kernel(int64_t M, int64_t N, int64_t K,
                                                        const float* __restrict__ A, int64_t lda,
                                                        const float* __restrict__ B1,
                                                        const float* __restrict__ B2, int64_t K1,
                                                        int64_t ldb, float* __restrict__ C,
                                                        int64_t ldc, float* __restrict__ P,
                                                        int64_t kps, int64_t nfull, ActEpi epi,
                                                        AdamEpi adam) {
  constexpr int NA = F_BM * F_BK / 4 / F_NT;   // A float4 per thread (2)
  constexpr int NBQ = F_BK * F_BN / 4 / F_NT;  // B k-quads per thread (4)
  constexpr int BQS = F_NT / F_BN;             // k-quad stride between them (2)
  __shared__ __attribute__((aligned(16))) float As[2][F_BM][F_LD];
  __shared__ __attribute__((aligned(16))) float Bs[2][F_BN][F_LD];
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform
  const int l16 = lane & 15, c = lane >> 4;
  // 1-D grid of work items (gemm_work), m fastest, so the row tiles that
  // read one weight panel run together on one XCD.
  const GemmWork wk = gemm_work<F_BM, F_BN, AT>(M, N, K, kps, nfull, C, ldc, P);
  const int64_t bm = wk.bm, bn = wk.bn, kbeg = wk.kbeg, kend = wk.kend;
  const int wm = (w & 1) * 64, wn = (w >> 1) * 64;

  // A: rows (t/8) + 64 i, k quad t%8.  B: column t % 256, k quads t/256 + 2i
  // (the quad index is uniform across a wave, so its source matrix is picked
  // with a scalar select).  Loads are buffer loads whose bounds are offsets:
  // out of range reads 0, a k-tile past the end is all zeros, and no branch
  // splits the prefetch pipeline.
  const int am = t >> 3, ak = 4 * (t & 7), bc = t % F_BN, bq0 = w / (F_BN / 64);
  const int64_t mrows = min((int64_t)F_BM, M - bm);
  // (with AT the rows' range is not used: a quad's resource is made per load)
  const brsrc_t ra = make_brsrc(A + bm * lda, AT ? 0u : (uint32_t)(((mrows - 1) * lda + K) * 4));
  const uint32_t bcoff = bn + bc < N ? (uint32_t)(bc * 4) : BUF_OOB;
  // (AT) column t % 128 of the tile, k quads t / 128 + 4 i (t / 128 = w / 2,
  // uniform across a wave, so each quad's resource is a scalar)
  const int atc = t % F_BM, aq0 = w >> 1;
  static_assert(F_BM == 128 && F_NT / F_BM * 8 == F_BK, "AT gather covers one k-tile");
  const uint32_t acoff = atc < mrows ? (uint32_t)(atc * 4) : BUF_OOB;
  // the rows of a k quad inside the k-range (a range of 0 to 4 rows: a
  // quad that runs past kend reads zeros there)
  auto qrows = [&](int64_t kq) -> uint32_t {
    const int64_t n = kend - kq;
    return n <= 0 ? 0u : (uint32_t)(n < 4 ? n : 4);
  };
  struct Stage {
    float4 a[NA], b[NBQ];
  };
  auto load = [&](Stage& r, int64_t k0) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      if constexpr (AT) {
        const int64_t kq = k0 + 4 * (aq0 + 4 * i);
        const brsrc_t rt = make_brsrc(A + kq * lda + bm, qrows(kq) * (uint32_t)(lda * 4));
        float v[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          v[jj] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
              rt, (int)(acoff + (uint32_t)(jj * lda * 4)), 0, 0));
        r.a[i] = make_float4(v[0], v[1], v[2], v[3]);
      } else {
        const int m = am + 64 * i;
        const int64_t k = k0 + ak;
        r.a[i] = bload_f4(ra, (m < mrows && k < kend) ? (uint32_t)((m * lda + k) * 4) : BUF_OOB);
      }
    }
#pragma unroll
    for (int i = 0; i < NBQ; ++i) {
      const int64_t kq = k0 + 4 * (bq0 + BQS * i);  // K1 is a multiple of 4
      const bool s1 = kq < K1;
      // without AT, K is a multiple of 4 (the layer's feature sizes): a
      // quad is whole or past the end
      const uint32_t brange = AT ? qrows(kq) * (uint32_t)(ldb * 4)
                                 : (kq < kend ? (uint32_t)(4 * ldb * 4) : 0u);
      const brsrc_t rb = make_brsrc((s1 ? B1 + kq * ldb : B2 + (kq - K1) * ldb) + bn, brange);
      float v[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        v[jj] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            rb, (int)(bcoff + (uint32_t)(jj * ldb * 4)), 0, 0));
      r.b[i] = make_float4(v[0], v[1], v[2], v[3]);
    }
  };
  auto stash = [&](const Stage& r, int buf) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      if constexpr (AT)
        *reinterpret_cast<float4*>(&As[buf][atc][4 * (aq0 + 4 * i)]) = r.a[i];
      else
        *reinterpret_cast<float4*>(&As[buf][am + 64 * i][ak]) = r.a[i];
    }
#pragma unroll
    for (int i = 0; i < NBQ; ++i)
      *reinterpret_cast<float4*>(&Bs[buf][bc][4 * (bq0 + BQS * i)]) = r.b[i];
  };
  floatx4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int buf) {
    // operands of both 16-k halves first
    float4 a[2][4], b[2][4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[kb][i] = *reinterpret_cast<const float4*>(&As[buf][wm + 16 * i + l16][16 * kb + 4 * c]);
        b[kb][i] = *reinterpret_cast<const float4*>(&Bs[buf][wn + 16 * i + l16][16 * kb + 4 * c]);
      }
    // one MFMA per accumulator per k step: 16 independent chains
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            acc[i][jj] = mfma16x16x4(f4at(a[kb][i], q), f4at(b[kb][jj], q), acc[i][jj]);
  };

  // Three k-tiles in flight: the LDS buffer in use and two register stages
  // (an odd tile count ends with a tile of zeros).
  Stage s0, s1;
  load(s0, kbeg);
  stash(s0, 0);
  load(s0, kbeg + F_BK);
  load(s1, kbeg + 2 * F_BK);
  __syncthreads();
  for (int64_t k0 = kbeg; k0 < kend; k0 += 2 * F_BK) {
    compute(0);
    stash(s0, 1);
    __syncthreads();
    load(s0, k0 + 3 * F_BK);
    compute(1);
    stash(s1, 0);
    __syncthreads();
    load(s1, k0 + 4 * F_BK);
  }
  if constexpr (EPI == 32)
    adam_tile_epilogue(adam, M, N, bm, bn, wm, wn, acc, &Bs[0][0][0]);
  else
    store_out<EPI>(epi, wk, M, N, wm, wn, acc, &Bs[0][0][0]);
}

// ---------------------------------------------------------------------------
// bf16 GEMM: 512 threads, tile 128 x 256, BK = 64, waves 2 x 4 of 64 x 64
// (v_mfma_f32_16x16x32_bf16).  A (bf16; launch_gemm rounds an fp32 A first)
// sits in LDS k-contiguous, As[m][k], and is read with one 16-byte load per
// operand.  B keeps its memory layout in LDS, Bs[k][n], filled with
// plain 16-byte copies; the LDS transpose read turns four k-rows of a column
// into one lane's operand half.  Double-buffered, one barrier per k-tile;
// the operands of each half k-tile are read into registers during the
// previous half's MFMAs (seq 2048 bf16 W_down 128.6 -> 122.6 us, gate/up
// 236 -> 223 us), and two register stages keep the global loads of the
// next two k-tiles in flight (gate/up 219.5 -> 212.3 us).
constexpr int H_BM = 128, H_BN = 256, H_BK = 64, H_NT = 512;
constexpr int H_LDA = H_BK + 8, H_LDB = H_BN + 16;
static_assert(2 * H_BK * H_LDB * 2 >= 64 * EPI_LD * 4, "activation stage fits in Bs");
static_assert(2 * H_BK * H_LDB >= H_BN * TC_LD, "transposed-copy stage fits in Bs");

template <bool SPLITB, int EPI>
__global__ __launch_bounds__(H_NT) void gemm_bf16_kernel(int64_t M, int64_t N, int64_t K,
                                                         const uint16_t* __restrict__ A, int64_t lda,
                                                         const uint16_t* __restrict__ B1,
                                                         const uint16_t* __restrict__ B2,
                                                         int64_t K1, int64_t ldb,
                                                         float* __restrict__ C, int64_t ldc,
                                                         float* __restrict__ P, int64_t kps,
                                                         int64_t nfull, ActEpi epi) {
  constexpr int NA = H_BM * H_BK / 8 / H_NT;  // A chunks of 8 per thread (2)
  constexpr int NB = H_BK * H_BN / 8 / H_NT;  // B chunks of 8 per thread (4)
  // One k-tile of global data in registers
  struct Stage {
    uint4 a[NA];
    uint4 b[NB];
  };
  __shared__ __attribute__((aligned(16))) uint16_t As[2][H_BM][H_LDA];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][H_BK][H_LDB];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int l16 = lane & 15, c = lane >> 4;
  const GemmWork wk = gemm_work<H_BM, H_BN>(M, N, K, kps, nfull, C, ldc, P);
  const int64_t bm = wk.bm, bn = wk.bn, kbeg = wk.kbeg, kend = wk.kend;
  const int wm = (w & 1) * 64, wn = (w >> 1) * 64;

  // Loads are buffer loads whose bounds are offsets (out of range reads 0):
  // no branch splits the prefetch pipeline, and a k-tile past the end is all
  // zeros.  A: the tile's rows as one range.  B: the rows of one k-tile,
  // from W1 (rows < K1) or W2; with SPLITB (K1 not a multiple of the tile)
  // every chunk reads both sources, each masked to its own rows.
  const int64_t mrows = min((int64_t)H_BM, M - bm);
  const brsrc_t ra = make_brsrc(A + bm * lda, (uint32_t)(((mrows - 1) * lda + K) * 2));
  auto brows = [&](const uint16_t* Bs_, int64_t r0, int64_t nrows) -> brsrc_t {
    return make_brsrc(Bs_ + r0 * ldb + bn, nrows > 0 ? (uint32_t)(nrows * ldb * 2) : 0u);
  };
  auto load = [&](Stage& r, int64_t k0) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int e = t + H_NT * i;
      const int m = e >> 3;
      const int64_t k = k0 + 8 * (e & 7);
      r.a[i] = bload_u4(ra, (m < mrows && k < kend) ? (uint32_t)((m * lda + k) * 2) : BUF_OOB);
    }
    if (!SPLITB) {
      // the whole tile lies in one source (K1 is a multiple of the tile)
      const bool s1 = k0 < K1;
      const int64_t r0 = s1 ? k0 : k0 - K1;
      const int64_t nrows = min(kend, s1 ? K1 : K) - k0;
      const brsrc_t rb = brows(s1 ? B1 : B2, r0, nrows);
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int e = t + H_NT * i;
        const int kk = e >> 5, n = 8 * (e & 31);  // N % 8 == 0: a chunk is whole
        const uint32_t off = (kk < nrows && bn + n < N) ? (uint32_t)((kk * ldb + n) * 2) : BUF_OOB;
        r.b[i] = bload_u4(rb, off);
      }
    } else {
      const int64_t n1 = min(kend, K1) - k0;   // rows of this tile in W1
      const int64_t r2 = k0 > K1 ? k0 - K1 : 0, lo2 = K1 > k0 ? K1 - k0 : 0;
      const brsrc_t rb1 = brows(B1, k0 < K1 ? k0 : 0, n1);
      const brsrc_t rb2 = brows(B2, r2, min(kend, K) - k0 - lo2);
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int e = t + H_NT * i;
        const int kk = e >> 5, n = 8 * (e & 31);
        const bool nok = bn + n < N && k0 + kk < kend;
        const uint32_t o1 = (nok && kk < n1) ? (uint32_t)((kk * ldb + n) * 2) : BUF_OOB;
        const uint32_t o2 = (nok && kk >= lo2) ? (uint32_t)(((kk - lo2) * ldb + n) * 2) : BUF_OOB;
        const uint4 v1 = bload_u4(rb1, o1), v2 = bload_u4(rb2, o2);
        r.b[i] = make_uint4(v1.x | v2.x, v1.y | v2.y, v1.z | v2.z, v1.w | v2.w);
      }
    }
  };
  auto stash = [&](const Stage& r, int buf) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int e = t + H_NT * i;
      *reinterpret_cast<uint4*>(&As[buf][e >> 3][8 * (e & 7)]) = r.a[i];
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int e = t + H_NT * i;
      const int row = e >> 5;  // column chunk swizzled as lds_colk8<true> reads it
      *reinterpret_cast<uint4*>(&Bs[buf][row][(8 * (e & 31)) ^ (64 * ((row >> 3) & 1))]) = r.b[i];
    }
  };
  floatx4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  // the MFMA operands of one half k-tile (k = 32 ks .. 32 ks + 31), read
  // from LDS into registers
  struct Half {
    ushortx8 a[4], b[4];
  };
  auto read_half = [&](Half& o, int buf, int ks) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o.a[i] = *reinterpret_cast<const ushortx8*>(&As[buf][wm + 16 * i + l16][32 * ks + 8 * c]);
      o.b[i] = lds_colk8<true>(&Bs[buf][0][0], H_LDB, 32 * ks, wn + 16 * i, lane);
    }
  };
  auto mma_half = [&](const Half& o) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32bf16(o.a[i], o.b[j], acc[i][j]);
  };

  // Pipeline in half k-tiles: the MFMAs of one half run from registers while
  // the operands of the next half are read from LDS, so the LDS reads never
  // wait for a barrier with the MFMA pipe idle.  Tile k sits in LDS buffer
  // X, tile k+1 in Y.  Phase A: read (k, second half) from X, MFMAs of (k,
  // first half); barrier (every read of X is complete).  Phase B: read
  // (k+1, first half) from Y, MFMAs of (k, second half), tile k+2 copied
  // from the register stage into X, tile k+3's global loads issued.  Loads
  // past the end read 0.
  Half h0, h1;
  auto step = [&](int buf, Stage& sx, int64_t knext) {
    read_half(h1, buf, 1);
    __builtin_amdgcn_sched_barrier(0);
    mma_half(h0);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    read_half(h0, buf ^ 1, 0);
    __builtin_amdgcn_sched_barrier(0);
    mma_half(h1);
    __builtin_amdgcn_sched_barrier(0);
    stash(sx, buf);
    load(sx, knext);
  };
  if constexpr (!SPLITB) {
    // two register stages used in turn: tiles k+2 and k+3 are in flight
    // while tile k is multiplied (an odd tile count ends with a tile of
    // zeros); the two-source loads of SPLITB leave no registers for it
    Stage s0, s1;
    load(s0, kbeg);
    stash(s0, 0);
    load(s0, kbeg + H_BK);
    load(s1, kbeg + 2 * H_BK);
    __syncthreads();
    stash(s0, 1);
    load(s0, kbeg + 3 * H_BK);
    read_half(h0, 0, 0);
    __syncthreads();
    for (int64_t k0 = kbeg; k0 < kend; k0 += 2 * H_BK) {
      step(0, s1, k0 + 4 * H_BK);
      step(1, s0, k0 + 5 * H_BK);
    }
  } else {
    Stage st;
    load(st, kbeg);
    stash(st, 0);
    load(st, kbeg + H_BK);
    __syncthreads();
    stash(st, 1);
    load(st, kbeg + 2 * H_BK);
    read_half(h0, 0, 0);
    __syncthreads();
    int buf = 0;
    for (int64_t k0 = kbeg; k0 < kend; k0 += H_BK) {
      step(buf, st, k0 + 3 * H_BK);
      buf ^= 1;
    }
  }
  store_out<EPI>(epi, wk, M, N, wm, wn, acc, reinterpret_cast<float*>(&Bs[0][0][0]));
}

// ---------------------------------------------------------------------------
// Wide bf16 GEMM for plain products (no epilogue, one B source per k-tile):
// tile 256 x 256, BK = 64, 8 waves of 128 x 64 (8 x 4 MFMA accumulators).
// Per MFMA a wave reads 25 % fewer LDS bytes than with 64 x 64 wave tiles,
// and the tile copies 27 % fewer bytes into LDS per flop.  The accumulators
// (128 registers) leave room for one register stage of global loads and one
// half k-tile of operands at two waves per SIMD: the operand reads of one
// wave overlap the MFMAs of the other.  LDS: A [2][256][72], B [2][64][272]
// (swizzled as lds_colk8<true> reads it), 143 KB.  One barrier per k-tile:
// tile k+1 goes from registers into the buffer read two tiles ago, tile k+2's
// loads are issued, tile k is multiplied.
constexpr int W_BM = 256, W_BN = 256;
static_assert(2 * W_BM * H_LDA * 2 >= 64 * EPI_LD * 4, "activation stage fits in As (both buffers)");
// EPI: 0 plain, or (7, 8) the activation epilogue of whole tiles as in the
// narrow kernel (bf16 gate/up and output).
template <int EPI>
__global__ __launch_bounds__(H_NT) void gemm_bf16w_kernel(int64_t M, int64_t N, int64_t K,
                                                          const uint16_t* __restrict__ A,
                                                          int64_t lda,
                                                          const uint16_t* __restrict__ B1,
                                                          const uint16_t* __restrict__ B2,
                                                          int64_t K1, int64_t ldb,
                                                          float* __restrict__ C, int64_t ldc,
                                                          float* __restrict__ P, int64_t kps,
                                                          int64_t nfull, ActEpi epi) {
  constexpr int NA = W_BM * H_BK / 8 / H_NT;  // A chunks of 8 per thread (4)
  constexpr int NB = H_BK * W_BN / 8 / H_NT;  // B chunks of 8 per thread (4)
  struct Stage {
    uint4 a[NA];
    uint4 b[NB];
  };
  __shared__ __attribute__((aligned(16))) uint16_t As[2][W_BM][H_LDA];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][H_BK][H_LDB];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int l16 = lane & 15, c = lane >> 4;
  const GemmWork wk = gemm_work<W_BM, W_BN>(M, N, K, kps, nfull, C, ldc, P);
  const int64_t bm = wk.bm, bn = wk.bn, kbeg = wk.kbeg, kend = wk.kend;
  const int wm = (w & 1) * 128, wn = (w >> 1) * 64;
  const int64_t mrows = min((int64_t)W_BM, M - bm);
  const brsrc_t ra = make_brsrc(A + bm * lda, (uint32_t)(((mrows - 1) * lda + K) * 2));
  auto load = [&](Stage& r, int64_t k0) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int e = t + H_NT * i;
      const int m = e >> 3;
      const int64_t k = k0 + 8 * (e & 7);
      r.a[i] = bload_u4(ra, (m < mrows && k < kend) ? (uint32_t)((m * lda + k) * 2) : BUF_OOB);
    }
    // the whole k-tile lies in one source (K1 is a multiple of the tile)
    const bool s1 = k0 < K1;
    const int64_t r0 = s1 ? k0 : k0 - K1;
    const int64_t nrows = min(kend, s1 ? K1 : K) - k0;
    const brsrc_t rb = make_brsrc((s1 ? B1 : B2) + r0 * ldb + bn,
                                  nrows > 0 ? (uint32_t)(nrows * ldb * 2) : 0u);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int e = t + H_NT * i;
      const int kk = e >> 5, n = 8 * (e & 31);  // N % 8 == 0: a chunk is whole
      const uint32_t off = (kk < nrows && bn + n < N) ? (uint32_t)((kk * ldb + n) * 2) : BUF_OOB;
      r.b[i] = bload_u4(rb, off);
    }
  };
  auto stash = [&](const Stage& r, int buf) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int e = t + H_NT * i;
      *reinterpret_cast<uint4*>(&As[buf][e >> 3][8 * (e & 7)]) = r.a[i];
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int e = t + H_NT * i;
      const int row = e >> 5;
      *reinterpret_cast<uint4*>(&Bs[buf][row][(8 * (e & 31)) ^ (64 * ((row >> 3) & 1))]) = r.b[i];
    }
  };
  floatx4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  // B operands of both halves first, then row block by row block: each A
  // operand is read just ahead of its four MFMAs
  auto compute = [&](int buf) {
    ushortx8 b[2][4];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[ks][j] = lds_colk8<true>(&Bs[buf][0][0], H_LDB, 32 * ks, wn + 16 * j, lane);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const ushortx8 a =
            *reinterpret_cast<const ushortx8*>(&As[buf][wm + 16 * i + l16][32 * ks + 8 * c]);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32bf16(a, b[ks][j], acc[i][j]);
      }
  };
  Stage st;
  load(st, kbeg);
  stash(st, 0);
  load(st, kbeg + H_BK);
  __syncthreads();
  int buf = 0;
  for (int64_t k0 = kbeg; k0 < kend; k0 += H_BK) {
    // buffer buf ^ 1 was last read in the previous iteration (before its
    // barrier): it takes tile k+1 now
    stash(st, buf ^ 1);
    load(st, k0 + 2 * H_BK);
    compute(buf);
    __syncthreads();
    buf ^= 1;
  }
  if constexpr (EPI != 0) {
    if (wk.whole) {
      constexpr int ACT = (EPI - 1) & 1;
      act_tile_epilogue<bf16, bf16, ACT, 8>(epi, M, N, bm, bn, wm, wn, acc,
                                            reinterpret_cast<float*>(&As[0][0][0]));
      return;
    }
  }
  // output: wave rows wm + 16 i .., columns wn + 16 j ..
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = bn + wn + 16 * j + l16;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t row = bm + wm + 16 * i + 4 * c + v;
        if (row < M && col < N) wk.out[row * wk.ldo + col] = acc[i][j][v];
      }
    }
}

// ---------------------------------------------------------------------------
// Fixed-order reduction of split-K partials: C[m, n] = sum_s P[s, m, n],
// over the split tiles only -- columns n >= n0, except the rows m < mskip of
// the first column panel [n0, n0 + bn), which were whole tiles.
template <int EPI>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(int64_t M, int64_t N, int splits,
                                                            const float* __restrict__ P,
                                                            float* __restrict__ C, int64_t ldc,
                                                            int64_t n0, int64_t bn, int64_t mskip,
                                                            ActEpi epi) {
  const int64_t q = (N - n0) / 4;
  const int64_t total = M * q;
  const int64_t stride = M * N;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = t / q, n = n0 + (t - m * q) * 4;
    if (m < mskip && n < n0 + bn) continue;
    const float* p = P + m * N + n;
    // the partials of up to 8 splits in flight at a time, added in split order
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int i0 = 0; i0 < splits; i0 += 8) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        // a split index past the end re-reads the last split (a valid
        // address, no branch) and its term is dropped below
        const int i = i0 + u < splits ? i0 + u : splits - 1;
        v[u] = *reinterpret_cast<const float4*>(p + i * stride);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const bool take = i0 + u < splits;
        s.x += take ? v[u].x : 0.f;
        s.y += take ? v[u].y : 0.f;
        s.z += take ? v[u].z : 0.f;
        s.w += take ? v[u].w : 0.f;
      }
    }
    if constexpr (EPI != 0) {
      // through the activation backward (see store_tile_act)
      constexpr int ACT = (EPI - 1) & 1;
      constexpr bool GB = ((EPI - 1) & 2) != 0, OB = ((EPI - 1) & 4) != 0;
      typedef typename std::conditional<GB, bf16, float>::type TG;
      const float4 g = Act<TG>::ld4((const TG*)epi.gate, m * N + n);
      const float4 u = Act<TG>::ld4((const TG*)epi.up, m * N + n);
      float4 dg, du;
      act_bwd1<ACT>(g.x, u.x, s.x, dg.x, du.x);
      act_bwd1<ACT>(g.y, u.y, s.y, dg.y, du.y);
      act_bwd1<ACT>(g.z, u.z, s.z, dg.z, du.z);
      act_bwd1<ACT>(g.w, u.w, s.w, dg.w, du.w);
      if constexpr (OB) {
        uint16_t* o = (uint16_t*)epi.out + m * 2 * N + n;
        *reinterpret_cast<uint2*>(o) = make_uint2(pk_bf16(dg.x, dg.y), pk_bf16(dg.z, dg.w));
        *reinterpret_cast<uint2*>(o + N) = make_uint2(pk_bf16(du.x, du.y), pk_bf16(du.z, du.w));
      } else {
        float* o = (float*)epi.out + m * 2 * N + n;
        *reinterpret_cast<float4*>(o) = dg;
        *reinterpret_cast<float4*>(o + N) = du;
      }
    } else {
      *reinterpret_cast<float4*>(C + m * ldc + n) = s;
    }
  }
}

static inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Work split from a small cost model.  The CUs take the workgroups in
// rounds of 256 (one per CU: LDS); a whole tile lasts its k-range at the rate
// measured for the kernel.  The first nfull tiles (whole rounds) run whole;
// the rest are split in nsp k-chunks so the ragged last round is short, at
// the cost of an HBM round trip of their partial sums.  nfull = 0 is plain
// split-K.
struct GemmPlan {
  int bm, bn, nsp;
  int64_t kps, nfull;
};
static GemmPlan gemm_plan(int64_t M, int64_t N, int64_t K, int b_dt, bool wide = false) {
  const bool f32 = b_dt == F32;
  const int bm = f32 ? F_BM : (wide ? W_BM : H_BM), bn = f32 ? F_BN : (wide ? W_BN : H_BN);
  const int bk = f32 ? F_BK : H_BK;
  const int64_t slots = 256;
  // ns per k index for one tile: 2 bm bn flops at the sustained MFMA rate
  const double ns_per_k = f32 ? 2.0 * bm * bn / (256.0 * 0.74 * 2.4)
                              : 2.0 * bm * bn / (4069.0 * 0.5 * 2.4);
  const int64_t tiles = cdiv(M, bm) * cdiv(N, bn);
  const double tile_bytes = (double)std::min((int64_t)bm, M) * std::min((int64_t)bn, N) * 4;
  GemmPlan best{bm, bn, 1, K, tiles};
  double best_t = (double)cdiv(tiles, slots) * K * ns_per_k * 1e-3;  // us
  for (int64_t r = 0; r * slots < tiles; ++r) {
    const int64_t nfull = r * slots, tail = tiles - nfull;
    for (int s = 2; s <= 16; ++s) {
      const int64_t kps = cdiv(cdiv(K, s), 64) * 64;
      const int nsp = (int)cdiv(K, kps);
      if (nsp != s) continue;
      if (kps < 4 * bk) break;
      double tt = ((double)r * K + (double)cdiv(tail * nsp, slots) * kps) * ns_per_k * 1e-3;
      tt += (2.0 * nsp + 1) * tail * tile_bytes / 6.0e6;  // us at 6 TB/s
      if (tt < best_t * 0.98) {
        best_t = tt;
        best = GemmPlan{bm, bn, nsp, kps, nfull};
      }
    }
  }
  return best;
}

// The wide bf16 kernel takes plain products with at least two of its tiles
// in each direction.
static bool wide_ok(int64_t M, int64_t N, int b_dt) {
  return b_dt == BF16 && M >= 2 * W_BM && N >= 2 * W_BN;
}

int gemm_splits(int64_t M, int64_t N, int64_t K, int b_dt) {
  const int s = gemm_plan(M, N, K, b_dt).nsp;
  const int sw = wide_ok(M, N, b_dt) ? gemm_plan(M, N, K, b_dt, true).nsp : 1;
  return s > sw ? s : sw;  // partial slots for whichever kernel runs
}

// Scratch of launch_gemm: the split-K partials, then (bf16 weights with an
// fp32 A) A rounded to bf16, [M][K] -- the MFMA kernel then reads 2 bytes per
// A element instead of 4 and keeps no conversion in its k-loop.
static size_t gemm_part_only(int64_t M, int64_t N, int64_t K, int b_dt) {
  const int s = gemm_splits(M, N, K, b_dt);
  return s > 1 ? ((size_t)s * M * N * sizeof(float) + 255) / 256 * 256 : 0;
}
size_t gemm_partial_bytes(int64_t M, int64_t N, int64_t K, int a_dt, int b_dt) {
  size_t b = gemm_part_only(M, N, K, b_dt);
  if (a_dt == F32 && b_dt != F32) b += ((size_t)M * K * 2 + 255) / 256 * 256;
  return b;
}

// A (fp32, row stride lda) -> bf16 [M][K], round to nearest even (K % 8 == 0)
__global__ __launch_bounds__(256) void cvt_a_bf16_kernel(int64_t M, int64_t K, const float* __restrict__ A,
                                                         int64_t lda, uint16_t* __restrict__ out) {
  const int64_t q = K / 8, total = M * q;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t m = i / q, k = (i - m * q) * 8;
    const float4 x = *reinterpret_cast<const float4*>(A + m * lda + k);
    const float4 y = *reinterpret_cast<const float4*>(A + m * lda + k + 4);
    *reinterpret_cast<uint4*>(out + m * K + k) =
        make_uint4(pk_bf16(x.x, x.y),
                   pk_bf16(x.z, x.w),
                   pk_bf16(y.x, y.y),
                   pk_bf16(y.z, y.w));
  }
}

hipError_t launch_gemm(int64_t M, int64_t N, int64_t K, const void* A, int a_dt, int64_t lda,
                       const void* B1, const void* B2, int64_t K1, int b_dt, int64_t ldb,
                       float* C, int64_t ldc, float* partials, hipStream_t s, int* deferred,
                       const ActEpi* act, bool* act_done, const TCopy* tc, bool* tc_done) {
  const int a_dt0 = a_dt;  // the operand as the caller holds it
  if (deferred) *deferred = 1;
  if (act_done) *act_done = false;
  if (tc_done) *tc_done = false;
  if (M == 0 || N == 0) return hipSuccess;
  // bf16 products with enough tiles and one source per k-tile take the wide
  // kernel (the transposed-copy store stays on the narrow one)
  const bool wide = wide_ok(M, N, b_dt) && (B2 == nullptr || K1 % H_BK == 0) && tc == nullptr;
  const GemmPlan pl = gemm_plan(M, N, K, b_dt, wide);
  const int64_t kps = pl.kps, nfull = pl.nfull;
  const int nsp = pl.nsp;
  // the activation epilogue: whole tiles apply it as they store, a split
  // tail is reduced through it; a plain split-K product leaves its partials
  // (the caller's activation pass adds them) -- and gate/up/out take the
  // weights' dtype
  const bool use_act = act != nullptr && (nsp == 1 || nfull > 0) &&
                       act->gdt == b_dt && act->odt == b_dt && ldc == N && N % 8 == 0 &&
                       (double)std::min<int64_t>(pl.bm, M) * N * 4 < BUF_MAX_BYTES;
  // the transposed bf16 copy: every tile whole, bf16 operands
  const bool use_tc = !use_act && tc != nullptr && tc_done != nullptr && nsp == 1 &&
                      b_dt == BF16 && a_dt == BF16 && M % 8 == 0 && tc->ld % 8 == 0;
  const int epi = use_act ? 1 + act->act + (b_dt == BF16 ? 6 : 0) : (use_tc ? 16 : 0);
  ActEpi ea = use_act ? *act : ActEpi{};
  if (use_tc) {
    ea.out = tc->dst;
    ea.ldt = tc->ld;
  }
  if (act_done) *act_done = use_act;
  if (tc_done) *tc_done = use_tc;
  // buffer ranges: one tile's rows of A (no more than M), one k-tile of B
  // (an fp32 A of the bf16 path is first rounded into a dense bf16 [M][K]
  // copy)
  if (b_dt == F32) {
    const double ar = (double)std::min<int64_t>(F_BM, M) - 1;
    if ((ar * lda + K) * 4 >= BUF_MAX_BYTES || 16.0 * ldb >= BUF_MAX_BYTES)
      return hipErrorInvalidValue;
  } else {
    const double la = a_dt == F32 ? (double)K : (double)lda;
    const double ar = (double)std::min<int64_t>(W_BM, M) - 1;
    if ((ar * la + K) * 2 >= BUF_MAX_BYTES || (double)H_BK * ldb * 2 >= BUF_MAX_BYTES)
      return hipErrorInvalidValue;
  }
  if (dry_run()) {
    if (deferred && nsp > 1 && nfull == 0) *deferred = nsp;
    return hipSuccess;
  }
  const int64_t tiles = cdiv(N, pl.bn) * cdiv(M, pl.bm);
  const dim3 grid1((unsigned)(nfull + (tiles - nfull) * nsp));
  if (B2 == nullptr) {
    B2 = B1;
    K1 = K;
  }
  const dim3 block(256);
  if (b_dt == F32) {
#define LBP_GEMM_F32(E)                                                                        \
  gemm_f32_kernel<E, false><<<grid1, dim3(F_NT), 0, s>>>(                                    \
      M, N, K, (const float*)A, lda, (const float*)B1, (const float*)B2, K1, ldb, C, ldc,      \
      partials, kps, nfull, ea, AdamEpi{})
    if (epi == 1) LBP_GEMM_F32(1);
    else if (epi == 2) LBP_GEMM_F32(2);
    else LBP_GEMM_F32(0);
#undef LBP_GEMM_F32
  } else {
    if (a_dt == F32) {
      // A to bf16 once, into the scratch after the partials
      uint16_t* a16 = (uint16_t*)((char*)partials + gemm_part_only(M, N, K, b_dt));
      int64_t blocks = cdiv(M * (K / 8), 256);
      if (blocks > 8192) blocks = 8192;
      cvt_a_bf16_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(M, K, (const float*)A, lda, a16);
      mark("cvt_a_bf16", 0, 0, s, (double)M * K * 6);  // a rounded copy of A
      if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
      A = a16;
      a_dt = BF16;
      lda = K;
    }
    const bool splitb = K1 % H_BK != 0;
    if (wide) {
#define LBP_GEMM_W(E)                                                                         \
  gemm_bf16w_kernel<E><<<grid1, dim3(H_NT), 0, s>>>(M, N, K, (const uint16_t*)A, lda,          \
                                                    (const uint16_t*)B1, (const uint16_t*)B2, K1, \
                                                    ldb, C, ldc, partials, kps, nfull, ea)
      if (epi == 7) LBP_GEMM_W(7);
      else if (epi == 8) LBP_GEMM_W(8);
      else LBP_GEMM_W(0);
#undef LBP_GEMM_W
    } else {
#define LBP_GEMM_BF16(SB, E)                                                                \
  gemm_bf16_kernel<SB, E><<<grid1, dim3(H_NT), 0, s>>>(M, N, K, (const uint16_t*)A, lda,      \
                                                      (const uint16_t*)B1, (const uint16_t*)B2, \
                                                      K1, ldb, C, ldc, partials, kps, nfull, ea)
    if (epi == 7) {
      if (splitb) LBP_GEMM_BF16(true, 7);
      else LBP_GEMM_BF16(false, 7);
    } else if (epi == 8) {
      if (splitb) LBP_GEMM_BF16(true, 8);
      else LBP_GEMM_BF16(false, 8);
    } else if (epi == 16) {
      if (splitb) LBP_GEMM_BF16(true, 16);
      else LBP_GEMM_BF16(false, 16);
    } else {
      if (splitb) LBP_GEMM_BF16(true, 0);
      else LBP_GEMM_BF16(false, 0);
    }
#undef LBP_GEMM_BF16
    }
  }
  hipError_t e = hipGetLastError();
  // with the activation epilogue the product's output is [dGate | dUp] from
  // gate and up (weights' dtype) instead of C
  const double es = b_dt == F32 ? 4 : 2;
  // A at the type the caller holds it (a rounded copy is implementation
  // traffic), B once, the result once (with the activation epilogue: gate and
  // up read, [dGate | dUp] written, in place of dHid); split-K partials and
  // the transposed bf16 copy are implementation traffic
  mark(b_dt == F32 ? "gemm_f32_mfma" : "gemm_bf16_mfma",
       (double)M * K * (a_dt0 == F32 ? 4 : 2) + (double)K * N * es +
           (use_act ? (double)M * N * 4 * es : (double)M * N * 4),
       2.0 * M * N * K, s,
       (use_tc ? (double)M * N * 2 : 0.0) +
           (nsp > 1 ? (double)(tiles - nfull) * pl.bm * pl.bn * 4 * nsp : 0.0));
  if (e != hipSuccess || nsp == 1) return e;
  if (deferred && nfull == 0) {
    // plain split-K: the caller adds the partials itself
    *deferred = nsp;
    return hipSuccess;
  }
  const int64_t nm = cdiv(M, pl.bm);
  const int64_t n0 = (nfull / nm) * pl.bn, mskip = (nfull % nm) * pl.bm;
  int64_t blocks = cdiv(M * ((N - n0) / 4), 256);
  if (blocks > 4096) blocks = 4096;
#define LBP_RED(E)                                                                          \
  splitk_reduce_kernel<E><<<dim3((unsigned)blocks), block, 0, s>>>(M, N, nsp, partials, C, ldc, \
                                                                  n0, pl.bn, mskip, ea)
  switch (epi) {
    case 1: LBP_RED(1); break;
    case 2: LBP_RED(2); break;
    case 7: LBP_RED(7); break;
    case 8: LBP_RED(8); break;
    default: LBP_RED(0);
  }
#undef LBP_RED
  mark("splitk_reduce", 0, 0, s, (double)(tiles - nfull) * pl.bm * pl.bn * 4 * (nsp + 1));
  return hipGetLastError();
}

hipError_t launch_gemm_at_adamw(int64_t M, int64_t N, int64_t K, const float* At, int64_t lda,
                                const float* B, int64_t ldb, const AdamEpi& ad, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  // buffer ranges: four rows of A^T and of B, and one tile's rows of W, m, v
  if (N % 8 != 0 || lda < M || ldb < N || 16.0 * lda >= BUF_MAX_BYTES ||
      16.0 * ldb >= BUF_MAX_BYTES || (double)std::min<int64_t>(F_BM, M) * N * 4 >= BUF_MAX_BYTES)
    return hipErrorInvalidValue;
  if (dry_run()) return hipSuccess;
  // every tile whole (the epilogue needs the finished dW tile)
  const int64_t tiles = cdiv(M, F_BM) * cdiv(N, F_BN);
  gemm_f32_kernel<32, true><<<dim3((unsigned)tiles), dim3(F_NT), 0, s>>>(
      M, N, K, At, lda, B, B, K, ldb, nullptr, N, nullptr, K, tiles, ActEpi{}, ad);
  // A^T and B once; W, m, v read and written (and the gradient copy)
  mark("gemm_f32_mfma_adamw", (double)K * (M + N) * 4 + (double)M * N * 4 * (ad.grad ? 7 : 6),
       2.0 * M * N * K, s);
  return hipGetLastError();
}

}  // namespace lbp
