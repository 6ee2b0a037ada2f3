// GQA attention backward from saved softmax weights.
//
// Hesper "Attention Backward GPU Kernels": "Attention Apply Backward"
// (dA = dCtx V^T), "Softmax Backward" (dS = P o (dA - delta)), "Attention
// Score Backward" (dQ = scale dS K); entrenar wgpu_backward.rs attention
// backward for dV = P^T dCtx.  Query head h reads KV head h / grp.
//
// Sequence path (s_q > 1), float32 (v_mfma_f32_16x16x4_f32):
//   attn_dq_f32_kernel  workgroup = 16*QW query rows x HW heads of one KV
//       group (HW*QW = 4 waves).  Each wave keeps its dCtx rows in
//       registers and walks 32-key tiles of K and V staged in LDS (the next
//       tile is fetched into registers while the current one is used).
//       The scores are formed transposed, dA^T = V dCtx^T, so that a lane
//       holds one query and four consecutive keys: P is read with one
//       16-byte load per lane straight into the accumulator layout, and the
//       resulting dS^T registers are already the A operand of dQ = dS K.
//       delta comes from <dCtx, ctx> (ctx = P V), so P is streamed once.
//       Under a causal mask the grid is ordered so that long and short
//       query tiles pair up on a CU.
//   attn_dv_f32_kernel  workgroup = 64 keys of one KV group and one chunk of
//       query rows; each wave owns 16 keys x all head dims and sums
//       P^T dCtx over the heads of the group; dCtx rows are staged in LDS.
//       Chunks give the launch enough workgroups; their partial sums are
//       added in chunk order by attn_dv_reduce_kernel.
// bfloat16 inputs use the kernels further down.  One query row (decode)
// goes to the kernels in decode.hip.
#include "common.h"
#include "kernels.h"

namespace lbp {

__host__ __device__ static inline int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Four consecutive floats of one P row from column `col`, zero past `ncol`.
// vec: the row start is 16-byte aligned (ncol % 4 == 0).
__device__ __forceinline__ float4 prow4(const float* rowp, int64_t col, int64_t ncol, bool vec) {
  float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
  if (vec) {
    if (col < ncol) r = *reinterpret_cast<const float4*>(rowp + col);
  } else {
    if (col < ncol) r.x = rowp[col];
    if (col + 1 < ncol) r.y = rowp[col + 1];
    if (col + 2 < ncol) r.z = rowp[col + 2];
    if (col + 3 < ncol) r.w = rowp[col + 3];
  }
  return r;
}

__device__ __forceinline__ float f4at(const float4& v, int j) {
  return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
}

constexpr int FQ_KT = 32;  // keys per tile, float32 dq kernel
constexpr int DV_KT = 64;  // keys per workgroup, dv kernels

template <int D, int HW, bool PVEC, bool KSPLIT>
__global__ __launch_bounds__(256) void attn_dq_f32_kernel(
    int64_t s_q, int64_t s_kv, int Hq, int grp, const float* __restrict__ dctx,
    const float* __restrict__ P, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ ctx, const float* __restrict__ delta_ws, float* __restrict__ dq,
    float* __restrict__ dq2, float scale, int causal, float* __restrict__ ds_out) {
  constexpr int KT = FQ_KT, DK = D / 4, ND = D / 16, QW = 4 / HW, LDK = D + 4;
  constexpr int NE = KT * D / 4;           // float4 per staged tile
  constexpr int SE = (NE + 255) / 256;     // per thread
  __shared__ float Vs[2][KT][LDK];
  __shared__ float Ks[2][KT][LDK];
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform: h, q0 are too
  const int l16 = lane & 15, c = lane >> 4;
  // 1-D grid over (query tile, head block), head block fastest: workgroups
  // go to the XCDs round-robin, so with eight head blocks each XCD works on
  // one KV group.  Causal, without KSPLIT: the first half of the grid takes
  // the query tiles from the end (longest first) and the second half the
  // complementary ones, so the two workgroups that share a CU add up to
  // about the same work.  KSPLIT (causal only): item L = (pair, half, head
  // block); the workgroup takes query tiles p and nqt-1-p of the pair but
  // only half of each one's key tiles, so every workgroup has the same work;
  // half 0 writes dq, half 1 the partial dq2 (the caller adds the two).
  const int nhb = Hq / HW;
  const int64_t nqt = cdiv64(s_q, 16 * QW);
  const int64_t L = blockIdx.x;
  int64_t qt, hb;
  int half = 0;
  if (KSPLIT) {
    hb = L % nhb;
    half = (int)((L / nhb) & 1);
    qt = L / (2 * nhb);  // the pair index; the second tile is nqt-1-qt
  } else if (causal) {
    const int64_t H = (int64_t)nhb * ((nqt + 1) / 2);
    if (L < H) {
      qt = nqt - 1 - L / nhb;
      hb = L % nhb;
    } else {
      qt = (L - H) / nhb;
      hb = (L - H) % nhb;
    }
  } else {
    qt = L / nhb;
    hb = L % nhb;
  }
  const int h = (int)hb * HW + (w % HW), g = h / grp;
  const int64_t ldq = (int64_t)Hq * D, ldk = (int64_t)(Hq / grp) * D;
  auto segment = [&](int64_t qtile, int hpart, float* __restrict__ out) {
  const int64_t qw0 = qtile * (16 * QW);
    const int64_t q0 = qw0 + 16 * (w / HW);
    const int64_t qrow = q0 + l16;
    const bool qok = qrow < s_q;
  
    // B operand of dA^T = V dCtx^T: lane (query qrow, group c) holds head dims
    // DK*c .. DK*c + DK - 1 (MFMA step j of that group is d = DK*c + j).
    float dc[DK];
#pragma unroll
    for (int i = 0; i < DK; i += 4) {
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (qok) v = *reinterpret_cast<const float4*>(dctx + qrow * ldq + h * D + DK * c + i);
      dc[i] = v.x;
      dc[i + 1] = v.y;
      dc[i + 2] = v.z;
      dc[i + 3] = v.w;
    }
    float dl = 0.f;
    if (ctx != nullptr) {
#pragma unroll
      for (int i = 0; i < DK; i += 4) {
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (qok) x = *reinterpret_cast<const float4*>(ctx + qrow * ldq + h * D + DK * c + i);
        dl += dc[i] * x.x + dc[i + 1] * x.y + dc[i + 2] * x.z + dc[i + 3] * x.w;
      }
      dl += __shfl_xor(dl, 16, 64);
      dl += __shfl_xor(dl, 32, 64);
    } else if (qok) {
      dl = delta_ws[(int64_t)h * s_q + qrow];
    }
  
    floatx4 acc[ND];
#pragma unroll
    for (int f = 0; f < ND; ++f) acc[f] = floatx4{0.f, 0.f, 0.f, 0.f};
  
    const int64_t off = s_kv - s_q;
    const int64_t qlast = min(s_q, qw0 + 16 * QW) - 1;
    const int64_t kend = causal ? min(s_kv, off + qlast + 1) : s_kv;
    const int ntile_all = (int)cdiv64(kend, KT);
    const int mid = (ntile_all + 1) / 2;
    const int kt0 = !KSPLIT ? 0 : (hpart == 0 ? 0 : mid);
    const int ntile = !KSPLIT ? ntile_all : (hpart == 0 ? mid : ntile_all);
    // Buffer ranges (bounds are offsets, out of range reads 0): the wave's 16
    // P rows, and one key tile of V and K.  Pipeline: the next tile's V/K
    // loads go out at the top of a step and its P as soon as this tile's dS is
    // formed (into the same registers), so both fly during the dQ products,
    // the barrier and the next dA products; one barrier per tile.
    const brsrc_t prs = make_brsrc(P + ((int64_t)h * s_q + q0) * s_kv, (uint32_t)(16 * s_kv * 4));
    float4 sv[SE], sk[SE], pc[2];
    auto fetch = [&](int64_t k0, bool valid) {
      const brsrc_t vr = make_brsrc(V + k0 * ldk + g * D, (uint32_t)(KT * ldk * 4));
      const brsrc_t kr = make_brsrc(K + k0 * ldk + g * D, (uint32_t)(KT * ldk * 4));
#pragma unroll
      for (int i = 0; i < SE; ++i) {
        const int e = t + 256 * i;
        const int kk = e / (D / 4), d = 4 * (e % (D / 4));
        const uint32_t off = (valid && e < NE && k0 + kk < s_kv) ? (uint32_t)((kk * ldk + d) * 4) : BUF_OOB;
        sv[i] = bload_f4(vr, off);
        sk[i] = bload_f4(kr, off);
      }
    };
    auto fetch_p = [&](int64_t k0) {
      const bool ok = qok && k0 < kend;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int64_t col = k0 + 16 * nt + 4 * c;
        const int64_t e = (int64_t)l16 * s_kv + col;
        if (PVEC) {
          pc[nt] = bload_f4(prs, (ok && col < s_kv) ? (uint32_t)(e * 4) : BUF_OOB);
        } else {
          float v[4];
#pragma unroll
          for (int j = 0; j < 4; ++j)
            v[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                prs, (ok && col + j < s_kv) ? (int)((e + j) * 4) : (int)BUF_OOB, 0, 0));
          pc[nt] = make_float4(v[0], v[1], v[2], v[3]);
        }
      }
    };
    auto stash = [&](int buf) {
#pragma unroll
      for (int i = 0; i < SE; ++i) {
        const int e = t + 256 * i;
        if (e < NE) {
          const int kr = e / (D / 4), d = 4 * (e % (D / 4));
          *reinterpret_cast<float4*>(&Vs[buf][kr][d]) = sv[i];
          *reinterpret_cast<float4*>(&Ks[buf][kr][d]) = sk[i];
        }
      }
    };
    fetch((int64_t)kt0 * KT, ntile > kt0);
    stash(0);
    fetch_p((int64_t)kt0 * KT);
    __syncthreads();
    int buf = 0;
    for (int it = kt0; it < ntile; ++it) {
      const int64_t k0 = (int64_t)it * KT;
      fetch(k0 + KT, it + 1 < ntile);
      // dA^T for two 16-key sub-tiles: row = key 16 nt + 4c + v, col = query l16.
      // Four partial accumulators per sub-tile keep eight MFMA chains in flight.
      floatx4 da[2][4];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int j = 0; j < 4; ++j) da[nt][j] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s4 = 0; s4 < DK / 4; ++s4)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const float4 v4 = *reinterpret_cast<const float4*>(&Vs[buf][16 * nt + l16][DK * c + 4 * s4]);
          da[nt][0] = mfma16x16x4(v4.x, dc[4 * s4 + 0], da[nt][0]);
          da[nt][1] = mfma16x16x4(v4.y, dc[4 * s4 + 1], da[nt][1]);
          da[nt][2] = mfma16x16x4(v4.z, dc[4 * s4 + 2], da[nt][2]);
          da[nt][3] = mfma16x16x4(v4.w, dc[4 * s4 + 3], da[nt][3]);
        }
      // dS^T = P^T o (dA^T - delta)
      float ds[2][4];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float a = (da[nt][0][v] + da[nt][1][v]) + (da[nt][2][v] + da[nt][3][v]);
          ds[nt][v] = f4at(pc[nt], v) * (a - dl);
        }
      fetch_p(k0 + KT);
      // scale dS, stored as P is ([head][query][key]) for the dK pass; the
      // tiles this workgroup computes cover every key a query sees
      if (ds_out != nullptr && qok) {
        float* dsr = ds_out + ((int64_t)h * s_q + qrow) * s_kv;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int64_t col = k0 + 16 * nt + 4 * c;
          if (PVEC) {
            if (col < s_kv)
              *reinterpret_cast<float4*>(dsr + col) =
                  make_float4(scale * ds[nt][0], scale * ds[nt][1], scale * ds[nt][2], scale * ds[nt][3]);
          } else {
#pragma unroll
            for (int v = 0; v < 4; ++v)
              if (col + v < s_kv) dsr[col + v] = scale * ds[nt][v];
          }
        }
      }
      // dQ += dS K with k index = key.  Column n of MFMA tile f is head dim
      // ND n + f, so a lane's K values for its ND tiles are contiguous
      // (vector LDS reads) and its dq values contiguous on store.
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float kv[ND];
#pragma unroll
          for (int f = 0; f < ND; ++f) kv[f] = Ks[buf][16 * nt + 4 * c + v][ND * l16 + f];
#pragma unroll
          for (int f = 0; f < ND; ++f) acc[f] = mfma16x16x4(ds[nt][v], kv[f], acc[f]);
        }
      stash(buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t row = q0 + 4 * c + v;
      if (row < s_q) {
#pragma unroll
        for (int f = 0; f < ND; ++f) out[row * ldq + h * D + ND * l16 + f] = scale * acc[f][v];
      }
    }
  };
  if (KSPLIT) {
    float* out = half == 0 ? dq : dq2;
    segment(qt, half, out);
    if (nqt - 1 - qt != qt) {
      __syncthreads();
      segment(nqt - 1 - qt, half, out);
    }
  } else {
    segment(qt, 0, dq);
  }
}

// Work of the dv kernels.  A workgroup owns a tile of kt keys of one KV
// group; the tile's query range starts at the first row that sees its first
// key (causal), rounded down to qround, and is walked in steps of (head,
// qblk-row block), head-major.  A work item is a chunk of cs consecutive
// steps of one tile.  Items are numbered full chunks first (every tile's, in
// tile order), then the tiles' shorter last chunks, the KV group varying
// fastest: workgroups go to the XCDs round-robin in launch order, so with
// eight KV groups each XCD works on one group and gets the same share of
// long items.
struct DvGeo {
  int kt, qround, qblk;
};
__host__ __device__ __forceinline__ int64_t dv_tile_qbeg(int64_t j, int64_t s_q, int64_t s_kv,
                                                         int causal, DvGeo q) {
  int64_t qbeg = causal ? j * q.kt - (s_kv - s_q) : 0;
  return qbeg < 0 ? 0 : qbeg / q.qround * q.qround;
}
__host__ __device__ __forceinline__ int64_t dv_tile_steps(int64_t j, int64_t s_q, int64_t s_kv,
                                                          int64_t grp, int causal, DvGeo q) {
  const int64_t qbeg = dv_tile_qbeg(j, s_q, s_kv, causal, q);
  return qbeg >= s_q ? 0 : grp * ((s_q - qbeg + q.qblk - 1) / q.qblk);
}
// Item L -> (KV group g, tile jt, chunk ch); false when L names no item.
__device__ __forceinline__ bool dv_item(int64_t L, int Hkv, int64_t s_q, int64_t s_kv, int grp,
                                        int causal, DvGeo q, int64_t cs, int64_t nfull, int& g,
                                        int64_t& jt, int64_t& ch) {
  const int64_t nt = (s_kv + q.kt - 1) / q.kt;
  g = (int)(L % Hkv);
  int64_t r = L / Hkv;
  jt = 0;
  ch = 0;
  if (r < nfull) {
    for (; jt < nt; ++jt) {
      const int64_t nf = dv_tile_steps(jt, s_q, s_kv, grp, causal, q) / cs;
      if (r < nf) break;
      r -= nf;
    }
    ch = r;
  } else {
    r -= nfull;
    for (; jt < nt; ++jt) {
      if (dv_tile_steps(jt, s_q, s_kv, grp, causal, q) % cs != 0) {
        if (r == 0) break;
        --r;
      }
    }
    if (jt < nt) ch = dv_tile_steps(jt, s_q, s_kv, grp, causal, q) / cs;
  }
  return jt < nt;
}

// dV for 64 keys of one KV group over one work item (chunk of steps, see
// dv_item).  MFMA rows = keys (wave w: 16w .. 16w+15), cols = head dims,
// k = query rows (step s, group c: row qb + 4s + c).  32 query rows of one
// head per step: their dCtx rows go to a double-buffered LDS tile, the P
// values straight into registers; one step of loads is in flight.  Output:
// dv itself when cmax == 1, else partial sums part[chunk][key][kv_dim].
constexpr int FV_QT = 32;  // query rows per step, fp32 dv kernel
constexpr DvGeo FV_GEO{DV_KT, 16, FV_QT};

// CMASK (causal only): read P only at keys the query sees (key <= s_kv - s_q
// + query), 0 elsewhere; the dK pass runs this kernel on (scale dS, Q), whose
// dS is written only where the dQ kernel computed it.
template <int D, bool CMASK>
__global__ __launch_bounds__(256) void attn_dv_f32_kernel(int64_t s_q, int64_t s_kv, int Hq,
                                                          int grp, int cmax, int64_t cs,
                                                          int64_t nfull,
                                                          const float* __restrict__ dctx,
                                                          const float* __restrict__ P,
                                                          float* __restrict__ out, int causal) {
  constexpr int ND = D / 16, LDC = D == 16 ? 48 : D + 16, QT = FV_QT;
  constexpr int NE = QT * D / 4;  // float4 per staged dCtx block
  constexpr int SE = (NE + 255) / 256;
  __shared__ float dCs[2][QT][LDC];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int l16 = lane & 15, c = lane >> 4;
  int g;
  int64_t jt, ch;
  if (!dv_item(blockIdx.x, Hq / grp, s_q, s_kv, grp, causal, FV_GEO, cs, nfull, g, jt, ch)) return;
  const int64_t ldq = (int64_t)Hq * D, ldk = (int64_t)(Hq / grp) * D;
  const int64_t k0 = jt * DV_KT;
  const int64_t qbeg = dv_tile_qbeg(jt, s_q, s_kv, causal, FV_GEO);
  const int64_t nqb = cdiv64(s_q - qbeg, QT);
  const int64_t st0 = ch * cs, st1 = min(nqb * grp, st0 + cs);
  const int64_t key = k0 + 16 * w + l16;
  const bool kok = key < s_kv;
  float* dst = out + (cmax > 1 ? ch * s_kv * ldk : 0);
  if (st0 >= st1) return;

  floatx4 acc[ND];
#pragma unroll
  for (int f = 0; f < ND; ++f) acc[f] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int64_t nit = st1 - st0;
  // One step = 32 query rows of one head: its dCtx rows go to LDS, the P
  // values of this lane's key straight into registers.  Two register stages
  // used in turn; every load is a branch-free buffer load (a step past the
  // end reads zeros), so the pipeline never drains on a branch.
  struct Stage {
    float4 d[SE];
    float p[QT / 4];
  };
  auto fetch = [&](Stage& r, int64_t it) {
    const bool valid = it < nit;
    const int64_t stp = st0 + (valid ? it : 0);
    const int h = g * grp + (int)(stp / nqb);
    const int64_t qb = qbeg + QT * (stp % nqb);
    const brsrc_t rd = make_brsrc(dctx + qb * ldq + h * D, (uint32_t)(QT * ldq * 4));
#pragma unroll
    for (int i = 0; i < SE; ++i) {
      const int e = t + 256 * i;
      const int rr = e / (D / 4);
      const bool ok = valid && e < NE && qb + rr < s_q;
      r.d[i] = bload_f4(rd, ok ? (uint32_t)((rr * ldq + 4 * (e % (D / 4))) * 4) : BUF_OOB);
    }
    const brsrc_t rp = make_brsrc(P + ((int64_t)h * s_q + qb) * s_kv + k0, (uint32_t)(QT * s_kv * 4));
#pragma unroll
    for (int s2 = 0; s2 < QT / 4; ++s2) {
      const int rr = 4 * s2 + c;
      const bool ok = valid && kok && qb + rr < s_q && (!CMASK || key <= s_kv - s_q + qb + rr);
      r.p[s2] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
          rp, ok ? (int)((rr * s_kv + 16 * w + l16) * 4) : (int)BUF_OOB, 0, 0));
    }
  };
  auto stash = [&](const Stage& r, int buf) {
#pragma unroll
    for (int i = 0; i < SE; ++i) {
      const int e = t + 256 * i;
      if (e < NE) *reinterpret_cast<float4*>(&dCs[buf][e / (D / 4)][4 * (e % (D / 4))]) = r.d[i];
    }
  };
  auto compute = [&](const Stage& r, int buf) {
#pragma unroll
    for (int s2 = 0; s2 < QT / 4; ++s2)
#pragma unroll
      for (int f = 0; f < ND; ++f)
        acc[f] = mfma16x16x4(r.p[s2], dCs[buf][4 * s2 + c][16 * f + l16], acc[f]);
  };
  Stage s0, s1;
  fetch(s0, 0);
  stash(s0, 0);
  fetch(s1, 1);
  __syncthreads();
  for (int64_t it = 0; it < nit; it += 2) {
    compute(s0, 0);
    stash(s1, 1);
    __syncthreads();
    fetch(s0, it + 2);
    compute(s1, 1);
    stash(s0, 0);
    __syncthreads();
    fetch(s1, it + 3);
  }
#pragma unroll
  for (int f = 0; f < ND; ++f)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t k = k0 + 16 * w + 4 * c + v;
      if (k < s_kv) dst[k * ldk + g * D + 16 * f + l16] = acc[f][v];
    }
}

// dv[key][:] = sum of the chunk partials that exist for the key's tile (a
// chunk is cs steps, see dv_item), in chunk order (zero when no query row
// sees the key).
__device__ __forceinline__ void dv_reduce_at(int64_t e, int64_t s_q, int64_t s_kv, int64_t ldk,
                                             int cmax, int64_t cs, const float* __restrict__ part,
                                             float* __restrict__ dv, int causal, int grp,
                                             DvGeo geo) {
  const int64_t n4 = s_kv * ldk / 4;
  if (e >= n4) return;
  const int64_t key = 4 * e / ldk;
  const int64_t nch = cdiv64(dv_tile_steps(key / geo.kt, s_q, s_kv, grp, causal, geo), cs);
  // up to 8 chunk partials in flight, added in chunk order (an index past
  // the last chunk re-reads chunk 0 and its term is dropped)
  const int n = (int)(nch < cmax ? nch : cmax);
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int c0 = 0; c0 < n; c0 += 8) {
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int ch = c0 + u < n ? c0 + u : 0;
      v[u] = reinterpret_cast<const float4*>(part + (int64_t)ch * s_kv * ldk)[e];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bool take = c0 + u < n;
      s.x += take ? v[u].x : 0.f;
      s.y += take ? v[u].y : 0.f;
      s.z += take ? v[u].z : 0.f;
      s.w += take ? v[u].w : 0.f;
    }
  }
  reinterpret_cast<float4*>(dv)[e] = s;
}

__global__ __launch_bounds__(256) void attn_dv_reduce_kernel(int64_t s_q, int64_t s_kv,
                                                             int64_t ldk, int cmax, int64_t cs,
                                                             const float* __restrict__ part,
                                                             float* __restrict__ dv, int causal,
                                                             int grp, DvGeo geo) {
  dv_reduce_at((int64_t)blockIdx.x * 256 + threadIdx.x, s_q, s_kv, ldk, cmax, cs, part, dv,
               causal, grp, geo);
}

// The same reduction in its first nred workgroups, and the inverse RoPE of
// dq (+ dq2) one row per workgroup after them: one launch instead of two.
struct RopeRows {
  const float* dy;
  const float* dy2;
  float* dx;
  int64_t n_heads;
  int head_dim, threads;
  int64_t pos0;
  double log2_base;
  RopeNorm norm;
};
__global__ __launch_bounds__(256) void attn_dv_reduce_rope_kernel(
    int64_t s_q, int64_t s_kv, int64_t ldk, int cmax, int64_t cs, const float* __restrict__ part,
    float* __restrict__ dv, int causal, int grp, DvGeo geo, int64_t nred, RopeRows r) {
  if ((int64_t)blockIdx.x < nred) {
    dv_reduce_at((int64_t)blockIdx.x * 256 + threadIdx.x, s_q, s_kv, ldk, cmax, cs, part, dv,
                 causal, grp, geo);
    return;
  }
  if ((int)threadIdx.x >= r.threads) return;
  rope_bwd_row((int64_t)blockIdx.x - nred, threadIdx.x, r.threads, r.n_heads, r.head_dim, r.dy,
               r.dy2, r.dx, r.pos0, r.log2_base, r.norm);
}

// The last launch of a dV with chunk partials: the reduction, with the
// inverse RoPE of dq (rows s_q) when rope is set.
static hipError_t launch_dv_reduce(int64_t s_q, int64_t s_kv, int Hq, int Hkv, int D, int cmax,
                                   int64_t cs, const float* part, float* dv, int causal, DvGeo geo,
                                   const float* dq, const float* dq2, const RopeArgs* rope,
                                   bool* rope_done, hipStream_t s) {
  const int64_t ldk = (int64_t)Hkv * D, n4 = s_kv * ldk / 4, nred = cdiv64(n4, 256);
  const double kvbytes = (double)s_kv * ldk * 4;
  if (rope == nullptr || rope_done == nullptr) {
    attn_dv_reduce_kernel<<<dim3((unsigned)nred), 256, 0, s>>>(s_q, s_kv, ldk, cmax, cs, part, dv,
                                                               causal, Hq / Hkv, geo);
    mark("attn_dv_reduce", 0, 0, s, kvbytes * (cmax + 1));  // dV counted at the dV launch
    return hipGetLastError();
  }
  const RopeNorm nm = rope->norm.x != nullptr
                          ? RopeNorm{rope->norm.x, rope->norm.x_bf16, rope->norm.gamma, rope->norm.eps}
                          : RopeNorm{nullptr, 0, nullptr, 0.f};
  const RopeRows r{dq, dq2, rope->dx, Hq, D, rope_threads(Hq, D), rope->pos0,
                   log2((double)rope->base), nm};
  attn_dv_reduce_rope_kernel<<<dim3((unsigned)(nred + s_q)), 256, 0, s>>>(
      s_q, s_kv, ldk, cmax, cs, part, dv, causal, Hq / Hkv, geo, nred, r);
  const double qe = (double)s_q * Hq * D;
  // the inverse RoPE reads dq and writes dq_pre (a split dq's second half on
  // top); dV was counted at the dV launch, its chunk partials are not
  mark("attn_dv_reduce_rope", qe * (8 + (nm.x ? (nm.x_bf16 ? 2 : 4) : 0)), qe * (nm.x ? 9 : 3), s,
       kvbytes * (cmax + 1) + (dq2 ? qe * 4 : 0.0));
  *rope_done = true;
  return hipGetLastError();
}

// ---------------------------------------------------------------- bfloat16
// bf16 inputs (P, K, V, ctx) run on v_mfma_f32_16x16x32_bf16; dCtx and dS are
// rounded to bf16 as MFMA operands, accumulation and softmax algebra stay
// fp32.  Operand lane layout: lane l holds row (or column) l%16 and the eight
// k indices 8(l/16) .. 8(l/16)+7; result lane l, register v holds row
// 4(l/16)+v, column l%16.
//
// transpose_bf16_kernel  dst[col][row] (bf16, rows padded with zeros to LR)
//     from src[row][col] (fp32 or bf16).  Gives K as Kt[kv head][d][key] and
//     dCtx as dCt[head][d][query] (both in one launch, ahead of dQ), so the
//     operands whose MFMA k index runs over keys or queries are 16-byte
//     reads.
// attn_dq_bf16_kernel  workgroup = HW heads of one KV group x QW wave groups;
//     a wave owns two 16-query blocks, i and n-1-i, so every wave does about
//     the same causal work.  64-key tiles of V and Kt are staged in LDS
//     (double-buffered, next tile fetched during the current one).  Inside a
//     tile the key of MFMA row m in sub-tile nt is 16(m/4) + 4 nt + m%4: a
//     lane's four sub-tiles then hold 16 consecutive keys of its query, so P
//     is read as 32 contiguous bytes, and the dS values for keys 16c + 8s ..
//     +7 are the A operand of dQ = dS K with Kt read as one 16-byte row.
// attn_dv_bf16_kernel  workgroup = 128 keys of one KV group x one chunk of
//     the tile's steps (head, 64-query block); waves 2 x 2 over (64 keys, D/2
//     dims), two workgroups per CU.  Per step the P block is copied to LDS as
//     stored ([query][key]) and read as P^T through the LDS transpose read;
//     dCt rows are copied.  The operands of each 32-query half are read during
//     the previous half's MFMAs.  Chunks hold equal step counts, sized so all
//     of them run in one round (the causal mask gives early key tiles more
//     steps); chunk partials as in fp32.
constexpr int TR_R = 64, TR_C = 32;

// One transposition of the launch below: src [rows][cols] (row stride ld)
// into dst [cols][LR] in tiles of TR_R rows x TR_C columns, gx x gy tiles.
struct TrJob {
  int64_t rows, LR, ld;
  const void* src;
  uint16_t* dst;
  int gx, gy;
};

// Kᵀ (bf16 source) and dCtxᵀ (fp32 source) in one launch: the first
// a.gx * a.gy workgroups take job a, the rest job b.
// Eight consecutive elements of a row as bf16 bit patterns (16-byte loads).
__device__ __forceinline__ void ld8_bf16(const float* p, uint16_t (&o)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  const uint32_t w[4] = {pk_bf16(a.x, a.y), pk_bf16(a.z, a.w), pk_bf16(b.x, b.y), pk_bf16(b.z, b.w)};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    o[2 * j] = (uint16_t)(w[j] & 0xffffu);
    o[2 * j + 1] = (uint16_t)(w[j] >> 16);
  }
}
__device__ __forceinline__ void ld8_bf16(const bf16* p, uint16_t (&o)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    o[2 * j] = (uint16_t)(w[j] & 0xffffu);
    o[2 * j + 1] = (uint16_t)(w[j] >> 16);
  }
}

// Each thread reads eight consecutive columns of one row with 16-byte loads
// (rows past the end give 0) and scatters them into the LDS tile
// transposed; each thread then writes eight consecutive rows of one column.
template <typename TA, typename TB>
__global__ __launch_bounds__(256) void transpose_bf16_kernel(TrJob a, TrJob b) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[TR_C][TR_R + 8];
  const int64_t na = (int64_t)a.gx * a.gy;
  const bool second = (int64_t)blockIdx.x >= na;
  const int64_t loc = second ? (int64_t)blockIdx.x - na : (int64_t)blockIdx.x;
  const TrJob& jb = second ? b : a;
  const int64_t rows = jb.rows, LR = jb.LR, ld = jb.ld;
  uint16_t* __restrict__ dst = jb.dst;
  const int t = threadIdx.x;
  const int64_t r0 = (loc % jb.gx) * TR_R, c0 = (loc / jb.gx) * TR_C;
  static_assert(TR_R * TR_C == 256 * 8, "one 8-column chunk per thread");
  const int row = t >> 2, c8 = 8 * (t & 3);
  uint16_t v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (r0 + row < rows) {
    if (second)
      ld8_bf16((const TB*)jb.src + (r0 + row) * ld + c0 + c8, v);
    else
      ld8_bf16((const TA*)jb.src + (r0 + row) * ld + c0 + c8, v);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) tile[c8 + j][row] = v[j];
  __syncthreads();
  const int rc = t & 7, cc = t >> 3;
  *reinterpret_cast<uint4*>(dst + (c0 + cc) * LR + r0 + 8 * rc) =
      *reinterpret_cast<const uint4*>(&tile[cc][8 * rc]);
}

__device__ __forceinline__ ushortx8 pack8(const float (&x)[8]) {
  const uint4 u = make_uint4(pk_bf16(x[0], x[1]), pk_bf16(x[2], x[3]), pk_bf16(x[4], x[5]),
                             pk_bf16(x[6], x[7]));
  return __builtin_bit_cast(ushortx8, u);
}

// Eight consecutive bf16 keys kc .. kc+7 of a P row at element offset
// `row` of resource r; keys at or past s_kv, and the whole chunk when !ok,
// read 0.  With PVEC (s_kv a multiple of 8) it is one 16-byte load.
template <bool PVEC>
__device__ __forceinline__ ushortx8 load_p8(brsrc_t r, bool ok, int64_t row, int64_t kc,
                                            int64_t s_kv) {
  if (PVEC) {
    const uint32_t off = (ok && kc < s_kv) ? (uint32_t)((row + kc) * 2) : BUF_OOB;
    return __builtin_bit_cast(ushortx8, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
  } else {
    ushortx8 v;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t off = (ok && kc + j < s_kv) ? (uint32_t)((row + kc + j) * 2) : BUF_OOB;
      v[j] = __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
    }
    return v;
  }
}

constexpr int HQ_KT = 64;  // keys per tile, bf16 dq kernel

// LDS of the bf16 dQ and dV workgroups (16-bit elements)
template <int D>
constexpr int dq_bf16_lds() {
  return 2 * HQ_KT * (D + 8) + 2 * D * (HQ_KT + 8);
}

// Workgroup blk of the bf16 dQ launch, on the LDS at smem (dq_bf16_lds).
template <int D, int HW, bool PVEC>
__device__ __forceinline__ void attn_dq_bf16_body(
    int64_t blk, int64_t s_q, int64_t s_kv, int Hq, int grp, int64_t LK, int npairs,
    const float* __restrict__ dctx, const uint16_t* __restrict__ P,
    const uint16_t* __restrict__ Kt, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ ctx, const float* __restrict__ delta_ws, float* __restrict__ dq,
    float scale, int causal, uint16_t* smem, uint16_t* __restrict__ ds_out) {
  constexpr int KT = HQ_KT, NK = D / 32, ND = D / 16, QW = 4 / HW;
  constexpr int VLD = D + 8, KLD = KT + 8;
  constexpr int NCH = KT * D / 8;            // 16-byte chunks per staged matrix
  constexpr int SE = (NCH + 255) / 256;
  auto& Vs = *reinterpret_cast<uint16_t(*)[2][KT][VLD]>(smem);
  auto& Ks = *reinterpret_cast<uint16_t(*)[2][D][KLD]>(smem + 2 * KT * VLD);
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform, so are h and the blocks
  const int l16 = lane & 15, c = lane >> 4;
  // 1-D grid, head group fastest: workgroups go to the XCDs round-robin, so
  // with eight head groups each XCD works on one KV group (its K and V stay
  // in that XCD's L2)
  const int nhg = Hq / HW;
  const int by = (int)(blk % nhg), bx = (int)(blk / nhg);
  const int h = by * HW + (w % HW), g = h / grp;
  const int64_t ldq = (int64_t)Hq * D, ldk = (int64_t)(Hq / grp) * D;
  const int nsub = (int)cdiv64(s_q, 16);
  const int64_t off = s_kv - s_q;
  // key range of a 16-query block: causal end after its last row
  auto kend_of = [&](int sb) -> int64_t {
    if (!causal) return s_kv;
    const int64_t last = min(s_q, (int64_t)16 * sb + 16) - 1;
    return min(s_kv, off + last + 1);
  };
  // this wave's two blocks (the second is absent for the middle of an odd count)
  const int pair = bx * QW + w / HW;
  int sub[2];
  bool has[2];
  sub[0] = pair;
  sub[1] = nsub - 1 - pair;
  has[0] = pair < npairs;
  has[1] = pair < npairs && sub[1] != sub[0];
  int64_t kend[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) kend[s] = has[s] ? kend_of(sub[s]) : 0;
  // the workgroup walks the longest key range among its waves
  int64_t kend_wg = 0;
  for (int j = 0; j < QW; ++j) {
    const int pj = bx * QW + j;
    if (pj < npairs) {
      kend_wg = max(kend_wg, kend_of(pj));
      if (nsub - 1 - pj != pj) kend_wg = max(kend_wg, kend_of(nsub - 1 - pj));
    }
  }
  const int ntile = (int)cdiv64(kend_wg, KT);

  // B operand of dA^T = V dCtx^T: dCtx[q][32 ks + 8c .. +7] as bf16; delta
  ushortx8 dcb[2][NK];
  float dl[2] = {0.f, 0.f};
  int64_t qrow[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    qrow[s] = (int64_t)16 * sub[s] + l16;
    const bool ok = has[s] && qrow[s] < s_q;
    float part = 0.f;
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (ok) {
        const float* p = dctx + qrow[s] * ldq + h * D + 32 * ks + 8 * c;
        const float4 u0 = *reinterpret_cast<const float4*>(p);
        const float4 u1 = *reinterpret_cast<const float4*>(p + 4);
        x[0] = u0.x; x[1] = u0.y; x[2] = u0.z; x[3] = u0.w;
        x[4] = u1.x; x[5] = u1.y; x[6] = u1.z; x[7] = u1.w;
        if (ctx != nullptr) {
          const float4 y0 = Act<bf16>::ld4((const bf16*)ctx, qrow[s] * ldq + h * D + 32 * ks + 8 * c);
          const float4 y1 = Act<bf16>::ld4((const bf16*)ctx, qrow[s] * ldq + h * D + 32 * ks + 8 * c + 4);
          part += x[0] * y0.x + x[1] * y0.y + x[2] * y0.z + x[3] * y0.w + x[4] * y1.x +
                  x[5] * y1.y + x[6] * y1.z + x[7] * y1.w;
        }
      }
      dcb[s][ks] = pack8(x);
    }
    if (ctx != nullptr) {
      part += __shfl_xor(part, 16, 64);
      part += __shfl_xor(part, 32, 64);
      dl[s] = part;
    } else if (ok) {
      dl[s] = delta_ws[(int64_t)h * s_q + qrow[s]];
    }
  }

  floatx4 acc[2][ND];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int f = 0; f < ND; ++f) acc[s][f] = floatx4{0.f, 0.f, 0.f, 0.f};

  // buffer resources: the 16 P rows of each of the wave's query blocks, and
  // the V and Kt tiles of the kv group (bounds become offsets, see common.h)
  brsrc_t prs[2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
    prs[s] = make_brsrc(P + ((int64_t)h * s_q + (has[s] ? 16 * (int64_t)sub[s] : 0)) * s_kv,
                        (uint32_t)(16 * s_kv * 2));
  uint4 sv[SE], sk[SE];
  // P of one tile: [block][half], keys 16c .. 16c+15 (0 past the block's keys)
  auto fetch_p = [&](int64_t k0, ushortx8 (&pc)[2][2]) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const bool ok = has[s] && qrow[s] < s_q && k0 < kend[s];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        pc[s][hf] = load_p8<PVEC>(prs[s], ok, (int64_t)l16 * s_kv, k0 + 16 * c + 8 * hf, s_kv);
    }
  };
  // V and Kt of the tile at k0 (all 0 when !valid)
  auto fetch = [&](int64_t k0, bool valid) {
    const brsrc_t vr = make_brsrc(V + k0 * ldk + g * D, (uint32_t)(KT * ldk * 2));
    const brsrc_t kr = make_brsrc(Kt + (int64_t)g * D * LK + k0, (uint32_t)(((D - 1) * LK + KT) * 2));
#pragma unroll
    for (int i = 0; i < SE; ++i) {
      const int e = t + 256 * i;
      const bool eok = valid && e < NCH;
      const int kk = e / (D / 8), d8 = e % (D / 8);
      sv[i] = bload_u4(vr, (eok && k0 + kk < s_kv) ? (uint32_t)((kk * ldk + 8 * d8) * 2) : BUF_OOB);
      const int d = e / (KT / 8), k8 = e % (KT / 8);
      sk[i] = bload_u4(kr, eok ? (uint32_t)((d * LK + 8 * k8) * 2) : BUF_OOB);
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < SE; ++i) {
      const int e = t + 256 * i;
      if (e < NCH) {
        const int kk = e / (D / 8), d8 = e % (D / 8);
        const int row = 16 * ((kk >> 2) & 3) + 4 * (kk >> 4) + (kk & 3);
        *reinterpret_cast<uint4*>(&Vs[buf][row][8 * d8]) = sv[i];
        const int d = e / (KT / 8), k8 = e % (KT / 8);
        *reinterpret_cast<uint4*>(&Ks[buf][d][8 * k8]) = sk[i];
      }
    }
  };

  // Pipeline: the next tile's V/Kt loads go out at the top of a step, and
  // the next tile's P as soon as this tile's dS is formed (into the same
  // registers), so both fly during the dQ products, the barrier and the next
  // step's dA products.  Loads are unconditional (past the end they read 0),
  // so no branch makes the compiler drain them.
  int buf = 0;
  ushortx8 pc[2][2];
  fetch(0, ntile > 0);
  stash(0);
  fetch_p(0, pc);
  __syncthreads();
  for (int it = 0; it < ntile; ++it) {
    const int64_t k0 = (int64_t)it * KT;
    fetch(k0 + KT, it + 1 < ntile);
    // Block 0 (the shorter key range) is active only on the first tiles, so
    // a wave-uniform branch per phase picks a body with or without its
    // products; block 1's run unconditionally (past its range, or when the
    // wave has no second block, its P and dCtx operands are 0 and so are
    // its contributions).
    const bool on0 = k0 < kend[0];
    // dA^T: sub-tile nt, row m -> key 16(m/4) + 4nt + m%4, column = query
    floatx4 da[2][4];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) da[s][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
    ushortx8 dsa[2][2];
    auto tile_ds = [&](auto both) {
      constexpr bool B = decltype(both)::value;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int ks = 0; ks < NK; ++ks) {
          const ushortx8 a = *reinterpret_cast<const ushortx8*>(&Vs[buf][16 * nt + l16][32 * ks + 8 * c]);
          if (B) da[0][nt] = mfma16x16x32bf16(a, dcb[0][ks], da[0][nt]);
          da[1][nt] = mfma16x16x32bf16(a, dcb[1][ks], da[1][nt]);
        }
      // dS (fp32 algebra), packed to bf16 in the A layout of dQ = dS K
#pragma unroll
      for (int s = B ? 0 : 1; s < 2; ++s)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          float x[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int nt = 2 * st + j / 4, v = j % 4;
            const float p = bf2f(pc[s][st][4 * (nt & 1) + v]);
            x[j] = p * (da[s][nt][v] - dl[s]);
          }
          dsa[s][st] = pack8(x);
          // scale dS as bf16, stored as P is ([head][query][key]) for the
          // dK pass: keys k0 + 16c + 8st .. +7 of query qrow[s]
          if (ds_out != nullptr && has[s] && qrow[s] < s_q && k0 < kend[s]) {
            uint16_t* dsr = ds_out + ((int64_t)h * s_q + qrow[s]) * s_kv;
            const int64_t kc = k0 + 16 * c + 8 * st;
            float y[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) y[j] = scale * x[j];
            if (PVEC) {
              if (kc < s_kv) *reinterpret_cast<ushortx8*>(dsr + kc) = pack8(y);
            } else {
#pragma unroll
              for (int j = 0; j < 8; ++j)
                if (kc + j < s_kv) dsr[kc + j] = f2bf(y[j]);
            }
          }
        }
    };
    auto tile_dq = [&](auto both) {
      constexpr bool B = decltype(both)::value;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int f = 0; f < ND; ++f) {
          const ushortx8 b = *reinterpret_cast<const ushortx8*>(&Ks[buf][16 * f + l16][16 * c + 8 * st]);
          if (B) acc[0][f] = mfma16x16x32bf16(dsa[0][st], b, acc[0][f]);
          acc[1][f] = mfma16x16x32bf16(dsa[1][st], b, acc[1][f]);
        }
    };
    if (on0) tile_ds(std::integral_constant<bool, true>{});
    else tile_ds(std::integral_constant<bool, false>{});
    fetch_p(k0 + KT, pc);
    if (on0) tile_dq(std::integral_constant<bool, true>{});
    else tile_dq(std::integral_constant<bool, false>{});
    stash(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    if (!has[s]) continue;
#pragma unroll
    for (int f = 0; f < ND; ++f)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t row = (int64_t)16 * sub[s] + 4 * c + v;
        if (row < s_q) dq[row * ldq + h * D + 16 * f + l16] = scale * acc[s][f][v];
      }
  }
}

template <int D, int HW, bool PVEC>
__global__ __launch_bounds__(256, 2) void attn_dq_bf16_kernel(
    int64_t s_q, int64_t s_kv, int Hq, int grp, int64_t LK, int npairs,
    const float* __restrict__ dctx, const uint16_t* __restrict__ P,
    const uint16_t* __restrict__ Kt, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ ctx, const float* __restrict__ delta_ws, float* __restrict__ dq,
    float scale, int causal, uint16_t* __restrict__ ds_out) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[dq_bf16_lds<D>()];
  attn_dq_bf16_body<D, HW, PVEC>(blockIdx.x, s_q, s_kv, Hq, grp, LK, npairs, dctx, P, Kt, V, ctx,
                                 delta_ws, dq, scale, causal, smem, ds_out);
}

constexpr int HV_QT = 64;   // queries per step, bf16 dv kernel
constexpr int HV_KT = 128;  // keys per workgroup, bf16 dv kernel
constexpr DvGeo HV_GEO{HV_KT, HV_QT, HV_QT};

template <int D>
constexpr int dv_bf16_lds() {
  return 2 * HV_QT * (HV_KT + 16) + 2 * D * (HV_QT + 8);
}

// Work item blk of the bf16 dV launch, on the LDS at smem (dv_bf16_lds).
// CMASK (causal only): P is read only at keys the query sees, 0 elsewhere
// (the dK pass on scale dS, written only where the dQ kernel computed it).
template <int D, bool PVEC, bool CMASK>
__device__ __forceinline__ void attn_dv_bf16_body(int64_t blk, int64_t s_q, int64_t s_kv, int Hq,
                                                  int grp, int cmax, int64_t cs, int64_t nfull,
                                                  int64_t LQ, const uint16_t* __restrict__ P,
                                                  const uint16_t* __restrict__ dCt,
                                                  float* __restrict__ out, int causal,
                                                  uint16_t* smem) {
  constexpr int QT = HV_QT, KT = HV_KT, LDP = KT + 16, LDT = QT + 8, NJ = D / 32;
  constexpr int NP = KT * QT / 8 / 256;  // P chunks of 8 keys per thread (4)
  constexpr int NC = D * QT / 8;         // dCt chunks of 8 queries
  constexpr int SC = (NC + 255) / 256;
  auto& Pn = *reinterpret_cast<uint16_t(*)[2][QT][LDP]>(smem);  // [query][key], swizzled
  auto& Ct = *reinterpret_cast<uint16_t(*)[2][D][LDT]>(smem + 2 * QT * LDP);
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int l16 = lane & 15, c = lane >> 4;
  const int Hkv = Hq / grp;
  int g;
  int64_t jt, ch;
  if (!dv_item(blk, Hkv, s_q, s_kv, grp, causal, HV_GEO, cs, nfull, g, jt, ch)) return;
  const int64_t ldk = (int64_t)Hkv * D;
  const int64_t k0 = jt * KT;
  const int64_t qbeg = dv_tile_qbeg(jt, s_q, s_kv, causal, HV_GEO);
  // the tile's steps (head, 64-query block), head-major; chunk ch takes
  // steps [ch cs, ch cs + cs)
  const int64_t nqb = cdiv64(s_q - qbeg, QT);
  const int64_t st0 = ch * cs, st1 = min(nqb * grp, st0 + cs);
  float* dst = out + (cmax > 1 ? ch * s_kv * ldk : 0);
  if (st0 >= st1) return;
  const int kh = w & 1, dh = w >> 1;

  floatx4 acc[4][NJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int64_t nit = st1 - st0;
  // one 64-query step of global data
  struct Stage {
    ushortx8 p[NP];
    uint4 c[SC];
  };
  // one step's loads (all 0 for a step past the last, so the pipeline runs
  // without branches)
  auto fetch = [&](Stage& r, int64_t it) {
    const bool valid = it < nit;
    const int64_t stp = st0 + (valid ? it : 0);
    const int h = g * grp + (int)(stp / nqb);
    const int64_t qb = qbeg + QT * (stp % nqb);
    const brsrc_t pr = make_brsrc(P + ((int64_t)h * s_q + qb) * s_kv, (uint32_t)(QT * s_kv * 2));
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int e = t + 256 * i;
      const int rr = e >> 4, k8 = e & 15;
      const int64_t kc = k0 + 8 * k8, lim = s_kv - s_q + qb + rr;  // last key the row sees
      r.p[i] = load_p8<PVEC>(pr, valid && qb + rr < s_q && (!CMASK || kc <= lim), (int64_t)rr * s_kv,
                             kc, s_kv);
      if (CMASK) {
#pragma unroll
        for (int j = 0; j < 8; ++j) r.p[i][j] = kc + j <= lim ? r.p[i][j] : (unsigned short)0;
      }
    }
    const brsrc_t cr = make_brsrc(dCt + (int64_t)h * D * LQ + qb, (uint32_t)(((D - 1) * LQ + QT) * 2));
#pragma unroll
    for (int i = 0; i < SC; ++i) {
      const int e = t + 256 * i;
      const int d = e / (QT / 8), q8 = e % (QT / 8);
      // rows past s_q are the zero padding; their P rows read 0
      const bool ok = valid && e < NC && qb + 8 * q8 < s_q;
      r.c[i] = bload_u4(cr, ok ? (uint32_t)((d * LQ + 8 * q8) * 2) : BUF_OOB);
    }
  };
  auto stash = [&](const Stage& r, int buf) {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int e = t + 256 * i;
      const int rr = e >> 4;  // key chunk swizzled as lds_colk8<true> reads it
      *reinterpret_cast<ushortx8*>(&Pn[buf][rr][(8 * (e & 15)) ^ (64 * ((rr >> 3) & 1))]) = r.p[i];
    }
#pragma unroll
    for (int i = 0; i < SC; ++i) {
      const int e = t + 256 * i;
      if (e < NC) {
        const int d = e / (QT / 8), q8 = e % (QT / 8);
        *reinterpret_cast<uint4*>(&Ct[buf][d][8 * q8]) = r.c[i];
      }
    }
  };
  // MFMA operands of one half step (queries 32 ks .. 32 ks + 31)
  struct Half {
    ushortx8 a[4], b[NJ];
  };
  auto read_half = [&](Half& o, int buf, int ks) {
    // P^T operand: eight consecutive queries of key column 64 kh + 16 mi + l%16
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
      o.a[mi] = lds_colk8<true>(&Pn[buf][0][0], LDP, 32 * ks, 64 * kh + 16 * mi, lane);
#pragma unroll
    for (int nj = 0; nj < NJ; ++nj)
      o.b[nj] = *reinterpret_cast<const ushortx8*>(&Ct[buf][(D / 2) * dh + 16 * nj + l16][32 * ks + 8 * c]);
  };
  auto mma = [&](const Half& o) {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int nj = 0; nj < NJ; ++nj) acc[mi][nj] = mfma16x16x32bf16(o.a[mi], o.b[nj], acc[mi][nj]);
  };
  // Step it sits in LDS buffer it % 2; register stages sa, sb hold the next
  // two steps to be copied in.  Within a step the operands of each half are
  // read during the previous half's MFMAs; one barrier per step (every read
  // of a buffer is complete before it is refilled).  An odd step count ends
  // with a step of zeros.
  Stage sa;
  Half h0, h1;
  fetch(sa, 0);
  stash(sa, 0);
  fetch(sa, 1);
  stash(sa, 1);
  fetch(sa, 2);
  __syncthreads();
  read_half(h0, 0, 0);
  int buf = 0;
  for (int64_t it = 0; it < nit; ++it) {
    read_half(h1, buf, 1);
    __builtin_amdgcn_sched_barrier(0);
    mma(h0);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    read_half(h0, buf ^ 1, 0);
    __builtin_amdgcn_sched_barrier(0);
    mma(h1);
    __builtin_amdgcn_sched_barrier(0);
    stash(sa, buf);
    fetch(sa, it + 3);
    buf ^= 1;
  }
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int nj = 0; nj < NJ; ++nj)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t k = k0 + 64 * kh + 16 * mi + 4 * c + v;
        if (k < s_kv) dst[k * ldk + g * D + (D / 2) * dh + 16 * nj + l16] = acc[mi][nj][v];
      }
}

template <int D, bool PVEC, bool CMASK>
__global__ __launch_bounds__(256, 2) void attn_dv_bf16_kernel(int64_t s_q, int64_t s_kv, int Hq,
                                                           int grp, int cmax, int64_t cs,
                                                           int64_t nfull, int64_t LQ,
                                                           const uint16_t* __restrict__ P,
                                                           const uint16_t* __restrict__ dCt,
                                                           float* __restrict__ out, int causal) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[dv_bf16_lds<D>()];
  attn_dv_bf16_body<D, PVEC, CMASK>(blockIdx.x, s_q, s_kv, Hq, grp, cmax, cs, nfull, LQ, P, dCt,
                                    out, causal, smem);
}

// dQ and dV in one launch: workgroups [0, ndq) are dQ's, the rest dV's work
// items, so dV work fills the CUs as the dQ workgroups of unequal causal
// length finish.
template <int D, int HW, bool PVEC>
__global__ __launch_bounds__(256, 2) void attn_dqdv_bf16_kernel(
    int64_t s_q, int64_t s_kv, int Hq, int grp, int64_t LK, int npairs,
    const float* __restrict__ dctx, const uint16_t* __restrict__ P,
    const uint16_t* __restrict__ Kt, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ ctx, const float* __restrict__ delta_ws, float* __restrict__ dq,
    float scale, int causal, int64_t ndq, int cmax, int64_t cs, int64_t nfull, int64_t LQ,
    const uint16_t* __restrict__ dCt, float* __restrict__ dvout, uint16_t* __restrict__ ds_out) {
  constexpr int LDS = dq_bf16_lds<D>() > dv_bf16_lds<D>() ? dq_bf16_lds<D>() : dv_bf16_lds<D>();
  __shared__ __attribute__((aligned(16))) uint16_t smem[LDS];
  if ((int64_t)blockIdx.x < ndq)
    attn_dq_bf16_body<D, HW, PVEC>(blockIdx.x, s_q, s_kv, Hq, grp, LK, npairs, dctx, P, Kt, V,
                                   ctx, delta_ws, dq, scale, causal, smem, ds_out);
  else
    attn_dv_bf16_body<D, PVEC, false>((int64_t)blockIdx.x - ndq, s_q, s_kv, Hq, grp, cmax, cs,
                                      nfull, LQ, P, dCt, dvout, causal, smem);
}

// ---------------------------------------------------------------- bfloat16, D = 16
// (head dim 16: one query tile per workgroup on the fp32 MFMA)


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

// Work chunking of the dv kernels (see dv_item).  Key tile j has T_j steps,
// fewer for later tiles under the causal mask; a chunk is cs steps, the
// smallest count with which all chunks fit in `target` workgroups, so no
// chunk is much longer than the others.
struct DvPlan {
  int cmax;              // chunks of the longest tile
  int64_t cs;            // steps per chunk
  int64_t nfull, items;  // full chunks per KV group, work items
};
constexpr int FV_WG_TARGET = 768, HV_WG_TARGET = 512;
static DvPlan dv_plan(int64_t s_q, int64_t s_kv, int64_t Hkv, int64_t grp, int causal, DvGeo q,
                      int64_t target) {
  const int64_t sq = s_q < 1 ? 1 : s_q, nt = cdiv64(s_kv, q.kt);
  auto steps = [&](int64_t j) { return dv_tile_steps(j, sq, s_kv, grp, causal, q); };
  const int64_t tmax = steps(0) > 0 ? steps(0) : 1;
  DvPlan p{};
  for (int64_t cs = 4;; ++cs) {
    int64_t n = 0;
    for (int64_t j = 0; j < nt; ++j) n += cdiv64(steps(j), cs);
    if (n * Hkv <= target || cs >= tmax) {
      p.cs = cs < tmax ? cs : tmax;
      p.cmax = (int)cdiv64(tmax, p.cs);
      int64_t np = 0;
      for (int64_t j = 0; j < nt; ++j) {
        p.nfull += steps(j) / p.cs;
        np += steps(j) % p.cs != 0;
      }
      p.items = (p.nfull + np) * Hkv;
      return p;
    }
  }
}

static bool bf16_mfma_path(int dt, int64_t D) { return dt == BF16 && D >= 32; }

// Workspace of the sequence path, 256-byte aligned pieces:
//   delta [Hq, s_q] f32 (callers without ctx) | dv chunk partials f32 |
//   bf16 MFMA path: Kt [Hkv, D, LK] bf16 | dCt [Hq, D, LQ] bf16
//   with dK: scale dS [Hq, s_q, s_kv] (f32, or bf16 on the bf16 MFMA path) |
//   bf16 MFMA path: Qt [Hq, D, LQ] bf16
struct AttnWs {
  size_t delta, part, kt, dct, dq2, ds, qt, end;
  int64_t LK, LQ;
};
static size_t al256(size_t b) { return (b + 255) / 256 * 256; }
static AttnWs attn_ws(int64_t s_q, int64_t s_kv, int64_t Hq, int64_t Hkv, int64_t D, int dt,
                      bool with_dk = false) {
  AttnWs w;
  const bool hb = bf16_mfma_path(dt, D);
  // sized for the larger chunk count of the causal and the full mask
  const DvGeo geo = hb ? HV_GEO : FV_GEO;
  const int64_t tgt = hb ? HV_WG_TARGET : FV_WG_TARGET;
  const DvPlan c1 = dv_plan(s_q, s_kv, Hkv, Hq / Hkv, 1, geo, tgt);
  const DvPlan c0 = dv_plan(s_q, s_kv, Hkv, Hq / Hkv, 0, geo, tgt);
  const DvPlan dp = c1.cmax > c0.cmax ? c1 : c0;
  w.LK = cdiv64(s_kv, 64) * 64;
  w.LQ = cdiv64(s_q, 64) * 64;
  w.delta = 0;
  w.part = al256((size_t)Hq * s_q * 4);
  const size_t pb = dp.cmax > 1 ? (size_t)dp.cmax * s_kv * Hkv * D * 4 : 0;
  w.kt = w.part + al256(pb);
  w.dct = w.kt + (hb ? al256((size_t)Hkv * D * w.LK * 2) : 0);
  w.dq2 = w.dct + (hb ? al256((size_t)Hq * D * w.LQ * 2) : 0);
  // fp32 path: the second key half's dq partial (causal key split)
  w.ds = w.dq2 + (hb ? 0 : al256((size_t)s_q * Hq * D * 4));
  w.qt = w.ds + (with_dk ? al256((size_t)Hq * s_q * s_kv * (dt == BF16 ? 2 : 4)) : 0);
  w.end = w.qt + (with_dk && hb ? al256((size_t)Hq * D * w.LQ * 2) : 0);
  return w;
}

size_t attn_ws_bytes(int64_t s_q, int64_t s_kv, int64_t n_heads, int64_t n_kv_heads,
                     int64_t head_dim, int dt, bool with_dk) {
  const size_t seq = attn_ws(s_q, s_kv, n_heads, n_kv_heads, head_dim, dt, with_dk).end;
  if (with_dk) return seq;
  if (s_q == 1) {
    const size_t d = dec_attn_ws_bytes(s_kv, n_heads, head_dim);
    return d > seq ? d : seq;
  }
  return seq;
}

// unmasked (query, key) pairs per head: the work the method must do
static double attn_pairs(int64_t s_q, int64_t s_kv, int causal) {
  return causal ? (double)s_q * (s_kv - s_q) + 0.5 * (double)s_q * (s_q + 1)
                : (double)s_q * s_kv;
}

template <int D, int HW>
static void launch_dq_f32(int64_t s_q, int64_t s_kv, int Hq, int grp, const float* dctx,
                          const float* P, const float* K, const float* V, const float* ctx,
                          const float* delta, float* dq, float* dq2, bool ksplit, float scale,
                          int causal, hipStream_t s, float* ds) {
  constexpr int QW = 4 / HW;
  const int64_t nqt = cdiv64(s_q, 16 * QW);
  const dim3 grid((unsigned)((ksplit ? 2 * ((nqt + 1) / 2) : nqt) * (Hq / HW)));
#define LBP_DQ32(PV, KS)                                                                       \
  attn_dq_f32_kernel<D, HW, PV, KS><<<grid, 256, 0, s>>>(s_q, s_kv, Hq, grp, dctx, P, K, V, ctx, \
                                                         delta, dq, dq2, scale, causal, ds)
  if (s_kv % 4 == 0) {
    if (ksplit) LBP_DQ32(true, true);
    else LBP_DQ32(true, false);
  } else {
    if (ksplit) LBP_DQ32(false, true);
    else LBP_DQ32(false, false);
  }
#undef LBP_DQ32
}

// dst += src, float4 per thread (n4 float4)
__global__ __launch_bounds__(256) void add_inplace_kernel(int64_t n4, float* __restrict__ dst,
                                                          const float* __restrict__ src) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    float4 a = reinterpret_cast<float4*>(dst)[i];
    const float4 b = reinterpret_cast<const float4*>(src)[i];
    a.x += b.x;
    a.y += b.y;
    a.z += b.z;
    a.w += b.w;
    reinterpret_cast<float4*>(dst)[i] = a;
  }
}

template <int D>
static hipError_t attn_launch_f32(int64_t s_q, int64_t s_kv, int Hq, int Hkv, const float* dctx,
                                  const float* P, const float* K, const float* V,
                                  const float* ctx, float* dq, float* dv, float scale, int causal,
                                  void* ws, hipStream_t s, const float** dq_second,
                                  const RopeArgs* rope, bool* rope_done, const float* Q,
                                  float* dk) {
  const int grp = Hq / Hkv;
  const AttnWs wl = attn_ws(s_q, s_kv, Hq, Hkv, D, F32, dk != nullptr);
  float* ds = dk != nullptr ? (float*)((char*)ws + wl.ds) : nullptr;
  float* delta = (float*)((char*)ws + wl.delta);
  const double pairs = attn_pairs(s_q, s_kv, causal);
  const double pbytes = pairs * Hq * 4, qbytes = (double)s_q * Hq * D * 4;
  const double kvbytes = (double)s_kv * Hkv * D * 4;
  hipError_t e;
  if (ctx == nullptr) {
    attn_delta_kernel<float, D><<<dim3((unsigned)cdiv64(s_q, 4), (unsigned)Hq), 256, 0, s>>>(
        s_q, s_kv, Hq, grp, dctx, P, V, delta, causal);
    mark("attn_delta", 0, 2.0 * D * pairs * Hq, s, pbytes + qbytes + kvbytes + (double)Hq * s_q * 4);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int hw = grp % 4 == 0 ? 4 : (grp % 2 == 0 ? 2 : 1);
  // causal: split each query tile pair's key range in two halves (equal
  // work per workgroup); the second half's partial is added afterwards
  const bool ksplit = causal && cdiv64(s_q, 16 * (4 / hw)) >= 2;
  float* dq2 = (float*)((char*)ws + wl.dq2);
  if (hw == 4)
    launch_dq_f32<D, 4>(s_q, s_kv, Hq, grp, dctx, P, K, V, ctx, delta, dq, dq2, ksplit, scale, causal, s, ds);
  else if (hw == 2)
    launch_dq_f32<D, 2>(s_q, s_kv, Hq, grp, dctx, P, K, V, ctx, delta, dq, dq2, ksplit, scale, causal, s, ds);
  else
    launch_dq_f32<D, 1>(s_q, s_kv, Hq, grp, dctx, P, K, V, ctx, delta, dq, dq2, ksplit, scale, causal, s, ds);
  // the attention's single pass: P, dCtx, ctx, K and V read once, dq
  // written (dV's write is counted at its launch; with dK, dS is written
  // for its pass)
  mark("attn_dq_f32", pbytes + qbytes * (ctx ? 3 : 2) + 2 * kvbytes, 4.0 * D * pairs * Hq, s,
       (ksplit ? qbytes : 0.0) + (ds ? pbytes : 0.0));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ksplit && dq_second != nullptr) {
    *dq_second = dq2;  // the caller adds it (the inverse RoPE pass does)
  } else if (ksplit) {
    const int64_t n4 = s_q * Hq * D / 4;
    int64_t blocks = cdiv64(n4, 256);
    if (blocks > 4096) blocks = 4096;
    add_inplace_kernel<<<dim3((unsigned)blocks), 256, 0, s>>>(n4, dq, dq2);
    mark("attn_dq_add", 0, 0, s, qbytes * 3);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const DvPlan dp = dv_plan(s_q, s_kv, Hkv, grp, causal, FV_GEO, FV_WG_TARGET);
  float* const partbuf = (float*)((char*)ws + wl.part);
  if (dv != nullptr) {
    float* part = dp.cmax > 1 ? partbuf : dv;
    attn_dv_f32_kernel<D, false><<<dim3((unsigned)dp.items), 256, 0, s>>>(
        s_q, s_kv, Hq, grp, dp.cmax, dp.cs, dp.nfull, dctx, P, part, causal);
    mark("attn_dv_f32", kvbytes, 2.0 * D * pairs * Hq, s,
         pbytes + qbytes + (dp.cmax > 1 ? kvbytes * (dp.cmax - 1) : 0.0));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (dp.cmax > 1 &&
        (e = launch_dv_reduce(s_q, s_kv, Hq, Hkv, D, dp.cmax, dp.cs, part, dv, causal, FV_GEO, dq,
                              ksplit && dq_second != nullptr ? dq2 : nullptr, rope, rope_done, s)) !=
            hipSuccess)
      return e;
  }
  if (dk == nullptr) return hipSuccess;
  // dK = scale dS^T Q: the dV kernel on (scale dS, Q), reading dS only at the
  // keys each query sees; chunk partials reduced as dV's are
  float* kpart = dp.cmax > 1 ? partbuf : dk;
  if (causal)
    attn_dv_f32_kernel<D, true><<<dim3((unsigned)dp.items), 256, 0, s>>>(
        s_q, s_kv, Hq, grp, dp.cmax, dp.cs, dp.nfull, Q, ds, kpart, causal);
  else
    attn_dv_f32_kernel<D, false><<<dim3((unsigned)dp.items), 256, 0, s>>>(
        s_q, s_kv, Hq, grp, dp.cmax, dp.cs, dp.nfull, Q, ds, kpart, causal);
  // dK written; Q once (dS is implementation traffic: the method never
  // stores it)
  mark("attn_dk_f32", kvbytes + qbytes, 2.0 * D * pairs * Hq, s,
       pbytes + (dp.cmax > 1 ? kvbytes * (dp.cmax - 1) : 0.0));
  if ((e = hipGetLastError()) != hipSuccess || dp.cmax == 1) return e;
  return launch_dv_reduce(s_q, s_kv, Hq, Hkv, D, dp.cmax, dp.cs, kpart, dk, causal, FV_GEO, dq,
                          nullptr, nullptr, nullptr, s);
}

template <int D, int HW>
static void launch_dq_bf16(int64_t s_q, int64_t s_kv, int Hq, int grp, int64_t LK,
                           const float* dctx, const uint16_t* P, const uint16_t* Kt,
                           const uint16_t* V, const uint16_t* ctx, const float* delta, float* dq,
                           float scale, int causal, hipStream_t s, const DvPlan* dp = nullptr,
                           int64_t LQ = 0, const uint16_t* dCt = nullptr, float* dvout = nullptr,
                           uint16_t* ds = nullptr) {
  constexpr int QW = 4 / HW;
  const int nsub = (int)cdiv64(s_q, 16);
  const int npairs = (nsub + 1) / 2;
  const int64_t ndq = cdiv64(npairs, QW) * (Hq / HW);
  if (dp != nullptr) {
    // dV's work items in the same launch, after dQ's workgroups
    const dim3 g2((unsigned)(ndq + dp->items));
    if (s_kv % 8 == 0)
      attn_dqdv_bf16_kernel<D, HW, true><<<g2, 256, 0, s>>>(
          s_q, s_kv, Hq, grp, LK, npairs, dctx, P, Kt, V, ctx, delta, dq, scale, causal, ndq,
          dp->cmax, dp->cs, dp->nfull, LQ, dCt, dvout, ds);
    else
      attn_dqdv_bf16_kernel<D, HW, false><<<g2, 256, 0, s>>>(
          s_q, s_kv, Hq, grp, LK, npairs, dctx, P, Kt, V, ctx, delta, dq, scale, causal, ndq,
          dp->cmax, dp->cs, dp->nfull, LQ, dCt, dvout, ds);
    return;
  }
  const dim3 grid((unsigned)ndq);
  if (s_kv % 8 == 0)
    attn_dq_bf16_kernel<D, HW, true><<<grid, 256, 0, s>>>(s_q, s_kv, Hq, grp, LK, npairs, dctx, P,
                                                          Kt, V, ctx, delta, dq, scale, causal, ds);
  else
    attn_dq_bf16_kernel<D, HW, false><<<grid, 256, 0, s>>>(s_q, s_kv, Hq, grp, LK, npairs, dctx, P,
                                                           Kt, V, ctx, delta, dq, scale, causal, ds);
}

template <int D>
static hipError_t attn_launch_bf16(int64_t s_q, int64_t s_kv, int Hq, int Hkv, const float* dctx,
                                   const uint16_t* P, const uint16_t* K, const uint16_t* V,
                                   const uint16_t* ctx, float* dq, float* dv, float scale,
                                   int causal, void* ws, hipStream_t s, const RopeArgs* rope,
                                   bool* rope_done, bool dct_ready, const uint16_t* Q, float* dk) {
  const int grp = Hq / Hkv;
  const AttnWs wl = attn_ws(s_q, s_kv, Hq, Hkv, D, BF16, dk != nullptr);
  char* wb = (char*)ws;
  uint16_t* ds = dk != nullptr ? (uint16_t*)(wb + wl.ds) : nullptr;
  float* delta = (float*)(wb + wl.delta);
  uint16_t* Kt = (uint16_t*)(wb + wl.kt);
  uint16_t* dCt = (uint16_t*)(wb + wl.dct);
  const double pairs = attn_pairs(s_q, s_kv, causal);
  const double pbytes = pairs * Hq * 2, qbytes = (double)s_q * Hq * D;
  const double kvbytes = (double)s_kv * Hkv * D;
  hipError_t e;
  // Kᵀ for dQ and, when dV is wanted, dCtxᵀ for it, in one launch
  const TrJob jk{s_kv, wl.LK, (int64_t)Hkv * D, K, Kt, (int)(wl.LK / TR_R), (int)(Hkv * D / TR_C)};
  const TrJob jd{s_q, wl.LQ, (int64_t)Hq * D, dctx, dCt, (int)(wl.LQ / TR_R),
                 dv != nullptr && !dct_ready ? (int)(Hq * D / TR_C) : 0};
  const int64_t ntr = (int64_t)jk.gx * jk.gy + (int64_t)jd.gx * jd.gy;
  transpose_bf16_kernel<bf16, float><<<dim3((unsigned)ntr), 256, 0, s>>>(jk, jd);
  mark("transpose_bf16", 0, 0, s,
       kvbytes * 2 + (double)Hkv * D * wl.LK * 2 +
           (jd.gy > 0 ? qbytes * 4 + (double)Hq * D * wl.LQ * 2 : 0.0));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ctx == nullptr) {
    attn_delta_kernel<bf16, D><<<dim3((unsigned)cdiv64(s_q, 4), (unsigned)Hq), 256, 0, s>>>(
        s_q, s_kv, Hq, grp, dctx, (const bf16*)P, (const bf16*)V, delta, causal);
    mark("attn_delta", 0, 2.0 * D * pairs * Hq, s,
         pbytes + qbytes * 4 + kvbytes * 2 + (double)Hq * s_q * 4);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // dQ, and with dv wanted dV in the same launch
  const DvPlan dp = dv_plan(s_q, s_kv, Hkv, grp, causal, HV_GEO, HV_WG_TARGET);
  float* part = dp.cmax > 1 ? (float*)(wb + wl.part) : dv;
  const DvPlan* dpp = dv != nullptr ? &dp : nullptr;
  const int hw = grp % 4 == 0 ? 4 : (grp % 2 == 0 ? 2 : 1);
  if (hw == 4)
    launch_dq_bf16<D, 4>(s_q, s_kv, Hq, grp, wl.LK, dctx, P, Kt, V, ctx, delta, dq, scale, causal, s,
                         dpp, wl.LQ, dCt, part, ds);
  else if (hw == 2)
    launch_dq_bf16<D, 2>(s_q, s_kv, Hq, grp, wl.LK, dctx, P, Kt, V, ctx, delta, dq, scale, causal, s,
                         dpp, wl.LQ, dCt, part, ds);
  else
    launch_dq_bf16<D, 1>(s_q, s_kv, Hq, grp, wl.LK, dctx, P, Kt, V, ctx, delta, dq, scale, causal, s,
                         dpp, wl.LQ, dCt, part, ds);
  // the attention's single pass: P, dCtx (fp32), ctx, K and V read once,
  // dq and dV written; the dV body's second read of P, the transposed
  // copies it reads and its chunk partials are implementation traffic
  const double alg = pbytes + qbytes * (4 + 4 + (ctx ? 2 : 0)) + 2 * kvbytes * 2 +
                     (dv != nullptr ? kvbytes * 4 : 0.0);
  if (dv == nullptr)
    mark("attn_dq_bf16", alg, 4.0 * D * pairs * Hq, s, ds ? pbytes : 0.0);
  else
    mark("attn_dqdv_bf16", alg, 6.0 * D * pairs * Hq, s,
         pbytes * (ds ? 2 : 1) + qbytes * 2 + (dp.cmax > 1 ? kvbytes * 4 * (dp.cmax - 1) : 0.0));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (dv != nullptr && dp.cmax > 1 &&
      (e = launch_dv_reduce(s_q, s_kv, Hq, Hkv, D, dp.cmax, dp.cs, part, dv, causal, HV_GEO, dq,
                            nullptr, rope, rope_done, s)) != hipSuccess)
    return e;
  if (dk == nullptr) return hipSuccess;
  // dK = scale dS^T Q: the dV body on (scale dS, Q^T), reading dS only at the
  // keys each query sees; Q^T [Hq, D, LQ] bf16 (zero padded) first
  uint16_t* Qt = (uint16_t*)(wb + wl.qt);
  const TrJob jq{s_q, wl.LQ, (int64_t)Hq * D, Q, Qt, (int)(wl.LQ / TR_R), (int)(Hq * D / TR_C)};
  const TrJob none{0, 0, 0, nullptr, nullptr, 0, 0};
  transpose_bf16_kernel<bf16, bf16><<<dim3((unsigned)((int64_t)jq.gx * jq.gy)), 256, 0, s>>>(jq, none);
  mark("transpose_bf16", 0, 0, s, qbytes * 2 + (double)Hq * D * wl.LQ * 2);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  float* kpart = dp.cmax > 1 ? (float*)(wb + wl.part) : dk;
#define LBP_DK16(PV, CM)                                                                      \
  attn_dv_bf16_kernel<D, PV, CM><<<dim3((unsigned)dp.items), 256, 0, s>>>(                     \
      s_q, s_kv, Hq, grp, dp.cmax, dp.cs, dp.nfull, wl.LQ, ds, Qt, kpart, causal)
  if (s_kv % 8 == 0) {
    if (causal) LBP_DK16(true, true);
    else LBP_DK16(true, false);
  } else {
    if (causal) LBP_DK16(false, true);
    else LBP_DK16(false, false);
  }
#undef LBP_DK16
  mark("attn_dk_bf16", kvbytes * 4 + qbytes * 2, 2.0 * D * pairs * Hq, s,
       pbytes + (dp.cmax > 1 ? kvbytes * 4 * (dp.cmax - 1) : 0.0));
  if ((e = hipGetLastError()) != hipSuccess || dp.cmax == 1) return e;
  return launch_dv_reduce(s_q, s_kv, Hq, Hkv, D, dp.cmax, dp.cs, kpart, dk, causal, HV_GEO, dq,
                          nullptr, nullptr, nullptr, s);
}

template <typename T, int D>
static hipError_t attn_launch(int64_t s_q, int64_t s_kv, int Hq, int Hkv, const float* dctx,
                              const T* P, const T* K, const T* V, const T* ctx, float* dq,
                              float* dv, float scale, int causal, float* ws, hipStream_t s) {
  const int grp = Hq / Hkv;
  const double es = sizeof(T);
  dim3 block(256);
  const double pairs = attn_pairs(s_q, s_kv, causal);
  const double pbytes = pairs * Hq * es, qbytes = (double)s_q * Hq * D;
  const double kvbytes = (double)s_kv * Hkv * D;
  dim3 gq((unsigned)((s_q + AQ - 1) / AQ), (unsigned)Hq);
  if (ctx != nullptr) {
    attn_dq_kernel<T, D, 1><<<gq, block, 0, s>>>(s_q, s_kv, Hq, grp, dctx, P, K, V, ctx, nullptr,
                                                  dq, scale, causal);
    mark("attn_dq_mfma", pbytes + qbytes * (8 + es) + 2 * kvbytes * es, 4.0 * D * pairs * Hq, s);  // P, dCtx, ctx, K, V once; dq
  } else {
    attn_delta_kernel<T, D><<<dim3((unsigned)((s_q + 3) / 4), (unsigned)Hq), block, 0, s>>>(
        s_q, s_kv, Hq, grp, dctx, P, V, ws, causal);
    mark("attn_delta", 0, 2.0 * D * pairs * Hq, s,
         pbytes + qbytes * 4 + kvbytes * es + (double)Hq * s_q * 4);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    attn_dq_kernel<T, D, 0><<<gq, block, 0, s>>>(s_q, s_kv, Hq, grp, dctx, P, K, V, nullptr, ws,
                                                  dq, scale, causal);
    mark("attn_dq_mfma", pbytes + qbytes * 8 + 2 * kvbytes * es, 4.0 * D * pairs * Hq, s,
         (double)Hq * s_q * 4);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || dv == nullptr) return e;
  constexpr int KB = 16 * (D >= 32 ? 2 : 4);
  attn_dv_kernel<T, D><<<dim3((unsigned)((s_kv + KB - 1) / KB), (unsigned)Hkv), block, 0, s>>>(
      s_q, s_kv, Hq, grp, dctx, P, dv, causal);
  mark("attn_dv_mfma", kvbytes * 4, 2.0 * D * pairs * Hq, s, pbytes + qbytes * 4);
  return hipGetLastError();
}

template <typename T>
static hipError_t attn_dispatch_d(int64_t s_q, int64_t s_kv, int Hq, int Hkv, int D,
                                  const float* dctx, const void* P, const void* K, const void* V,
                                  const void* ctx, float* dq, float* dv, float scale, int causal,
                                  void* ws, hipStream_t s, const float** dq_second,
                                  const RopeArgs* rope, bool* rope_done, bool dct_ready,
                                  const void* Q, float* dk) {
#define LBP_ATTN_D(DD)                                                                         \
  case DD:                                                                                     \
    if constexpr (sizeof(T) == 4)                                                              \
      return attn_launch_f32<DD>(s_q, s_kv, Hq, Hkv, dctx, (const float*)P, (const float*)K,   \
                                 (const float*)V, (const float*)ctx, dq, dv, scale, causal, ws, \
                                 s, dq_second, rope, rope_done, (const float*)Q, dk);          \
    else if constexpr (DD >= 32)                                                               \
      return attn_launch_bf16<DD>(s_q, s_kv, Hq, Hkv, dctx, (const uint16_t*)P,                \
                                  (const uint16_t*)K, (const uint16_t*)V, (const uint16_t*)ctx, \
                                  dq, dv, scale, causal, ws, s, rope, rope_done, dct_ready,    \
                                  (const uint16_t*)Q, dk);                                     \
    else if (dk != nullptr)                                                                    \
      return hipErrorInvalidValue; /* dK is not built for bf16 with head_dim 16 */             \
    else                                                                                       \
      return attn_launch<T, DD>(s_q, s_kv, Hq, Hkv, dctx, (const T*)P, (const T*)K,            \
                                (const T*)V, (const T*)ctx, dq, dv, scale, causal, (float*)ws, s);
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
                           float scale, int causal, void* ws, hipStream_t s,
                           const float** dq_second, const RopeArgs* rope, bool* rope_done,
                           bool dct_ready, const void* Q, float* dk) {
  if (dq_second != nullptr) *dq_second = nullptr;
  if (rope_done != nullptr) *rope_done = false;
  if (s_q == 0) {
    hipError_t e = hipSuccess;
    if (dv != nullptr) e = launch_fill_zero(s_kv * n_kv_heads * head_dim, dv, s);
    if (e == hipSuccess && dk != nullptr) e = launch_fill_zero(s_kv * n_kv_heads * head_dim, dk, s);
    return e;
  }
  if (dk != nullptr && (Q == nullptr || (dt == BF16 && head_dim < 32))) return hipErrorInvalidValue;
  if (s_q == 1 && dk == nullptr && dec_attn_fits(s_kv, n_heads, n_kv_heads, head_dim)) {
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
  // buffer ranges (a block of 64 query rows of P, dctx and ctx; 64 key rows
  // of K and V; one head of the transposed bf16 copies) and grid rows (heads)
  const double es = dt == F32 ? 4 : 2, lq = (double)n_heads * head_dim;
  const double lk = (double)n_kv_heads * head_dim;
  if (64.0 * s_kv * es >= BUF_MAX_BYTES || 64.0 * lq * 4 >= BUF_MAX_BYTES ||
      64.0 * lk * 4 >= BUF_MAX_BYTES || (double)head_dim * (s_kv + 64) * 2 >= BUF_MAX_BYTES ||
      (double)head_dim * (s_q + 64) * 2 >= BUF_MAX_BYTES || n_heads > 65535)
    return hipErrorInvalidValue;
  if (dry_run()) return hipSuccess;
  if (dt == F32)
    return attn_dispatch_d<float>(s_q, s_kv, (int)n_heads, (int)n_kv_heads, (int)head_dim, dctx,
                                  P, K, V, ctx, dq, dv, scale, causal, ws, s, dq_second, rope,
                                  rope_done, false, Q, dk);
  return attn_dispatch_d<bf16>(s_q, s_kv, (int)n_heads, (int)n_kv_heads, (int)head_dim, dctx, P,
                               K, V, ctx, dq, dv, scale, causal, ws, s, dq_second, rope,
                               rope_done, dct_ready, Q, dk);
}

uint16_t* attn_dct_buffer(void* ws, int64_t s_q, int64_t s_kv, int64_t n_heads,
                          int64_t n_kv_heads, int64_t head_dim, int dt, int64_t* LQ) {
  // the bf16 MFMA launch is the one that takes dCtxᵀ (sequence rows)
  if (s_q <= 1 || dt != BF16 || !bf16_mfma_path(dt, head_dim)) return nullptr;
  const AttnWs wl = attn_ws(s_q, s_kv, n_heads, n_kv_heads, head_dim, dt);
  *LQ = wl.LQ;
  return (uint16_t*)((char*)ws + wl.dct);
}

}  // namespace lbp
