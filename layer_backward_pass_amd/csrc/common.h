// Device helpers shared by the lorabwd kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lbp {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short ushortx8 __attribute__((ext_vector_type(8)));
typedef unsigned short ushortx4 __attribute__((ext_vector_type(4)));

// bfloat16 is carried as its 16-bit pattern.
struct bf16 {
  uint16_t bits;
};

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// float32 -> bfloat16 by the hardware conversion (v_cvt_pk_bf16_f32): round
// to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
// two floats rounded to bf16 and packed (a in the low half), one instruction
typedef float lbp_float2v __attribute__((ext_vector_type(2)));
typedef __bf16 lbp_bf16x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  const lbp_float2v f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, lbp_bf16x2v));
}

// Scalar and vector loads of an activation element (float or bf16) as float.
template <typename T> struct Act;
template <> struct Act<float> {
  static __device__ __forceinline__ float ld(const float* p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ float4 ld4(const float* p, int64_t i) {
    return *reinterpret_cast<const float4*>(p + i);
  }
};
template <> struct Act<bf16> {
  static __device__ __forceinline__ float ld(const bf16* p, int64_t i) { return bf2f(p[i].bits); }
  static __device__ __forceinline__ float4 ld4(const bf16* p, int64_t i) {
    uint2 u = *reinterpret_cast<const uint2*>(p + i);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
  }
};

// Buffer loads (MUBUF, offsets in bytes from a resource base).  A load whose
// per-lane offset is at or past the resource's size reads 0 and touches no
// memory, so a bound becomes an offset instead of a branch: a branch around
// a load makes the compiler wait for every load still in flight where the
// two paths join, which empties a register prefetch pipeline.  Only the
// per-lane (VGPR) offset carries bounds here; resources stay below 1 GiB so
// a valid offset plus BUF_OOB never wraps into range.
typedef __amdgpu_buffer_rsrc_t brsrc_t;
// cache policy of a load that streams data read once (the nt bit): weight
// rows of a GEMV are not worth keeping in L2 (decode [W_gate;W_up]:
// 25.5 -> 23.6 us)
constexpr int BUF_NT = 2;
constexpr uint32_t BUF_OOB = 0x80000000u;
constexpr uint32_t BUF_MAX_BYTES = 0x40000000u;
__device__ __forceinline__ brsrc_t make_brsrc(const void* base, uint32_t bytes) {
  // word 3 = 0x00020000: 32-bit raw data format for the gfx9 family
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
template <int AUX = 0>
__device__ __forceinline__ float4 bload_f4(brsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, AUX);
  return make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]),
                     __uint_as_float(v[3]));
}
template <int AUX = 0>
__device__ __forceinline__ uint2 bload_u2(brsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, AUX);
  return make_uint2(v[0], v[1]);
}
__device__ __forceinline__ float2 bload_f2(brsrc_t r, uint32_t off) {
  const uint2 v = bload_u2(r, off);
  return make_float2(__uint_as_float(v.x), __uint_as_float(v.y));
}
__device__ __forceinline__ uint4 bload_u4(brsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ float4 bf4_to_f4(uint2 u) {
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}
// 4 consecutive elements (float or bf16) at element index i as float; the
// raw type is kept until use so that the load is not waited on early
template <typename T> struct BufVec;
template <> struct BufVec<float> {
  typedef float4 raw;
  static __device__ __forceinline__ raw load(brsrc_t r, uint32_t off) { return bload_f4(r, off); }
  static __device__ __forceinline__ raw load_stream(brsrc_t r, uint32_t off) { return bload_f4<BUF_NT>(r, off); }
  static __device__ __forceinline__ float4 cvt(raw v) { return v; }
  static __device__ __forceinline__ raw zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }
};
template <> struct BufVec<bf16> {
  typedef uint2 raw;
  static __device__ __forceinline__ raw load(brsrc_t r, uint32_t off) { return bload_u2(r, off); }
  static __device__ __forceinline__ raw load_stream(brsrc_t r, uint32_t off) { return bload_u2<BUF_NT>(r, off); }
  static __device__ __forceinline__ float4 cvt(raw v) { return bf4_to_f4(v); }
  static __device__ __forceinline__ raw zero() { return make_uint2(0u, 0u); }
};

// Packed ternary weights (lorabwd_pack_ternary): 2-bit sign codes, column
// 4c + j in bits 2j .. 2j+1 of byte c of a row (00 -> 0, 01 -> +1, 11 -> -1).
// A lane's four columns of one row are one byte; each field is sign-extended
// (v_bfe_i32) to its value in {-1, 0, +1}.  The matrix's scale is applied by
// the user of the values.
struct tern2 {
  uint8_t bits;
};
template <> struct BufVec<tern2> {
  typedef uint32_t raw;
  static __device__ __forceinline__ raw load(brsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b8(r, (int)off, 0, 0);
  }
  static __device__ __forceinline__ raw load_stream(brsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b8(r, (int)off, 0, BUF_NT);
  }
  // (the builtin's result type is unsigned: the field is read back as int
  // before the conversion, or -1 would convert as 2^32 - 1)
  static __device__ __forceinline__ float4 cvt(raw v) {
    const int b = (int)v;
    return make_float4((float)(int)__builtin_amdgcn_sbfe(b, 0, 2), (float)(int)__builtin_amdgcn_sbfe(b, 2, 2),
                       (float)(int)__builtin_amdgcn_sbfe(b, 4, 2), (float)(int)__builtin_amdgcn_sbfe(b, 6, 2));
  }
  static __device__ __forceinline__ raw zero() { return 0u; }
};
// bytes that four consecutive columns of a weight row take
template <typename T> struct ColBytes4 { static constexpr int v = 4 * (int)sizeof(T); };
template <> struct ColBytes4<tern2> { static constexpr int v = 1; };

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Sum over a block of NW waves; result valid in every thread.  `red` must
// hold NW floats; the call ends with a barrier so `red` can be reused.
template <int NW>
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NW; ++i) s += red[i];
  __syncthreads();
  return s;
}

// Workgroups are handed to the 8 XCDs round-robin by linear id.  Renumber
// them so that XCD x runs one contiguous block of the T work items: items
// that share operands (consecutive ids) then share that XCD's L2.
__device__ __forceinline__ int64_t xcd_remap(int64_t L, int64_t T) {
  const int64_t x = L & 7, j = L >> 3, q = T >> 3, r = T & 7;
  return x * q + (x < r ? x : r) + j;
}

__device__ __forceinline__ floatx4 mfma16x16x4(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// gfx950 LDS transpose read (16-bit elements).  Within each group of 16
// lanes, result lane i, element j is the 16-bit value at offset i%4 from the
// address given by lane 4j + i/4 of the group.  With the 16 lanes pointing
// at four rows k .. k+3 of a row-major tile (lane i': row k + i'/4, columns
// n0 + 4(i'%4) .. +3), lane i receives column n0 + i of rows k .. k+3.
__device__ __forceinline__ ushortx4 lds_read_tr16(const uint16_t* p) {
  typedef short s4 __attribute__((ext_vector_type(4)));
  const s4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s4*)(p));
  return __builtin_bit_cast(ushortx4, r);
}

// MFMA bf16 operand (eight consecutive k of column n0 + l%16, k from row
// k0 + 8(l/16)) out of a row-major [k][n] LDS tile with row stride ld.
// SWZ: the tile stores row k, column n at column n ^ (64 ((k / 8) % 2))
// (rows >= 128 wide, k0 % 16 == 0), so that the four lane groups, whose
// rows are 8 apart, do not read the same banks.
template <bool SWZ = false>
__device__ __forceinline__ ushortx8 lds_colk8(const uint16_t* tile, int ld, int k0, int n0,
                                              int lane) {
  const int l16 = lane & 15, c = lane >> 4;
  const int nc = SWZ ? (n0 ^ (64 * (c & 1))) : n0;
  const uint16_t* p = tile + (k0 + 8 * c + (l16 >> 2)) * ld + nc + 4 * (l16 & 3);
  const ushortx4 lo = lds_read_tr16(p);
  const ushortx4 hi = lds_read_tr16(p + 4 * ld);
  return ushortx8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ floatx4 mfma16x16x32bf16(ushortx8 a, ushortx8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Inverse NeoX RoPE of one row, all heads.  Hesper "Attention Backward GPU
// Kernels", section "RoPE Backward (inverse rotation)", of dy (+ dy2: the two
// key halves of a split attention dq, added here).  Thread tid < nthr is
// (d, hg) = (tid % half, tid / half): it forms theta_d = pos * base^(-2d/D)
// and its cosine and sine in float64 once, then rotates the (d, d + half)
// pair of every head hg, hg + HG, ...  The angle of a late position needs
// float64: at pos ~2e3 one float32 ulp of theta is ~1e-4 rad.
//
// With norm.x set (QK-norm: the rotated values are the gradient of a per-head
// RMSNorm's output), each head's rotated slice g then goes through that
// norm's backward, dx = (gamma g - x <gamma g, x> / (D r^2)) / r with
// r = sqrt(mean(x^2) + eps) over the head's D features of the norm input x
// (the saved projection output) and one scale vector gamma [D] for every
// head.  A head's `half` threads are consecutive lanes of one wave (half
// divides 64 and every thread of a head runs the same iterations), so its
// two sums are a shuffle reduction within that lane group.
struct RopeNorm {
  const void* x;  // [rows, n_heads * head_dim] float or bf16; NULL: no norm
  int x_bf16;
  const float* gamma;  // [head_dim]
  float eps;
};

__device__ __forceinline__ float group_sum(float v, int width) {
  for (int m = width >> 1; m > 0; m >>= 1) v += __shfl_xor(v, m, width);
  return v;
}

__device__ __forceinline__ void rope_bwd_row(int64_t row, int tid, int nthr, int64_t n_heads,
                                             int head_dim, const float* dy, const float* dy2,
                                             float* dx, int64_t pos0, double log2_base,
                                             const RopeNorm& nm = RopeNorm{nullptr, 0, nullptr, 0.f}) {
  const int half = head_dim >> 1;
  const int d = tid % half;
  const int hg = tid / half;
  const int HG = nthr / half;
  const double pos = (double)(pos0 + row);
  const double inv_freq = exp2(-(2.0 * d / head_dim) * log2_base);
  double sn, cs;
  sincos(pos * inv_freq, &sn, &cs);
  const float c = (float)cs, s = (float)sn;
  const int64_t base = row * n_heads * head_dim;
  const bool norm = nm.x != nullptr;
  const float g_lo = norm ? nm.gamma[d] : 0.f, g_hi = norm ? nm.gamma[d + half] : 0.f;
  for (int64_t h = hg; h < n_heads; h += HG) {
    const int64_t i = base + h * head_dim + d;
    float lo = dy[i], hi = dy[i + half];
    if (dy2 != nullptr) {
      lo += dy2[i];
      hi += dy2[i + half];
    }
    float o_lo = lo * c + hi * s;
    float o_hi = -lo * s + hi * c;
    if (norm) {
      float x_lo, x_hi;
      if (nm.x_bf16) {
        const uint16_t* xb = (const uint16_t*)nm.x;
        x_lo = bf2f(xb[i]);
        x_hi = bf2f(xb[i + half]);
      } else {
        const float* xf = (const float*)nm.x;
        x_lo = xf[i];
        x_hi = xf[i + half];
      }
      const float gl = g_lo * o_lo, gh = g_hi * o_hi;
      const float sxx = group_sum(x_lo * x_lo + x_hi * x_hi, half);
      const float sgx = group_sum(gl * x_lo + gh * x_hi, half);
      const float r2 = sxx / (float)head_dim + nm.eps;
      const float inv_r = 1.0f / sqrtf(r2);
      const float k = sgx / ((float)head_dim * r2);
      o_lo = (gl - x_lo * k) * inv_r;
      o_hi = (gh - x_hi * k) * inv_r;
    }
    dx[i] = o_lo;
    dx[i + half] = o_hi;
  }
}

// Gated activation backward of one element.
//   SwiGLU (entrenar wgpu_backward.rs, "SiLU backward"): s = sigmoid(g),
//     dGate = dH up s (1 + g (1 - s)),  dUp = dH g s
//   ReLU^2 x up (Hesper "FFN Backward GPU Kernels", "ReLU²×Mul Backward"):
//     dGate = dH up 2 max(0,g),  dUp = dH max(0,g)^2
template <int ACT>
__device__ __forceinline__ void act_bwd1(float g, float u, float dh, float& dg, float& du) {
  if (ACT == 0) {
    const float sg = 1.0f / (1.0f + expf(-g));
    dg = dh * u * sg * (1.0f + g * (1.0f - sg));
    du = dh * g * sg;
  } else {
    const float r = fmaxf(g, 0.0f);
    dg = dh * u * 2.0f * r;
    du = dh * r * r;
  }
}

}  // namespace lbp
