// Device helpers shared by the CSA2 HIP kernels (gfx950 / CDNA4).
//
// MFMA operand convention used by every kernel: one 16x16 output tile takes a
// "k-step" of 32 contraction elements; lane l supplies row (l % 16) of A and
// column (l % 16) of B, each with the 8 consecutive k-slots 8*(l/16) .. +7.  The
// accumulator gives lane l the outputs C[4*(l/16) + i][l % 16], i < 4.  For
// bf16 this is one v_mfma_f32_16x16x32_bf16; for fp32 the same 8 slots feed
// eight v_mfma_f32_16x16x4f32 (k-slot j of every lane in step j).  Because a
// contraction does not care how k is numbered, a kernel may map the 32 k-slots
// of a step to any 32 source elements as long as A and B use the same map.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

typedef __bf16 bf16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;

struct f32x8 { float v[8]; };

template <typename T> struct Frag;                 // 8 k-slots of one lane
template <> struct Frag<bf16> { typedef bf16x8 type; };
template <> struct Frag<float> { typedef f32x8 type; };

__device__ __forceinline__ f32x4 mma16(const bf16x8& a, const bf16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(const f32x8& a, const f32x8& b, f32x4 c) {
#pragma unroll
  for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], c, 0, 0, 0);
  return c;
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // RNE

// Load 8 consecutive elements (16 B for bf16, 32 B for fp32) as an operand fragment.
__device__ __forceinline__ bf16x8 load_frag(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ f32x8 load_frag(const float* p) {
  f32x8 r;
  const float4* q = reinterpret_cast<const float4*>(p);
  float4 a = q[0], b = q[1];
  r.v[0] = a.x; r.v[1] = a.y; r.v[2] = a.z; r.v[3] = a.w;
  r.v[4] = b.x; r.v[5] = b.y; r.v[6] = b.z; r.v[7] = b.w;
  return r;
}
__device__ __forceinline__ void zero_frag(bf16x8& f) {
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = (bf16)0.0f;
}
__device__ __forceinline__ void zero_frag(f32x8& f) {
#pragma unroll
  for (int i = 0; i < 8; ++i) f.v[i] = 0.0f;
}

// ---------------------------------------------------------------- FP8 / FP4
// E4M3FN (OCP FP8): bias 7, max finite 448, no infinities.
// Non-negative finite input, round to nearest even, saturate at 448.
__device__ __forceinline__ uint32_t e4m3_encode_nonneg(float v) {
  if (!(v < 448.0f)) return 0x7Eu;
  uint32_t bits = __float_as_uint(v);
  int ex = (int)((bits >> 23) & 0xFF);
  if (ex >= 121) {                       // v >= 2^-6: normal E4M3 range
    uint32_t mant = bits & 0x7FFFFFu;
    uint32_t keep = mant >> 20, rest = mant & 0xFFFFFu;
    uint32_t r = ((uint32_t)(ex - 120) << 3) | keep;
    if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) r += 1u;  // carry may bump the exponent
    return r > 0x7Eu ? 0x7Eu : r;
  }
  // subnormal grid: multiples of 2^-9 (8 * 2^-9 is the smallest normal, byte 0x08)
  float m = __builtin_rintf(v * 512.0f);  // exact scaling, RNE
  return (uint32_t)m;
}
__device__ __forceinline__ float e4m3_decode(uint32_t b) {
  uint32_t e = (b >> 3) & 15u, m = b & 7u;
  float v = (e == 0) ? (float)m * 0.001953125f : ldexpf((float)(8u + m), (int)e - 10);
  return (b & 0x80u) ? -v : v;
}
// E2M1 (OCP MX FP4) of a float32, nearest with ties to the even code, saturating
// at 6; bit 3 carries the sign even when the magnitude rounds to zero.
__device__ __forceinline__ uint32_t e2m1_encode(float x) {
  float a = fabsf(x);
  uint32_t c = (a <= 0.25f) ? 0u : (a < 0.75f) ? 1u : (a <= 1.25f) ? 2u : (a < 1.75f) ? 3u
             : (a <= 2.5f) ? 4u : (a < 3.5f) ? 5u : (a <= 5.0f) ? 6u : 7u;
  return c | ((__float_as_uint(x) >> 28) & 8u);
}

// Value of an E2M1 code as a float32: magnitude bits e1 e0 m give m/2 for e = 0
// and 2^(e-1) (1 + m/2) otherwise; bit 3 is the sign.
__device__ __forceinline__ float e2m1_value(uint32_t c) {
  const uint32_t e = (c >> 1) & 3u, m = c & 1u;
  const uint32_t bits = (e == 0u) ? (m ? 0x3F000000u : 0u) : (((e + 126u) << 23) | (m << 22));
  return __uint_as_float(bits | ((c & 8u) << 28));
}

// Quantise one 32-value block held 2 values per lane by 16 lanes of a 16-lane
// group: returns the scale byte (all 16 lanes) and the two codes of this lane.
// `amax` must already be the maximum of |v| over the block.
__device__ __forceinline__ uint32_t fp4_scale_byte(float amax) {
  return e4m3_encode_nonneg(__fdiv_rn(amax, 6.0f));
}
__device__ __forceinline__ uint32_t fp4_code(float v, float s) {
  return (s == 0.0f) ? 0u : e2m1_encode(__fdiv_rn(v, s));
}

// UE8M0 (a bare biased exponent): value 2^(b - 127), byte 255 unused.
__device__ __forceinline__ float ue8m0_decode(uint32_t b) {
  return b == 0u ? __uint_as_float(0x00400000u) : __uint_as_float(b << 23);   // 2^-127 is subnormal
}
// Byte of the smallest power of two at or above sigma >= 0, clamped to 2^-127 ..
// 2^127; sigma == 0 gives byte 0.
__device__ __forceinline__ uint32_t ue8m0_encode_ceil(float sigma) {
  if (!(sigma > 0.0f)) return 0u;
  const uint32_t bits = __float_as_uint(sigma);
  const int ex = (int)((bits >> 23) & 0xFFu);
  const uint32_t mant = bits & 0x7FFFFFu;
  // ceil(log2 sigma): normal 1.m x 2^(ex-127); subnormal mant x 2^-149
  int e = ex != 0 ? ex - 127 + (mant != 0u ? 1 : 0) : (32 - __clz((int)(mant - 1u))) - 149;
  e = e < -127 ? -127 : (e > 127 ? 127 : e);
  return (uint32_t)(e + 127);
}
// One index-K block's scale byte and scale value in format sfmt (0 = E4M3, 1 = UE8M0).
__device__ __forceinline__ uint32_t ik_scale_byte(float amax, int sfmt) {
  return sfmt ? ue8m0_encode_ceil(__fdiv_rn(amax, 6.0f)) : fp4_scale_byte(amax);
}
__device__ __forceinline__ float ik_scale_value(uint32_t b, int sfmt) {
  return sfmt ? ue8m0_decode(b) : e4m3_decode(b);
}

// ---------------------------------------------------------------- RoPE
// Angle of rotary pair i (of n_rope/2) at position pos, computed in double so
// that large positions (up to 2^20 and beyond) keep full float accuracy.
__device__ __forceinline__ void rope_cos_sin(int64_t pos, int pair, int n_rope, double base, float& c, float& s) {
  double theta = pow(base, -2.0 * (double)pair / (double)n_rope);
  double ang = (double)pos * theta;
  double sd, cd;
  sincos(ang, &sd, &cd);
  c = (float)cd;
  s = (float)sd;
}

// ---------------------------------------------------------------- misc
__device__ __forceinline__ float wave_sum_xor(float v, int width_mask) {
  // butterfly over lanes differing in the bits of width_mask (powers of two)
  for (int off = 1; off < 64; off <<= 1)
    if (width_mask & off) v += __shfl_xor(v, off, 64);
  return v;
}
__device__ __forceinline__ float wave_max_xor(float v, int width_mask) {
  for (int off = 1; off < 64; off <<= 1)
    if (width_mask & off) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// Order-preserving map of a float score to uint32 (larger score -> larger key);
// -0 is mapped like +0.
__device__ __forceinline__ uint32_t score_key(float s) {
  if (s == 0.0f) s = 0.0f;  // -0 -> +0
  uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

}  // namespace csa2
