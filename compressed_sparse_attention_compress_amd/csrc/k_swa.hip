// Sliding-window KV in FP8 ([P3] "DeepSeek-V4.1-Flash：把百万 Token 的记忆…",
// section seven: the local window KV is more sensitive to quantisation than the
// main KV and is kept in FP8).  Stored as E4M3FN bytes with no scale, one per
// dimension, in a per-layer ring of L_w rows: the row of position u sits in slot
// u mod L_w.
//
// swa_fp8_append: quantises new rows into their slots (one wave per row, 8 dims
//   per lane, nearest-even with saturation at +-448, the sign kept for a value
//   that rounds to zero).
// swa_fp8_window: reads L_w rows of each sequence out of the ring, in position
//   order from p0 = max(swa_pos0, newest - L_w + 1) (newest = the largest query
//   position of that sequence in the call), into dense rows of the attention
//   dtype, and writes p0 as that sequence's first dense position.  E4M3 values
//   are exact in bf16 and fp32, so attention over them sees exactly the stored
//   values.
#include "csa2_internal.h"
#include "device_common.h"

namespace csa2 {

namespace {

__device__ __forceinline__ uint32_t e4m3_encode_signed(float v) {
  return e4m3_encode_nonneg(fabsf(v)) | ((__float_as_uint(v) >> 24) & 0x80u);
}

template <typename T>
__global__ __launch_bounds__(64) void swa_fp8_append(const T* __restrict__ rows, const int32_t* __restrict__ pos,
                                                     uint8_t* __restrict__ ring, int T_len, int L_w) {
  const int bt = blockIdx.x;
  const int b = bt / T_len;
  const int u = pos[bt];
  if (u < 0) return;
  const int lane = threadIdx.x;
  const T* src = rows + (size_t)bt * 512 + lane * 8;
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i >> 2] |= e4m3_encode_signed(to_f32(src[i])) << (8 * (i & 3));
  uint8_t* dst = ring + ((size_t)b * L_w + (u % L_w)) * 512 + lane * 8;
  *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
}

// One workgroup per (sequence, 8 consecutive dense rows); 256 threads, 16 dims each.
template <typename T>
__global__ __launch_bounds__(256) void swa_fp8_window(const uint8_t* __restrict__ ring,
                                                      const int32_t* __restrict__ q_pos,
                                                      const int32_t* __restrict__ swa_pos0, T* __restrict__ dense,
                                                      int32_t* __restrict__ pos0_out, int T_len, int L_w) {
  __shared__ int red[4];
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  int nw = -2147483647 - 1;
  for (int t = tid; t < T_len; t += 256) nw = max(nw, q_pos[(size_t)b * T_len + t]);
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) nw = max(nw, __shfl_xor(nw, off, 64));
  if ((tid & 63) == 0) red[tid >> 6] = nw;
  __syncthreads();
  const int newest = max(max(red[0], red[1]), max(red[2], red[3]));
  // first dense position: the ring holds newest - L_w + 1 .. newest, and nothing
  // before swa_pos0 was ever written.  Dense row j holds position p0 + j; rows past
  // newest are never attended (a window ends at its query's position).
  const int p0 = max(swa_pos0[b], newest - L_w + 1);
  if (blockIdx.x == 0 && tid == 0) pos0_out[b] = p0;
  const int j = blockIdx.x * 8 + (tid >> 5);
  if (j >= L_w) return;
  const int u = p0 + j;
  const int slot = ((u % L_w) + L_w) % L_w;   // non-negative for any position
  const int d0 = (tid & 31) * 16;
  const uint4 c = *reinterpret_cast<const uint4*>(ring + ((size_t)b * L_w + slot) * 512 + d0);
  const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
  T* out = dense + ((size_t)b * L_w + j) * 512 + d0;
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    typedef float v2f __attribute__((ext_vector_type(2)));
    const v2f lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)cw[q4], false);
    const v2f hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)cw[q4], true);
    out[4 * q4 + 0] = from_f32<T>(lo.x);
    out[4 * q4 + 1] = from_f32<T>(lo.y);
    out[4 * q4 + 2] = from_f32<T>(hi.x);
    out[4 * q4 + 3] = from_f32<T>(hi.y);
  }
}

}  // namespace

hipError_t launch_swa_append(int dtype, const void* rows, const int32_t* pos, uint8_t* ring, int B, int T_len,
                             int L_w, hipStream_t st) {
  if (B == 0 || T_len == 0) return hipSuccess;
  const dim3 grid((unsigned)(B * T_len));
  if (dtype == 1)
    hipLaunchKernelGGL(swa_fp8_append<bf16>, grid, dim3(64), 0, st, static_cast<const bf16*>(rows), pos, ring, T_len,
                       L_w);
  else
    hipLaunchKernelGGL(swa_fp8_append<float>, grid, dim3(64), 0, st, static_cast<const float*>(rows), pos, ring,
                       T_len, L_w);
  return hipGetLastError();
}

hipError_t launch_swa_window(int dtype, const uint8_t* ring, const int32_t* q_pos, const int32_t* swa_pos0,
                             void* dense, int32_t* pos0_out, int B, int T_len, int L_w, hipStream_t st) {
  if (B == 0 || T_len == 0) return hipSuccess;
  const dim3 grid((unsigned)((L_w + 7) / 8), (unsigned)B);
  if (dtype == 1)
    hipLaunchKernelGGL(swa_fp8_window<bf16>, grid, dim3(256), 0, st, ring, q_pos, swa_pos0, static_cast<bf16*>(dense),
                       pos0_out, T_len, L_w);
  else
    hipLaunchKernelGGL(swa_fp8_window<float>, grid, dim3(256), 0, st, ring, q_pos, swa_pos0,
                       static_cast<float*>(dense), pos0_out, T_len, L_w);
  return hipGetLastError();
}

}  // namespace csa2
