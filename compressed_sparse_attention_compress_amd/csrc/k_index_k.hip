// (b) Index K: 512 -> 128 projection of the pre-RoPE latent, RoPE on its last 64
// dims at the entry position, FP4 (E2M1) codes with one E4M3 (or UE8M0) scale per 32 dims.
//
// Method ([P1] "DeepSeek-V4.1 模型结构（2）…", section "indexer K 改由 main KV
// 投影": the projection reads the main-KV entry before its RoPE, index K then gets
// its own RoPE on the last 64 dims, no Hadamard rotation, FP4 with one scale per
// 32 dims; [P3] "DeepSeek-V4.1-Flash：把百万 Token 的记忆…", section six: 68 B per
// entry).  Quantisation of a 32-dim block: scale = E4M3(amax / 6) (round to
// nearest even, saturating), code_i = E2M1(u_i / scale) (nearest even, saturating,
// sign kept), all divisions float32 round-to-nearest; a zero scale zeroes the
// block.  The code of dim 2j is the low nibble of byte j.
//
// Kernel: a workgroup of 4 waves per 16 entries; the 16 x 32 rotary angles are
// evaluated once into LDS by all threads; wave q computes the 32
// output dims of quantisation block q.  MFMA with the 16 entries as rows and the
// block's 32 dims as 2 column tiles; the float32 latent is split into a bf16 high
// part and a bf16 remainder (two MFMAs) so bf16 weights lose nothing beyond ~2^-17
// relative; fp32 weights use the fp32 MFMA.  The accumulator layout puts the 32
// dims of the block in one 16-lane group, so amax, RoPE pairs and nibble packing
// are lane shuffles.
#include "csa2_internal.h"
#include "device_common.h"

namespace csa2 {

namespace {

__device__ __forceinline__ void split_hi_lo(const f32x8& a, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    bf16 h = (bf16)a.v[i];
    hi[i] = h;
    lo[i] = (bf16)(a.v[i] - (float)h);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void index_k_kernel(const float* __restrict__ lat, const T* __restrict__ w_ik,
                                                      uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                      int N, int m, int entry0, int N_cap, double base,
                                                      int sfmt) {
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int q = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // quantisation block of this wave
  const int e0 = blockIdx.x * 16;
  const int b = blockIdx.y;
  __shared__ float2 rot[16][32];
  const float* lb = lat + (size_t)b * N * 512;
  const int arow = e0 + lr;
  // rows past N read row N - 1: they only feed outputs of entries that are not stored
  const float* arow_p = lb + (size_t)min(arow, N - 1) * 512;
  f32x4 acc[2];
  acc[0] = f32x4{0.f, 0.f, 0.f, 0.f};
  acc[1] = f32x4{0.f, 0.f, 0.f, 0.f};

  // eight k-steps per round: all their loads are issued before the first MFMA
  f32x8 a[8];
  typename Frag<T>::type bw[8][2];
  auto load_round = [&](int k0) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      a[u] = load_frag(arow_p + (k0 + u) * 32 + 8 * lg);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bw[u][j] = load_frag(w_ik + (size_t)((2 * q + j) * 16 + lr) * 512 + (k0 + u) * 32 + 8 * lg);
    }
  };
  auto mma_round = [&]() {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if constexpr (sizeof(T) == 2) {
        bf16x8 hi, lo;
        split_hi_lo(a[u], hi, lo);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[j] = mma16(hi, bw[u][j], acc[j]);
          acc[j] = mma16(lo, bw[u][j], acc[j]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[j] = mma16(a[u], bw[u][j], acc[j]);
      }
    }
  };
  load_round(0);
  // rotary angles of the 16 entries x 32 pairs, two per thread, into LDS, while
  // the first round's loads are in flight (read after the barrier below)
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int idx = threadIdx.x + 256 * r, ee = idx >> 5, pair = idx & 31;
    float c = 1.f, s = 0.f;
    if (e0 + ee < N) rope_cos_sin((int64_t)(entry0 + e0 + ee) * m, pair, 64, base, c, s);
    rot[ee][pair] = make_float2(c, s);
  }
  mma_round();
  load_round(8);
  mma_round();
  __syncthreads();   // the rotary table is complete

  // RoPE on dims 64..127 (blocks 2 and 3): pair (64+2p, 65+2p) lives in lanes l, l^1
  if (q >= 2) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int pair = (2 * q + j - 4) * 8 + (lr >> 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float2 cs = rot[4 * lg + i][pair];
        const float c = cs.x, s = cs.y;
        float mine = acc[j][i];
        float other = __shfl_xor(mine, 1, 64);
        acc[j][i] = (lr & 1) ? (other * s + mine * c) : (mine * c - other * s);
      }
    }
  }

  // quantise block q; entry 4*lg+i lives in the lane's 16-lane group
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = e0 + 4 * lg + i;
    float v0 = acc[0][i], v1 = acc[1][i];
    float amax = fmaxf(fabsf(v0), fabsf(v1));
    amax = wave_max_xor(amax, 15);  // within the 16-lane group
    const uint32_t sb = ik_scale_byte(amax, sfmt);
    const float s = ik_scale_value(sb, sfmt);
    const uint32_t c0 = fp4_code(v0, s), c1 = fp4_code(v1, s);
    const uint32_t o0 = __shfl_xor((int)c0, 1, 64), o1 = __shfl_xor((int)c1, 1, 64);
    if (e < N) {
      uint8_t* crow = codes + ((size_t)b * N_cap + entry0 + e) * 64 + 16 * q;
      if ((lr & 1) == 0) {
        crow[lr >> 1] = (uint8_t)(c0 | (o0 << 4));
        crow[8 + (lr >> 1)] = (uint8_t)(c1 | (o1 << 4));
      }
      if (lr == 0) scales[((size_t)b * N_cap + entry0 + e) * 4 + q] = (uint8_t)sb;
    }
  }
}

// Stand-alone packer: one thread per 32-value block.
__global__ __launch_bounds__(256) void fp4_pack_kernel(const float* __restrict__ rows, int64_t n_blocks,
                                                       uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n_blocks) return;
  const float* src = rows + t * 32;
  float v[32];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; i += 4) {
    float4 p = *reinterpret_cast<const float4*>(src + i);
    v[i] = p.x; v[i + 1] = p.y; v[i + 2] = p.z; v[i + 3] = p.w;
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(p.x), fabsf(p.y)), fmaxf(fabsf(p.z), fabsf(p.w))));
  }
  const uint32_t sb = fp4_scale_byte(amax);
  const float s = e4m3_decode(sb);
  uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 32; ++i) w[i >> 3] |= fp4_code(v[i], s) << (4 * (i & 7));
  *reinterpret_cast<uint4*>(codes + t * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  scales[t] = (uint8_t)sb;
}

// FP4 main KV: one thread per 16-value block of a 512-d row (one E4M3 scale per
// block, 8 code bytes, even dimension in the low nibble).
__global__ __launch_bounds__(256) void kv_fp4_pack_kernel(const float* __restrict__ rows, int64_t n_blocks,
                                                          uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n_blocks) return;
  const float4* src = reinterpret_cast<const float4*>(rows + t * 16);
  float v[16];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 p = src[i];
    v[4 * i] = p.x; v[4 * i + 1] = p.y; v[4 * i + 2] = p.z; v[4 * i + 3] = p.w;
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(p.x), fabsf(p.y)), fmaxf(fabsf(p.z), fabsf(p.w))));
  }
  const uint32_t sb = fp4_scale_byte(amax);
  const float s = e4m3_decode(sb);
  uint32_t w[2] = {0, 0};
#pragma unroll
  for (int i = 0; i < 16; ++i) w[i >> 3] |= fp4_code(v[i], s) << (4 * (i & 7));
  *reinterpret_cast<uint2*>(codes + t * 8) = make_uint2(w[0], w[1]);
  scales[t] = (uint8_t)sb;
}

// FP4 main KV -> dense rows (bf16 or float32): one thread per 16-dim block.  The
// products are exact in both types.
template <typename T>
__global__ __launch_bounds__(256) void kv_fp4_dequant_kernel(const uint8_t* __restrict__ codes,
                                                             const uint8_t* __restrict__ scales, int64_t n_blocks,
                                                             T* __restrict__ out) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n_blocks) return;
  const uint2 w = *reinterpret_cast<const uint2*>(codes + t * 8);
  const float s = e4m3_decode(scales[t]);
  T* dst = out + t * 16;
#pragma unroll
  for (int i = 0; i < 16; ++i) dst[i] = from_f32<T>(e2m1_value(((i < 8 ? w.x : w.y) >> (4 * (i & 7))) & 0xFu) * s);
}

}  // namespace

hipError_t launch_kv_fp4_pack(const float* rows, int64_t n_rows, uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  const int64_t nb = n_rows * 32;
  if (nb == 0) return hipSuccess;
  hipLaunchKernelGGL(kv_fp4_pack_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, stream, rows, nb, codes,
                     scales);
  return hipGetLastError();
}

hipError_t launch_kv_fp4_dequant(int dtype, const uint8_t* codes, const uint8_t* scales, int64_t n_rows, void* out,
                                 hipStream_t stream) {
  const int64_t nb = n_rows * 32;
  if (nb == 0) return hipSuccess;
  const dim3 grid((unsigned)((nb + 255) / 256));
  if (dtype == 1)
    hipLaunchKernelGGL(kv_fp4_dequant_kernel<bf16>, grid, dim3(256), 0, stream, codes, scales, nb,
                       static_cast<bf16*>(out));
  else
    hipLaunchKernelGGL(kv_fp4_dequant_kernel<float>, grid, dim3(256), 0, stream, codes, scales, nb,
                       static_cast<float*>(out));
  return hipGetLastError();
}

hipError_t launch_index_k(int dtype, const float* latent_pre, const void* w_ik, uint8_t* codes, uint8_t* scales,
                          int B, int N, int m, int entry0, int N_cap, float rope_base, hipStream_t stream, int sfmt) {
  if (N == 0 || B == 0) return hipSuccess;
  dim3 grid((N + 15) / 16, B), blk(256);
  if (dtype == 1)
    hipLaunchKernelGGL((index_k_kernel<bf16>), grid, blk, 0, stream, latent_pre, static_cast<const bf16*>(w_ik),
                       codes, scales, N, m, entry0, N_cap, (double)rope_base, sfmt);
  else
    hipLaunchKernelGGL((index_k_kernel<float>), grid, blk, 0, stream, latent_pre, static_cast<const float*>(w_ik),
                       codes, scales, N, m, entry0, N_cap, (double)rope_base, sfmt);
  return hipGetLastError();
}

hipError_t launch_fp4_pack(const float* rows, int64_t n_rows, uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  const int64_t nb = n_rows * 4;
  if (nb == 0) return hipSuccess;
  hipLaunchKernelGGL(fp4_pack_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, stream, rows, nb, codes,
                     scales);
  return hipGetLastError();
}

}  // namespace csa2
