// (a) Compressor: projection GEMM with a fused per-channel group softmax-pool
// epilogue, then RMSNorm + RoPE.
//
// Method ([P1] "DeepSeek-V4.1 模型结构（2）…CSA2 的三种模式", section on the
// compressor without overlap or position bias; [P4] "CSA2 — l'attention creuse
// compressée…", table in "Ce qui change par rapport à V4"): C = x W_kv and
// Z = x W_gate per token; each disjoint group of m tokens is pooled as
// sum_i softmax_i(Z[:, c]) * C[i, c] per channel c, with no position bias; the
// entry is RMS-normalised and the last 64 dims are rotated at the position of the
// group's first token.  m == 1 is the plain projection plus norm.
//
// Kernel 1 (compress_gemm_pool): a 128-token x 128-column tile per workgroup,
// 4 waves of 64x64, MFMA 16x16x32 bf16 (or 8x 16x16x4 fp32), K staged through LDS
// with a register prefetch of the next K tile.  The 128 columns of a gated tile
// are 64 channels of C followed, per wave, by the same channels of Z, so each
// lane holds C and Z of one channel for 4 consecutive tokens and pools groups of
// 2 or 4 tokens entirely in registers.  Output: the pooled entry in float32.
// Kernel 2 (compress_finalize): one wave per entry: RMSNorm in float32, write the
// pre-RoPE latent (float32, in place) and the cache row with RoPE applied.
// m == 1 with a bf16 cache (compress_m1_bf16): one kernel; a workgroup holds 128
// whole 512-channel rows and finishes them in its epilogue.
#include "csa2_internal.h"
#include "device_common.h"
#include "lds_dma.h"

namespace csa2 {

namespace {

constexpr int BM = 128;     // tokens per workgroup tile
constexpr int BN = 128;     // output columns per workgroup tile
constexpr int ROWB = 128;   // bytes of K per LDS row per stage
constexpr int PADB = 16;    // LDS row padding (bytes)

template <typename T>
struct Tile {
  static constexpr int BK = ROWB / (int)sizeof(T);               // elements per stage
  static constexpr int LDK = (ROWB + PADB) / (int)sizeof(T);     // LDS row stride (elements)
  static constexpr int CHUNK = 16 / (int)sizeof(T);              // elements per 16-B chunk
  static constexpr int KSTEPS = BK / 32;
};

template <typename T, int M_RATIO>
__global__ __launch_bounds__(256) void compress_gemm_pool(
    const T* __restrict__ x, const T* __restrict__ w_kv, const T* __restrict__ w_gate,
    float* __restrict__ e_out, int T_len, int D) {
  typedef Tile<T> TL;
  typedef typename Frag<T>::type FragT;
  __shared__ __attribute__((aligned(16))) T As[BM * TL::LDK];
  __shared__ __attribute__((aligned(16))) T Bs[BN * TL::LDK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int b = blockIdx.z;
  const int row0 = blockIdx.x * BM;
  constexpr bool gated = M_RATIO > 1;
  constexpr int CH_PER_WG = gated ? 64 : 128;
  const int ch0 = blockIdx.y * CH_PER_WG;

  const T* xb = x + (size_t)b * T_len * D;

  // source row of B-tile row j (0..127)
  auto wrow = [&](int j) -> const T* {
    if (gated) {
      int wj = j >> 6, jj = j & 63;
      int ch = ch0 + 32 * wj + (jj & 31);
      return (jj < 32 ? w_kv : w_gate) + (size_t)ch * D;
    }
    return w_kv + (size_t)(ch0 + j) * D;
  };

  // global -> register staging: 4 A chunks and 4 B chunks of 16 B per thread
  uint4 ra[4], rb[4];
  auto load_tiles = [&](int k0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int c = tid + 256 * j;
      int r = c >> 3, cc = c & 7;
      int tok = row0 + r;
      if (tok < T_len)
        ra[j] = *reinterpret_cast<const uint4*>(xb + (size_t)tok * D + k0 + cc * TL::CHUNK);
      else
        ra[j] = make_uint4(0, 0, 0, 0);
      rb[j] = *reinterpret_cast<const uint4*>(wrow(r) + k0 + cc * TL::CHUNK);
    }
  };
  auto store_tiles = [&]() {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int c = tid + 256 * j;
      int r = c >> 3, cc = c & 7;
      *reinterpret_cast<uint4*>(&As[r * TL::LDK + cc * TL::CHUNK]) = ra[j];
      *reinterpret_cast<uint4*>(&Bs[r * TL::LDK + cc * TL::CHUNK]) = rb[j];
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = D / TL::BK;
  load_tiles(0);
  store_tiles();
  __syncthreads();
  const int lr = lane & 15, lg = lane >> 4;
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) load_tiles((kt + 1) * TL::BK);
#pragma unroll
    for (int ks = 0; ks < TL::KSTEPS; ++ks) {
      FragT a[4], bb[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        a[mt] = load_frag(&As[(wm * 64 + mt * 16 + lr) * TL::LDK + ks * 32 + 8 * lg]);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        bb[nt] = load_frag(&Bs[(wn * 64 + nt * 16 + lr) * TL::LDK + ks * 32 + 8 * lg]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = mma16(a[mt], bb[nt], acc[mt][nt]);
    }
    __syncthreads();
    if (kt + 1 < nk) {
      store_tiles();
      __syncthreads();
    }
  }

  // epilogue: lane holds tokens row0 + wm*64 + mt*16 + 4*lg + i, column l%16 of n-tile nt
  const int n_entries = T_len / M_RATIO;
  float* eb = e_out + (size_t)b * n_entries * 512;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int tok0 = row0 + wm * 64 + mt * 16 + 4 * lg;  // first of the lane's 4 tokens
    if (gated) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int ch = ch0 + 32 * wn + 16 * nt + lr;
        const f32x4 c = acc[mt][nt], z = acc[mt][nt + 2];
#pragma unroll
        for (int g0 = 0; g0 < 4; g0 += M_RATIO) {
          if (tok0 + g0 >= T_len) continue;
          float zmax = z[g0];
#pragma unroll
          for (int i = 1; i < M_RATIO; ++i) zmax = fmaxf(zmax, z[g0 + i]);
          float num = 0.f, den = 0.f;
#pragma unroll
          for (int i = 0; i < M_RATIO; ++i) {
            float p = __expf(z[g0 + i] - zmax);
            den += p;
            num += p * c[g0 + i];
          }
          eb[(size_t)((tok0 + g0) / M_RATIO) * 512 + ch] = num / den;
        }
      }
    } else {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int ch = ch0 + 64 * wn + 16 * nt + lr;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (tok0 + i < T_len) eb[(size_t)(tok0 + i) * 512 + ch] = acc[mt][nt][i];
      }
    }
  }
}

// ---- bf16 projection: 256-token x 128-column tiles, 8 waves of 64 x 64, operands
// gathered straight into LDS (3-stage ring of 48 KB stages, one barrier per
// 64-wide k step).  LDS rows are 128 B = 8 units of 16 B; unit u of row r is
// stored in slot u ^ (r & 7), so the 8 lanes that share an LDS cycle in a
// fragment read hit 8 different slots.  The gather makes this layout by letting
// lane i (which the load instruction writes to slot i & 7 of row i >> 3) fetch
// unit (i & 7) ^ (row & 7) of its row.
constexpr int G_BM = 256;
constexpr int G_BN = 128;
constexpr int G_A_BYTES = G_BM * 128;
constexpr int G_STAGE = G_A_BYTES + G_BN * 128;   // 48 KB

template <int M_RATIO>
__global__ __launch_bounds__(512) void compress_gemm_pool_bf16(const bf16* __restrict__ x,
                                                               const bf16* __restrict__ w_kv,
                                                               const bf16* __restrict__ w_gate,
                                                               float* __restrict__ e_out, int T_len, int D) {
  __shared__ __attribute__((aligned(16))) unsigned char st0[G_STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char st1[G_STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char st2[G_STAGE];

  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int b = blockIdx.z;
  const int row0 = blockIdx.x * G_BM;
  constexpr bool gated = M_RATIO > 1;
  const int ch0 = blockIdx.y * (gated ? 64 : 128);
  const bf16* xb = x + (size_t)b * T_len * D;

  // this lane's 6 source rows (4 of the token tile, 2 of the weight tile), with
  // its swizzled 16-B unit folded in; the k offset is added per stage
  const unsigned char* gsrc[6];
#pragma unroll
  for (int q = 0; q < 6; ++q) {
    const int j = wave + 8 * q;             // gather instruction: stage rows 8j .. 8j+7
    const int r = 8 * (j & 31) + (lane >> 3);
    const int unit = (lane & 7) ^ (r & 7);
    const bf16* rowp;
    if (q < 4) {
      const int tok = min(row0 + r, T_len - 1);   // rows past the end repeat the last token (discarded)
      rowp = xb + (size_t)tok * D;
    } else if (gated) {
      const int ch = ch0 + 32 * (r >> 6) + (r & 31);
      rowp = ((r & 63) < 32 ? w_kv : w_gate) + (size_t)ch * D;
    } else {
      rowp = w_kv + (size_t)(ch0 + r) * D;
    }
    gsrc[q] = reinterpret_cast<const unsigned char*>(rowp) + unit * 16;
  }
  auto issue = [&](int kt, unsigned char* st) {
#pragma unroll
    for (int q = 0; q < 6; ++q) dma16_asm(gsrc[q] + (size_t)kt * 128, (const lds_u8*)(st + (wave + 8 * q) * 1024));
  };

  // fragment offsets: row (tile row) * 128 + slot * 16; r & 7 == lr & 7 for every fragment row
  int aoff[2], boff[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int slot = (ks * 4 + lg) ^ (lr & 7);
    aoff[ks] = (wm * 64 + lr) * 128 + slot * 16;
    boff[ks] = G_A_BYTES + (wn * 64 + lr) * 128 + slot * 16;
  }
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = D / 64;
  auto step = [&](int kt, const unsigned char* cur, unsigned char* nxt2) {
    if (kt + 1 < nk) WAIT_VMCNT(6);   // this wave's gathers of stage kt are in (kt+1's may fly)
    else WAIT_VMCNT(0);
    COMPILER_FENCE();
    __builtin_amdgcn_s_barrier();
    COMPILER_FENCE();
    // every wave is past stage kt-1, whose buffer takes stage kt+2; its gathers
    // are issued after the first half-step (an asm statement between the
    // fragment reads and their MFMAs would make the compiler wait for every
    // outstanding read)
    // the 8 fragments of the first half-step are read up front; those of the
    // second half are read two at a time between the first half's MFMAs, so they
    // arrive under them (the LDS counter tracks at most 15 reads)
    bf16x8 a[2][4], bb[2][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) a[0][mt] = *reinterpret_cast<const bf16x8*>(cur + aoff[0] + mt * 16 * 128);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) bb[0][nt] = *reinterpret_cast<const bf16x8*>(cur + boff[0] + nt * 16 * 128);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      __builtin_amdgcn_sched_barrier(0);
      a[1][mt] = *reinterpret_cast<const bf16x8*>(cur + aoff[1] + mt * 16 * 128);
      bb[1][mt] = *reinterpret_cast<const bf16x8*>(cur + boff[1] + mt * 16 * 128);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = mma16(a[0][mt], bb[0][nt], acc[mt][nt]);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (kt + 2 < nk) issue(kt + 2, nxt2);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = mma16(a[1][mt], bb[1][nt], acc[mt][nt]);
  };
  issue(0, st0);
  if (nk > 1) issue(1, st1);
  for (int kt = 0; kt < nk; kt += 3) {
    step(kt, st0, st2);
    if (kt + 1 < nk) step(kt + 1, st1, st0);
    if (kt + 2 < nk) step(kt + 2, st2, st1);
  }

  // epilogue: lane holds tokens row0 + wm*64 + mt*16 + 4*lg + i, column l%16 of n-tile nt
  const int n_entries = T_len / M_RATIO;
  float* eb = e_out + (size_t)b * n_entries * 512;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int tok0 = row0 + wm * 64 + mt * 16 + 4 * lg;
    if (gated) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int ch = ch0 + 32 * wn + 16 * nt + lr;
        const f32x4 c = acc[mt][nt], z = acc[mt][nt + 2];
#pragma unroll
        for (int g0 = 0; g0 < 4; g0 += M_RATIO) {
          if (tok0 + g0 >= T_len) continue;
          float zmax = z[g0];
#pragma unroll
          for (int i = 1; i < M_RATIO; ++i) zmax = fmaxf(zmax, z[g0 + i]);
          float num = 0.f, den = 0.f;
#pragma unroll
          for (int i = 0; i < M_RATIO; ++i) {
            const float p = __expf(z[g0 + i] - zmax);
            den += p;
            num += p * c[g0 + i];
          }
          eb[(size_t)((tok0 + g0) / M_RATIO) * 512 + ch] = num / den;
        }
      }
    } else {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int ch = ch0 + 64 * wn + 16 * nt + lr;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (tok0 + i < T_len) eb[(size_t)(tok0 + i) * 512 + ch] = acc[mt][nt][i];
      }
    }
  }
}

// m == 1 with bf16 operands and a bf16 cache: one workgroup owns 128 tokens and
// all 512 channels, so RMSNorm, the pre-RoPE latent, RoPE and the cache row come
// out of the accumulators in the epilogue (no finalize pass, no second read of
// the latent, and every token row of x is read from memory once).  8 waves of
// 64 tokens x 128 channels on v_mfma_f32_16x16x32_bf16.  Operands go straight
// from global memory into two 80 KB LDS stages of 64-wide k-steps (16 KB of
// tokens, 64 KB of weights), one barrier per k-step, the loads of step k + 1
// issued right after it.  LDS rows are 128 B with the swizzle of the gated
// kernel above (unit u of row r in slot u ^ (r & 7)).  The epilogue reuses the
// stages: the rotary table, the per-wave sums of squares, and a row-major
// staging area through which 32 token rows at a time leave as whole rows.
// With w_ik given (the Full layer's own call) the epilogue also makes the index-K
// rows from the staged pre-RoPE latent (the same float32 hi + lo bf16 split, MFMA
// order, RoPE and FP4 block rule as index_k_kernel), so no second pass reads the
// latent back.
constexpr int F_BM = 128;                          // tokens per workgroup
constexpr int F_ROWB = 128;                        // bytes of a row per stage (64 bf16)
constexpr int F_A_BYTES = F_BM * F_ROWB;           // 16 KB of tokens
constexpr int F_STAGE = F_A_BYTES + 512 * F_ROWB;  // + 64 KB of weights
constexpr int F_NS = 2;                            // stages (160 KB)
constexpr int F_LROW = 512 * 4 + 16;               // epilogue row stride (bytes): fp32 row + pad

__global__ __launch_bounds__(512) void compress_m1_bf16(const bf16* __restrict__ x, const bf16* __restrict__ w_kv,
                                                        const float* __restrict__ gamma, float* __restrict__ lat,
                                                        bf16* __restrict__ kv_cache, const bf16* __restrict__ w_ik,
                                                        uint8_t* __restrict__ ik_codes, uint8_t* __restrict__ ik_scales,
                                                        int sfmt, int T_len, int D, int entry0, int N_cap, float eps,
                                                        double base) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[F_NS * F_STAGE];
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int b = blockIdx.y;
  const int row0 = blockIdx.x * F_BM;
  const bf16* xb = x + (size_t)b * T_len * D;

  // DMA instruction j (0..79) of a stage fills stage rows 8j .. 8j+7 (1 KB): rows
  // 0..127 are tokens, rows 128..639 weight rows (channels).  Wave w issues
  // instructions w, w + 8, .., w + 72; lane i writes slot i % 8 of row 8j + i / 8.
  const unsigned char* gsrc[10];
#pragma unroll
  for (int q = 0; q < 10; ++q) {
    const int j = wave + 8 * q;
    const int r = 8 * j + (lane >> 3);
    const int unit = (lane & 7) ^ (r & 7);
    const bf16* rowp = r < F_BM ? xb + (size_t)min(row0 + r, T_len - 1) * D   // rows past the end: discarded
                                : w_kv + (size_t)(r - F_BM) * D;
    gsrc[q] = reinterpret_cast<const unsigned char*>(rowp) + unit * 16;
  }
  auto issue = [&](int kt) {
    unsigned char* st = smem + (kt & (F_NS - 1)) * F_STAGE;
#pragma unroll
    for (int q = 0; q < 10; ++q) dma16_asm(gsrc[q] + (size_t)kt * F_ROWB, (const lds_u8*)(st + (wave + 8 * q) * 1024));
  };
  // fragment rows: tile row r has r & 7 == lr & 7
  int aoff[2], boff[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int slot = (ks * 4 + lg) ^ (lr & 7);
    aoff[ks] = (wm * 64 + lr) * F_ROWB + slot * 16;
    boff[ks] = F_A_BYTES + (wn * 128 + lr) * F_ROWB + slot * 16;
  }
  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = D / 64;
  issue(0);
  for (int kt = 0; kt < nk; ++kt) {
    WAIT_VMCNT(0);   // this wave's loads of step kt are in
    COMPILER_FENCE();
    __builtin_amdgcn_s_barrier();   // every wave's loads of step kt are in; every wave is past step kt - 1
    COMPILER_FENCE();
    if (kt + 1 < nk) issue(kt + 1);   // into the stage of step kt - 1
    const unsigned char* cur = smem + (kt & (F_NS - 1)) * F_STAGE;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 a[4], bb[8];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) a[mt] = *reinterpret_cast<const bf16x8*>(cur + aoff[ks] + mt * 16 * F_ROWB);
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) bb[nt] = *reinterpret_cast<const bf16x8*>(cur + boff[ks] + nt * 16 * F_ROWB);
#pragma unroll
      for (int nt = 0; nt < 8; ++nt)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[mt][nt] = mma16(a[mt], bb[nt], acc[mt][nt]);
    }
  }
  __syncthreads();   // the ring is free: the epilogue reuses its LDS

  // lane holds token wm*64 + mt*16 + 4*lg + i, channel wn*128 + nt*16 + lr
  float* ssq = reinterpret_cast<float*>(smem);                    // [4 wn][128 tokens]
  float2* rot = reinterpret_cast<float2*>(smem + 2048);           // [128 tokens][32 pairs]
  unsigned char* lbuf = smem + 2048 + F_BM * 32 * 8;              // [32 rows][F_LROW]
  for (int i = threadIdx.x; i < F_BM * 32; i += 512) {
    const int r = i >> 5;
    float c = 1.f, sn = 0.f;
    if (row0 + r < T_len) rope_cos_sin((int64_t)(entry0 + row0 + r), i & 31, 64, base, c, sn);
    rot[i] = make_float2(c, sn);
  }
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float sq = 0.f;
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) sq += acc[mt][nt][i] * acc[mt][nt][i];
      sq = wave_sum_xor(sq, 15);
      if (lr == 0) ssq[wn * F_BM + wm * 64 + mt * 16 + 4 * lg + i] = sq;
    }
  float g[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) g[nt] = gamma[wn * 128 + nt * 16 + lr];
  __syncthreads();
  float rinv[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = wm * 64 + mt * 16 + 4 * lg + i;
      const float ss = ssq[t] + ssq[F_BM + t] + ssq[2 * F_BM + t] + ssq[3 * F_BM + t];
      rinv[mt][i] = 1.0f / sqrtf(ss * (1.0f / 512.0f) + eps);
    }
  const int n_entries = T_len;
  // four passes of 32 token rows (16 per wm) staged row-major, then written out
  // 16 B (latent) and 8 B (cache row) per thread
#pragma unroll
  for (int p = 0; p < 4; ++p) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float* lrow = reinterpret_cast<float*>(lbuf + (wm * 16 + 4 * lg + i) * F_LROW) + wn * 128 + lr;
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) lrow[nt * 16] = acc[p][nt][i] * rinv[p][i] * g[nt];
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int piece = threadIdx.x + 512 * u;
      const int lrw = piece >> 7, c4 = piece & 127;
      const int tl = (lrw >> 4) * 64 + p * 16 + (lrw & 15);
      const int tok = row0 + tl;
      if (tok < T_len) {
        float4 v = *reinterpret_cast<const float4*>(lbuf + lrw * F_LROW + c4 * 16);
        reinterpret_cast<float4*>(lat + ((size_t)b * n_entries + tok) * 512)[c4] = v;
        if (c4 >= 112) {   // dims 448..511: pairs 2c4 - 224 and 2c4 - 223
          const float2 r0 = rot[tl * 32 + 2 * c4 - 224], r1 = rot[tl * 32 + 2 * c4 - 223];
          const float x0 = v.x, x1 = v.y, x2 = v.z, x3 = v.w;
          v.x = x0 * r0.x - x1 * r0.y;
          v.y = x0 * r0.y + x1 * r0.x;
          v.z = x2 * r1.x - x3 * r1.y;
          v.w = x2 * r1.y + x3 * r1.x;
        }
        bf16x2 p0, p1;
        p0[0] = (bf16)v.x; p0[1] = (bf16)v.y;
        p1[0] = (bf16)v.z; p1[1] = (bf16)v.w;
        uint2 w2;
        __builtin_memcpy(&w2.x, &p0, 4);
        __builtin_memcpy(&w2.y, &p1, 4);
        *reinterpret_cast<uint2*>(kv_cache + ((size_t)b * N_cap + entry0 + tok) * 512 + 4 * c4) = w2;
      }
    }
    if (w_ik != nullptr) {
      // index K of the 32 staged rows: wave (rt, q) = rows 16rt .. 16rt+15, dims
      // 32q .. 32q+31 (quantisation block q) as two column tiles
      const int q = wave & 3, rt = wave >> 2;
      const unsigned char* arow = lbuf + (16 * rt + lr) * F_LROW + 32 * lg;
      f32x4 u[2];
      u[0] = f32x4{0.f, 0.f, 0.f, 0.f};
      u[1] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int k0 = 0; k0 < 16; k0 += 4) {   // four k-steps of weights in flight per round
        bf16x8 bw[4][2];
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            bw[v][j] = *reinterpret_cast<const bf16x8*>(w_ik + (size_t)((2 * q + j) * 16 + lr) * 512 + (k0 + v) * 32 +
                                                        8 * lg);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float4 a0 = *reinterpret_cast<const float4*>(arow + (k0 + v) * 128);
          const float4 a1 = *reinterpret_cast<const float4*>(arow + (k0 + v) * 128 + 16);
          const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
          bf16x8 hi, lo;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const bf16 h = (bf16)av[e];
            hi[e] = h;
            lo[e] = (bf16)(av[e] - (float)h);
          }
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            u[j] = mma16(hi, bw[v][j], u[j]);
            u[j] = mma16(lo, bw[v][j], u[j]);
          }
        }
      }
      // lane: rows 16rt + 4lg + i, dims 32q + 16j + lr.  RoPE on dims 64..127 (blocks
      // 2 and 3): pair (64 + 2p, 65 + 2p) lives in lanes l, l ^ 1
      if (q >= 2) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int pair = (2 * q + j - 4) * 8 + (lr >> 1);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float2 cs = rot[(rt * 64 + p * 16 + 4 * lg + i) * 32 + pair];
            const float mine = u[j][i], other = __shfl_xor(mine, 1, 64);
            u[j][i] = (lr & 1) ? (other * cs.y + mine * cs.x) : (mine * cs.x - other * cs.y);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = row0 + rt * 64 + p * 16 + 4 * lg + i;
        const float v0 = u[0][i], v1 = u[1][i];
        const float amax = wave_max_xor(fmaxf(fabsf(v0), fabsf(v1)), 15);   // the block: 16 lanes x 2
        const uint32_t sb = ik_scale_byte(amax, sfmt);
        const float sc = ik_scale_value(sb, sfmt);
        const uint32_t c0 = fp4_code(v0, sc), c1 = fp4_code(v1, sc);
        const uint32_t o0 = __shfl_xor((int)c0, 1, 64), o1 = __shfl_xor((int)c1, 1, 64);
        if (tok < T_len) {
          uint8_t* crow = ik_codes + ((size_t)b * N_cap + entry0 + tok) * 64 + 16 * q;
          if ((lr & 1) == 0) {
            crow[lr >> 1] = (uint8_t)(c0 | (o0 << 4));
            crow[8 + (lr >> 1)] = (uint8_t)(c1 | (o1 << 4));
          }
          if (lr == 0) ik_scales[((size_t)b * N_cap + entry0 + tok) * 4 + q] = (uint8_t)sb;
        }
      }
    }
    __syncthreads();
  }
}

// One wave per entry: RMSNorm, RoPE on dims 448..511, write latent (fp32, in
// place over the pooled values) and the cache row.  The 4 x 32 rotary angles of
// the workgroup's entries are evaluated once, one per thread, into LDS.
template <typename T>
__global__ __launch_bounds__(256) void compress_finalize(float* __restrict__ lat, const float* __restrict__ gamma,
                                                         T* __restrict__ kv_cache, uint8_t* __restrict__ kv_scales,
                                                         int n_entries, int entry0, int m, int N_cap, float eps,
                                                         double base) {
  __shared__ float2 rot[4][32];
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int b = blockIdx.y;
  if (threadIdx.x < 128) {
    const int ee = blockIdx.x * 4 + (threadIdx.x >> 5), pair = threadIdx.x & 31;
    float c = 1.f, s = 0.f;
    if (ee < n_entries) rope_cos_sin((int64_t)(entry0 + ee) * m, pair, 64, base, c, s);
    rot[threadIdx.x >> 5][pair] = make_float2(c, s);
  }
  __syncthreads();
  if (e >= n_entries) return;
  float* row = lat + ((size_t)b * n_entries + e) * 512;
  float v[8];
  const float4* r4 = reinterpret_cast<const float4*>(row + lane * 8);
  float4 p0 = r4[0], p1 = r4[1];
  v[0] = p0.x; v[1] = p0.y; v[2] = p0.z; v[3] = p0.w; v[4] = p1.x; v[5] = p1.y; v[6] = p1.z; v[7] = p1.w;
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ss += v[i] * v[i];
  ss = wave_sum_xor(ss, 63);
  const float rinv = 1.0f / sqrtf(ss * (1.0f / 512.0f) + eps);
  const float4* g4 = reinterpret_cast<const float4*>(gamma + lane * 8);
  float4 g0 = g4[0], g1 = g4[1];
  float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = v[i] * rinv * g[i];
  float4* w4 = reinterpret_cast<float4*>(row + lane * 8);
  w4[0] = make_float4(v[0], v[1], v[2], v[3]);
  w4[1] = make_float4(v[4], v[5], v[6], v[7]);
  if (lane >= 56) {  // dims 448..511: 4 rotary pairs per lane
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float2 cs = rot[threadIdx.x >> 6][(lane - 56) * 4 + j];
      const float c = cs.x, s = cs.y;
      float x0 = v[2 * j], x1 = v[2 * j + 1];
      v[2 * j] = x0 * c - x1 * s;
      v[2 * j + 1] = x0 * s + x1 * c;
    }
  }
  const size_t er = (size_t)b * N_cap + entry0 + e;
  if (kv_scales != nullptr) {
    // FP4 main KV: a 16-dim block is lanes 2j, 2j + 1; even dimension in the low nibble
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    const uint32_t sb = fp4_scale_byte(amax);
    const float sc = e4m3_decode(sb);
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) w |= fp4_code(v[i], sc) << (4 * i);
    reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(kv_cache) + er * 256)[lane] = w;
    if ((lane & 1) == 0) kv_scales[er * 32 + (lane >> 1)] = (uint8_t)sb;
    return;
  }
  T* out = kv_cache + er * 512 + lane * 8;
#pragma unroll
  for (int i = 0; i < 8; ++i) out[i] = from_f32<T>(v[i]);
}

template <typename T>
hipError_t launch_t(const void* x, const void* w_kv, const void* w_gate, const float* gamma, float* lat,
                    void* kv, uint8_t* kv_scales, int B, int T_len, int D, int m, int start_pos, int N_cap, float eps,
                    float base, hipStream_t st, const void* w_ik = nullptr, uint8_t* ik_codes = nullptr,
                    uint8_t* ik_scales = nullptr, int sfmt = 0) {
  const int n_entries = T_len / m;
  if (n_entries == 0 || B == 0) return hipSuccess;
  dim3 blk(256);
  dim3 grid((T_len + BM - 1) / BM, m > 1 ? 512 / 64 : 512 / 128, B);
  const T* xx = static_cast<const T*>(x);
  const T* wk = static_cast<const T*>(w_kv);
  const T* wg = static_cast<const T*>(w_gate);
  if constexpr (sizeof(T) == 2) {
    if (m == 1 && kv_scales == nullptr) {   // whole rows per workgroup: the epilogue finishes the entries
      hipLaunchKernelGGL(compress_m1_bf16, dim3((T_len + F_BM - 1) / F_BM, B), dim3(512), 0, st, xx, wk, gamma, lat,
                         static_cast<bf16*>(kv), static_cast<const bf16*>(w_ik), ik_codes, ik_scales, sfmt, T_len, D,
                         start_pos, N_cap, eps, (double)base);
      return hipGetLastError();
    }
    dim3 gb((T_len + G_BM - 1) / G_BM, m > 1 ? 512 / 64 : 512 / 128, B);
    if (m == 1) hipLaunchKernelGGL((compress_gemm_pool_bf16<1>), gb, dim3(512), 0, st, xx, wk, wg, lat, T_len, D);
    else if (m == 2) hipLaunchKernelGGL((compress_gemm_pool_bf16<2>), gb, dim3(512), 0, st, xx, wk, wg, lat, T_len, D);
    else hipLaunchKernelGGL((compress_gemm_pool_bf16<4>), gb, dim3(512), 0, st, xx, wk, wg, lat, T_len, D);
  } else {
    if (m == 1) hipLaunchKernelGGL((compress_gemm_pool<T, 1>), grid, blk, 0, st, xx, wk, wg, lat, T_len, D);
    else if (m == 2) hipLaunchKernelGGL((compress_gemm_pool<T, 2>), grid, blk, 0, st, xx, wk, wg, lat, T_len, D);
    else hipLaunchKernelGGL((compress_gemm_pool<T, 4>), grid, blk, 0, st, xx, wk, wg, lat, T_len, D);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  dim3 g2((n_entries + 3) / 4, B);
  hipLaunchKernelGGL((compress_finalize<T>), g2, blk, 0, st, lat, gamma, static_cast<T*>(kv), kv_scales, n_entries,
                     start_pos / m, m, N_cap, eps, (double)base);
  return hipGetLastError();
}


// ---------------------------------------------------------------- decode append
// One new token per sequence after the prefill.  Step 1 (compress_step_proj):
// partial C and Z of every sequence's token, cz[q][b][n] for K quarter q of the
// hidden dims (n < 512: C channel n, else Z channel n - 512).  Workgroup
// (column group, q) computes 16 output columns over quarter q for all sequences
// with MFMA (sequences as the rows of 16-row tiles, 4 tiles per pass); its 4
// waves split the quarter's 32-wide k-steps into contiguous runs (so a wave reads
// long pieces of each weight row), issue the loads of eight k-steps before
// their MFMAs, and their partial sums meet in LDS.  The weights are read once;
// the four quarters give 4x more workgroups than column groups.
constexpr int STEP_KQ = 4;   // K quarters (partial sums summed by compress_step_entry)
constexpr int STEP_KB = 8;   // k-steps whose loads are in flight together
template <typename T>
__global__ __launch_bounds__(256) void compress_step_proj(const T* __restrict__ x, const T* __restrict__ w_kv,
                                                          const T* __restrict__ w_gate, float* __restrict__ cz,
                                                          int B, int D) {
  typedef typename Frag<T>::type FragT;
  __shared__ f32x4 red[3][4 * 64];
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = blockIdx.x * 16 + lr;
  const int kq = blockIdx.y;
  const T* wrow = n < 512 ? w_kv + (size_t)n * D : w_gate + (size_t)(n - 512) * D;
  const int nks = D / 32;
  const int q0 = kq * nks / STEP_KQ, q1 = (kq + 1) * nks / STEP_KQ;
  const int ks0 = q0 + wave * (q1 - q0) / 4, ks1 = q0 + (wave + 1) * (q1 - q0) / 4;   // this wave's k-steps
  float* czq = cz + (size_t)kq * B * 1024;
  for (int b0 = 0; b0 < B; b0 += 64) {
    f32x4 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int kb = ks0; kb < ks1; kb += STEP_KB) {   // k-steps kb .. kb + STEP_KB - 1
      FragT wf[STEP_KB], xf[STEP_KB][4];
#pragma unroll
      for (int u = 0; u < STEP_KB; ++u) {
        const int ks = min(kb + u, ks1 - 1);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int seq = min(b0 + t * 16 + lr, B - 1);   // rows past B repeat the last token (discarded)
          xf[u][t] = load_frag(x + (size_t)seq * D + ks * 32 + 8 * lg);
        }
        wf[u] = load_frag(wrow + ks * 32 + 8 * lg);
      }
#pragma unroll
      for (int u = 0; u < STEP_KB; ++u) {
        if (kb + u >= ks1) break;
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = mma16(xf[u][t], wf[u], acc[t]);
      }
    }
    if (wave > 0) {
#pragma unroll
      for (int t = 0; t < 4; ++t) red[wave - 1][t * 64 + lane] = acc[t];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const f32x4 v = acc[t] + red[0][t * 64 + lane] + red[1][t * 64 + lane] + red[2][t * 64 + lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int seq = b0 + t * 16 + 4 * lg + i;   // accumulator row 4*lg+i, column lr
          if (seq < B) czq[(size_t)seq * 1024 + n] = v[i];
        }
      }
    }
    __syncthreads();
  }
}

__device__ __forceinline__ float frag_elem(const bf16x8& f, int i) { return (float)f[i]; }
__device__ __forceinline__ float frag_elem(const f32x8& f, int i) { return f.v[i]; }

// Step 2 (compress_step_entry), one workgroup per sequence; thread t owns channels
// t and t + 256.  The token joins its group's running softmax pool per channel
// (maximum of Z, sum of exp(Z - max), sum of exp(Z - max) C): the exact softmax
// pool of the group, reached one token at a time.  At the group's last token the
// pooled vector is normalised (RMSNorm), written before RoPE to latent_pre and
// after RoPE on dims 448..511 (at position g*m) to the cache row g; then its
// index-K row: 512 -> 128 (thread pair per output dim, halves of the dot product
// added by a shuffle), RoPE on dims 64..127, FP4 codes with one E4M3 (or UE8M0) scale per
// 32 dims (wave q holds block q).
template <typename T>
__global__ __launch_bounds__(256) void compress_step_entry(const float* __restrict__ cz, const int32_t* __restrict__ pos_arr,
                                                           const float* __restrict__ gamma, const T* __restrict__ w_ik,
                                                           float* __restrict__ state, T* __restrict__ kv_cache,
                                                           uint8_t* __restrict__ kv_scales,
                                                           uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                           float* __restrict__ latent_pre, int B, int m, int N_cap,
                                                           float eps, double base, int sfmt) {
  typedef typename Frag<T>::type FragT;
  __shared__ float lat_s[512];
  __shared__ float red[4];
  __shared__ float2 rot[32];   // cos, sin of the 32 rotary pairs at position g*m (latent and index K alike)
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pos = pos_arr[b];
  if (pos < 0) return;
  const int gi = pos % m, g = pos / m;
  const bool closes = gi == m - 1 && g < N_cap;   // this token completes a group whose row is stored
  // a closing token needs the index-K weights: their loads start now, under the pool and norm
  const int o = tid >> 1, h = tid & 1;
  constexpr int NPF = sizeof(T) == 2 ? 32 : 16;   // fragments of the 256 weights per load round
  const T* wr = w_ik + (size_t)o * 512 + h * 256;
  FragT wf[NPF];
  if (closes) {
#pragma unroll
    for (int u = 0; u < NPF; ++u) wf[u] = load_frag(wr + 8 * u);
    if (tid < 32) {
      float c, s;
      rope_cos_sin((int64_t)g * m, tid, 64, base, c, s);
      rot[tid] = make_float2(c, s);
    }
  }
  // C and Z of the token: the sum of the projection's K-quarter partials
  auto cz_at = [&](int col) -> float {
    float v = 0.f;
#pragma unroll
    for (int q = 0; q < STEP_KQ; ++q) v += cz[((size_t)q * B + b) * 1024 + col];
    return v;
  };
  float e[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int ch = tid + 256 * j;
    const float c = cz_at(ch);
    if (m == 1) {
      e[j] = c;
      continue;
    }
    float* st = state + (size_t)b * 1536;
    const float z = cz_at(512 + ch);
    float zm, den, num;
    if (gi == 0) {
      zm = z;
      den = 1.f;
      num = c;
    } else {
      const float zo = st[ch];
      zm = fmaxf(zo, z);
      const float ao = __expf(zo - zm), an = __expf(z - zm);
      den = st[512 + ch] * ao + an;
      num = st[1024 + ch] * ao + c * an;
    }
    if (gi < m - 1) {
      st[ch] = zm;
      st[512 + ch] = den;
      st[1024 + ch] = num;
    }
    e[j] = num / den;
  }
  if (!closes) return;   // the group goes on (or its row is outside the cache)

  float ss = e[0] * e[0] + e[1] * e[1];
  ss = wave_sum_xor(ss, 63);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  const float rinv = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) * (1.0f / 512.0f) + eps);
  float v[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int ch = tid + 256 * j;
    v[j] = e[j] * rinv * gamma[ch];
    lat_s[ch] = v[j];
    if (latent_pre != nullptr) latent_pre[(size_t)b * 512 + ch] = v[j];
  }
  {
    // RoPE pair (448 + 2p, 449 + 2p) = channels tid + 256 of threads tid, tid ^ 1
    const float other = __shfl_xor(v[1], 1, 64);
    const int ch = tid + 256;
    if (ch >= 448) {
      const float2 cs = rot[(ch - 448) >> 1];
      v[1] = (ch & 1) ? (other * cs.y + v[1] * cs.x) : (v[1] * cs.x - other * cs.y);
    }
  }
  if (kv_scales != nullptr) {
    // FP4 main KV: a 16-dim block is 16 consecutive threads; the even thread of a
    // pair writes the byte (even dimension in the low nibble)
    uint8_t* crow = reinterpret_cast<uint8_t*>(kv_cache) + ((size_t)b * N_cap + g) * 256;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float amax = fabsf(v[j]);
#pragma unroll
      for (int o2 = 1; o2 < 16; o2 <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o2, 64));
      const uint32_t sb = fp4_scale_byte(amax);
      const uint32_t code = fp4_code(v[j], e4m3_decode(sb));
      const uint32_t other = __shfl_xor(code, 1, 64);
      const int ch = tid + 256 * j;
      if ((tid & 1) == 0) crow[ch >> 1] = (uint8_t)(code | (other << 4));
      if ((tid & 15) == 0) kv_scales[((size_t)b * N_cap + g) * 32 + (ch >> 4)] = (uint8_t)sb;
    }
  } else {
    T* kvrow = kv_cache + ((size_t)b * N_cap + g) * 512;
    kvrow[tid] = from_f32<T>(v[0]);
    kvrow[tid + 256] = from_f32<T>(v[1]);
  }
  __syncthreads();   // lat_s complete

  const float* lh = lat_s + h * 256;
  float acc = 0.f;
#pragma unroll
  for (int r = 0; r < 32 / NPF; ++r) {
    if (r > 0) {
#pragma unroll
      for (int u = 0; u < NPF; ++u) wf[u] = load_frag(wr + 8 * (r * NPF + u));
    }
#pragma unroll
    for (int u = 0; u < NPF; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc = fmaf(lh[8 * (r * NPF + u) + i], frag_elem(wf[u], i), acc);
  }
  float u = acc + __shfl_xor(acc, 1, 64);
  {
    // RoPE pair (64 + 2p, 65 + 2p) = outputs o, o ^ 1 = threads tid, tid ^ 2
    const float uo = __shfl_xor(u, 2, 64);
    if (o >= 64) {
      const float2 cs = rot[(o - 64) >> 1];
      u = (o & 1) ? (uo * cs.y + u * cs.x) : (u * cs.x - uo * cs.y);
    }
  }
  const float amax = wave_max_xor(fabsf(u), 63);   // block `wave` = outputs 32*wave .. +31
  const uint32_t sb = ik_scale_byte(amax, sfmt);
  const uint32_t code = fp4_code(u, ik_scale_value(sb, sfmt));
  const uint32_t code_next = (uint32_t)__shfl_xor((int)code, 2, 64);   // output o + 1 for even o
  if (h == 0 && (o & 1) == 0) codes[((size_t)b * N_cap + g) * 64 + (o >> 1)] = (uint8_t)(code | (code_next << 4));
  if (lane == 0) scales[((size_t)b * N_cap + g) * 4 + wave] = (uint8_t)sb;
}

}  // namespace

hipError_t launch_compress(int dtype, const void* x, const void* w_kv, const void* w_gate, const float* gamma,
                           float* latent_pre, void* kv_cache, uint8_t* kv_scales, int B, int T, int D, int m,
                           int start_pos, int N_cap, float eps, float rope_base, hipStream_t stream) {
  if (dtype == 1)
    return launch_t<bf16>(x, w_kv, w_gate, gamma, latent_pre, kv_cache, kv_scales, B, T, D, m, start_pos, N_cap, eps,
                          rope_base, stream);
  return launch_t<float>(x, w_kv, w_gate, gamma, latent_pre, kv_cache, kv_scales, B, T, D, m, start_pos, N_cap, eps,
                         rope_base, stream);
}


bool compress_makes_index_k(int dtype, int m, bool kv_fp4) { return dtype == 1 && m == 1 && !kv_fp4; }

hipError_t launch_compress_index_k(const void* x, const void* w_kv, const float* gamma, float* latent_pre,
                                   void* kv_cache, const void* w_ik, uint8_t* codes, uint8_t* scales, int B, int T,
                                   int D, int start_pos, int N_cap, float eps, float rope_base, hipStream_t stream,
                                   int scale_fmt) {
  return launch_t<bf16>(x, w_kv, nullptr, gamma, latent_pre, kv_cache, nullptr, B, T, D, 1, start_pos, N_cap, eps,
                        rope_base, stream, w_ik, codes, scales, scale_fmt);
}

hipError_t launch_compress_step(int dtype, const void* x, const int32_t* pos, const void* w_kv, const void* w_gate,
                                const float* gamma, const void* w_ik, float* state, void* kv_cache, uint8_t* kv_scales,
                                uint8_t* codes, uint8_t* scales, float* latent_pre, float* cz, int B, int D, int m, int N_cap,
                                float eps, float rope_base, hipStream_t stream, int sfmt) {
  if (B == 0) return hipSuccess;
  const dim3 g1((m > 1 ? 1024 : 512) / 16, STEP_KQ), g2(B), blk(256);
  if (dtype == 1) {
    hipLaunchKernelGGL((compress_step_proj<bf16>), g1, blk, 0, stream, static_cast<const bf16*>(x),
                       static_cast<const bf16*>(w_kv), static_cast<const bf16*>(w_gate), cz, B, D);
    hipLaunchKernelGGL((compress_step_entry<bf16>), g2, blk, 0, stream, cz, pos, gamma,
                       static_cast<const bf16*>(w_ik), state, static_cast<bf16*>(kv_cache), kv_scales, codes, scales,
                       latent_pre, B, m, N_cap, eps, (double)rope_base, sfmt);
  } else {
    hipLaunchKernelGGL((compress_step_proj<float>), g1, blk, 0, stream, static_cast<const float*>(x),
                       static_cast<const float*>(w_kv), static_cast<const float*>(w_gate), cz, B, D);
    hipLaunchKernelGGL((compress_step_entry<float>), g2, blk, 0, stream, cz, pos, gamma,
                       static_cast<const float*>(w_ik), state, static_cast<float*>(kv_cache), kv_scales, codes, scales,
                       latent_pre, B, m, N_cap, eps, (double)rope_base, sfmt);
  }
  return hipGetLastError();
}

}  // namespace csa2
