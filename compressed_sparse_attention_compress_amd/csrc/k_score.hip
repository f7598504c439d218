// (c) Indexer score, (c') HSI candidate pool and (d) causal top-k.
//
// Method ([P1] "DeepSeek-V4.1 模型结构（2）…", indexer-K section: score of entry s
// for query t = sum over the H_I indexer heads j of w[t,j] * ReLU(q^I[t,j] . k^I[s]);
// each query keeps the 512 best; [P2] "DeepSeek v4.1 Flash技术剖析——架构篇",
// CSA2-FULL: only causally visible entries compete; CSA2-ReIndex: blocks of s
// entries scored by their best entry, the n_b best blocks (the block with the
// newest visible entry always included) form the pool a Reindex layer selects in,
// scores outside it being -inf; [P3] "…分级缓存", section five).
// Ties go to the smaller entry id; -0 and +0 are equal.
//
// Kernel 1 (score_chunk): one workgroup per (query, chunk of C entries).  Each
// wave scores tiles of 16 entries with MFMA 16x16x32: rows = 16 indexer heads
// (two row tiles for 32 heads), columns = 16 entries, one k-step per 32-dim
// quantisation block.  The FP4 codes are expanded with v_cvt_scalef32_pk_bf16_fp4
// (unit scale: exact) and the block's E4M3 scale, which is per entry and so per
// accumulator column, multiplies the block's partial product afterwards.  The
// accumulator gives each lane 8 heads of one entry, so ReLU * w and the head sum
// are in-lane plus two cross-lane adds.  Scores go to LDS as order-preserving
// keys; a radix select (11-bit digits over key|local-index composites, all
// distinct so no tie pass is needed) keeps the chunk's best min(k, C), and for
// HSI the chunk's block maxima are written too.
// Kernel 2 (topk_merge): one workgroup per query: the same select over all chunk
// candidates (key|entry-id composites), indices sorted ascending and padded with
// -1; with HSI BUILD also the n_b best blocks (newest block forced) as the pool.
#include "csa2_internal.h"
#include "device_common.h"

namespace csa2 {

namespace {

constexpr int SEL_BINS = 2048;   // 11-bit digits
constexpr int SEL_BITS = 11;

template <int NT>
struct SelSmem {
  uint32_t hist[SEL_BINS];
  uint32_t wtot[NT / 64];
  uint32_t digit, above, n_valid, done;
  uint32_t count;
};

// Exclusive suffix sum over the threads of a block (thread t gets the sum of the
// values of threads > t).
template <int NT>
__device__ __forceinline__ uint32_t block_suffix_excl(uint32_t v, SelSmem<NT>& sm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    uint32_t u = __shfl_down(x, off, 64);
    if (lane + off < 64) x += u;
  }
  if (lane == 0) sm.wtot[wave] = x;  // inclusive suffix of lane 0 = wave total
  __syncthreads();
  uint32_t higher = 0;
  for (int w = wave + 1; w < NT / 64; ++w) higher += sm.wtot[w];
  __syncthreads();
  return x - v + higher;
}

// Block-wide selection of the R largest non-zero 64-bit composites (R = min(k,
// number of non-zero items)).  On return every thread has (prefix, mask): item c
// is selected iff c != 0 and (c & mask) >= prefix.  R == 0 gives mask = 0,
// prefix = ~0 (selects nothing).
template <int NT, typename Get>
__device__ void block_select(Get get, int n, uint32_t k, int total_bits, SelSmem<NT>& sm, uint64_t& prefix,
                             uint64_t& mask) {
  prefix = 0;
  mask = 0;
  uint32_t need = 0;
  constexpr int BPT = SEL_BINS / NT;
  for (int pass = 0;; ++pass) {
    int shift = total_bits - SEL_BITS * (pass + 1);
    int width = SEL_BITS;
    if (shift < 0) {
      width += shift;
      shift = 0;
    }
    const uint64_t dmask = (width >= 64) ? ~0ull : ((1ull << width) - 1);
    for (int i = threadIdx.x; i < SEL_BINS; i += NT) sm.hist[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += NT) {
      uint64_t c = get(i);
      if (c != 0 && (c & mask) == prefix) atomicAdd(&sm.hist[(uint32_t)((c >> shift) & dmask)], 1u);
    }
    __syncthreads();
    uint32_t own[BPT];
    uint32_t tot = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      own[j] = sm.hist[threadIdx.x * BPT + j];
      tot += own[j];
    }
    if (pass == 0) {
      // total number of valid items
      uint32_t above_all = block_suffix_excl<NT>(tot, sm);
      if (threadIdx.x == 0) sm.n_valid = above_all + tot;
      __syncthreads();
      uint32_t nv = sm.n_valid;
      need = nv < k ? nv : k;
      if (need == 0) {
        prefix = ~0ull;
        mask = 0;
        __syncthreads();
        return;
      }
    }
    uint32_t above = block_suffix_excl<NT>(tot, sm);
    uint32_t cum = above;
#pragma unroll
    for (int j = BPT - 1; j >= 0; --j) {
      if (cum < need && cum + own[j] >= need) {
        sm.digit = threadIdx.x * BPT + j;
        sm.above = cum;
        sm.done = (cum + own[j] == need) ? 1u : 0u;
      }
      cum += own[j];
    }
    __syncthreads();
    const uint32_t d = sm.digit;
    need -= sm.above;
    prefix |= (uint64_t)d << shift;
    mask |= dmask << shift;
    const uint32_t done = sm.done;
    __syncthreads();
    if (done || shift == 0) return;
  }
}

// Bitonic sort (ascending) of n_pow2 ints in LDS, n_pow2 <= 2 * NT * 4.
template <int NT>
__device__ void block_bitonic_sort(int* a, int n_pow2) {
  for (int size = 2; size <= n_pow2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = threadIdx.x; t < n_pow2 / 2; t += NT) {
        int lo = 2 * t - (t & (stride - 1));
        int hi = lo + stride;
        bool up = ((lo & size) == 0);
        int x = a[lo], y = a[hi];
        if ((x > y) == up) {
          a[lo] = y;
          a[hi] = x;
        }
      }
      __syncthreads();
    }
  }
}

__device__ __forceinline__ bf16x8 fp4x8_to_bf16(uint32_t w) {
  bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0);
  bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1);
  bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2);
  bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3);
  bf16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}
__device__ __forceinline__ f32x8 fp4x8_to_f32(uint32_t w) {
  f32x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  f32x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  f32x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  f32x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  f32x8 r;
  r.v[0] = p0[0]; r.v[1] = p0[1]; r.v[2] = p1[0]; r.v[3] = p1[1];
  r.v[4] = p2[0]; r.v[5] = p2[1]; r.v[6] = p3[0]; r.v[7] = p3[1];
  return r;
}
template <typename T> struct Fp4;
template <> struct Fp4<bf16> { static __device__ __forceinline__ bf16x8 cvt(uint32_t w) { return fp4x8_to_bf16(w); } };
template <> struct Fp4<float> { static __device__ __forceinline__ f32x8 cvt(uint32_t w) { return fp4x8_to_f32(w); } };

constexpr int MAX_CHUNK = 4096;
constexpr int SC_THREADS = 256;
constexpr int NBINS = 2048;
constexpr int SPT = 4;                          // tiles (of 16 entries) per super-tile
constexpr int ST_BYTES = SPT * 1024 + 256;      // one super-tile in LDS: codes + scales

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) unsigned char lds_u8;
#define WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | 0x70 | 0xF00)
#define WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(0xC07F)
__device__ __forceinline__ void dma16(const void* g, lds_u8* l) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)l, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* g, lds_u8* l) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)l, 4, 0, 0);
}

// Visible entries of query (b, t).
__device__ __forceinline__ int visible(const int32_t* q_pos, int bt, int m, int n_entries) {
  int p = q_pos[bt];
  int nv = p < 0 ? 0 : (int)(((int64_t)p + 1) / m);
  return nv < n_entries ? nv : n_entries;
}

// Sum over lanes l, l^16, l^32, l^48 with the gfx950 permlane swaps (VALU, no LDS).
__device__ __forceinline__ float sum_lane_groups(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  float y = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  auto r2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(r2[0]) + __uint_as_float(r2[1]);
}

struct ChunkSmem {
  uint32_t keys[MAX_CHUNK];
  uint32_t hist[NBINS];
  uint32_t wtot[SC_THREADS / 64];
  uint32_t red[3][SC_THREADS / 64];
  uint32_t digit, above, done, lb, count, running;
};

__device__ __forceinline__ uint32_t suffix_excl(uint32_t v, ChunkSmem& sm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    uint32_t u = __shfl_down(x, off, 64);
    if (lane + off < 64) x += u;
  }
  if (lane == 0) sm.wtot[wave] = x;
  __syncthreads();
  uint32_t higher = 0;
#pragma unroll
  for (int w = 0; w < SC_THREADS / 64; ++w)
    if (w > wave) higher += sm.wtot[w];
  __syncthreads();
  return x - v + higher;
}

// Number of chunks a query scans, and the rank whose per-chunk lower bounds the
// merge combines: r0 = ceil(k / chunks), so chunks x r0 >= k entries lie at or
// above the smallest of those bounds, which therefore bounds the k-th best key.
__device__ __forceinline__ int rank_for_bound(int k, int nc) { return nc > 0 ? (k + nc - 1) / nc : k; }

template <typename T, bool POOL, bool BUILD>
__global__ __launch_bounds__(SC_THREADS) void score_chunk(
    const T* __restrict__ q_idx, const float* __restrict__ w, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const int32_t* __restrict__ q_pos, const int32_t* __restrict__ cands,
    uint32_t* __restrict__ cand_key, int32_t* __restrict__ cand_idx, uint32_t* __restrict__ chunk_lb,
    uint32_t* __restrict__ blkmax, int T_len, int H_I, int N_cap, int n_entries, int m, int C, int k_chunk,
    int n_chunks, int k, int hsi_s, int hsi_nb, int nblk_max) {
  typedef typename Frag<T>::type FragT;
  __shared__ ChunkSmem sm;
  __shared__ __attribute__((aligned(16))) unsigned char ring0[4 * ST_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char ring1[4 * ST_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char ring2[4 * ST_BYTES];

  const int c = blockIdx.x, t = blockIdx.y, b = blockIdx.z;
  const int bt = b * T_len + t;
  const int n_t = visible(q_pos, bt, m, n_entries);
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int base = c * C;
  if (!POOL && base >= n_t) return;  // chunk beyond the visible range: never read by the merge
  const int nc_q = POOL ? n_chunks : (n_t + C - 1) / C;

  // indexer query fragments: row tile mt = heads 16mt.., k-step kb = dims 32kb + 8lg ..
  FragT qf[2][4];
  float wv[2][4];
  const T* qb = q_idx + (size_t)bt * H_I * 128;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int h = mt * 16 + lr;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      if (h < H_I) qf[mt][kb] = load_frag(qb + (size_t)h * 128 + kb * 32 + 8 * lg);
      else zero_frag(qf[mt][kb]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = mt * 16 + 4 * lg + i;
      wv[mt][i] = hh < H_I ? w[(size_t)bt * H_I + hh] : 0.0f;
    }
  }
  const int32_t* cq = POOL ? cands + (size_t)bt * hsi_nb : nullptr;
  const uint8_t* cb = codes + (size_t)b * N_cap * 64;
  const uint8_t* sb = scales + (size_t)b * N_cap * 4;

  // ---- scoring.  Wave w takes super-tiles w, w+4, ... of 64 entries (4 tiles of
  // 16).  A super-tile is staged in the wave's LDS ring by 5 DMA instructions: one
  // per tile moves its 1 KB of codes (16-B piece i of the tile lands in unit i,
  // piece = (entry e, block b) with unit 4e + ((b + e/4) & 3), which makes the
  // MFMA-pattern dword reads below conflict-free) and one moves the 64 scale words.
  const int n_st = C / 64;
  const int st_w = (n_st - wave + 3) / 4;   // super-tiles of this wave
  auto entry_at = [&](int j, bool& valid) -> int {   // chunk position -> entry id
    if (POOL) {
      const int vj = base + j;
      const int pb = vj / hsi_s;
      const int blk = pb < hsi_nb ? cq[pb] : -1;
      valid = blk >= 0 && blk <= (n_t - 1) / hsi_s;   // ids outside the visible blocks are ignored
      const int ent = valid ? blk * hsi_s + vj % hsi_s : 0;
      valid = valid && ent < n_t;
      return valid ? ent : 0;
    }
    const int ent = base + j;
    valid = ent < n_t;
    return valid ? ent : 0;
  };
  const int dma_e = lane >> 2, dma_b = ((lane & 3) - (dma_e >> 2)) & 3;
  auto issue = [&](int i, unsigned char* ring) {
    const int st = wave + 4 * i;
    unsigned char* dst = ring + wave * ST_BYTES;
#pragma unroll
    for (int tt = 0; tt < SPT; ++tt) {
      bool v;
      const int ent = entry_at(st * 64 + tt * 16 + dma_e, v);
      dma16(cb + (size_t)ent * 64 + 16 * dma_b, (lds_u8*)(dst + tt * 1024));
    }
    bool v;
    const int ent = entry_at(st * 64 + lane, v);
    dma4(sb + (size_t)ent * 4, (lds_u8*)(dst + SPT * 1024));
  };
  auto compute = [&](int i, const unsigned char* ring) {
    const int st = wave + 4 * i;
    const unsigned char* src = ring + wave * ST_BYTES;
#pragma unroll
    for (int tt = 0; tt < SPT; ++tt) {
      const unsigned char* tb = src + tt * 1024;
      uint32_t cw[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        cw[kb] = *reinterpret_cast<const uint32_t*>(tb + ((4 * lr + ((kb + (lr >> 2)) & 3)) << 4) + 4 * lg);
      const uint32_t sw = *reinterpret_cast<const uint32_t*>(src + SPT * 1024 + (tt * 16 + lr) * 4);
      const float sc0 = __builtin_amdgcn_cvt_f32_fp8((int)sw, 0);
      const float sc1 = __builtin_amdgcn_cvt_f32_fp8((int)sw, 1);
      const float sc2 = __builtin_amdgcn_cvt_f32_fp8((int)sw, 2);
      const float sc3 = __builtin_amdgcn_cvt_f32_fp8((int)sw, 3);
      const float scv[4] = {sc0, sc1, sc2, sc3};
      f32x4 acc[2];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const auto kf = Fp4<T>::cvt(cw[kb]);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const f32x4 tmp = mma16(qf[mt][kb], kf, f32x4{0.f, 0.f, 0.f, 0.f});
          if (kb == 0) acc[mt] = tmp * scv[0];
          else acc[mt] += tmp * scv[kb];
        }
      }
      float part = 0.f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) part += wv[mt][ii] * fmaxf(acc[mt][ii], 0.0f);
      part = sum_lane_groups(part);
      const int j = st * 64 + tt * 16 + lr;
      bool valid;
      entry_at(j, valid);
      if (lg == 0) sm.keys[j] = valid ? score_key(part) : 0u;
    }
  };
  // 3-slot ring, unrolled so that each slot is a distinct LDS object
  if (st_w > 0) issue(0, ring0);
  if (st_w > 1) issue(1, ring1);
  auto step = [&](int i, const unsigned char* cur, unsigned char* nxt) {
    if (i + 2 < st_w) {
      issue(i + 2, nxt);
      WAIT_VMCNT(2 * (SPT + 1));
    } else if (i + 1 < st_w) {
      WAIT_VMCNT(SPT + 1);
    } else {
      WAIT_VMCNT(0);
    }
    compute(i, cur);
    WAIT_LGKM0();
  };
  for (int i = 0; i < st_w; i += 3) {
    step(i, ring0, ring2);
    if (i + 1 < st_w) step(i + 1, ring1, ring0);
    if (i + 2 < st_w) step(i + 2, ring2, ring1);
  }
  __syncthreads();

  if (BUILD) {
    // block maxima of this chunk (C is a multiple of hsi_s)
    const int nb_chunk = C / hsi_s;
    const int nvis_blk = (n_t + hsi_s - 1) / hsi_s;
    for (int jb = threadIdx.x; jb < nb_chunk; jb += SC_THREADS) {
      const int gblk = base / hsi_s + jb;
      if (gblk >= nvis_blk) break;
      uint32_t mx = 0;
      for (int e = 0; e < hsi_s; ++e) mx = max(mx, sm.keys[jb * hsi_s + e]);
      blkmax[(size_t)bt * nblk_max + gblk] = mx;
    }
  }

  // ---- adaptive radix select of the chunk's best min(k_chunk, valid) keys
  uint32_t mn = 0xFFFFFFFFu, mx = 0u, nv = 0u;
  for (int i = threadIdx.x; i < C; i += SC_THREADS) {
    const uint32_t kk = sm.keys[i];
    if (kk) {
      mn = min(mn, kk);
      mx = max(mx, kk);
      ++nv;
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, off, 64));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 64));
    nv += (uint32_t)__shfl_xor((int)nv, off, 64);
  }
  if (lane == 0) {
    sm.red[0][wave] = mn;
    sm.red[1][wave] = mx;
    sm.red[2][wave] = nv;
  }
  __syncthreads();
  mn = sm.red[0][0]; mx = sm.red[1][0]; nv = sm.red[2][0];
#pragma unroll
  for (int w2 = 1; w2 < SC_THREADS / 64; ++w2) {
    mn = min(mn, sm.red[0][w2]);
    mx = max(mx, sm.red[1][w2]);
    nv += sm.red[2][w2];
  }
  const int r0 = rank_for_bound(k, nc_q);
  uint32_t need = nv < (uint32_t)k_chunk ? nv : (uint32_t)k_chunk;
  const size_t obase = ((size_t)bt * n_chunks + c) * k_chunk;
  uint32_t thresh = 0;
  bool eq_mode = false;
  if (threadIdx.x == 0) sm.lb = 0;
  const bool have = nv > 0;
  if (have) {
    uint32_t lo = mn, hi = mx;
    for (int pass = 0;; ++pass) {
      const uint32_t R = hi - lo;
      const int shift = (R >> 11) == 0 ? 0 : 32 - __clz((int)(R >> 11));
      for (int i = threadIdx.x; i < NBINS; i += SC_THREADS) sm.hist[i] = 0;
      __syncthreads();
      for (int i = threadIdx.x; i < C; i += SC_THREADS) {
        const uint32_t kk = sm.keys[i];
        if (kk && kk >= lo && kk <= hi) atomicAdd(&sm.hist[(kk - lo) >> shift], 1u);
      }
      __syncthreads();
      constexpr int BPT = NBINS / SC_THREADS;
      uint32_t own[BPT], tot = 0;
#pragma unroll
      for (int j = 0; j < BPT; ++j) {
        own[j] = sm.hist[threadIdx.x * BPT + j];
        tot += own[j];
      }
      const uint32_t above = suffix_excl(tot, sm);
      uint32_t cum = above;
#pragma unroll
      for (int j = BPT - 1; j >= 0; --j) {
        if (cum < need && cum + own[j] >= need) {
          sm.digit = threadIdx.x * BPT + j;
          sm.above = cum;
          sm.done = (cum + own[j] == need) ? 1u : 0u;
        }
        if (pass == 0 && nv >= (uint32_t)r0 && cum < (uint32_t)r0 && cum + own[j] >= (uint32_t)r0)
          sm.lb = lo + ((uint32_t)(threadIdx.x * BPT + j) << shift);
        cum += own[j];
      }
      __syncthreads();
      const uint32_t d = sm.digit;
      need -= sm.above;
      const uint32_t new_lo = lo + (d << shift);
      const uint64_t top = (uint64_t)new_lo + ((1ull << shift) - 1);
      const uint32_t new_hi = top < (uint64_t)hi ? (uint32_t)top : hi;
      const uint32_t done = sm.done;
      __syncthreads();
      if (done) {
        thresh = new_lo;   // every key >= new_lo is taken
        break;
      }
      if (shift == 0) {
        thresh = new_lo;   // keys > thresh, and the first `need` keys == thresh in index order
        eq_mode = true;
        break;
      }
      lo = new_lo;
      hi = new_hi;
    }
  }
  if (threadIdx.x == 0) {
    sm.count = 0;
    sm.running = 0;
    chunk_lb[(size_t)bt * n_chunks + c] = sm.lb;
  }
  __syncthreads();
  auto entry_of = [&](int i) -> int {
    if (POOL) {
      const int vj = base + i;
      return cq[vj / hsi_s] * hsi_s + vj % hsi_s;
    }
    return base + i;
  };
  if (have) {
    for (int i = threadIdx.x; i < C; i += SC_THREADS) {
      const uint32_t kk = sm.keys[i];
      if (kk && (eq_mode ? kk > thresh : kk >= thresh)) {
        const uint32_t slot = atomicAdd(&sm.count, 1u);
        if (slot < (uint32_t)k_chunk) {
          cand_key[obase + slot] = kk;
          cand_idx[obase + slot] = entry_of(i);
        }
      }
    }
    if (eq_mode) {
      // ties at the threshold: the smallest positions (= smallest entry ids) first
      for (int i0 = 0; i0 < C; i0 += SC_THREADS) {
        const int i = i0 + threadIdx.x;
        const bool eq = sm.keys[i] == thresh;
        const unsigned long long bal = __ballot(eq);
        const uint32_t before = __popcll(bal & ((1ull << lane) - 1ull));
        if (lane == 0) sm.wtot[wave] = __popcll(bal);
        __syncthreads();
        uint32_t wbase = sm.running;
        for (int w2 = 0; w2 < wave; ++w2) wbase += sm.wtot[w2];
        const uint32_t rank = wbase + before;
        if (eq && rank < need) {
          const uint32_t slot = atomicAdd(&sm.count, 1u);
          if (slot < (uint32_t)k_chunk) {
            cand_key[obase + slot] = thresh;
            cand_idx[obase + slot] = entry_of(i);
          }
        }
        __syncthreads();
        if (threadIdx.x == 0)
          for (int w2 = 0; w2 < SC_THREADS / 64; ++w2) sm.running += sm.wtot[w2];
        __syncthreads();
        if (sm.running >= need) break;
      }
    }
  }
  __syncthreads();
  for (int i = (int)min(sm.count, (uint32_t)k_chunk) + threadIdx.x; i < k_chunk; i += SC_THREADS) {
    cand_key[obase + i] = 0u;
    cand_idx[obase + i] = -1;
  }
}

constexpr int MG_THREADS = 512;
constexpr int MAX_SORT = 1024;   // >= k and >= n_b (checked by the host)
constexpr int MG_CAP = 12288;    // candidates staged in LDS

struct MergeSmem {
  int list[MAX_SORT];
  uint32_t count;
  uint32_t tlb;
};

template <bool POOL, bool BUILD>
__global__ __launch_bounds__(MG_THREADS) void topk_merge(const uint32_t* __restrict__ cand_key,
                                                         const int32_t* __restrict__ cand_idx,
                                                         const uint32_t* __restrict__ chunk_lb,
                                                         const uint32_t* __restrict__ blkmax,
                                                         const int32_t* __restrict__ q_pos, int32_t* __restrict__ topk,
                                                         int32_t* __restrict__ cands_out, int T_len, int n_entries,
                                                         int m, int k, int C, int k_chunk, int n_chunks, int hsi_s,
                                                         int hsi_nb, int nblk_max, int cap) {
  __shared__ SelSmem<MG_THREADS> sel;
  __shared__ MergeSmem sm;
  extern __shared__ uint64_t comp_dyn[];   // staged candidates, `cap` of them (dynamic LDS)
  const int t = blockIdx.x, b = blockIdx.y;
  const int bt = b * T_len + t;
  const int n_t = visible(q_pos, bt, m, n_entries);
  const int nc = POOL ? n_chunks : (n_t + C - 1) / C;
  const int n_items = nc * k_chunk;
  const uint32_t* kb = cand_key + (size_t)bt * n_chunks * k_chunk;
  const int32_t* ib = cand_idx + (size_t)bt * n_chunks * k_chunk;

  auto emit_sorted = [&](int32_t* out, int kk, uint32_t cnt) {
    int np2 = 1;
    while (np2 < kk) np2 <<= 1;
    for (int i = cnt + threadIdx.x; i < np2; i += MG_THREADS) sm.list[i] = 0x7FFFFFFF;
    __syncthreads();
    block_bitonic_sort<MG_THREADS>(sm.list, np2);
    for (int i = threadIdx.x; i < kk; i += MG_THREADS) out[i] = (i < (int)cnt) ? sm.list[i] : -1;
    __syncthreads();
  };
  // select from `n` composites produced by get(i), emit the low 32 bits' entry ids sorted
  auto select_emit = [&](auto get, int n, uint32_t kk, int32_t* out, auto id_of) {
    uint64_t prefix, mask;
    block_select<MG_THREADS>(get, n, kk, 64, sel, prefix, mask);
    if (threadIdx.x == 0) sm.count = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += MG_THREADS) {
      const uint64_t cc = get(i);
      if (cc != 0 && (cc & mask) >= prefix) {
        const uint32_t slot = atomicAdd(&sm.count, 1u);
        if (slot < kk) sm.list[slot] = id_of(i, cc);
      }
    }
    __syncthreads();
    const uint32_t cnt = min(sm.count, kk);
    __syncthreads();
    emit_sorted(out, (int)kk, cnt);
  };

  {
    // lower bound of the k-th best key: min over chunks of their rank-r0 bounds
    if (threadIdx.x == 0) {
      sm.count = 0;
      uint32_t tl = 0xFFFFFFFFu;
      for (int c = 0; c < nc; ++c) tl = min(tl, chunk_lb[(size_t)bt * n_chunks + c]);
      sm.tlb = nc > 0 ? tl : 0u;
    }
    __syncthreads();
    const uint32_t tlb = sm.tlb;
    for (int i = threadIdx.x; i < n_items; i += MG_THREADS) {
      const uint32_t kk = kb[i];
      if (kk != 0 && kk >= tlb) {
        const uint32_t slot = atomicAdd(&sm.count, 1u);
        if (slot < (uint32_t)cap) comp_dyn[slot] = ((uint64_t)kk << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)ib[i]);
      }
    }
    __syncthreads();
    const uint32_t staged = sm.count;
    __syncthreads();
    auto id_of = [&](int, uint64_t cc) -> int { return (int)(0xFFFFFFFFu - (uint32_t)(cc & 0xFFFFFFFFu)); };
    if (staged <= (uint32_t)cap) {
      auto get = [&](int i) -> uint64_t { return comp_dyn[i]; };
      select_emit(get, (int)staged, (uint32_t)k, topk + (size_t)bt * k, id_of);
    } else {
      auto get = [&](int i) -> uint64_t {
        const uint32_t kk = kb[i];
        return (kk == 0 || kk < tlb) ? 0ull : (((uint64_t)kk << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)ib[i]));
      };
      select_emit(get, n_items, (uint32_t)k, topk + (size_t)bt * k, id_of);
    }
  }
  if (BUILD) {
    const int nblk = (n_t + hsi_s - 1) / hsi_s;
    const uint32_t* bm = blkmax + (size_t)bt * nblk_max;
    auto bget = [&](int i) -> uint64_t {
      const uint32_t kk = (i == nblk - 1) ? 0xFFFFFFFFu : bm[i];  // newest block forced in
      return kk == 0 ? 0ull : (((uint64_t)kk << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i));
    };
    auto id_of = [&](int i, uint64_t) -> int { return i; };
    if (nblk <= cap) {
      for (int i = threadIdx.x; i < nblk; i += MG_THREADS) comp_dyn[i] = bget(i);
      __syncthreads();
      auto get = [&](int i) -> uint64_t { return comp_dyn[i]; };
      select_emit(get, nblk, (uint32_t)hsi_nb, cands_out + (size_t)bt * hsi_nb, id_of);
    } else {
      select_emit(bget, nblk, (uint32_t)hsi_nb, cands_out + (size_t)bt * hsi_nb, id_of);
    }
  }
}

template <typename T, bool POOL, bool BUILD>
hipError_t launch_impl(const void* q_idx, const float* w, const uint8_t* codes, const uint8_t* scales,
                       const int32_t* q_pos, int32_t* topk, int32_t* cands, int B, int T_len, int H_I, int N_cap,
                       int n_entries, int m, int k, int hsi_s, int hsi_nb, void* ws, const ScorePlan& p,
                       hipStream_t st) {
  char* wsb = static_cast<char*>(ws);
  const size_t n_slots = p.cand_bytes / 8;
  uint32_t* cand_key = reinterpret_cast<uint32_t*>(wsb);
  int32_t* cand_idx = reinterpret_cast<int32_t*>(wsb + n_slots * 4);
  uint32_t* chunk_lb = reinterpret_cast<uint32_t*>(wsb + p.cand_bytes);
  uint32_t* blkmax = reinterpret_cast<uint32_t*>(wsb + p.cand_bytes + p.lb_bytes);
  const int nblk_max = BUILD ? (n_entries + hsi_s - 1) / hsi_s : 0;
  dim3 g1(p.n_chunks, T_len, B);
  hipLaunchKernelGGL((score_chunk<T, POOL, BUILD>), g1, dim3(SC_THREADS), 0, st, static_cast<const T*>(q_idx), w,
                     codes, scales, q_pos, cands, cand_key, cand_idx, chunk_lb, blkmax, T_len, H_I, N_cap, n_entries, m,
                     p.chunk, p.k_chunk, p.n_chunks, k, hsi_s, hsi_nb, nblk_max);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // LDS for staged candidates: enough for all of them (or all block maxima) up to MG_CAP
  long long want = (long long)p.n_chunks * p.k_chunk;
  if (nblk_max > want) want = nblk_max;
  const int cap = (int)(want < MG_CAP ? want : MG_CAP);
  const size_t dyn = (size_t)cap * 8;
  static bool attr_set = false;
  if (!attr_set) {
    hipFuncSetAttribute(reinterpret_cast<const void*>(&topk_merge<POOL, BUILD>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, MG_CAP * 8);
    attr_set = true;
  }
  dim3 g2(T_len, B);
  hipLaunchKernelGGL((topk_merge<POOL, BUILD>), g2, dim3(MG_THREADS), dyn, st, cand_key, cand_idx, chunk_lb, blkmax,
                     q_pos, topk, cands, T_len, n_entries, m, k, p.chunk, p.k_chunk, p.n_chunks, hsi_s, hsi_nb,
                     nblk_max, cap);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_mode(int hsi, const void* q_idx, const float* w, const uint8_t* codes, const uint8_t* scales,
                       const int32_t* q_pos, int32_t* topk, int32_t* cands, int B, int T_len, int H_I, int N_cap,
                       int n_entries, int m, int k, int hsi_s, int hsi_nb, void* ws, const ScorePlan& p,
                       hipStream_t st) {
  if (hsi == 1)
    return launch_impl<T, false, true>(q_idx, w, codes, scales, q_pos, topk, cands, B, T_len, H_I, N_cap, n_entries,
                                       m, k, hsi_s, hsi_nb, ws, p, st);
  if (hsi == 2)
    return launch_impl<T, true, false>(q_idx, w, codes, scales, q_pos, topk, cands, B, T_len, H_I, N_cap, n_entries,
                                       m, k, hsi_s, hsi_nb, ws, p, st);
  return launch_impl<T, false, false>(q_idx, w, codes, scales, q_pos, topk, cands, B, T_len, H_I, N_cap, n_entries, m,
                                      k, hsi_s, hsi_nb, ws, p, st);
}

}  // namespace

ScorePlan plan_score(int B, int T, int n_scan, int k, int hsi, int hsi_s, int hsi_nb) {
  ScorePlan p{};
  const long long Q = (long long)B * T;
  int C = MAX_CHUNK;
  while (C > 256 && C / 2 >= n_scan) C /= 2;                       // no chunk much larger than the scan
  while (C > 1024 && Q * ((n_scan + C - 1) / C) < 1024) C /= 2;   // enough workgroups to fill the GPU
  if (hsi != 0 && C < hsi_s) C = hsi_s;                           // chunks hold whole blocks
  p.chunk = C;
  p.n_chunks = n_scan <= 0 ? 1 : (n_scan + C - 1) / C;
  p.k_chunk = k < C ? k : C;
  p.cand_bytes = (size_t)Q * p.n_chunks * p.k_chunk * 8;
  p.lb_bytes = ((size_t)Q * p.n_chunks * 4 + 255) / 256 * 256;
  const long long nblk = (hsi == 1) ? ((long long)n_scan + hsi_s - 1) / hsi_s : 0;
  p.blk_bytes = (size_t)(Q * nblk * 4);
  p.total_bytes = p.cand_bytes + p.lb_bytes + p.blk_bytes + 256;
  return p;
}

hipError_t launch_score_topk(int dtype, const void* q_idx, const float* w, const uint8_t* codes,
                             const uint8_t* scales, const int32_t* q_pos, int32_t* topk, int32_t* candidates, int B,
                             int T, int H_I, int N_cap, int n_entries, int m, int k, int hsi, int hsi_s, int hsi_nb,
                             void* workspace, const ScorePlan& plan, hipStream_t stream) {
  if (B == 0 || T == 0) return hipSuccess;
  if (dtype == 1)
    return launch_mode<bf16>(hsi, q_idx, w, codes, scales, q_pos, topk, candidates, B, T, H_I, N_cap, n_entries, m,
                             k, hsi_s, hsi_nb, workspace, plan, stream);
  return launch_mode<float>(hsi, q_idx, w, codes, scales, q_pos, topk, candidates, B, T, H_I, N_cap, n_entries, m, k,
                            hsi_s, hsi_nb, workspace, plan, stream);
}

}  // namespace csa2
