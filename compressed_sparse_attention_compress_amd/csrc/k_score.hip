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

constexpr int MAX_CHUNK = 8192;
constexpr int SC_THREADS = 256;

// Visible entries of query (b, t).
__device__ __forceinline__ int visible(const int32_t* q_pos, int bt, int m, int n_entries) {
  int p = q_pos[bt];
  int nv = p < 0 ? 0 : (int)(((int64_t)p + 1) / m);
  return nv < n_entries ? nv : n_entries;
}

template <typename T, bool POOL, bool BUILD>
__global__ __launch_bounds__(SC_THREADS) void score_chunk(
    const T* __restrict__ q_idx, const float* __restrict__ w, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const int32_t* __restrict__ q_pos, const int32_t* __restrict__ cands,
    uint32_t* __restrict__ cand_key, int32_t* __restrict__ cand_idx, uint32_t* __restrict__ blkmax, int T_len,
    int H_I, int N_cap, int n_entries, int m, int C, int k_chunk, int n_chunks, int hsi_s, int hsi_nb,
    int nblk_max) {
  typedef typename Frag<T>::type FragT;
  __shared__ uint32_t keys[MAX_CHUNK];
  __shared__ SelSmem<SC_THREADS> sm;

  const int c = blockIdx.x, t = blockIdx.y, b = blockIdx.z;
  const int bt = b * T_len + t;
  const int n_t = visible(q_pos, bt, m, n_entries);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, lr = lane & 15, lg = lane >> 4;
  const int base = c * C;
  if (!POOL && base >= n_t) return;  // chunk beyond the visible range: never read by the merge

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

  const int tiles = C / 16;
  for (int tt = wave; tt < tiles; tt += 4) {
    const int j = tt * 16 + lr;
    int ent;
    bool valid;
    if (POOL) {
      const int vj = base + j;
      const int pb = vj / hsi_s;
      const int blk = pb < hsi_nb ? cq[pb] : -1;
      valid = blk >= 0 && blk <= (n_t - 1) / hsi_s;   // ids outside the visible blocks are ignored
      ent = valid ? blk * hsi_s + vj % hsi_s : 0;
      valid = valid && ent < n_t;
    } else {
      ent = base + j;
      valid = ent < n_t;
    }
    uint32_t cw[4] = {0, 0, 0, 0}, sw = 0;
    if (valid) {
      const uint8_t* crow = cb + (size_t)ent * 64 + 4 * lg;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) cw[kb] = *reinterpret_cast<const uint32_t*>(crow + 16 * kb);
      sw = *reinterpret_cast<const uint32_t*>(sb + (size_t)ent * 4);
    }
    const float s0 = __builtin_amdgcn_cvt_f32_fp8((int)sw, 0);
    const float s1 = __builtin_amdgcn_cvt_f32_fp8((int)sw, 1);
    const float s2 = __builtin_amdgcn_cvt_f32_fp8((int)sw, 2);
    const float s3 = __builtin_amdgcn_cvt_f32_fp8((int)sw, 3);
    const float sc[4] = {s0, s1, s2, s3};
    f32x4 acc[2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const auto kf = Fp4<T>::cvt(cw[kb]);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        f32x4 tmp = mma16(qf[mt][kb], kf, f32x4{0.f, 0.f, 0.f, 0.f});
        if (kb == 0) acc[mt] = tmp * sc[0];
        else acc[mt] += tmp * sc[kb];
      }
    }
    float part = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) part += wv[mt][i] * fmaxf(acc[mt][i], 0.0f);
    part += __shfl_xor(part, 16, 64);
    part += __shfl_xor(part, 32, 64);
    if (lg == 0) keys[j] = valid ? score_key(part) : 0u;
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
      for (int e = 0; e < hsi_s; ++e) mx = max(mx, keys[jb * hsi_s + e]);
      blkmax[(size_t)bt * nblk_max + gblk] = mx;
    }
  }

  // composite (key << 13 | (8191 - local index)) << 10: 55 bits, all distinct
  auto get = [&](int i) -> uint64_t {
    const uint32_t kk = keys[i];
    return kk == 0 ? 0ull : ((((uint64_t)kk << 13) | (uint64_t)(8191 - i)) << 10);
  };
  uint64_t prefix, mask;
  block_select<SC_THREADS>(get, C, (uint32_t)k_chunk, 55, sm, prefix, mask);
  if (threadIdx.x == 0) sm.count = 0;
  __syncthreads();
  const size_t obase = ((size_t)bt * n_chunks + c) * k_chunk;
  for (int i = threadIdx.x; i < C; i += SC_THREADS) {
    const uint64_t cc = get(i);
    if (cc != 0 && (cc & mask) >= prefix) {
      const uint32_t slot = atomicAdd(&sm.count, 1u);
      if (slot >= (uint32_t)k_chunk) continue;
      int ent;
      if (POOL) {
        const int vj = base + i;
        ent = cq[vj / hsi_s] * hsi_s + vj % hsi_s;
      } else {
        ent = base + i;
      }
      cand_key[obase + slot] = keys[i];
      cand_idx[obase + slot] = ent;
    }
  }
  __syncthreads();
  for (int i = (int)min(sm.count, (uint32_t)k_chunk) + threadIdx.x; i < k_chunk; i += SC_THREADS) {
    cand_key[obase + i] = 0u;
    cand_idx[obase + i] = -1;
  }
}

constexpr int MG_THREADS = 256;
constexpr int MAX_SORT = 1024;  // >= k and >= n_b (checked by the host)

template <bool POOL, bool BUILD>
__global__ __launch_bounds__(MG_THREADS) void topk_merge(const uint32_t* __restrict__ cand_key,
                                                         const int32_t* __restrict__ cand_idx,
                                                         const uint32_t* __restrict__ blkmax,
                                                         const int32_t* __restrict__ q_pos, int32_t* __restrict__ topk,
                                                         int32_t* __restrict__ cands_out, int T_len, int n_entries,
                                                         int m, int k, int C, int k_chunk, int n_chunks, int hsi_s,
                                                         int hsi_nb, int nblk_max) {
  __shared__ SelSmem<MG_THREADS> sm;
  __shared__ int list[MAX_SORT];
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
    for (int i = cnt + threadIdx.x; i < np2; i += MG_THREADS) list[i] = 0x7FFFFFFF;
    __syncthreads();
    block_bitonic_sort<MG_THREADS>(list, np2);
    for (int i = threadIdx.x; i < kk; i += MG_THREADS) out[i] = (i < (int)cnt) ? list[i] : -1;
    __syncthreads();
  };

  {
    auto get = [&](int i) -> uint64_t {
      const uint32_t kk = kb[i];
      return kk == 0 ? 0ull : (((uint64_t)kk << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)ib[i]));
    };
    uint64_t prefix, mask;
    block_select<MG_THREADS>(get, n_items, (uint32_t)k, 64, sm, prefix, mask);
    if (threadIdx.x == 0) sm.count = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n_items; i += MG_THREADS) {
      const uint64_t cc = get(i);
      if (cc != 0 && (cc & mask) >= prefix) {
        const uint32_t slot = atomicAdd(&sm.count, 1u);
        if (slot < (uint32_t)k) list[slot] = ib[i];
      }
    }
    __syncthreads();
    const uint32_t cnt = min(sm.count, (uint32_t)k);
    __syncthreads();
    emit_sorted(topk + (size_t)bt * k, k, cnt);
  }
  if (BUILD) {
    const int nblk = (n_t + hsi_s - 1) / hsi_s;
    const uint32_t* bm = blkmax + (size_t)bt * nblk_max;
    auto get = [&](int i) -> uint64_t {
      const uint32_t kk = (i == nblk - 1) ? 0xFFFFFFFFu : bm[i];  // newest block forced in
      return kk == 0 ? 0ull : (((uint64_t)kk << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i));
    };
    uint64_t prefix, mask;
    block_select<MG_THREADS>(get, nblk, (uint32_t)hsi_nb, 64, sm, prefix, mask);
    if (threadIdx.x == 0) sm.count = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < nblk; i += MG_THREADS) {
      const uint64_t cc = get(i);
      if (cc != 0 && (cc & mask) >= prefix) {
        const uint32_t slot = atomicAdd(&sm.count, 1u);
        if (slot < (uint32_t)hsi_nb) list[slot] = i;
      }
    }
    __syncthreads();
    const uint32_t cnt = min(sm.count, (uint32_t)hsi_nb);
    __syncthreads();
    emit_sorted(cands_out + (size_t)bt * hsi_nb, hsi_nb, cnt);
  }
}

template <typename T, bool POOL, bool BUILD>
hipError_t launch_impl(const void* q_idx, const float* w, const uint8_t* codes, const uint8_t* scales,
                       const int32_t* q_pos, int32_t* topk, int32_t* cands, int B, int T_len, int H_I, int N_cap,
                       int n_entries, int m, int k, int hsi_s, int hsi_nb, void* ws, const ScorePlan& p,
                       hipStream_t st) {
  uint32_t* cand_key = static_cast<uint32_t*>(ws);
  int32_t* cand_idx = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + p.cand_bytes / 2);
  uint32_t* blkmax = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + p.cand_bytes);
  const int nblk_max = BUILD ? (n_entries + hsi_s - 1) / hsi_s : 0;
  dim3 g1(p.n_chunks, T_len, B);
  hipLaunchKernelGGL((score_chunk<T, POOL, BUILD>), g1, dim3(SC_THREADS), 0, st, static_cast<const T*>(q_idx), w,
                     codes, scales, q_pos, cands, cand_key, cand_idx, blkmax, T_len, H_I, N_cap, n_entries, m,
                     p.chunk, p.k_chunk, p.n_chunks, hsi_s, hsi_nb, nblk_max);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2(T_len, B);
  hipLaunchKernelGGL((topk_merge<POOL, BUILD>), g2, dim3(MG_THREADS), 0, st, cand_key, cand_idx, blkmax, q_pos, topk,
                     cands, T_len, n_entries, m, k, p.chunk, p.k_chunk, p.n_chunks, hsi_s, hsi_nb, nblk_max);
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
  if (hsi == 1 && C < hsi_s) C = hsi_s;
  if (hsi == 2) {
    // chunks hold whole pool blocks
    if (C < hsi_s) C = hsi_s;
  }
  p.chunk = C;
  p.n_chunks = n_scan <= 0 ? 1 : (n_scan + C - 1) / C;
  p.k_chunk = k < C ? k : C;
  p.cand_bytes = (size_t)Q * p.n_chunks * p.k_chunk * 8;
  const long long nblk = (hsi == 1) ? ((long long)n_scan + hsi_s - 1) / hsi_s : 0;
  p.blk_bytes = (size_t)(Q * nblk * 4);
  p.total_bytes = p.cand_bytes + p.blk_bytes + 256;
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
