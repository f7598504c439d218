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
// Dequantisation (every bf16 path): a key element is an E2M1 value times an E4M3
// block scale, exact in fp16 (UE8M0 scales: see below).  v_cvt_scalef32_pk_f16_fp4 expands the codes and
// applies the power of two of the scale, one v_pk_mul_f16 applies its sign and
// significand, so the block scale sits inside the MFMA operand and the four
// 32-dim blocks of a key chain into one v_mfma_f32_16x16x32_f16 accumulator.  The
// bf16 query is exact in fp16 once each head is moved into range by a power of
// two, which the head weight takes back (it commutes with the ReLU).  The fp32
// path expands to fp32 and multiplies the block scale into each block's partial
// product instead.
//
// Kernel score_chunk: one workgroup per (query, chunk of C entries); codes and
// scales are loaded straight into registers through buffer resources.  Each
// 16-entry tile is one MFMA column block with the indexer heads as rows; the
// weighted ReLU sums are head-summed with permlane swaps and written to LDS as
// order-preserving keys; a radix select (11-bit digits) keeps the chunk's best
// min(k, C) with a lower bound for the merge, and for HSI the chunk's block
// maxima are written too.
// Kernel score_qtile_bf16 + select_rows (many queries over a cache of at most
// 8192 entries): 4 queries per workgroup share each dequantised tile; keys go to
// a key matrix, then one wave per query selects its k best.
// Kernel score_stream (very many queries over caches longer than the tiled path
// takes): one workgroup per (query, part of up to 65536 entries) keeps only the
// entries scoring at least the k-th best seen so far and cuts them back to the k
// best a few times per part, so a query costs a few selections instead of one per
// chunk plus a merge.
// Kernel topk_prefilter (queries with many chunks): workgroups over groups of
// chunks drop the candidates below the merge bound before the merge stages them.
// Kernel topk_merge: one workgroup per query: the select over all chunk
// candidates at or above the merge bound, indices sorted ascending and padded
// with -1; with HSI BUILD also the n_b best blocks (newest block forced) as the
// pool.
// Index-K scales are E4M3 or UE8M0 (a template argument of every scorer); with
// UE8M0 the fp16 operand takes each block's power of two relative to the entry's
// largest, which multiplies the entry's dot products afterwards.
#include "csa2_internal.h"
#include "device_common.h"
#include "lds_dma.h"

namespace csa2 {

namespace {

constexpr int NBINS = 2048;   // radix digit of 11 bits

// Shared memory of the block-wide selection helpers below.
template <int NT>
struct SelSmem {
  uint32_t hist[NBINS];
  uint32_t wsum[NT / 64];
  uint32_t red[3][NT / 64];
  uint32_t digit, above, done, lb, lb_above;
};

// Exclusive prefix sum over the threads of a block; `total` gets the block sum.
template <int NT>
__device__ __forceinline__ uint32_t block_prefix_excl(uint32_t v, SelSmem<NT>& sm, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t u = __shfl_up(x, off, 64);
    if (lane >= off) x += u;
  }
  if (lane == 63) sm.wsum[wave] = x;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const uint32_t s = sm.wsum[w];
    if (w < wave) before += s;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return x - v + before;
}

// Minimum, maximum and number of the non-zero keys key_at(0..n).
template <int NT, typename Get>
__device__ void key_stats(Get key_at, int n, SelSmem<NT>& sm, uint32_t& mn, uint32_t& mx, uint32_t& nv) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  mn = 0xFFFFFFFFu;
  mx = 0u;
  nv = 0u;
#pragma unroll 8   // several key reads in flight
  for (int i = threadIdx.x; i < n; i += NT) {
    const uint32_t kk = key_at(i);
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
  mn = sm.red[0][0];
  mx = sm.red[1][0];
  nv = sm.red[2][0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) {
    mn = min(mn, sm.red[0][w]);
    mx = max(mx, sm.red[1][w]);
    nv += sm.red[2][w];
  }
  __syncthreads();
}

// Result of a selection: a key is chosen iff it is non-zero and either greater than
// `thresh`, or equal to it and among the first `eq_take` keys equal to it in
// position order.  `lb` is a lower bound of the rank-r0 largest key (0 when there
// are fewer than r0 keys or no bound was asked for).
struct SelOut {
  uint32_t thresh, eq_take, lb;
};

// Radix select of the `need` (<= number of non-zero keys) largest non-zero keys,
// ties resolved in position order.  The digit of each pass covers the live key
// range [lo, hi] (starting from the keys' [min, max]) with 2048 bins, so a pass
// usually shrinks the range by ~2^11 and the loop ends when the count at the
// boundary bin is exact or the bin holds a single value.  The rank-r0 bound is
// the lower edge of the first pass's bin that holds the rank-r0 key; with
// `fine_lb` one more histogram over that bin makes it 2^11 times finer.
template <int NT, typename Get>
__device__ SelOut select_threshold(Get key_at, int n, uint32_t need, uint32_t mn, uint32_t mx, uint32_t r0,
                                   SelSmem<NT>& sm, bool fine_lb = false) {
  if (need == 0) return SelOut{0xFFFFFFFFu, 0u, 0u};
  if (threadIdx.x == 0) sm.lb = 0;
  uint32_t lo = mn, hi = mx;
  constexpr int BPT = NBINS / NT;
  for (int pass = 0;; ++pass) {
    const uint32_t R = hi - lo;
    const int shift = (R >> 11) == 0 ? 0 : 32 - __clz((int)(R >> 11));
    for (int i = threadIdx.x; i < NBINS; i += NT) sm.hist[i] = 0;
    __syncthreads();
#pragma unroll 8   // several key reads in flight
    for (int i = threadIdx.x; i < n; i += NT) {
      const uint32_t kk = key_at(i);
      if (kk && kk >= lo && kk <= hi) atomicAdd(&sm.hist[(kk - lo) >> shift], 1u);
    }
    __syncthreads();
    uint32_t own[BPT], tot = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      own[j] = sm.hist[threadIdx.x * BPT + j];
      tot += own[j];
    }
    uint32_t total;
    const uint32_t pre = block_prefix_excl<NT>(tot, sm, total);
    uint32_t cum = total - pre - tot;   // keys in higher bins
#pragma unroll
    for (int j = BPT - 1; j >= 0; --j) {
      if (cum < need && cum + own[j] >= need) {
        sm.digit = threadIdx.x * BPT + j;
        sm.above = cum;
        sm.done = (cum + own[j] == need) ? 1u : 0u;
      }
      if (pass == 0 && r0 != 0 && cum < r0 && cum + own[j] >= r0) {
        sm.lb = lo + ((uint32_t)(threadIdx.x * BPT + j) << shift);
        sm.lb_above = cum;
      }
      cum += own[j];
    }
    __syncthreads();
    const uint32_t d = sm.digit;
    need -= sm.above;
    const uint32_t new_lo = lo + (d << shift);
    const uint64_t top = (uint64_t)new_lo + ((1ull << shift) - 1);
    const uint32_t new_hi = top < (uint64_t)hi ? (uint32_t)top : hi;
    const uint32_t done = sm.done;
    uint32_t lb = sm.lb;
    const uint32_t lb_above = sm.lb_above;
    __syncthreads();
    if (pass == 0 && fine_lb && lb != 0 && shift > 0) {
      // keys of the rank-r0 bin [blo, bhi] at 2^11 finer bins; lb_above keys lie above it
      const uint32_t blo = lb;
      const uint64_t btop = (uint64_t)blo + ((1ull << shift) - 1);
      const uint32_t bhi = btop < (uint64_t)hi ? (uint32_t)btop : hi;
      const int shift1 = shift > 11 ? shift - 11 : 0;
      for (int i = threadIdx.x; i < NBINS; i += NT) sm.hist[i] = 0;
      __syncthreads();
#pragma unroll 8
      for (int i = threadIdx.x; i < n; i += NT) {
        const uint32_t kk = key_at(i);
        if (kk && kk >= blo && kk <= bhi) atomicAdd(&sm.hist[(kk - blo) >> shift1], 1u);
      }
      __syncthreads();
      uint32_t own1[BPT], tot1 = 0;
#pragma unroll
      for (int j = 0; j < BPT; ++j) {
        own1[j] = sm.hist[threadIdx.x * BPT + j];
        tot1 += own1[j];
      }
      uint32_t total1;
      const uint32_t pre1 = block_prefix_excl<NT>(tot1, sm, total1);
      uint32_t cum1 = lb_above + (total1 - pre1 - tot1);
#pragma unroll
      for (int j = BPT - 1; j >= 0; --j) {
        if (cum1 < r0 && cum1 + own1[j] >= r0) sm.lb = blo + ((uint32_t)(threadIdx.x * BPT + j) << shift1);
        cum1 += own1[j];
      }
      __syncthreads();
      lb = sm.lb;
      __syncthreads();
    }
    if (done) return SelOut{new_lo, 0xFFFFFFFFu, lb};   // every key >= new_lo
    if (shift == 0) return SelOut{new_lo, need, lb};    // keys > new_lo and the first `need` equal to it
    lo = new_lo;
    hi = new_hi;
  }
}

// Calls emit(i, slot) for every chosen position i in increasing i, with slot =
// the number of chosen positions before i; returns the number chosen.  Wave w owns
// a contiguous range of positions and walks it 64 at a time, so the reads are
// unit-stride and one block-wide exchange of per-wave counts orders the output.
template <int NT, typename Get, typename Emit>
__device__ uint32_t emit_ordered(Get key_at, int n, const SelOut& s, SelSmem<NT>& sm, Emit emit) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int per_w = (((n + NW - 1) / NW) + 63) & ~63;
  const int w0 = wave * per_w, w1 = min(n, w0 + per_w);
  uint32_t g = 0, e = 0;
  for (int i0 = w0; i0 < w1; i0 += 64) {
    const int i = i0 + lane;
    const uint32_t kk = i < w1 ? key_at(i) : 0u;
    g += __popcll(__ballot(kk != 0 && kk > s.thresh));
    e += __popcll(__ballot(kk != 0 && kk == s.thresh));
  }
  if (lane == 0) {
    sm.red[0][wave] = g;
    sm.red[1][wave] = e;
  }
  __syncthreads();
  uint32_t G = 0, E = 0, GT = 0, ET = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t gw = sm.red[0][w], ew = sm.red[1][w];
    if (w < wave) {
      G += gw;
      E += ew;
    }
    GT += gw;
    ET += ew;
  }
  __syncthreads();
  const uint64_t lt = (1ull << lane) - 1ull;
  for (int i0 = w0; i0 < w1; i0 += 64) {
    const int i = i0 + lane;
    const uint32_t kk = i < w1 ? key_at(i) : 0u;
    const bool is_gt = kk != 0 && kk > s.thresh, is_eq = kk != 0 && kk == s.thresh;
    const uint64_t mg = __ballot(is_gt), me = __ballot(is_eq);
    const uint32_t gl = G + __popcll(mg & lt), el = E + __popcll(me & lt);
    if (is_gt) emit(i, gl + min(el, s.eq_take));
    else if (is_eq && el < s.eq_take) emit(i, gl + el);
    G += __popcll(mg);
    E += __popcll(me);
  }
  return GT + min(ET, s.eq_take);
}

// emit_ordered for a selection without a partial tie (every non-zero key >= thresh
// is chosen) over keys in LDS: one pass in which wave w compacts its chosen keys
// to the front of its own range of `keys` (in place: a key is written at or
// before the position it was read from, in the same or an earlier step) and their
// positions to its segment of `stage`, then one block-wide copy calls
// emit(slot, key, position) for slots 0, 1, ... in position order.  Each lane
// reads 4 consecutive keys per step; position order is lane-major.  Needs at most
// `seg` chosen keys (the per-wave segment of `stage`).
template <int NT, typename Emit>
__device__ uint32_t emit_compact(uint32_t* keys, int n, uint32_t thresh, uint32_t* stage, int seg, SelSmem<NT>& sm,
                                 Emit emit) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int per_w = (((n + NW - 1) / NW) + 255) & ~255;
  const int w0 = wave * per_w, w1 = min(n, w0 + per_w);
  const uint64_t lt = (1ull << lane) - 1ull;
  uint32_t cnt = 0;
  for (int i0 = w0; i0 < w1; i0 += 256) {
    const int i = i0 + 4 * lane;
    const uint4 kv = i < w1 ? *reinterpret_cast<const uint4*>(keys + i) : make_uint4(0, 0, 0, 0);
    const uint32_t kk[4] = {kv.x, kv.y, kv.z, kv.w};
    bool s[4];
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      s[q] = i + q < w1 && kk[q] != 0u && kk[q] >= thresh;
      const uint64_t m = __ballot(s[q]);
      before += __popcll(m & lt);
      tot += __popcll(m);
    }
    uint32_t slot = cnt + before;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (s[q]) {
        keys[w0 + slot] = kk[q];
        stage[wave * seg + slot] = (uint32_t)(i + q);
        ++slot;
      }
    }
    cnt += tot;
  }
  if (lane == 0) sm.red[0][wave] = cnt;
  __syncthreads();
  uint32_t off[NW + 1];
  off[0] = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) off[w + 1] = off[w] + sm.red[0][w];
  const uint32_t total = off[NW];
  for (uint32_t t = threadIdx.x; t < total; t += NT) {
    int w = 0;
#pragma unroll
    for (int v = 1; v < NW; ++v) w += t >= off[v] ? 1 : 0;
    const uint32_t j = t - off[w];
    emit(t, keys[w * per_w + j], stage[w * seg + j]);
  }
  __syncthreads();
  return total;
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
constexpr int SPT = 4;                          // tiles (of 16 entries) per super-tile
constexpr int ST_BYTES = SPT * 1024 + 256;      // one super-tile in LDS: codes + scales


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

// ---- fp16 scoring of bf16 queries against FP4 keys.
// A key element is code x E4M3 scale: at most 2 + 4 significant bits with an
// exponent in [-10, 12], so it is exact in fp16.  The convert instruction applies
// the scale's power of two (it takes only the exponent of its f32 scale operand);
// one packed fp16 multiply applies the scale's sign and 1.mmm significand.  A bf16
// query has 8 significant bits, so it is exact in fp16 once each head is moved by
// a power of two 2^-s into fp16's range; the head's weight takes the 2^s back
// (ReLU commutes with a positive factor).  With the block scale inside the
// operand, the four 32-dim blocks of a key chain into one MFMA accumulator.
typedef _Float16 f16;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
template <typename T> struct ScoreQ;
template <> struct ScoreQ<bf16> { typedef f16x8 type; };
template <> struct ScoreQ<float> { typedef f32x8 type; };

__device__ __forceinline__ f32x4 mma16h(const f16x8& a, const f16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// 8 FP4 codes (dim 2t in the low nibble of byte t) times the scale whose power of
// two is p2 and whose signed significand is mm.
__device__ __forceinline__ f16x8 fp4x8_scaled_f16(uint32_t w, float p2, f16x2 mm) {
  const f16x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, p2, 0) * mm;
  const f16x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, p2, 1) * mm;
  const f16x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, p2, 2) * mm;
  const f16x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, p2, 3) * mm;
  f16x8 r;
  r[0] = v0[0]; r[1] = v0[1]; r[2] = v1[0]; r[3] = v1[1];
  r[4] = v2[0]; r[5] = v2[1]; r[6] = v3[0]; r[7] = v3[1];
  return r;
}
// Power of two and signed significand of an E4M3 scale byte (exact split of its
// f32 value; a zero scale gives the power 0, whose products flush to 0).
__device__ __forceinline__ void split_e4m3(uint32_t byte, float& p2, f16x2& mm) {
  const uint32_t bits = __float_as_uint(__builtin_amdgcn_cvt_f32_fp8((int)byte, 0));
  p2 = __uint_as_float(bits & 0x7F800000u);
  const f16 m = (f16)__uint_as_float((bits & 0x807FFFFFu) | 0x3F800000u);
  mm = f16x2{m, m};
}
// Scale of an index-K block for the fp16 operand.  E4M3 (SF 0): the exact split
// above.  UE8M0 (SF 1): p2 = 2^(e - e_ref), mm = 1, with e_ref the entry's largest
// block exponent byte; the entry's dot products are multiplied by 2^(e_ref - 127)
// afterwards (entry_post), so every operand stays within fp16 (a block more than
// ~2^24 below the entry's largest flushes to 0).
__device__ __forceinline__ uint32_t max_byte4(uint32_t w) {
  return max(max(w & 0xFFu, (w >> 8) & 0xFFu), max((w >> 16) & 0xFFu, w >> 24));
}
template <int SF>
__device__ __forceinline__ void split_scale(uint32_t byte, uint32_t eref, float& p2, f16x2& mm) {
  if constexpr (SF == 0) {
    split_e4m3(byte, p2, mm);
  } else {
    const int d = (int)byte - (int)eref + 127;
    p2 = d > 0 ? __uint_as_float((uint32_t)d << 23) : 0.0f;
    mm = f16x2{(f16)1.0f, (f16)1.0f};
  }
}
__device__ __forceinline__ float entry_post(uint32_t eref) {
  return eref != 0u ? __uint_as_float(eref << 23) : 0.0f;
}
// A block scale as a float32 (the fp32 scoring path).
template <int SF, int I>
__device__ __forceinline__ float block_scale_f32(uint32_t w) {
  if constexpr (SF == 0) return __builtin_amdgcn_cvt_f32_fp8((int)w, I);
  else return ue8m0_decode((w >> (8 * I)) & 0xFFu);
}

// Max over lanes l, l^16, l^32, l^48 with the gfx950 permlane swaps.
__device__ __forceinline__ float max_lane_groups(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  float y = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  auto r2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(r2[0]), __uint_as_float(r2[1]));
}

// Lower bound for the merge.  In a scan over nc chunks every chunk but the last
// is full, so with r0 = ceil(k / (nc - 1)) the first nc - 1 chunks hold at least
// k entries at or above the smallest of their rank-r0 keys: that smallest value
// bounds the k-th best key from below and the merge drops every candidate under it.
__device__ __forceinline__ uint32_t rank_for_bound(int k, int nc) { return nc > 1 ? (uint32_t)((k + nc - 2) / (nc - 1)) : 0u; }

// Indexer query fragments of query bt: row tile mt = heads 16mt.., k-step kb =
// dims 32kb + 8lg ..  bf16: k-step j of lane group g holds dims 32g + 8j .. +7
// (block g), fp16 as described above; fp32: k-step kb holds block kb (dims
// 32kb + 8g .. +7).  wv[mt][i] is the weight of head 16mt + 4lg + i (times the
// head's power of two for bf16).
template <typename T>
__device__ __forceinline__ void load_qfrags(const T* __restrict__ qb, const float* __restrict__ wrow, int H_I,
                                            int lr, int lg, typename ScoreQ<T>::type (&qf)[2][4],
                                            float (&wv)[2][4]) {
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int h = mt * 16 + lr;
    if constexpr (sizeof(T) == 2) {
      bf16x8 raw[4];
      float amax = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (h < H_I) raw[j] = load_frag(qb + (size_t)h * 128 + 32 * lg + 8 * j);
        else zero_frag(raw[j]);
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf((float)raw[j][i]));
      }
      amax = max_lane_groups(amax);
      int ex = 0;
      frexpf(amax, &ex);                          // amax < 2^ex
      const int s = amax > 0.0f ? min(max(ex - 15, -96), 96) : 0;   // |q| 2^-s < 2^15
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) qf[mt][j][i] = (f16)ldexpf((float)raw[j][i], -s);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hh = mt * 16 + 4 * lg + i;
        const int sh = __shfl(s, 4 * lg + i, 64);
        wv[mt][i] = hh < H_I ? ldexpf(wrow[hh], sh) : 0.0f;
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        if (h < H_I) qf[mt][kb] = load_frag(qb + (size_t)h * 128 + kb * 32 + 8 * lg);
        else zero_frag(qf[mt][kb]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hh = mt * 16 + 4 * lg + i;
        wv[mt][i] = hh < H_I ? wrow[hh] : 0.0f;
      }
    }
  }
}

// One super-tile of 64 consecutive entries in registers: lane (e = l % 16,
// g = l / 16) holds, for tile tt, the 16 code bytes of quantisation block g of
// entry 16tt + e and that entry's 4 scale bytes.
struct StLoad {
  uint4 c[SPT];
  uint32_t s[SPT];
};

// Score of entry 64st + lane of a loaded super-tile, in every lane.  bf16: the
// lane's dword j feeds k-step j, scaled by block g's scale inside the operand;
// the weighted ReLU sums of the 4 tiles are head-summed over the 4 lane groups at
// once with two rounds of permlane swaps.  fp32: four permlane swaps transpose the
// 4 x 4 pattern (lane group x dword) so that dword kb of lane group g holds dims
// 32kb + 8g .. +7 and k-step kb covers block kb, whose per-entry scale multiplies
// the step's partial product.  ReLU is an integer max on the float's bits
// (negative floats are negative integers).
template <typename T, int SF>
__device__ __forceinline__ float score_supertile(const typename ScoreQ<T>::type (&qf)[2][4],
                                                 const float (&wv)[2][4], const StLoad& L, int lg) {
  if constexpr (sizeof(T) == 2) {
    float part[SPT];
#pragma unroll
    for (int tt = 0; tt < SPT; ++tt) {
      const uint32_t cw[4] = {L.c[tt].x, L.c[tt].y, L.c[tt].z, L.c[tt].w};
      float p2;
      f16x2 mm;
      const uint32_t eref = SF ? max_byte4(L.s[tt]) : 0u;
      split_scale<SF>((L.s[tt] >> (8 * lg)) & 0xFFu, eref, p2, mm);
      f32x4 acc[2];
      acc[0] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f16x8 kf = fp4x8_scaled_f16(cw[j], p2, mm);
        acc[0] = mma16h(qf[0][j], kf, acc[0]);
        acc[1] = mma16h(qf[1][j], kf, acc[1]);
      }
      if constexpr (SF != 0) {
        const float post = entry_post(eref);
        acc[0] *= post;
        acc[1] *= post;
      }
      float p = 0.f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
          p = fmaf(wv[mt][ii], __int_as_float(max(__float_as_int(acc[mt][ii]), 0)), p);
      part[tt] = p;
    }
    // after two rounds of swaps and adds lane group g holds tile g's sums
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]), __float_as_uint(part[2]), false, false);
    const auto b2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[1]), __float_as_uint(part[3]), false, false);
    const float s02 = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const float s13 = __uint_as_float(b2[0]) + __uint_as_float(b2[1]);
    const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(s02), __float_as_uint(s13), false, false);
    return __uint_as_float(c[0]) + __uint_as_float(c[1]);
  } else {
    float mine = 0.f;
#pragma unroll
    for (int tt = 0; tt < SPT; ++tt) {
      uint32_t cw[4] = {L.c[tt].x, L.c[tt].y, L.c[tt].z, L.c[tt].w};
      f32x4 acc[2];
      auto a = __builtin_amdgcn_permlane32_swap(cw[0], cw[2], false, false);
      auto b2 = __builtin_amdgcn_permlane32_swap(cw[1], cw[3], false, false);
      auto c0 = __builtin_amdgcn_permlane16_swap(a[0], b2[0], false, false);
      auto c1 = __builtin_amdgcn_permlane16_swap(a[1], b2[1], false, false);
      cw[0] = c0[0]; cw[1] = c0[1]; cw[2] = c1[0]; cw[3] = c1[1];
      const uint32_t sw = L.s[tt];
      const float scv[4] = {block_scale_f32<SF, 0>(sw), block_scale_f32<SF, 1>(sw), block_scale_f32<SF, 2>(sw),
                            block_scale_f32<SF, 3>(sw)};
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
      part = sum_lane_groups(part);   // entry 16tt + e, in all four lane groups
      if (lg == tt) mine = part;
    }
    return mine;
  }
}

template <typename T, bool POOL, bool BUILD, int SF>
__global__ __launch_bounds__(SC_THREADS) void score_chunk(
    const T* __restrict__ q_idx, const float* __restrict__ w, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const int32_t* __restrict__ q_pos, const int32_t* __restrict__ cands,
    uint32_t* __restrict__ cand_key, int32_t* __restrict__ cand_idx, uint32_t* __restrict__ chunk_lb,
    uint32_t* __restrict__ blkmax, int32_t* __restrict__ topk, float* __restrict__ scores_out, int T_len, int H_I,
    int N_cap, int n_entries, int m, int C, int k_chunk, int n_chunks, int k, int hsi_s, int hsi_nb, int nblk_max) {
  typedef typename Frag<T>::type FragT;
  __shared__ SelSmem<SC_THREADS> sm;
  __shared__ __attribute__((aligned(16))) uint32_t keys[MAX_CHUNK];

  const int c = blockIdx.x, t = blockIdx.y, b = blockIdx.z;
  const int bt = b * T_len + t;
  const int n_t = visible(q_pos, bt, m, n_entries);
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int base = c * C;
  const int nc_q = POOL ? n_chunks : (n_t + C - 1) / C;
  // a query whose candidates fit one chunk gets its top-k written here; the merge skips it
  const bool direct = !BUILD && nc_q <= 1;
  if (!POOL && base >= n_t) {
    if (direct && c == 0)   // nothing visible
      for (int i = threadIdx.x; i < k; i += SC_THREADS) topk[(size_t)bt * k + i] = -1;
    return;   // chunk beyond the visible range: never read by the merge
  }
  // positions of this chunk that hold visible entries, rounded up to whole super-tiles
  // (and whole HSI blocks); keys past them are never read
  const int gran = BUILD ? (hsi_s > 64 ? hsi_s : 64) : 64;
  const int n_here = POOL ? C : min(C, n_t - base);
  const int Ce = min(C, (n_here + gran - 1) / gran * gran);

  // indexer query fragments: row tile mt = heads 16mt.., k-step kb = dims 32kb + 8lg ..
  // bf16: k-step j of lane group g holds dims 32g + 8j .. +7 (block g), fp16 as
  // described above; fp32: k-step kb holds block kb (dims 32kb + 8g .. +7)
  typename ScoreQ<T>::type qf[2][4];
  float wv[2][4];
  const T* qb = q_idx + (size_t)bt * H_I * 128;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int h = mt * 16 + lr;
    if constexpr (sizeof(T) == 2) {
      bf16x8 raw[4];
      float amax = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (h < H_I) raw[j] = load_frag(qb + (size_t)h * 128 + 32 * lg + 8 * j);
        else zero_frag(raw[j]);
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf((float)raw[j][i]));
      }
      amax = max_lane_groups(amax);
      int ex = 0;
      frexpf(amax, &ex);                          // amax < 2^ex
      const int s = amax > 0.0f ? min(max(ex - 15, -96), 96) : 0;   // |q| 2^-s < 2^15
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) qf[mt][j][i] = (f16)ldexpf((float)raw[j][i], -s);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hh = mt * 16 + 4 * lg + i;
        const int sh = __shfl(s, 4 * lg + i, 64);
        wv[mt][i] = hh < H_I ? ldexpf(w[(size_t)bt * H_I + hh], sh) : 0.0f;
      }
    } else {
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
  }
  const int32_t* cq = POOL ? cands + (size_t)bt * hsi_nb : nullptr;
  const uint8_t* cb = codes + (size_t)b * N_cap * 64;
  const uint8_t* sb = scales + (size_t)b * N_cap * 4;

  // ---- scoring.  Wave w takes super-tiles w, w+4, ... of 64 entries (4 tiles of
  // 16), straight into registers: lane (e = l % 16, g = l / 16) of a tile loads the
  // 16 code bytes of quantisation block g of entry e (a tile of consecutive entries
  // is one contiguous 1 KB) and the entry's 4 scale bytes.  bf16: the lane's dword
  // j feeds k-step j, scaled by block g's scale inside the operand.  fp32: four
  // permlane swaps transpose the 4 x 4 pattern (lane group x dword) so that dword
  // kb of lane group g holds dims 32kb + 8g .. +7 and k-step kb covers block kb,
  // whose per-entry scale multiplies the step's partial product.  The next
  // super-tile's loads are in flight while one is computed.
  const int n_st = Ce / 64;
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
  // Flat selection reads consecutive entries through buffer resources over this
  // sequence's codes and scales: one offset per super-tile, immediate offsets per
  // tile, and reads past the N_cap entries return 0 (their keys are masked anyway).
  // The loads of a super-tile past the wave's last one are issued too, with an
  // offset past the buffer (no memory access) or entry 0, so that every load is
  // unconditional: the compiler's wait counts then let the next super-tile's loads
  // stay in flight while one is computed (a conditional load makes it assume the
  // shorter queue and wait for them).
  const bool use_buf = !POOL && N_cap <= (1 << 25);
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)cb, (short)0, use_buf ? N_cap * 64 : 0, 0x00020000);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)sb, (short)0, use_buf ? N_cap * 4 : 0, 0x00020000);
  auto load_buf = [&](int i, StLoad& L) {
    const int st = wave + 4 * i;
    const bool live = i < st_w;
    const int e = base + st * 64 + lr;
    const int oc = live ? e * 64 + 16 * lg : (int)0x80000000;
    const int os = live ? e * 4 : (int)0x80000000;
#pragma unroll
    for (int tt = 0; tt < SPT; ++tt) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rc, oc + tt * 1024, 0, 0);
      L.c[tt] = make_uint4(v[0], v[1], v[2], v[3]);
      L.s[tt] = __builtin_amdgcn_raw_buffer_load_b32(rs, os + tt * 64, 0, 0);
    }
  };
  auto load_glob = [&](int i, StLoad& L) {
    const int st = wave + 4 * i;
    const bool live = i < st_w;
#pragma unroll
    for (int tt = 0; tt < SPT; ++tt) {
      bool v;
      const int ent = live ? entry_at(st * 64 + tt * 16 + lr, v) : 0;
      L.c[tt] = *reinterpret_cast<const uint4*>(cb + (size_t)ent * 64 + 16 * lg);
      L.s[tt] = *reinterpret_cast<const uint32_t*>(sb + (size_t)ent * 4);
    }
  };
  auto compute = [&](int i, const StLoad& L) {
    const int st = wave + 4 * i;
    if constexpr (sizeof(T) == 2) {
      // per tile: 8 heads x 1 entry per lane; ReLU as an integer max on the float's
      // bits (negative floats are negative integers)
      float part[SPT];
#pragma unroll
      for (int tt = 0; tt < SPT; ++tt) {
        const uint32_t cw[4] = {L.c[tt].x, L.c[tt].y, L.c[tt].z, L.c[tt].w};
        float p2;
        f16x2 mm;
        const uint32_t eref = SF ? max_byte4(L.s[tt]) : 0u;
        split_scale<SF>((L.s[tt] >> (8 * lg)) & 0xFFu, eref, p2, mm);
        f32x4 acc[2];
        acc[0] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f16x8 kf = fp4x8_scaled_f16(cw[j], p2, mm);
          acc[0] = mma16h(qf[0][j], kf, acc[0]);
          acc[1] = mma16h(qf[1][j], kf, acc[1]);
        }
        if constexpr (SF != 0) {
          const float post = entry_post(eref);
          acc[0] *= post;
          acc[1] *= post;
        }
        float p = 0.f;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int ii = 0; ii < 4; ++ii)
            p = fmaf(wv[mt][ii], __int_as_float(max(__float_as_int(acc[mt][ii]), 0)), p);
        part[tt] = p;
      }
      // head sums of the 4 tiles over the 4 lane groups at once: after two rounds
      // of swaps and adds lane group g holds tile g's sums, i.e. entry st*64 + lane
      const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]), __float_as_uint(part[2]), false, false);
      const auto b2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[1]), __float_as_uint(part[3]), false, false);
      const float s02 = __uint_as_float(a[0]) + __uint_as_float(a[1]);
      const float s13 = __uint_as_float(b2[0]) + __uint_as_float(b2[1]);
      const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(s02), __float_as_uint(s13), false, false);
      const float s = __uint_as_float(c[0]) + __uint_as_float(c[1]);
      const int j = st * 64 + lane;
      bool valid;
      entry_at(j, valid);
      keys[j] = valid ? score_key(s) : 0u;
    } else {
#pragma unroll
    for (int tt = 0; tt < SPT; ++tt) {
      uint32_t cw[4] = {L.c[tt].x, L.c[tt].y, L.c[tt].z, L.c[tt].w};
      f32x4 acc[2];
      {
        auto a = __builtin_amdgcn_permlane32_swap(cw[0], cw[2], false, false);
        auto b2 = __builtin_amdgcn_permlane32_swap(cw[1], cw[3], false, false);
        auto c0 = __builtin_amdgcn_permlane16_swap(a[0], b2[0], false, false);
        auto c1 = __builtin_amdgcn_permlane16_swap(a[1], b2[1], false, false);
        cw[0] = c0[0]; cw[1] = c0[1]; cw[2] = c1[0]; cw[3] = c1[1];
        const uint32_t sw = L.s[tt];
        const float sc0 = block_scale_f32<SF, 0>(sw);
        const float sc1 = block_scale_f32<SF, 1>(sw);
        const float sc2 = block_scale_f32<SF, 2>(sw);
        const float sc3 = block_scale_f32<SF, 3>(sw);
        const float scv[4] = {sc0, sc1, sc2, sc3};
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
      if (lg == 0) keys[j] = valid ? score_key(part) : 0u;
    }
    }   // fp32
  };
  // one loop per load form, so that each loop's wait counts see one kind of load
  auto scan = [&](auto load_st) {
    StLoad L0, L1;
    load_st(0, L0);
    for (int i = 0; i < st_w; i += 2) {
      load_st(i + 1, L1);
      __builtin_amdgcn_sched_barrier(0);
      compute(i, L0);
      load_st(i + 2, L0);
      __builtin_amdgcn_sched_barrier(0);
      if (i + 1 < st_w) compute(i + 1, L1);
    }
  };
  if (use_buf) scan(load_buf);
  else scan(load_glob);
  __syncthreads();
  if (scores_out != nullptr) {   // debug dump: the scores of this chunk's valid positions
    float* srow = scores_out + (size_t)bt * (POOL ? hsi_nb * hsi_s : n_entries) + base;
    for (int j = threadIdx.x; j < Ce; j += SC_THREADS)
      if (keys[j] != 0u) srow[j] = key_score(keys[j]);
  }

  if (BUILD) {
    // block maxima of this chunk (C is a multiple of hsi_s)
    const int nb_chunk = Ce / hsi_s;
    const int nvis_blk = (n_t + hsi_s - 1) / hsi_s;
    for (int jb = threadIdx.x; jb < nb_chunk; jb += SC_THREADS) {
      const int gblk = base / hsi_s + jb;
      if (gblk >= nvis_blk) break;
      uint32_t mx = 0;
      for (int e = 0; e < hsi_s; ++e) mx = max(mx, keys[jb * hsi_s + e]);
      blkmax[(size_t)bt * nblk_max + gblk] = mx;
    }
  }

  // ---- the chunk's best min(k_chunk, valid) keys, emitted in entry order
  auto key_at = [&](int i) -> uint32_t { return keys[i]; };
  uint32_t mn, mx, nv;
  key_stats<SC_THREADS>(key_at, Ce, sm, mn, mx, nv);
  // a direct query's row holds k ids; a chunk's candidate list k_chunk (>= min(k, C))
  const uint32_t lim = direct ? (uint32_t)k : (uint32_t)k_chunk;
  const uint32_t need = nv < lim ? nv : lim;
  const uint32_t r0 = (direct || c == nc_q - 1) ? 0u : rank_for_bound(k, nc_q);
  SelOut sel;
  if (need == nv && r0 == 0) sel = SelOut{mn, 0xFFFFFFFFu, 0u};   // every valid key
  else sel = select_threshold<SC_THREADS>(key_at, Ce, need, mn, mx, r0, sm, nc_q > 32);
  auto entry_of = [&](int i) -> int {
    if (POOL) {
      const int vj = base + i;
      return cq[vj / hsi_s] * hsi_s + vj % hsi_s;
    }
    return base + i;
  };
  // without a partial tie and with at most NBINS / 4 chosen keys the positions can
  // be staged in the histogram
  constexpr int SEG = NBINS / (SC_THREADS / 64);
  const bool compact = sel.eq_take == 0xFFFFFFFFu && need <= (uint32_t)SEG;
  if (direct) {
    int32_t* out = topk + (size_t)bt * k;
    const uint32_t cnt =
        compact ? emit_compact<SC_THREADS>(keys, Ce, sel.thresh, sm.hist, SEG, sm,
                                           [&](uint32_t slot, uint32_t, uint32_t i) { out[slot] = entry_of((int)i); })
                : emit_ordered<SC_THREADS>(key_at, Ce, sel, sm, [&](int i, uint32_t slot) { out[slot] = entry_of(i); });
    for (int i = (int)cnt + threadIdx.x; i < k; i += SC_THREADS) out[i] = -1;
  } else {
    const size_t obase = ((size_t)bt * n_chunks + c) * k_chunk;
    if (threadIdx.x == 0) chunk_lb[(size_t)bt * n_chunks + c] = sel.lb;
    const uint32_t cnt =
        compact ? emit_compact<SC_THREADS>(keys, Ce, sel.thresh, sm.hist, SEG, sm,
                                           [&](uint32_t slot, uint32_t key, uint32_t i) {
                                             cand_key[obase + slot] = key;
                                             cand_idx[obase + slot] = entry_of((int)i);
                                           })
                : emit_ordered<SC_THREADS>(key_at, Ce, sel, sm, [&](int i, uint32_t slot) {
                    cand_key[obase + slot] = keys[i];
                    cand_idx[obase + slot] = entry_of(i);
                  });
    for (int i = (int)cnt + threadIdx.x; i < k_chunk; i += SC_THREADS) {
      cand_key[obase + i] = 0u;
      cand_idx[obase + i] = -1;
    }
  }
}

// ---------------------------------------------------------------------------
// Pre-filter before the merge (queries with many chunks): one workgroup per
// (query, group of pf_cpg chunks) drops the group's candidates below the merge
// bound (the smallest rank-r0 key over the query's full chunks, which no chosen
// key is below) and compacts the rest, in order, to the front of the group's
// own candidate range, with their count in seg_cnt.  The merge then stages only
// the survivors instead of streaming every chunk's list through one workgroup.
constexpr int PF_THREADS = 256;
constexpr int PF_PER = 16;                          // candidates per thread
constexpr int PF_ITEMS = PF_THREADS * PF_PER;       // candidates per group at most
constexpr long long PF_MIN_ITEMS = 32768;           // pre-filter above this many candidates per query
constexpr int PF_MAX_GROUPS = 512;                  // groups per query at most (offsets in the merge's LDS)

template <bool POOL>
__global__ __launch_bounds__(PF_THREADS) void topk_prefilter(uint32_t* __restrict__ cand_key,
                                                             int32_t* __restrict__ cand_idx,
                                                             const uint32_t* __restrict__ chunk_lb,
                                                             const int32_t* __restrict__ q_pos,
                                                             uint32_t* __restrict__ seg_cnt, int T_len, int n_entries,
                                                             int m, int C, int k_chunk, int n_chunks, int cpg,
                                                             int n_groups, int single_direct) {
  __shared__ uint32_t s_bound;
  __shared__ uint32_t wsum[PF_THREADS / 64];
  const int g = blockIdx.x, t = blockIdx.y, b = blockIdx.z;
  const int bt = b * T_len + t;
  const int n_t = visible(q_pos, bt, m, n_entries);
  const int nc = POOL ? n_chunks : (n_t + C - 1) / C;
  const int c0 = g * cpg, c1 = min(nc, c0 + cpg);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // no chunk of this query here, or a single chunk that wrote the query's top-k
  // itself (the merge reads every group's count, and skips such a query)
  if (c0 >= c1 || (single_direct && nc <= 1)) {
    if (threadIdx.x == 0) seg_cnt[(size_t)bt * n_groups + g] = 0u;
    return;
  }
  // the merge bound, as the merge computes it
  uint32_t tl = 0xFFFFFFFFu;
  for (int cc = threadIdx.x; cc < nc - 1; cc += PF_THREADS) tl = min(tl, chunk_lb[(size_t)bt * n_chunks + cc]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) tl = min(tl, (uint32_t)__shfl_xor((int)tl, off, 64));
  if (threadIdx.x == 0) s_bound = 0xFFFFFFFFu;
  __syncthreads();
  if (lane == 0) atomicMin(&s_bound, tl);
  __syncthreads();
  const uint32_t bound = nc > 1 ? s_bound : 0u;
  // thread i holds candidates [PF_PER i, PF_PER i + PF_PER) of the group (k_chunk % 4 == 0)
  const size_t base = ((size_t)bt * n_chunks + c0) * k_chunk;
  const int n_items = (c1 - c0) * k_chunk;
  const int i0 = threadIdx.x * PF_PER;
  uint4 kv[PF_PER / 4];
  int4 iv[PF_PER / 4];
#pragma unroll
  for (int j = 0; j < PF_PER / 4; ++j) {
    const bool in = i0 + 4 * j < n_items;
    kv[j] = in ? *reinterpret_cast<const uint4*>(cand_key + base + i0 + 4 * j) : make_uint4(0, 0, 0, 0);
    iv[j] = in ? *reinterpret_cast<const int4*>(cand_idx + base + i0 + 4 * j) : make_int4(-1, -1, -1, -1);
  }
  uint32_t own = 0;
#pragma unroll
  for (int j = 0; j < PF_PER / 4; ++j) {
    own += (kv[j].x != 0u && kv[j].x >= bound) + (kv[j].y != 0u && kv[j].y >= bound) +
           (kv[j].z != 0u && kv[j].z >= bound) + (kv[j].w != 0u && kv[j].w >= bound);
  }
  // exclusive prefix of the per-thread counts (thread order is candidate order)
  uint32_t x = own;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t u = __shfl_up(x, off, 64);
    if (lane >= off) x += u;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();   // also: every read of the group's range is done before any write below
  uint32_t slot = x - own, total = 0;
#pragma unroll
  for (int w = 0; w < PF_THREADS / 64; ++w) {
    slot += w < wave ? wsum[w] : 0u;
    total += wsum[w];
  }
#pragma unroll
  for (int j = 0; j < PF_PER / 4; ++j) {
    const uint32_t kk[4] = {kv[j].x, kv[j].y, kv[j].z, kv[j].w};
    const int32_t ii[4] = {iv[j].x, iv[j].y, iv[j].z, iv[j].w};
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (kk[u] != 0u && kk[u] >= bound) {
        cand_key[base + slot] = kk[u];
        cand_idx[base + slot] = ii[u];
        ++slot;
      }
  }
  if (threadIdx.x == 0) seg_cnt[(size_t)bt * n_groups + g] = total;
}

constexpr int MG_THREADS = 512;
constexpr int MG_TILE = 4096;    // candidate keys read into LDS per round (LDS-tile form)
constexpr int MG_CAP = 4096;     // staged candidates kept in LDS (LDS-tile form)
constexpr int MG_CAP_R = 8192;   // staged candidates kept in LDS (register form)

// One workgroup per query: candidates of all chunks at or above the bound are
// staged in LDS in entry order, then the same radix select picks the k best and
// emits their ids ascending.  With HSI BUILD a second workgroup per query picks
// the n_b best blocks (newest forced) the same way from the block maxima, staged
// in the whole 80 KB candidate area (up to 20480 blocks).
template <bool POOL, bool BUILD>
__global__ __launch_bounds__(MG_THREADS) void topk_merge(const uint32_t* __restrict__ cand_key,
                                                         const int32_t* __restrict__ cand_idx,
                                                         const uint32_t* __restrict__ chunk_lb,
                                                         const uint32_t* __restrict__ blkmax,
                                                         const int32_t* __restrict__ q_pos, int32_t* __restrict__ topk,
                                                         int32_t* __restrict__ cands_out, int T_len, int n_entries,
                                                         int m, int k, int C, int k_chunk, int n_chunks, int hsi_s,
                                                         int hsi_nb, int nblk_max, const uint32_t* __restrict__ seg_cnt,
                                                         int pf_cpg, int pf_groups) {
  __shared__ SelSmem<MG_THREADS> sel;
  // one 80 KB area: [tile | staged keys | staged candidate positions]; the block
  // selection of HSI BUILD (a workgroup of its own) uses all of it
  constexpr int BLK_CAP = MG_TILE + 2 * MG_CAP_R;
  __shared__ __attribute__((aligned(16))) uint32_t area[BLK_CAP];
  uint32_t* tile = area;
  uint32_t* skey = area + MG_TILE;
  int32_t* sidx = reinterpret_cast<int32_t*>(area + MG_TILE + MG_CAP_R);   // candidate positions
  __shared__ uint32_t s_bound;
  const int t = blockIdx.x, b = blockIdx.y;
  const int bt = b * T_len + t;
  const int n_t = visible(q_pos, bt, m, n_entries);
  const int nc = POOL ? n_chunks : (n_t + C - 1) / C;

  // with HSI BUILD, blockIdx.z == 0 merges the candidates and blockIdx.z == 1
  // selects the blocks, side by side
  if ((BUILD || nc > 1) && blockIdx.z == 0) {
    const int n_items = nc * k_chunk;
    const uint32_t* kb = cand_key + (size_t)bt * n_chunks * k_chunk;
    const int32_t* ib = cand_idx + (size_t)bt * n_chunks * k_chunk;
    int32_t* out = topk + (size_t)bt * k;
    // bound: smallest rank-r0 key over the full chunks (0 = none)
    uint32_t bound = 0;
    if (nc > 1) {
      uint32_t tl = 0xFFFFFFFFu;
      for (int cc = threadIdx.x; cc < nc - 1; cc += MG_THREADS) tl = min(tl, chunk_lb[(size_t)bt * n_chunks + cc]);
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) tl = min(tl, (uint32_t)__shfl_xor((int)tl, off, 64));
      if (threadIdx.x == 0) s_bound = 0xFFFFFFFFu;
      __syncthreads();
      if ((threadIdx.x & 63) == 0) atomicMin(&s_bound, tl);
      __syncthreads();
      bound = s_bound;
    }
    // stage candidates >= bound in entry order
    uint32_t staged = 0;
    const uint32_t cap = (k_chunk & 3) == 0 ? (uint32_t)MG_CAP_R : (uint32_t)MG_CAP;
    const SelOut keep{bound, 0xFFFFFFFFu, 0u};
    constexpr int MG_NW = MG_THREADS / 64;
    constexpr int MG_REG = 8;   // uint4 loads per lane: 32 candidates
    constexpr int MG_ROUND = MG_THREADS * 4 * MG_REG;   // 16384 candidates per register round
    const bool pf = pf_cpg > 0;   // pre-filtered: group g's survivors at the front of its range
    const bool in_regs = !pf && (k_chunk & 3) == 0;
    const int seg_len = pf_cpg * k_chunk;   // candidate range of one pre-filter group
    uint32_t* seg_off = tile;               // group offsets among the survivors (pre-filtered)
    const int ng = pf ? (nc + pf_cpg - 1) / pf_cpg : 0;
    if (pf) {
      // survivors per group -> offsets (ng <= MG_TILE); a wave copies group g's
      // survivors for g = wave, wave + 8, ... (entry order: group-major)
      const uint32_t* cnt_row = seg_cnt + (size_t)bt * pf_groups;
      for (int g = threadIdx.x; g < ng; g += MG_THREADS) seg_off[g] = cnt_row[g];
      __syncthreads();
      if (threadIdx.x == 0) {
        uint32_t acc = 0;
        for (int g = 0; g < ng; ++g) {
          const uint32_t c = seg_off[g];
          seg_off[g] = acc;
          acc += c;
        }
        s_bound = acc;
      }
      __syncthreads();
      staged = s_bound;
      if (staged <= cap) {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        for (int g = wave; g < ng; g += MG_NW) {
          const uint32_t o = seg_off[g];
          const uint32_t n = (g + 1 < ng ? seg_off[g + 1] : staged) - o;
          for (uint32_t i = lane; i < n; i += 64) {
            skey[o + i] = kb[(size_t)g * seg_len + i];
            sidx[o + i] = g * seg_len + (int)i;
          }
        }
      }
      __syncthreads();
    }
    if (in_regs && n_items > 0) {
      // rounds of up to 16384 candidates at once: wave w holds items
      // [w * 2048, w * 2048 + 2048) of the round, lane l the 4 consecutive items
      // 4 * (64 j + l) .. + 3 of step j, so entry order is (j, lane, u); a count
      // pass and one exchange of the per-wave counts give each wave its first
      // slot, a second pass over the registers writes the kept candidates (key and
      // candidate position; ids are read for the chosen k only) in order.  The keys
      // of the next round load while one is processed, through a buffer resource
      // over the query's candidates, so reads past them return 0 without a memory
      // access and every load is unconditional.
      const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
      const uint64_t lt = (1ull << lane) - 1ull;
      const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)kb, (short)0, n_items * 4, 0x00020000);
      auto kept = [&](uint32_t kk) { return kk != 0u && kk >= bound; };
      auto load_keys = [&](int r0, uint4* dst) {
#pragma unroll
        for (int j = 0; j < MG_REG; ++j) {
          const int i = r0 + wave * (256 * MG_REG) + 256 * j + 4 * lane;
          const auto v = __builtin_amdgcn_raw_buffer_load_b128(rk, i < n_items ? i * 4 : (int)0x80000000, 0, 0);
          dst[j] = make_uint4(v[0], v[1], v[2], v[3]);
        }
      };
      uint4 kn[MG_REG];
      load_keys(0, kn);
      for (int r0 = 0; r0 < n_items; r0 += MG_ROUND) {
        uint4 kv[MG_REG];
#pragma unroll
        for (int j = 0; j < MG_REG; ++j) kv[j] = kn[j];
        __builtin_amdgcn_sched_barrier(0);
        load_keys(r0 + MG_ROUND, kn);
        __builtin_amdgcn_sched_barrier(0);
        uint32_t wc = 0;
#pragma unroll
        for (int j = 0; j < MG_REG; ++j)
          wc += __popcll(__ballot(kept(kv[j].x))) + __popcll(__ballot(kept(kv[j].y))) +
                __popcll(__ballot(kept(kv[j].z))) + __popcll(__ballot(kept(kv[j].w)));
        if (lane == 0) sel.red[0][wave] = wc;
        __syncthreads();
        uint32_t slot = staged, total = 0;
#pragma unroll
        for (int w = 0; w < MG_NW; ++w) {
          const uint32_t c = sel.red[0][w];
          slot += w < wave ? c : 0u;
          total += c;
        }
        if (staged + total <= cap) {
#pragma unroll
          for (int j = 0; j < MG_REG; ++j) {
            const uint32_t kk[4] = {kv[j].x, kv[j].y, kv[j].z, kv[j].w};
            const int i0 = r0 + wave * (256 * MG_REG) + 256 * j + 4 * lane;
            bool s[4];
            uint32_t before = 0, tot = 0;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              s[u] = kept(kk[u]);
              const uint64_t msk = __ballot(s[u]);
              before += __popcll(msk & lt);
              tot += __popcll(msk);
            }
            uint32_t sl = slot + before;
#pragma unroll
            for (int u = 0; u < 4; ++u)
              if (s[u]) {
                skey[sl] = kk[u];
                sidx[sl] = i0 + u;
                ++sl;
              }
            slot += tot;
          }
        }
        staged += total;
        __syncthreads();
      }
    }
    for (int r = 0; r < (in_regs || pf ? 0 : n_items); r += MG_TILE) {
      const int len = min(MG_TILE, n_items - r);
      for (int i0 = 0; i0 < len; i0 += 4 * MG_THREADS) {   // all loads of a round in flight together
        uint32_t kk[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = i0 + u * MG_THREADS + threadIdx.x;
          kk[u] = i < len ? kb[r + i] : 0u;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = i0 + u * MG_THREADS + threadIdx.x;
          if (i < len) tile[i] = kk[u];
        }
      }
      __syncthreads();
      const uint32_t base_slot = staged;
      staged += emit_ordered<MG_THREADS>([&](int i) -> uint32_t { return tile[i]; }, len, keep, sel,
                                         [&](int i, uint32_t slot) {
                                           slot += base_slot;
                                           if (slot < (uint32_t)MG_CAP) {
                                             skey[slot] = tile[i];
                                             sidx[slot] = r + i;
                                           }
                                         });
      __syncthreads();
    }
    uint32_t cnt;
    if (staged <= cap) {
      auto key_at = [&](int i) -> uint32_t { return skey[i]; };
      uint32_t mn, mx, nv;
      key_stats<MG_THREADS>(key_at, (int)staged, sel, mn, mx, nv);
      const uint32_t need = nv < (uint32_t)k ? nv : (uint32_t)k;
      const SelOut s = need == nv ? SelOut{mn, 0xFFFFFFFFu, 0u}
                                  : select_threshold<MG_THREADS>(key_at, (int)staged, need, mn, mx, 0u, sel);
      // without a partial tie the chosen positions are staged in tile[] (8 waves x 512)
      if (s.eq_take == 0xFFFFFFFFu && need <= (uint32_t)(MG_TILE / (MG_THREADS / 64)))
        cnt = emit_compact<MG_THREADS>(skey, (int)staged, s.thresh, tile, MG_TILE / (MG_THREADS / 64), sel,
                                       [&](uint32_t slot, uint32_t, uint32_t i) { out[slot] = ib[sidx[i]]; });
      else
        cnt = emit_ordered<MG_THREADS>(key_at, (int)staged, s, sel,
                                       [&](int i, uint32_t slot) { out[slot] = ib[sidx[i]]; });
    } else if (pf) {
      // more survivors than LDS holds: select straight from the groups' ranges
      auto key_at = [&](int i) -> uint32_t {
        const int g = i / seg_len, r = i - g * seg_len;
        const uint32_t o = seg_off[g];
        const uint32_t n = (g + 1 < ng ? seg_off[g + 1] : staged) - o;
        return (uint32_t)r < n ? kb[i] : 0u;
      };
      uint32_t mn, mx, nv;
      key_stats<MG_THREADS>(key_at, n_items, sel, mn, mx, nv);
      const uint32_t need = nv < (uint32_t)k ? nv : (uint32_t)k;
      const SelOut s = need == nv ? SelOut{mn, 0xFFFFFFFFu, 0u}
                                  : select_threshold<MG_THREADS>(key_at, n_items, need, mn, mx, 0u, sel);
      cnt = emit_ordered<MG_THREADS>(key_at, n_items, s, sel, [&](int i, uint32_t slot) { out[slot] = ib[i]; });
    } else {
      // more candidates than LDS holds: select straight from the workspace
      auto key_at = [&](int i) -> uint32_t { const uint32_t kk = kb[i]; return kk >= bound ? kk : 0u; };
      uint32_t mn, mx, nv;
      key_stats<MG_THREADS>(key_at, n_items, sel, mn, mx, nv);
      const uint32_t need = nv < (uint32_t)k ? nv : (uint32_t)k;
      const SelOut s = need == nv ? SelOut{mn, 0xFFFFFFFFu, 0u}
                                  : select_threshold<MG_THREADS>(key_at, n_items, need, mn, mx, 0u, sel);
      cnt = emit_ordered<MG_THREADS>(key_at, n_items, s, sel, [&](int i, uint32_t slot) { out[slot] = ib[i]; });
    }
    for (int i = (int)cnt + threadIdx.x; i < k; i += MG_THREADS) out[i] = -1;
  }
  if (BUILD && blockIdx.z == 1) {
    const int nblk = (n_t + hsi_s - 1) / hsi_s;
    const uint32_t* bm = blkmax + (size_t)bt * nblk_max;
    int32_t* out = cands_out + (size_t)bt * hsi_nb;
    auto bkey = [&](int i) -> uint32_t { return (i == nblk - 1) ? 0xFFFFFFFFu : bm[i]; };  // newest block forced in
    uint32_t cnt;
    if (nblk <= BLK_CAP) {
      for (int i0 = 0; i0 < nblk; i0 += 4 * MG_THREADS) {   // 4 loads per thread in flight
        uint32_t v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = i0 + u * MG_THREADS + threadIdx.x;
          v[u] = i < nblk ? bkey(i) : 0u;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = i0 + u * MG_THREADS + threadIdx.x;
          if (i < nblk) area[i] = v[u];
        }
      }
      __syncthreads();
      auto key_at = [&](int i) -> uint32_t { return area[i]; };
      uint32_t mn, mx, nv;
      key_stats<MG_THREADS>(key_at, nblk, sel, mn, mx, nv);
      const uint32_t need = nv < (uint32_t)hsi_nb ? nv : (uint32_t)hsi_nb;
      const SelOut s = need == nv ? SelOut{mn, 0xFFFFFFFFu, 0u}
                                  : select_threshold<MG_THREADS>(key_at, nblk, need, mn, mx, 0u, sel);
      cnt = emit_ordered<MG_THREADS>(key_at, nblk, s, sel, [&](int i, uint32_t slot) { out[slot] = i; });
    } else {
      uint32_t mn, mx, nv;
      key_stats<MG_THREADS>(bkey, nblk, sel, mn, mx, nv);
      const uint32_t need = nv < (uint32_t)hsi_nb ? nv : (uint32_t)hsi_nb;
      const SelOut s = need == nv ? SelOut{mn, 0xFFFFFFFFu, 0u}
                                  : select_threshold<MG_THREADS>(bkey, nblk, need, mn, mx, 0u, sel);
      cnt = emit_ordered<MG_THREADS>(bkey, nblk, s, sel, [&](int i, uint32_t slot) { out[slot] = i; });
    }
    for (int i = (int)cnt + threadIdx.x; i < hsi_nb; i += MG_THREADS) out[i] = -1;
  }
}

// ---------------------------------------------------------------------------
// Streaming path (no HSI): one workgroup of 8 waves per (query, part of up to
// ST_MAXR consecutive entries).  Scores are filtered as they are computed: an
// entry is staged in LDS (key and id) only if its key is at least theta, the k-th
// best key among the entries the workgroup had scored at its last cutback.  Every
// entry it drops scores below the query's k-th best, so it cannot be chosen.  The
// staged count is checked every ST_CHECK rounds; when the next ST_CHECK rounds
// could overflow the staging (and once after the first 4096 entries, to set
// theta), the staged set is cut back to its k best, which raises theta; so the block-wide
// selection runs a few times per part instead of once per 4096 entries, and the
// scan keeps the loads streaming.  The part's k best leave in id order: as the
// query's top-k when one part covers its visible entries, else as a candidate
// list for topk_merge with a lower bound of the part's rank-r0 key.
constexpr int ST_THREADS = 512;    // two workgroups per CU (bf16; see the launch bounds)
constexpr int ST_NW = ST_THREADS / 64;
constexpr int ST_ROUND = ST_NW * 64;   // entries scored per round: one super-tile per wave
constexpr int ST_CAP = 4096;           // staged candidates
constexpr int ST_MAXR = 65536;         // entries per part at most (an id bitmap of 2048 words)
constexpr int ST_WPT = ST_MAXR / 32 / ST_THREADS;   // bitmap words per thread
constexpr int ST_FIRST = 4096;         // entries scored before theta is first set
constexpr int ST_CHECK = 4;            // rounds between checks of the staged count
static_assert(ST_CAP - ST_CHECK * ST_ROUND >= CSA2_MAX_TOPK, "a cutback must leave room for ST_CHECK rounds");

struct StreamSmem {
  SelSmem<ST_THREADS> sel;
  uint32_t key[ST_CAP];
  int32_t id[ST_CAP];
  uint32_t bits[ST_MAXR / 32];
  uint32_t wpre[ST_MAXR / 32];
  uint32_t tkey[CSA2_MAX_TOPK];
  int32_t tid[CSA2_MAX_TOPK];
  uint32_t cnt, theta;
};

// The staging one selection works on: keys and ids of the staged candidates,
// the id bitmap and its word prefix counts, and the block-wide selection memory.
struct StView {
  SelSmem<ST_THREADS>* sel;
  uint32_t* key;
  int32_t* id;
  uint32_t* bits;
  uint32_t* wpre;
};

// Exclusive prefix counts of the set bits of words [0, nw) of S.bits into S.wpre
// (WPT bitmap words per thread).
template <int WPT>
__device__ __forceinline__ void st_bit_prefix(const StView& S, int nw) {
  uint32_t pc[WPT], tot = 0;
#pragma unroll
  for (int j = 0; j < WPT; ++j) {
    const int wi = threadIdx.x * WPT + j;
    pc[j] = wi < nw ? (uint32_t)__popc(S.bits[wi]) : 0u;
    tot += pc[j];
  }
  uint32_t total;
  uint32_t pre = block_prefix_excl<ST_THREADS>(tot, *S.sel, total);
#pragma unroll
  for (int j = 0; j < WPT; ++j) {
    const int wi = threadIdx.x * WPT + j;
    if (wi < nw) S.wpre[wi] = pre;
    pre += pc[j];
  }
  __syncthreads();
}

// Rank of id offset r among the set bits of S.bits (valid after st_bit_prefix).
__device__ __forceinline__ uint32_t st_rank(const StView& S, int r) {
  return S.wpre[r >> 5] + (uint32_t)__popc(S.bits[r >> 5] & ((1u << (r & 31)) - 1u));
}

// Chooses the `need` best of the c staged candidates (ties to the smaller id; ids
// lie in [base, base + range), range <= 32 WPT ST_THREADS) and calls put(rank,
// key, id) for each, rank being its position in id order; returns how many were
// chosen.  thresh receives a value at or below the smallest chosen key; with
// r0 != 0, lb a lower bound of the rank-r0 key.
template <int WPT, typename Put>
__device__ uint32_t st_choose(const StView& S, int c, uint32_t need, uint32_t r0, int base, int range,
                              uint32_t& thresh, uint32_t& lb, Put put) {
  auto key_at = [&](int i) -> uint32_t { return S.key[i]; };
  uint32_t mn, mx, nv;
  key_stats<ST_THREADS>(key_at, c, *S.sel, mn, mx, nv);
  if (need > nv) need = nv;
  const SelOut sel = (need == nv && r0 == 0) ? SelOut{mn, 0xFFFFFFFFu, 0u}
                                             : select_threshold<ST_THREADS>(key_at, c, need, mn, mx, r0, *S.sel, true);
  thresh = sel.thresh;
  lb = sel.lb;
  const int nw = (range + 31) >> 5;
  for (int i = threadIdx.x; i < nw; i += ST_THREADS) S.bits[i] = 0u;
  __syncthreads();
  if (sel.eq_take != 0xFFFFFFFFu) {
    // a partial tie at the threshold: keep the eq_take smallest ids among the tied
    for (int i = threadIdx.x; i < c; i += ST_THREADS)
      if (S.key[i] == sel.thresh) {
        const int r = S.id[i] - base;
        atomicOr(&S.bits[r >> 5], 1u << (r & 31));
      }
    __syncthreads();
    st_bit_prefix<WPT>(S, nw);
    for (int i = threadIdx.x; i < c; i += ST_THREADS)
      if (S.key[i] == sel.thresh && st_rank(S, S.id[i] - base) >= sel.eq_take) S.key[i] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < nw; i += ST_THREADS) S.bits[i] = 0u;
    __syncthreads();
  }
  for (int i = threadIdx.x; i < c; i += ST_THREADS) {
    const uint32_t kk = S.key[i];
    if (kk != 0u && kk >= sel.thresh) {
      const int r = S.id[i] - base;
      atomicOr(&S.bits[r >> 5], 1u << (r & 31));
    }
  }
  __syncthreads();
  st_bit_prefix<WPT>(S, nw);
  for (int i = threadIdx.x; i < c; i += ST_THREADS) {
    const uint32_t kk = S.key[i];
    if (kk != 0u && kk >= sel.thresh) put(st_rank(S, S.id[i] - base), kk, S.id[i]);
  }
  __syncthreads();
  return need;
}

// bf16: at most 128 VGPRs, so that two workgroups (16 waves) share a CU; the
// compiler's own choice (145) left room for one, and the scan ran 27% slower
template <typename T, int SF>
__global__ __launch_bounds__(ST_THREADS, sizeof(T) == 2 ? 4 : 2) void score_stream(
    const T* __restrict__ q_idx, const float* __restrict__ w, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const int32_t* __restrict__ q_pos, uint32_t* __restrict__ cand_key,
    int32_t* __restrict__ cand_idx, uint32_t* __restrict__ chunk_lb, int32_t* __restrict__ topk,
    float* __restrict__ scores_out, int T_len, int H_I, int N_cap, int n_entries, int m, int R, int n_parts, int k,
    int k_chunk) {
  __shared__ StreamSmem S;
  const StView V{&S.sel, S.key, S.id, S.bits, S.wpre};
  const int part = blockIdx.x, t = blockIdx.y, b = blockIdx.z;
  const int bt = b * T_len + t;
  const int n_t = visible(q_pos, bt, m, n_entries);
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int base = part * R;
  const int np_q = (n_t + R - 1) / R;
  const bool direct = np_q <= 1;   // one part covers the query: its top-k is written here
  if (base >= n_t) {
    if (direct && part == 0)   // nothing visible
      for (int i = threadIdx.x; i < k; i += ST_THREADS) topk[(size_t)bt * k + i] = -1;
    return;                    // a part beyond the visible range: never read by the merge
  }
  const int n_here = min(R, n_t - base);
  const int n_rounds = (n_here + ST_ROUND - 1) / ST_ROUND;

  typename ScoreQ<T>::type qf[2][4];
  float wv[2][4];
  load_qfrags<T>(q_idx + (size_t)bt * H_I * 128, w + (size_t)bt * H_I, H_I, lr, lg, qf, wv);
  const uint8_t* cb = codes + (size_t)b * N_cap * 64;
  const uint8_t* sb = scales + (size_t)b * N_cap * 4;
  if (threadIdx.x == 0) {
    S.cnt = 0u;
    S.theta = 0u;
  }
  __syncthreads();

  // Round i: wave w scores super-tile ST_NW i + w of the part.  Loads as in
  // score_chunk: through buffer resources (reads past the N_cap entries, and the
  // dead loads past the last round, return 0 with no memory access), else plain
  // loads of entry 0 for the dead ones.
  const bool use_buf = N_cap <= (1 << 25);
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)cb, (short)0, use_buf ? N_cap * 64 : 0, 0x00020000);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)sb, (short)0, use_buf ? N_cap * 4 : 0, 0x00020000);
  auto load_buf = [&](int i, StLoad& L) {
    const bool live = i < n_rounds;
    const int e = base + (i * ST_NW + wave) * 64 + lr;
    const int oc = live ? e * 64 + 16 * lg : (int)0x80000000;
    const int os = live ? e * 4 : (int)0x80000000;
#pragma unroll
    for (int tt = 0; tt < SPT; ++tt) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rc, oc + tt * 1024, 0, 0);
      L.c[tt] = make_uint4(v[0], v[1], v[2], v[3]);
      L.s[tt] = __builtin_amdgcn_raw_buffer_load_b32(rs, os + tt * 64, 0, 0);
    }
  };
  auto load_glob = [&](int i, StLoad& L) {
    const bool live = i < n_rounds;
#pragma unroll
    for (int tt = 0; tt < SPT; ++tt) {
      const int e = base + (i * ST_NW + wave) * 64 + tt * 16 + lr;
      const int ent = live && e < n_t ? e : 0;
      L.c[tt] = *reinterpret_cast<const uint4*>(cb + (size_t)ent * 64 + 16 * lg);
      L.s[tt] = *reinterpret_cast<const uint32_t*>(sb + (size_t)ent * 4);
    }
  };
  const uint64_t lt = (1ull << lane) - 1ull;
  uint32_t theta = 0u;
  auto round = [&](int i, const StLoad& L) {
    const float sc = score_supertile<T, SF>(qf, wv, L, lg);
    const int j = (i * ST_NW + wave) * 64 + lane;   // position in the part
    const uint32_t kk = j < n_here ? score_key(sc) : 0u;
    if (scores_out != nullptr && j < n_here) scores_out[(size_t)bt * n_entries + base + j] = key_score(kk);
    const bool pass = kk != 0u && kk >= theta;
    const uint64_t msk = __ballot(pass);
    if (msk != 0ull) {
      uint32_t slot0 = 0u;
      if (lane == 0) slot0 = atomicAdd(&S.cnt, (uint32_t)__popcll(msk));
      slot0 = __shfl(slot0, 0, 64);
      if (pass) {
        const uint32_t sl = slot0 + (uint32_t)__popcll(msk & lt);
        S.key[sl] = kk;
        S.id[sl] = base + j;
      }
    }
    // the staged count is checked (two barriers) every ST_CHECK rounds and after the
    // last; a cutback leaves room for ST_CHECK more rounds, so the staging between
    // two checks cannot overflow
    if (i % ST_CHECK != ST_CHECK - 1 && i + 1 < n_rounds) return;
    __syncthreads();
    const uint32_t c = S.cnt;
    __syncthreads();   // every thread has read the count before the next round adds to it
    const int seen = min(n_here, (i + 1) * ST_ROUND);
    if (i + 1 < n_rounds && (c > (uint32_t)(ST_CAP - ST_CHECK * ST_ROUND) ||
                             (theta == 0u && seen >= ST_FIRST && c >= (uint32_t)k))) {
      uint32_t th, lb_unused;
      const uint32_t got = st_choose<ST_WPT>(V, (int)c, (uint32_t)k, 0u, base, n_here, th, lb_unused,
                                     [&](uint32_t r, uint32_t key, int32_t id) {
                                       S.tkey[r] = key;
                                       S.tid[r] = id;
                                     });
      for (uint32_t q = threadIdx.x; q < got; q += ST_THREADS) {
        S.key[q] = S.tkey[q];
        S.id[q] = S.tid[q];
      }
      if (threadIdx.x == 0) {
        S.cnt = got;
        S.theta = got >= (uint32_t)k ? th : 0u;
      }
      __syncthreads();
    }
    theta = S.theta;
  };
  auto scan = [&](auto load_st) {
    StLoad L0, L1;
    load_st(0, L0);
    for (int i = 0; i < n_rounds; i += 2) {
      load_st(i + 1, L1);
      __builtin_amdgcn_sched_barrier(0);
      round(i, L0);
      load_st(i + 2, L0);
      __builtin_amdgcn_sched_barrier(0);
      if (i + 1 < n_rounds) round(i + 1, L1);
    }
  };
  if (use_buf) scan(load_buf);
  else scan(load_glob);

  // ---- the part's k best in id order
  const int c = (int)S.cnt;
  const uint32_t r0 = (direct || part == np_q - 1) ? 0u : rank_for_bound(k, np_q);
  uint32_t th, lb;
  if (direct) {
    int32_t* out = topk + (size_t)bt * k;
    const uint32_t got = st_choose<ST_WPT>(V, c, (uint32_t)k, 0u, base, n_here, th, lb,
                                   [&](uint32_t r, uint32_t, int32_t id) { out[r] = id; });
    for (int i = (int)got + threadIdx.x; i < k; i += ST_THREADS) out[i] = -1;
  } else {
    const size_t obase = ((size_t)bt * n_parts + part) * k_chunk;
    const uint32_t got = st_choose<ST_WPT>(V, c, (uint32_t)k, r0, base, n_here, th, lb,
                                   [&](uint32_t r, uint32_t key, int32_t id) {
                                     cand_key[obase + r] = key;
                                     cand_idx[obase + r] = id;
                                   });
    if (threadIdx.x == 0) chunk_lb[(size_t)bt * n_parts + part] = lb;
    for (int i = (int)got + threadIdx.x; i < k_chunk; i += ST_THREADS) {
      cand_key[obase + i] = 0u;
      cand_idx[obase + i] = -1;
    }
  }
}

// ---------------------------------------------------------------------------
// Two-phase path for many queries over one cache (prefill, bf16, flat selection):
// score_qtile scores QT = 4 consecutive queries per workgroup, so each staged and
// dequantised K tile feeds 4 queries x 2 head tiles = 8 MFMAs; the key of every
// visible (query, entry) pair goes to a key matrix in the workspace, and
// select_rows then picks each query's top-k from its row.
//
// The FP4 codes are dequantised to fp16 with the block scale applied before the
// MFMA (exact, as in score_chunk), so one MFMA chain covers all 4 blocks of the
// 128 dims; the queries are moved into fp16 range per head as there.
constexpr int QT = 4;                 // queries per workgroup
constexpr int QT_CE = 4096;           // entries per workgroup (64 super-tiles of 64)
constexpr int SEL_MAX = 8192;         // keys per query row held in registers by select_rows


template <int SF>
__global__ __launch_bounds__(SC_THREADS, 2) void score_qtile_bf16(
    const bf16* __restrict__ q_idx, const float* __restrict__ w, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const int32_t* __restrict__ q_pos, uint32_t* __restrict__ keys,
    int T_len, int H_I, int N_cap, int n_entries, int m, int n_scan) {
  __shared__ __attribute__((aligned(16))) unsigned char ring0[4 * ST_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char ring1[4 * ST_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char ring2[4 * ST_BYTES];
  // query tiles in reverse order: the latest queries (most visible entries) start
  // first and the short ones fill the tail
  const int c = blockIdx.x, t0 = (int)(gridDim.y - 1 - blockIdx.y) * QT, b = blockIdx.z;
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int n_q[QT];
  int n_max = 0;
#pragma unroll
  for (int qi = 0; qi < QT; ++qi) {
    n_q[qi] = t0 + qi < T_len ? visible(q_pos, b * T_len + t0 + qi, m, n_entries) : 0;
    n_max = max(n_max, n_q[qi]);
  }
  const int base = c * QT_CE;
  if (base >= n_max) return;
  const int n_here = min(QT_CE, n_max - base);
  const int n_st = (n_here + 63) / 64;
  const int st_w = (n_st - wave + 3) / 4;   // super-tiles of this wave: wave, wave + 4, ...

  // k-step kb of lane group g: dims 32kb + 8g .. +7 (block kb)
  f16x8 qf[QT][2][4];
  float wv[QT][2][4];
#pragma unroll
  for (int qi = 0; qi < QT; ++qi) {
    const int bt = b * T_len + min(t0 + qi, T_len - 1);
    const bf16* qb = q_idx + (size_t)bt * H_I * 128;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int h = mt * 16 + lr;
      bf16x8 raw[4];
      float amax = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        if (h < H_I) raw[kb] = load_frag(qb + (size_t)h * 128 + kb * 32 + 8 * lg);
        else zero_frag(raw[kb]);
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf((float)raw[kb][i]));
      }
      amax = max_lane_groups(amax);
      int ex = 0;
      frexpf(amax, &ex);
      const int s = amax > 0.0f ? min(max(ex - 15, -96), 96) : 0;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 8; ++i) qf[qi][mt][kb][i] = (f16)ldexpf((float)raw[kb][i], -s);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hh = mt * 16 + 4 * lg + i;
        const int sh = __shfl(s, 4 * lg + i, 64);
        wv[qi][mt][i] = hh < H_I ? ldexpf(w[(size_t)bt * H_I + hh], sh) : 0.0f;
      }
    }
  }
  const uint8_t* cb = codes + (size_t)b * N_cap * 64;
  const uint8_t* sb = scales + (size_t)b * N_cap * 4;
  // staging as in score_chunk: one DMA per 16-entry tile (swizzled 16-B pieces) and one for the scales
  const int dma_e = lane >> 2, dma_b = ((lane & 3) - (dma_e >> 2)) & 3;
  auto issue = [&](int i, unsigned char* ring) {
    const int st = wave + 4 * i;
    unsigned char* dst = ring + wave * ST_BYTES;
#pragma unroll
    for (int tt = 0; tt < SPT; ++tt) {
      const int ent = min(base + st * 64 + tt * 16 + dma_e, n_entries - 1);
      dma16_asm(cb + (size_t)ent * 64 + 16 * dma_b, (const lds_u8*)(dst + tt * 1024));
    }
    const int ent = min(base + st * 64 + lane, n_entries - 1);
    dma4_asm(sb + (size_t)ent * 4, (const lds_u8*)(dst + SPT * 1024));
  };
  // lane group g writes the keys of query t0 + g
  static_assert(QT == 4, "one query per lane group");
  const int nq_lane = t0 + lg < T_len ? visible(q_pos, b * T_len + t0 + lg, m, n_entries) : 0;
  uint32_t* krow_lane = keys + (size_t)(b * T_len + min(t0 + lg, T_len - 1)) * n_scan;
  auto compute = [&](int i, const unsigned char* ring) {
    const int st = wave + 4 * i;
    const unsigned char* src = ring + wave * ST_BYTES;
    // the super-tile's code and scale words, read from LDS together up front
    uint32_t cwa[SPT][4], swa[SPT];
#pragma unroll
    for (int tt = 0; tt < SPT; ++tt) {
      swa[tt] = *reinterpret_cast<const uint32_t*>(src + SPT * 1024 + (tt * 16 + lr) * 4);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        cwa[tt][kb] = *reinterpret_cast<const uint32_t*>(src + tt * 1024 + ((4 * lr + ((kb + (lr >> 2)) & 3)) << 4) + 4 * lg);
    }
#pragma unroll
    for (int tt = 0; tt < SPT; ++tt) {
      const uint32_t sw = swa[tt];
      const uint32_t eref = SF ? max_byte4(sw) : 0u;
      f32x4 acc[QT][2];
#pragma unroll
      for (int qi = 0; qi < QT; ++qi) {
        acc[qi][0] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc[qi][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const uint32_t cw = cwa[tt][kb];
        float p2;
        f16x2 mm;
        split_scale<SF>((sw >> (8 * kb)) & 0xFFu, eref, p2, mm);
        const f16x8 kf = fp4x8_scaled_f16(cw, p2, mm);
#pragma unroll
        for (int qi = 0; qi < QT; ++qi) {
          acc[qi][0] = mma16h(qf[qi][0][kb], kf, acc[qi][0]);
          acc[qi][1] = mma16h(qf[qi][1][kb], kf, acc[qi][1]);
        }
      }
      if constexpr (SF != 0) {
        const float post = entry_post(eref);
#pragma unroll
        for (int qi = 0; qi < QT; ++qi) {
          acc[qi][0] *= post;
          acc[qi][1] *= post;
        }
      }
      // per query: weighted ReLU (integer max on the float bits) summed over the
      // lane's 8 heads, then the 4 queries' head sums over the lane groups at once:
      // lane group g ends up with query g's score of entry e
      float part[QT];
#pragma unroll
      for (int qi = 0; qi < QT; ++qi) {
        float pq = 0.f;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int ii = 0; ii < 4; ++ii)
            pq = fmaf(wv[qi][mt][ii], __int_as_float(max(__float_as_int(acc[qi][mt][ii]), 0)), pq);
        part[qi] = pq;
      }
      const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]), __float_as_uint(part[2]), false, false);
      const auto b2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[1]), __float_as_uint(part[3]), false, false);
      const float s02 = __uint_as_float(a[0]) + __uint_as_float(a[1]);
      const float s13 = __uint_as_float(b2[0]) + __uint_as_float(b2[1]);
      const auto cc = __builtin_amdgcn_permlane16_swap(__float_as_uint(s02), __float_as_uint(s13), false, false);
      const float sc = __uint_as_float(cc[0]) + __uint_as_float(cc[1]);
      const int e = base + st * 64 + tt * 16 + lr;
      if (e < nq_lane) krow_lane[e] = score_key(sc);
    }
  };
  if (st_w > 0) issue(0, ring0);
  if (st_w > 1) issue(1, ring1);
  // Each wave reads only the super-tiles it loaded itself, so its own wait is
  // enough: loads complete in issue order, so at most the younger stages' loads
  // outstanding (the key stores in between may be either way) means super-tile i
  // is in LDS.  The LDS-read wait at the end frees the buffer for the next DMA.
  auto step = [&](int i, const unsigned char* cur, unsigned char* nxt) {
    if (i + 2 < st_w) {
      issue(i + 2, nxt);
      WAIT_VMCNT(2 * (SPT + 1));
    } else if (i + 1 < st_w) {
      WAIT_VMCNT(SPT + 1);
    } else {
      WAIT_VMCNT(0);
    }
    COMPILER_FENCE();
    compute(i, cur);
    WAIT_LGKM0();
    COMPILER_FENCE();
  };
  for (int i = 0; i < st_w; i += 3) {
    step(i, ring0, ring2);
    if (i + 1 < st_w) step(i + 1, ring1, ring0);
    if (i + 2 < st_w) step(i + 2, ring2, ring1);
  }
}

// One wave per query (4 per workgroup, no block-wide barriers): lane l holds the
// keys of positions 64j + l in registers (coalesced row reads).
//  1. One histogram pass over score values: bin = floor((v - vmin) * 255.99 /
//     (vmax - vmin)) is monotone in the key, so the boundary bin (where the count
//     of better keys reaches k) holds a contiguous key range.
//  2. The keys of that bin are compacted into the wave's LDS list and split
//     exactly by radix passes over their key range (8-bit digits; a pass stops once
//     the count at the boundary bin is exact or the bin holds a single value).
//     When more keys share the bin than the list holds, the passes run over the
//     registers instead.
//  3. Emission: ballots give, for each register column j, the 64-bit masks of
//     chosen keys among positions 64j..64j+63; lane j keeps column j's masks, so
//     after the loop each lane owns 64 consecutive positions and writes its ids
//     in order after a wave prefix sum.  Ties at the threshold go to the smaller
//     position.
constexpr int SW_BINS = 256;
constexpr int SW_CAP = 256;   // boundary-bin keys held in the wave's LDS list

__device__ __forceinline__ uint32_t wave_excl_prefix(uint32_t v, int lane) {
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t u = __shfl_up(x, off, 64);
    if (lane >= off) x += u;
  }
  return x - v;
}

// Boundary bin of a 256-bin histogram held 4 bins per lane: the bin where the
// count of keys in higher bins first reaches `need`.  Returns the bin, sets
// `above` (keys in higher bins) and `exact` (above + bin count == need).
__device__ __forceinline__ int wave_boundary_bin(const uint32_t* hist, uint32_t need, int lane, uint32_t& above,
                                                 uint32_t& exact) {
  uint32_t own[SW_BINS / 64], tot = 0;
#pragma unroll
  for (int i = 0; i < SW_BINS / 64; ++i) {
    own[i] = hist[lane * (SW_BINS / 64) + i];
    tot += own[i];
  }
  uint32_t x = tot;   // inclusive suffix sum over lanes >= lane
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t u = __shfl_down(x, off, 64);
    if (lane + off < 64) x += u;
  }
  uint32_t cum = x - tot;
  int hit = -1;
  uint32_t ha = 0, he = 0;
#pragma unroll
  for (int i = SW_BINS / 64 - 1; i >= 0; --i) {
    if (cum < need && cum + own[i] >= need) {
      hit = lane * (SW_BINS / 64) + i;
      ha = cum;
      he = (cum + own[i] == need) ? 1u : 0u;
    }
    cum += own[i];
  }
  const int src = __ffsll((long long)__ballot(hit >= 0)) - 1;   // exactly one lane
  above = (uint32_t)__shfl((int)ha, src, 64);
  exact = (uint32_t)__shfl((int)he, src, 64);
  return __shfl(hit, src, 64);
}

// Rows of up to 4096 keys: at most 128 VGPRs, so that four workgroups share a CU
// (the compiler's own choice, 175, left room for two: 10% slower).
template <int KPT>
__global__ __launch_bounds__(SC_THREADS, KPT <= 64 ? 4 : 1) void select_rows(const uint32_t* __restrict__ keys,
                                                          const int32_t* __restrict__ q_pos,
                                                          int32_t* __restrict__ topk, int T_len, int n_entries,
                                                          int m, int n_scan, int k) {
  __shared__ uint32_t hist_all[SC_THREADS / 64][SW_BINS];
  __shared__ uint32_t cand_all[SC_THREADS / 64][SW_CAP];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // latest queries (longest rows) first
  const int t = (int)(gridDim.x - 1 - blockIdx.x) * (SC_THREADS / 64) + wave, b = blockIdx.y;
  if (t >= T_len) return;
  uint32_t* hist = hist_all[wave];
  uint32_t* cand = cand_all[wave];
  const int bt = b * T_len + t;
  const int n_t = min(visible(q_pos, bt, m, n_entries), n_scan);
  const uint32_t* row = keys + (size_t)bt * n_scan;
  uint32_t kv[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int p = 64 * j + lane;
    kv[j] = p < n_t ? row[p] : 0u;
  }
  uint32_t mn = 0xFFFFFFFFu, mx = 0u, nv = 0u;
#pragma unroll
  for (int j = 0; j < KPT; ++j)
    if (kv[j]) {
      mn = min(mn, kv[j]);
      mx = max(mx, kv[j]);
      ++nv;
    }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, off, 64));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 64));
    nv += (uint32_t)__shfl_xor((int)nv, off, 64);
  }
  uint32_t need = nv < (uint32_t)k ? nv : (uint32_t)k;
  const uint32_t want = need;
  uint32_t thresh = mn, eq_take = 0xFFFFFFFFu;   // need == nv: every non-zero key
  if (need == 0) {
    thresh = 0xFFFFFFFFu;
    eq_take = 0;
  } else if (need < nv) {
    // ---- 1. value pass
    const float vmin = key_score(mn), vmax = key_score(mx);
    // (a span too small to scale puts every key in bin 0; the key passes then split it)
    const float span = vmax - vmin;
    const float sc = span > 1e-30f ? 255.99f / span : 0.0f;
    auto vbin = [&](uint32_t kk) -> int { return min(SW_BINS - 1, (int)((key_score(kk) - vmin) * sc)); };
#pragma unroll
    for (int i = 0; i < SW_BINS / 64; ++i) hist[lane * (SW_BINS / 64) + i] = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if (kv[j]) atomicAdd(&hist[vbin(kv[j])], 1u);
    uint32_t above, exact;
    const int d = wave_boundary_bin(hist, need, lane, above, exact);
    need -= above;
    // ---- 2. keys of the boundary bin: their range, and a compact list when it fits
    uint32_t lo = 0xFFFFFFFFu, hi = 0u, nb = 0u;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const bool in = kv[j] != 0u && vbin(kv[j]) == d;
      const uint64_t mk = __ballot(in);
      if (in) {
        lo = min(lo, kv[j]);
        hi = max(hi, kv[j]);
        const uint32_t slot = nb + __popcll(mk & ((1ull << lane) - 1ull));
        if (slot < (uint32_t)SW_CAP) cand[slot] = kv[j];
      }
      nb += __popcll(mk);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      lo = min(lo, (uint32_t)__shfl_xor((int)lo, off, 64));
      hi = max(hi, (uint32_t)__shfl_xor((int)hi, off, 64));
    }
    if (exact) {
      thresh = lo;   // every key of the bin and above
    } else {
      const bool listed = nb <= (uint32_t)SW_CAP;
      uint32_t cl[SW_CAP / 64];   // the list, 4 per lane (0 = empty slot)
#pragma unroll
      for (int i = 0; i < SW_CAP / 64; ++i) cl[i] = (uint32_t)(64 * i + lane) < nb ? cand[64 * i + lane] : 0u;
      for (;;) {
        const uint32_t R = hi - lo;
        const int shift = (R >> 8) == 0 ? 0 : 32 - __clz((int)(R >> 8));
#pragma unroll
        for (int i = 0; i < SW_BINS / 64; ++i) hist[lane * (SW_BINS / 64) + i] = 0;
        if (listed) {
#pragma unroll
          for (int i = 0; i < SW_CAP / 64; ++i)
            if (cl[i] && cl[i] >= lo && cl[i] <= hi) atomicAdd(&hist[(cl[i] - lo) >> shift], 1u);
        } else {
#pragma unroll
          for (int j = 0; j < KPT; ++j)
            if (kv[j] && kv[j] >= lo && kv[j] <= hi) atomicAdd(&hist[(kv[j] - lo) >> shift], 1u);
        }
        const int dd = wave_boundary_bin(hist, need, lane, above, exact);
        need -= above;
        const uint32_t new_lo = lo + ((uint32_t)dd << shift);
        const uint64_t top = (uint64_t)new_lo + ((1ull << shift) - 1);
        const uint32_t new_hi = top < (uint64_t)hi ? (uint32_t)top : hi;
        if (exact) {
          thresh = new_lo;
          break;
        }
        if (shift == 0) {
          thresh = new_lo;
          eq_take = need;
          break;
        }
        lo = new_lo;
        hi = new_hi;
      }
    }
  }
  // ---- 3. ordered emission
  uint64_t my_gt = 0, my_eq = 0;   // lane j: masks of register column j (positions 64j..64j+63)
  if (eq_take == 0xFFFFFFFFu) {
    // no partial tie: every key >= thresh is chosen, one ballot per column
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const uint64_t mg = __ballot(kv[j] != 0u && kv[j] >= thresh);
      if (lane == j) my_gt = mg;
    }
  } else {
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const uint64_t mg = __ballot(kv[j] != 0u && kv[j] > thresh);
      const uint64_t me = __ballot(kv[j] != 0u && kv[j] == thresh);
      if (lane == j) {
        my_gt = mg;
        my_eq = me;
      }
    }
  }
  int32_t* out = topk + (size_t)bt * k;
  if (KPT <= 64) {
    const uint32_t eq_before = wave_excl_prefix((uint32_t)__popcll(my_eq), lane);
    // keep the first (eq_take - eq_before) ties of this lane's 64 positions
    uint64_t keep_eq = my_eq;
    const uint32_t room = eq_take > eq_before ? eq_take - eq_before : 0u;
    if ((uint32_t)__popcll(keep_eq) > room) {
      uint64_t x = keep_eq, r = 0;
      for (uint32_t n = 0; n < room; ++n) {
        const uint64_t low = x & (~x + 1ull);
        r |= low;
        x ^= low;
      }
      keep_eq = r;
    }
    uint64_t sel = my_gt | keep_eq;
    uint32_t pos = wave_excl_prefix((uint32_t)__popcll(sel), lane);
    while (sel) {
      const int bit = __ffsll((long long)sel) - 1;
      out[pos++] = 64 * lane + bit;
      sel &= sel - 1ull;
    }
  } else {
    // more register columns than lanes: emit column by column
    const uint64_t lt = (1ull << lane) - 1ull;
    uint32_t G = 0, E = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const uint32_t kk = kv[j];
      const bool is_gt = kk != 0u && kk > thresh, is_eq = kk != 0u && kk == thresh;
      const uint64_t mg = __ballot(is_gt), me = __ballot(is_eq);
      const uint32_t gl = G + __popcll(mg & lt), el = E + __popcll(me & lt);
      if (is_gt) out[gl + min(el, eq_take)] = 64 * j + lane;
      else if (is_eq && el < eq_take) out[gl + el] = 64 * j + lane;
      G += __popcll(mg);
      E += __popcll(me);
    }
  }
  for (int i = (int)want + lane; i < k; i += 64) out[i] = -1;
}

template <int SF>
hipError_t launch_tiled(const void* q_idx, const float* w, const uint8_t* codes, const uint8_t* scales,
                        const int32_t* q_pos, int32_t* topk, int B, int T_len, int H_I, int N_cap, int n_entries,
                        int m, int k, int n_scan, void* ws, const ScorePlan& p, hipStream_t st) {
  uint32_t* keys = static_cast<uint32_t*>(ws);
  dim3 g1((n_scan + QT_CE - 1) / QT_CE, (T_len + QT - 1) / QT, B);
  hipLaunchKernelGGL(score_qtile_bf16<SF>, g1, dim3(SC_THREADS), 0, st, static_cast<const bf16*>(q_idx), w, codes,
                     scales, q_pos, keys, T_len, H_I, N_cap, n_entries, m, n_scan);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 g2((T_len + SC_THREADS / 64 - 1) / (SC_THREADS / 64), B);
  if (n_scan <= 64 * 64)
    hipLaunchKernelGGL(select_rows<64>, g2, dim3(SC_THREADS), 0, st, keys, q_pos, topk, T_len, n_entries, m, n_scan, k);
  else
    hipLaunchKernelGGL(select_rows<SEL_MAX / 64>, g2, dim3(SC_THREADS), 0, st, keys, q_pos, topk, T_len, n_entries, m,
                       n_scan, k);
  return hipGetLastError();
}

template <typename T, bool POOL, bool BUILD, int SF>
hipError_t launch_impl(const void* q_idx, const float* w, const uint8_t* codes, const uint8_t* scales,
                       const int32_t* q_pos, int32_t* topk, int32_t* cands, int B, int T_len, int H_I, int N_cap,
                       int n_entries, int m, int k, int hsi_s, int hsi_nb, void* ws, const ScorePlan& p,
                       hipStream_t st, float* scores_out) {
  char* wsb = static_cast<char*>(ws);
  const size_t n_slots = p.cand_bytes / 8;
  uint32_t* cand_key = reinterpret_cast<uint32_t*>(wsb);
  int32_t* cand_idx = reinterpret_cast<int32_t*>(wsb + n_slots * 4);
  uint32_t* chunk_lb = reinterpret_cast<uint32_t*>(wsb + p.cand_bytes);
  uint32_t* blkmax = reinterpret_cast<uint32_t*>(wsb + p.cand_bytes + p.lb_bytes);
  uint32_t* seg_cnt = reinterpret_cast<uint32_t*>(wsb + p.cand_bytes + p.lb_bytes + (p.blk_bytes + 255) / 256 * 256);
  const int nblk_max = BUILD ? (n_entries + hsi_s - 1) / hsi_s : 0;
  dim3 g1(p.n_chunks, T_len, B);
  hipLaunchKernelGGL((score_chunk<T, POOL, BUILD, SF>), g1, dim3(SC_THREADS), 0, st, static_cast<const T*>(q_idx), w,
                     codes, scales, q_pos, cands, cand_key, cand_idx, chunk_lb, blkmax, topk, scores_out, T_len, H_I,
                     N_cap, n_entries, m, p.chunk, p.k_chunk, p.n_chunks, k, hsi_s, hsi_nb, nblk_max);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (!BUILD && p.n_chunks <= 1) return hipSuccess;   // every query was finished by its single chunk
  if (p.pf_cpg > 0) {
    hipLaunchKernelGGL((topk_prefilter<POOL>), dim3(p.pf_groups, T_len, B), dim3(PF_THREADS), 0, st, cand_key,
                       cand_idx, chunk_lb, q_pos, seg_cnt, T_len, n_entries, m, p.chunk, p.k_chunk, p.n_chunks,
                       p.pf_cpg, p.pf_groups, BUILD ? 0 : 1);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  dim3 g2(T_len, B, BUILD ? 2 : 1);
  hipLaunchKernelGGL((topk_merge<POOL, BUILD>), g2, dim3(MG_THREADS), 0, st, cand_key, cand_idx, chunk_lb, blkmax,
                     q_pos, topk, cands, T_len, n_entries, m, k, p.chunk, p.k_chunk, p.n_chunks, hsi_s, hsi_nb,
                     nblk_max, (const uint32_t*)seg_cnt, p.pf_cpg, p.pf_groups);
  return hipGetLastError();
}

// Debug score dump helpers.
__global__ __launch_bounds__(256) void fill_neg_inf(float* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = -INFINITY;
}
// Key matrix [Q, n_scan] of the tiled path -> scores (positions past a query's
// visible range, which the scorer does not write, read -inf).
__global__ __launch_bounds__(256) void keys_to_scores(const uint32_t* __restrict__ keys,
                                                      const int32_t* __restrict__ q_pos, float* __restrict__ out,
                                                      int T_len, int n_entries, int m, int n_scan) {
  const int bt = blockIdx.y;
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= n_scan) return;
  const int n_t = visible(q_pos, bt, m, n_entries);
  out[(size_t)bt * n_scan + j] = j < n_t ? key_score(keys[(size_t)bt * n_scan + j]) : -INFINITY;
}

template <typename T, int SF>
hipError_t launch_stream(const void* q_idx, const float* w, const uint8_t* codes, const uint8_t* scales,
                         const int32_t* q_pos, int32_t* topk, int B, int T_len, int H_I, int N_cap, int n_entries,
                         int m, int k, void* ws, const ScorePlan& p, hipStream_t st, float* scores_out) {
  char* wsb = static_cast<char*>(ws);
  const size_t n_slots = p.cand_bytes / 8;
  uint32_t* cand_key = reinterpret_cast<uint32_t*>(wsb);
  int32_t* cand_idx = reinterpret_cast<int32_t*>(wsb + n_slots * 4);
  uint32_t* chunk_lb = reinterpret_cast<uint32_t*>(wsb + p.cand_bytes);
  dim3 g1(p.n_chunks, T_len, B);
  hipLaunchKernelGGL((score_stream<T, SF>), g1, dim3(ST_THREADS), 0, st, static_cast<const T*>(q_idx), w, codes, scales,
                     q_pos, cand_key, cand_idx, chunk_lb, topk, scores_out, T_len, H_I, N_cap, n_entries, m, p.chunk,
                     p.n_chunks, k, p.k_chunk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.n_chunks <= 1) return hipSuccess;   // every query was finished by its single part
  dim3 g2(T_len, B, 1);
  hipLaunchKernelGGL((topk_merge<false, false>), g2, dim3(MG_THREADS), 0, st, cand_key, cand_idx, chunk_lb,
                     (const uint32_t*)nullptr, q_pos, topk, (int32_t*)nullptr, T_len, n_entries, m, k, p.chunk,
                     p.k_chunk, p.n_chunks, 0, 0, 0, (const uint32_t*)nullptr, 0, 0);
  return hipGetLastError();
}

template <typename T, int SF>
hipError_t launch_mode(int hsi, const void* q_idx, const float* w, const uint8_t* codes, const uint8_t* scales,
                       const int32_t* q_pos, int32_t* topk, int32_t* cands, int B, int T_len, int H_I, int N_cap,
                       int n_entries, int m, int k, int hsi_s, int hsi_nb, void* ws, const ScorePlan& p,
                       hipStream_t st, float* scores_out) {
  if (hsi == 1)
    return launch_impl<T, false, true, SF>(q_idx, w, codes, scales, q_pos, topk, cands, B, T_len, H_I, N_cap, n_entries,
                                       m, k, hsi_s, hsi_nb, ws, p, st, scores_out);
  if (hsi == 2)
    return launch_impl<T, true, false, SF>(q_idx, w, codes, scales, q_pos, topk, cands, B, T_len, H_I, N_cap, n_entries,
                                       m, k, hsi_s, hsi_nb, ws, p, st, scores_out);
  return launch_impl<T, false, false, SF>(q_idx, w, codes, scales, q_pos, topk, cands, B, T_len, H_I, N_cap, n_entries, m,
                                      k, hsi_s, hsi_nb, ws, p, st, scores_out);
}

}  // namespace

ScorePlan plan_score(int dtype, int B, int T, int n_scan, int k, int hsi, int hsi_s, int hsi_nb) {
  ScorePlan p{};
  const long long Q = (long long)B * T;
  // many queries over a cache of at most SEL_MAX entries: two-phase path
  if (dtype == 1 && hsi == 0 && Q >= 256 && n_scan >= 1 && n_scan <= SEL_MAX) {
    p.tiled = true;
    p.chunk = n_scan;
    p.n_chunks = 1;
    p.k_chunk = k;
    p.key_bytes = (size_t)Q * n_scan * 4;
    p.total_bytes = p.key_bytes + 256;
    return p;
  }
  const int k4 = (k + 3) & ~3;   // candidate lists in whole uint4s (the merge reads them so)
  if (hsi == 0 && Q >= 8192) {
    // streaming path (very many queries): parts of R entries (whole rounds, at most
    // ST_MAXR), about 512 workgroups in all (two per CU); fewer selections per query
    // than the chunked path, whose per-chunk selections dominate there
    const long long want = n_scan <= 0 ? 1 : (Q * (long long)n_scan + 511) / 512;
    long long R = (want + ST_ROUND - 1) / ST_ROUND * ST_ROUND;
    if (R > ST_MAXR) R = ST_MAXR;
    p.stream = true;
    p.chunk = (int)R;
    p.n_chunks = n_scan <= 0 ? 1 : (int)((n_scan + R - 1) / R);
    p.k_chunk = k4;   // <= CSA2_MAX_TOPK <= R
    p.cand_bytes = (size_t)Q * p.n_chunks * p.k_chunk * 8;
    p.lb_bytes = ((size_t)Q * p.n_chunks * 4 + 255) / 256 * 256;
    p.total_bytes = p.cand_bytes + p.lb_bytes + 256;
    return p;
  }
  int C = MAX_CHUNK;
  while (C > 256 && C / 2 >= n_scan) C /= 2;                       // no chunk much larger than the scan
  // enough workgroups to fill the GPU; a pool scan (a small gathered set, so the
  // merge input stays small) goes down to 256-entry chunks
  while (C > (hsi == 2 ? 256 : 1024) && Q * ((n_scan + C - 1) / C) < 1024) C /= 2;
  if (hsi != 0 && C < hsi_s) C = hsi_s;                           // chunks hold whole blocks
  p.chunk = C;
  p.n_chunks = n_scan <= 0 ? 1 : (n_scan + C - 1) / C;
  p.k_chunk = k4 < C ? k4 : C;
  p.cand_bytes = (size_t)Q * p.n_chunks * p.k_chunk * 8;
  p.lb_bytes = ((size_t)Q * p.n_chunks * 4 + 255) / 256 * 256;
  const long long nblk = (hsi == 1) ? ((long long)n_scan + hsi_s - 1) / hsi_s : 0;
  p.blk_bytes = (size_t)(Q * nblk * 4);
  // pre-filter the candidate lists when the merge would stream many of them
  // through its one workgroup per query: groups of PF_ITEMS candidates
  const long long n_items = (long long)p.n_chunks * p.k_chunk;
  const int cpg = PF_ITEMS / p.k_chunk;
  if (n_items > PF_MIN_ITEMS && (p.k_chunk & 3) == 0 && cpg >= 1 && (p.n_chunks + cpg - 1) / cpg <= PF_MAX_GROUPS) {
    p.pf_cpg = cpg;
    p.pf_groups = (p.n_chunks + cpg - 1) / cpg;
    p.seg_bytes = ((size_t)Q * p.pf_groups * 4 + 255) / 256 * 256;
  }
  p.total_bytes = p.cand_bytes + p.lb_bytes + (p.blk_bytes + 255) / 256 * 256 + p.seg_bytes + 256;
  return p;
}

namespace {

template <int SF>
hipError_t launch_fmt(int dtype, const void* q_idx, const float* w, const uint8_t* codes, const uint8_t* scales,
                      const int32_t* q_pos, int32_t* topk, int32_t* candidates, int B, int T, int H_I, int N_cap,
                      int n_entries, int m, int k, int hsi, int hsi_s, int hsi_nb, void* workspace,
                      const ScorePlan& plan, hipStream_t stream, float* scores_out) {
  const int n_scan = hsi == 2 ? hsi_nb * hsi_s : n_entries;
  if (plan.tiled) {
    hipError_t e = launch_tiled<SF>(q_idx, w, codes, scales, q_pos, topk, B, T, H_I, N_cap, n_entries, m, k,
                                    plan.chunk, workspace, plan, stream);
    if (e != hipSuccess || scores_out == nullptr) return e;
    // the key matrix holds every visible (query, entry) key
    hipLaunchKernelGGL(keys_to_scores, dim3((unsigned)((n_scan + 255) / 256), (unsigned)(B * T)), dim3(256), 0, stream,
                       static_cast<const uint32_t*>(workspace), q_pos, scores_out, T, n_entries, m, n_scan);
    return hipGetLastError();
  }
  if (scores_out != nullptr) {
    // positions no scorer writes (invisible, past the cache, empty pool slots) read -inf
    const size_t n = (size_t)B * T * n_scan;
    hipLaunchKernelGGL(fill_neg_inf, dim3((unsigned)std::min<size_t>((n + 255) / 256, 65536)), dim3(256), 0, stream,
                       scores_out, n);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (plan.stream)
    return dtype == 1 ? launch_stream<bf16, SF>(q_idx, w, codes, scales, q_pos, topk, B, T, H_I, N_cap, n_entries, m,
                                                k, workspace, plan, stream, scores_out)
                      : launch_stream<float, SF>(q_idx, w, codes, scales, q_pos, topk, B, T, H_I, N_cap, n_entries,
                                                 m, k, workspace, plan, stream, scores_out);
  if (dtype == 1)
    return launch_mode<bf16, SF>(hsi, q_idx, w, codes, scales, q_pos, topk, candidates, B, T, H_I, N_cap, n_entries,
                                 m, k, hsi_s, hsi_nb, workspace, plan, stream, scores_out);
  return launch_mode<float, SF>(hsi, q_idx, w, codes, scales, q_pos, topk, candidates, B, T, H_I, N_cap, n_entries,
                                m, k, hsi_s, hsi_nb, workspace, plan, stream, scores_out);
}

}  // namespace

hipError_t launch_score_topk(int dtype, const void* q_idx, const float* w, const uint8_t* codes,
                             const uint8_t* scales, const int32_t* q_pos, int32_t* topk, int32_t* candidates, int B,
                             int T, int H_I, int N_cap, int n_entries, int m, int k, int hsi, int hsi_s, int hsi_nb,
                             void* workspace, const ScorePlan& plan, hipStream_t stream, float* scores_out,
                             int scale_fmt) {
  if (B == 0 || T == 0) return hipSuccess;
  return scale_fmt == 1
             ? launch_fmt<1>(dtype, q_idx, w, codes, scales, q_pos, topk, candidates, B, T, H_I, N_cap, n_entries, m,
                             k, hsi, hsi_s, hsi_nb, workspace, plan, stream, scores_out)
             : launch_fmt<0>(dtype, q_idx, w, codes, scales, q_pos, topk, candidates, B, T, H_I, N_cap, n_entries, m,
                             k, hsi, hsi_s, hsi_nb, workspace, plan, stream, scores_out);
}

}  // namespace csa2
