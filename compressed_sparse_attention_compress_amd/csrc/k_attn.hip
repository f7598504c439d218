// (e) Sparse attention of one query token over its selected cache entries plus
// its sliding window, with key = value = the 512-d latent row.
//
// Method ([P1] "DeepSeek-V4.1 模型结构（2）…", section "一层全局注意力算四样东西":
// the layer's own query reads the k selected entries and the 128 rows of its
// sliding window; [P2] "DeepSeek v4.1 Flash技术剖析——架构篇", CSA2-FULL: one vector
// serves as key and value; [P3] "…分级缓存", section four: p_j proportional to
// exp(c_j . q / sqrt(d)), o = sum_j p_j c_j).
//
// The rows of a token (selected entries, then window positions) are streamed
// through LDS with direct global->LDS loads (global_load_lds_dwordx4: one wave
// instruction moves one 1 KB bf16 row), double-buffered so the next chunk is in
// flight while the current one is used.  S^T = R Q^T has cache rows as MFMA rows
// and 16 heads as columns; its accumulator already is the P^T operand of
// O^T = R^T P^T once the k-slots of the PV step are numbered (row 4g+i of tile 0,
// row 4g+i of tile 1) for lane group g.  The R^T operand is read from the
// row-major LDS copy with ds_read_b64_tr_b16 (each 16-lane group transposes 4 rows
// x 16 dims), so no transposed copy is stored.  Online softmax in base 2, float32
// throughout; each lane owns one head of a tile, so running max, sum and rescale
// are per-lane scalars.
//
// attn_prefill: one workgroup per token; wave (hp, dh) owns heads 32hp..32hp+31
//   and latent dims 256dh..256dh+255 (split-K: the two half-dim score partials are
//   swapped through LDS), 32-row chunks, two workgroups per CU; runs of tokens
//   are dealt to the XCDs round-robin, latest tokens first.
// attn_decode: one workgroup per (token, row split) for all heads (wave w owns
//   heads 16w..16w+15), rows gathered once into a 4-stage ring of 32-row chunks
//   with three chunks in flight.  Row splits, when used, write partials (bf16
//   normalised output, float32 log-sum-exp) that attn_combine merges.
#include <type_traits>

#include "csa2_internal.h"
#include "device_common.h"
#include "lds_dma.h"

namespace csa2 {

namespace {

constexpr int MAX_ROWS = 2048;   // selected + window rows per query (host-checked)

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;



// Max over lanes l and l^16, then l^32, with the gfx950 permlane swaps (VALU, no LDS).
__device__ __forceinline__ float max_lane_groups(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  auto r2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(r2[0]), __uint_as_float(r2[1]));
}

// Transposed read: lane i of each 16-lane group receives 4 consecutive rows
// (row0 .. row0+3) of dim d0 + i, bf16 (see file comment).  `p` is this lane's
// own address: row0 + (i / 4), dim d0 + 4 * (i % 4).
__device__ __forceinline__ v4s tr_read(const lds_u8* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)p);
}

// Rows live in LDS as 64 units of 16 B with the unit index XOR-swizzled by
// swz(row & 15), a bijection on 4 bits chosen so that both read patterns are
// free of bank conflicts: 16 lanes reading one 16-B unit of 16 consecutive rows
// (ds_read_b128) hit 16 different units, and the transposed reads (4 rows x two
// 16-B units per 16-lane group, two groups at a time) hit 16 different units.
// The DMA writes lane i's 16 B to unit i, so lane i fetches logical unit
// i ^ swz(row) from global memory.
__device__ __forceinline__ int swz(int r) { return (((r >> 2) & 1) << 3) | ((r & 3) << 1) | ((r >> 3) & 1); }

// Row list of one query: valid selected ids (order kept), then window rows
// encoded as -(j+1) for swa row j: dense row j = position pos0 + j, or with
// `ring` the ring slot of that position (position u sits in slot u mod L_w).
// Returns the number of rows.  Needs a __syncthreads() before use by other waves
// (done by the callers).  after_issue() runs once in every wave: in wave 0 right
// after the first 512 ids are requested (so loads it issues queue behind them),
// elsewhere at once.
template <typename F>
__device__ __forceinline__ int build_rowlist(int* rowlist, int* n_sel_s, const int32_t* tk, int k, int N_cap, int p,
                                             int pos0, int L_w, int W, F&& after_issue, bool ring = false) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wave == 0) {
    int cnt = 0;
    for (int j0 = 0; j0 < k; j0 += 512) {   // 8 loads per lane in flight, then the ballots
      int g[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = j0 + 64 * u + lane;
        g[u] = j < k ? tk[j] : -1;
      }
      if (j0 == 0) after_issue();
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const bool ok = g[u] >= 0 && g[u] < N_cap;
        const unsigned long long bal = __ballot(ok);
        const int before = __popcll(bal & ((1ull << lane) - 1ull));
        if (ok) rowlist[cnt + before] = g[u];
        cnt += __popcll(bal);
      }
    }
    if (k <= 0) after_issue();   // no id loads: the loop above did not run
    if (lane == 0) *n_sel_s = cnt;
  } else {
    after_issue();
  }
  __syncthreads();
  const int n_sel = *n_sel_s;
  int lo = p - W + 1;
  if (lo < 0) lo = 0;
  if (lo < pos0) lo = pos0;
  int hi = p;
  if (hi > pos0 + L_w - 1) hi = pos0 + L_w - 1;
  const int n_win = hi >= lo ? hi - lo + 1 : 0;
  for (int j = threadIdx.x; j < n_win; j += blockDim.x)
    rowlist[n_sel + j] = -(ring ? (lo + j) % L_w : lo - pos0 + j) - 1;
  __syncthreads();
  return n_sel + n_win;
}

template <typename T>
__device__ __forceinline__ const T* row_ptr(int id, const T* kvb, const T* swb) {
  return id >= 0 ? kvb + (size_t)id * 512 : swb + (size_t)(-id - 1) * 512;
}

// Final softmax normalisation of one head, base 2: the rows' running maximum m and
// sum l (relative to m), and the head's sink logit s2 (log2 units; -inf without a
// sink), which enters the denominator only.  Returns the factor that turns the
// accumulator (weights relative to m) into the output and sets lse2 to the
// log2-sum-exp over the rows and the sink (-inf when both are empty).
__device__ __forceinline__ float softmax_norm(float m, float l, float s2, float& lse2) {
  if (!(l > 0.f)) {   // no rows: zero output, the sink alone in the log-sum-exp
    lse2 = s2;
    return 0.f;
  }
  const float M = fmaxf(m, s2);
  const float a = exp2f(m - M);
  const float den = l * a + exp2f(s2 - M);
  lse2 = M + log2f(den);
  return a / den;
}
__device__ __forceinline__ float sink_log2(const float* sink, int head, int H) {
  return (sink != nullptr && head < H) ? sink[head] * 1.4426950408889634f : -INFINITY;
}

// ----------------------------------------------------------------- prefill

constexpr int PRC = 32;                 // rows per chunk
constexpr int PRS = 1024;               // LDS row stride (bytes) for bf16 rows (swizzled, no padding)
constexpr float RESCALE_SLACK = 8.0f;   // log2 units the running max may lag behind before rescaling

// Prefill: a workgroup of 2 x NW/2 waves per token; wave (hp, dh) owns heads
// 32hp..32hp+31 and the 256 latent dims 256dh..256dh+255.  S^T for its 32 heads is
// the sum of two half-dim products: each wave computes its half, the halves are
// swapped through LDS and added (a + b == b + a, so both waves hold bit-identical
// scores and run the same softmax), and PV covers the wave's own 256 dims.  Per
// 32-row chunk a wave reads 16 KB of rows for S and 16 KB for PV (half of what a
// 16-heads x 512-dims wave reads), two chunk buffers + the exchange area take 80 KB
// of LDS, so two workgroups share a CU.  Row ids come from the top-k row itself:
// lanes 0..31 hold the 32 ids of a chunk (read one chunk ahead), readlane gives
// each gather its row, and a ballot gives the chunk's validity mask.  The selected
// part spans the slots up to the last valid id; invalid ids inside it load row 0
// and are masked to probability 0.
template <int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void attn_prefill_bf16(
    const bf16* __restrict__ q, const bf16* __restrict__ kv, const int32_t* __restrict__ topk,
    const bf16* __restrict__ swa, const int32_t* __restrict__ swa_pos0, const int32_t* __restrict__ q_pos,
    bf16* __restrict__ o, float* __restrict__ lse, const float* __restrict__ sink, int T_len, int H, int N_cap,
    int k, int L_w, int W, float scale_log2, int tbl) {
  __shared__ __attribute__((aligned(16))) unsigned char buf0[PRC * PRS];
  __shared__ __attribute__((aligned(16))) unsigned char buf1[PRC * PRS];
  __shared__ f32x4 xbuf[NW][4 * 64];    // per wave: its half-dim S partial, [tile mt*2+ht][lane]
  constexpr int RPW = PRC / NW;          // rows gathered per wave per chunk

  // workgroups are dealt to the 8 XCDs round-robin by id; give each XCD runs of
  // tbl consecutive tokens, so the window rows (shared by neighbouring tokens)
  // stay in that XCD's L2, with the runs dealt round-robin so that every XCD gets
  // early (short, causal) and late tokens alike, and the latest tokens (the most
  // rows) go first so that the short ones fill the tail
  const int jx = blockIdx.x >> 3;
  const int t = T_len - 1 - (((jx / tbl) * 8 + (int)(blockIdx.x & 7)) * tbl + jx % tbl);
  const int b = blockIdx.y;
  if (t < 0 || t >= T_len) return;
  const int bt = b * T_len + t;
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hp = wave >> 1, dh = wave & 1;
  const int32_t* tk = topk + (size_t)bt * k;
  const bf16* kvb = kv + (size_t)b * N_cap * 512;
  const bf16* swb = swa + (size_t)b * L_w * 512;

  // rows: selected slots [0, k_eff) (k_eff = one past the last valid id), then the window
  int k_eff = 0;
  for (int j0 = 0; j0 < k; j0 += 512) {   // 8 loads per lane in flight, then the ballots
    int g[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = j0 + 64 * u + lane;
      g[u] = j < k ? tk[j] : -1;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const unsigned long long bal = __ballot(g[u] >= 0 && g[u] < N_cap);
      if (bal) k_eff = j0 + 64 * u + 64 - __clzll(bal);
    }
  }
  const int p = q_pos[bt], pos0 = swa_pos0[b];
  int lo = p - W + 1;
  if (lo < 0) lo = 0;
  if (lo < pos0) lo = pos0;
  int hi = p;
  if (hi > pos0 + L_w - 1) hi = pos0 + L_w - 1;
  const int n_win = hi >= lo ? hi - lo + 1 : 0;
  const int n_rows = k_eff + n_win;
  const bf16* dummy = n_win > 0 ? swb + (size_t)(lo - pos0) * 512 : kvb;

  bf16x8 qf[2][8];
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    const int head = hp * 32 + ht * 16 + lr;
    const bf16* qrow = q + ((size_t)bt * H + head) * 512 + dh * 256;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (head < H) qf[ht][ks] = load_frag(qrow + ks * 32 + 8 * lg);
      else zero_frag(qf[ht][ks]);
    }
  }
  f32x4 oacc[16][2];
#pragma unroll
  for (int dt = 0; dt < 16; ++dt) {
    oacc[dt][0] = f32x4{0.f, 0.f, 0.f, 0.f};
    oacc[dt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
  // the query fragments are complete before any gather is issued, so no wait in
  // the chunk loop has to cover them (which would also wait for the gathers)
  WAIT_VMCNT(0);

  f32x4* xown = xbuf[wave];
  const f32x4* xpart = xbuf[wave ^ 1];

  const int nch = (n_rows + PRC - 1) / PRC;
  // lane l (mod 32) holds the id slot of row 32c + l (selected part only)
  auto load_ids = [&](int c) -> int {
    const int r = c * PRC + (lane & 31);
    return tk[r < k_eff ? r : 0];
  };
  // gathers chunk c's rows of this wave into buf; returns the chunk's validity mask
  auto issue = [&](int c, unsigned char* buf, int ids) -> uint32_t {
    // lane l (mod 32) works out the source of row 32c + l without branches; each
    // gather instruction then takes its row's address with two readlanes.  The
    // opaque lane copy keeps the per-row offsets from being hoisted out of the loop
    // (they would not fit beside the accumulators).
    int lv = lane;
    __asm__ volatile("" : "+v"(lv));
    const int r_l = c * PRC + (lv & 31);
    const bool in_sel = r_l < k_eff;
    const bool ok_sel = ids >= 0 && ids < N_cap;
    const int jw = r_l - k_eff;
    const bool ok_win = !in_sel && jw < n_win;
    const uint32_t mask = (uint32_t)__ballot(in_sel ? ok_sel : ok_win);
    const bf16* src_l = in_sel ? kvb + (size_t)(ok_sel ? ids : 0) * 512
                               : (ok_win ? swb + (size_t)(lo - pos0 + jw) * 512 : dummy);
    const uint64_t a_l = reinterpret_cast<uint64_t>(src_l);
    const uint32_t lane16 = (uint32_t)lv << 4;
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
      const int rr = wave * RPW + j;
      const uint32_t alo = __builtin_amdgcn_readlane((uint32_t)a_l, rr);
      const uint32_t ahi = __builtin_amdgcn_readlane((uint32_t)(a_l >> 32), rr);
      dma16_asm_s(((uint64_t)ahi << 32) | alo, lane16 ^ ((uint32_t)swz(rr & 15) << 4), (const lds_u8*)(buf + rr * PRS));
    }
    return mask;
  };
  int ids_next = 0;
  uint32_t mask_cur = 0, mask_next = 0;
  auto step = [&](int c, unsigned char* cur, unsigned char* nxt) {
    // The id loads are ordinary loads: before ids(c+1) is used the compiler waits
    // for it and everything older, i.e. also chunk c's gathers, which are needed
    // now anyway.  Chunk c+1's gathers and ids(c+2) then stay in flight while
    // chunk c is computed; the explicit waits restate that chunk c is complete.
    if (c + 1 < nch) {
      mask_next = issue(c + 1, nxt, ids_next);
      if (c + 2 < nch) {
        ids_next = load_ids(c + 2);
        WAIT_VMCNT(RPW + 1);
      } else {
        WAIT_VMCNT(RPW);
      }
    } else {
      WAIT_VMCNT(0);
    }
    __builtin_amdgcn_s_barrier();
    COMPILER_FENCE();
    const lds_u8* lcur = (const lds_u8*)cur;
    // swizzled unit offsets, recomputed per chunk (an opaque copy of the lane id
    // keeps them from being held live across the loop, where they would spill)
    int lv = lane;
    __asm__ volatile("" : "+v"(lv));
    const int vlr = lv & 15, vlg = (lv >> 4) & 3;
    int soff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) soff[i] = ((4 * i + vlg) ^ swz(vlr)) << 4;

    // ---- this wave's half of S^T = R Q^T (k-steps 8dh .. 8dh+7 of the row)
    // fragment f = (mt, ks) = (f / 8, f % 8); the next one is read while the
    // current one feeds its two MFMAs
    f32x4 s[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      s[mt][0] = f32x4{0.f, 0.f, 0.f, 0.f};
      s[mt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const unsigned char* sbase = cur + vlr * PRS + dh * 512;
    auto rd = [&](int f) -> bf16x8 {
      return *reinterpret_cast<const bf16x8*>(sbase + (f >> 3) * 16 * PRS + soff[f & 3] + ((f & 7) >> 2) * 256);
    };
    bf16x8 a0 = rd(0), a1 = rd(1);
#pragma unroll
    for (int f = 0; f < 16; ++f) {
      bf16x8 a2;
      if (f + 2 < 16) a2 = rd(f + 2);
      __builtin_amdgcn_sched_barrier(0);
      const int mt = f >> 3, ks = f & 7;
      s[mt][0] = mma16(a0, qf[0][ks], s[mt][0]);
      s[mt][1] = mma16(a0, qf[1][ks], s[mt][1]);
      __builtin_amdgcn_sched_barrier(0);
      a0 = a1;
      if (f + 2 < 16) a1 = a2;
    }
    // ---- swap halves with the partner wave
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) xown[(mt * 2 + ht) * 64 + lane] = s[mt][ht];
    WAIT_LGKM0();
    COMPILER_FENCE();
    __builtin_amdgcn_s_barrier();
    COMPILER_FENCE();
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) s[mt][ht] += xpart[(mt * 2 + ht) * 64 + lane];

    // ---- online softmax with lazy rescale, per head tile.  A chunk without a
    // valid row is skipped, so every head sees a finite chunk maximum and exp2 of
    // (-inf - finite) gives the 0 of a masked row.
    if (mask_cur != 0u) {
    float cmax[2];
    bool grow[2];
    if (mask_cur != 0xFFFFFFFFu) {
      const uint32_t m4 = mask_cur >> (4 * vlg);   // bit mt*16+i: row mt*16 + 4*lg + i
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (!((m4 >> (mt * 16 + i)) & 1u)) {
            s[mt][0][i] = -INFINITY;
            s[mt][1][i] = -INFINITY;
          }
    }
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      // raw scores; the scale is positive, so the scaled maximum is the scaled raw one
      cmax[ht] = fmaxf(fmaxf(fmaxf(s[0][ht][0], s[0][ht][1]), fmaxf(s[0][ht][2], s[0][ht][3])),
                       fmaxf(fmaxf(s[1][ht][0], s[1][ht][1]), fmaxf(s[1][ht][2], s[1][ht][3])));
      cmax[ht] = max_lane_groups(cmax[ht]) * scale_log2;
      grow[ht] = cmax[ht] > m_run[ht] + RESCALE_SLACK;
    }
    if (__builtin_amdgcn_ballot_w64(grow[0] || grow[1])) {
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) {
        const float m_new = grow[ht] ? cmax[ht] : m_run[ht];
        const float alpha = grow[ht] ? __builtin_amdgcn_exp2f(m_run[ht] - m_new) : 1.0f;  // 0 on the first rows
        l_run[ht] *= alpha;
#pragma unroll
        for (int dt = 0; dt < 16; ++dt) oacc[dt][ht] *= alpha;
        m_run[ht] = m_new;
      }
    }
    bf16x8 pf[2];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float pv = __builtin_amdgcn_exp2f(fmaf(s[i >> 2][ht][i & 3], scale_log2, -m_run[ht]));
        psum += pv;
        pf[ht][i] = (bf16)pv;
      }
      l_run[ht] += psum;
    }
    // ---- O^T += R^T P^T over this wave's 256 dims
    const lds_u8* tb = lcur + (4 * vlg + (vlr >> 2)) * PRS + 8 * (vlr & 1) + dh * 512;
    const int tsw = swz(4 * vlg + (vlr >> 2)), th = (vlr & 3) >> 1;
    const lds_u8* tpa[8];
#pragma unroll
    for (int d8 = 0; d8 < 8; ++d8) tpa[d8] = tb + (((2 * d8 + th) ^ tsw) << 4);
    auto rdt = [&](int dt) -> bf16x8 {
      const v4s lo4 = tr_read(tpa[dt & 7] + (dt >> 3) * 256);
      const v4s hi4 = tr_read(tpa[dt & 7] + (dt >> 3) * 256 + 16 * PRS);
      bf16x8 a;
      __builtin_memcpy(&a, &lo4, 8);
      __builtin_memcpy(reinterpret_cast<char*>(&a) + 8, &hi4, 8);
      return a;
    };
    bf16x8 v0 = rdt(0), v1 = rdt(1);
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) {
      bf16x8 v2;
      if (dt + 2 < 16) v2 = rdt(dt + 2);
      __builtin_amdgcn_sched_barrier(0);
      oacc[dt][0] = mma16(v0, pf[0], oacc[dt][0]);
      oacc[dt][1] = mma16(v0, pf[1], oacc[dt][1]);
      __builtin_amdgcn_sched_barrier(0);
      v0 = v1;
      if (dt + 2 < 16) v1 = v2;
    }
    }   // mask_cur != 0
    WAIT_LGKM0();
    COMPILER_FENCE();
    __builtin_amdgcn_s_barrier();
    mask_cur = mask_next;
  };
  if (nch > 0) {
    const int ids0 = load_ids(0);
    ids_next = nch > 1 ? load_ids(1) : 0;
    mask_cur = issue(0, buf0, ids0);
  }
  for (int c = 0; c < nch; c += 2) {
    step(c, buf0, buf1);
    if (c + 1 < nch) step(c + 1, buf1, buf0);
  }

#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    float l_tot = l_run[ht] + __shfl_xor(l_run[ht], 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    const int head = hp * 32 + ht * 16 + lr;
    float lse2;
    const float inv = softmax_norm(m_run[ht], l_tot, sink_log2(sink, head, H), lse2);
    if (head < H) {
      bf16* orow = o + ((size_t)bt * H + head) * 512 + dh * 256;
#pragma unroll
      for (int dt = 0; dt < 16; ++dt) {
        const int d = dt * 16 + 4 * lg;
        bf16x2 p0, p1;
        p0[0] = (bf16)(oacc[dt][ht][0] * inv); p0[1] = (bf16)(oacc[dt][ht][1] * inv);
        p1[0] = (bf16)(oacc[dt][ht][2] * inv); p1[1] = (bf16)(oacc[dt][ht][3] * inv);
        uint2 u;
        __builtin_memcpy(&u.x, &p0, 4);
        __builtin_memcpy(&u.y, &p1, 4);
        *reinterpret_cast<uint2*>(orow + d) = u;
      }
      if (lse != nullptr && lg == 0 && dh == 0)
        lse[(size_t)bt * H + head] = lse2 * 0.69314718055994531f;
    }
  }
}

// ----------------------------------------------------------------- decode

constexpr int DRC = 32;                 // rows per stage
constexpr int DNS = 4;                  // stages: three in flight while one is used
constexpr int RAW4 = DRC * 288;         // FP4 chunk: 32 x 256 B of codes, then 32 x 32 scale bytes

// One workgroup per (query, row split); wave w owns heads 16w..16w+15, so each
// row is fetched once per workgroup and read from LDS by every wave.  Stage s of
// the 4-stage ring holds chunk c (32 rows) for c = s mod 4; the gathers of chunk
// c + 3 are issued right after the barrier that opens chunk c, into the stage
// that chunk c - 1 used.  NW = 4, 2 or 1 waves (H > 32, > 16, <= 16); wave w
// gathers rows w, w + NW, ... of each chunk.
//
// FP4 main KV (FP4 = true): the first n_fp4 splits of a query cover its selected
// rows, the others its window rows (bf16, the ring as above).  A selected-row
// chunk lands raw (288 B per row) in a 4-stage ring of 9 KiB stages; after the
// barrier that opens it, every thread dequantises 64 dims of one row into a
// single bf16 chunk buffer (same swizzled layout as a gathered bf16 chunk), and
// a second barrier hands that buffer to the MFMA steps.  E2M1 x E4M3 values are
// exact in bf16, so the MFMA inputs are exactly the dequantised cache.
//
// FP8 window ring (W8 = true): `swa` is the layer's ring of L_w E4M3 rows (512 B,
// position u in slot u mod L_w) and the window rows go to splits of their own
// (the last n_splits - n_fp4).  The ring's first position is p0 = max(swa_pos0,
// newest - L_w + 1), newest = the sequence's largest query position in the call
// (what a dense copy of the ring would start at).  A window chunk lands raw (32 x
// 512 B, two rows per DMA instruction) in a 4-stage ring of 16 KiB stages and is
// widened to bf16 (E4M3 values are exact in bf16) into the two chunk buffers the
// same way as an FP4 chunk.
template <int NW, bool FP4, bool W8>
__global__ __launch_bounds__(64 * NW, 1) void attn_decode_bf16(
    const bf16* __restrict__ q, const void* __restrict__ kv, const uint8_t* __restrict__ kv_scales,
    const int32_t* __restrict__ topk, const void* __restrict__ swa, const int32_t* __restrict__ swa_pos0,
    const int32_t* __restrict__ q_pos, bf16* __restrict__ o, float* __restrict__ lse, const float* __restrict__ sink,
    bf16* __restrict__ part_o, float* __restrict__ part_lse, int T_len, int H, int N_cap, int k, int L_w, int W,
    float scale_log2, int n_splits, int n_fp4) {
  constexpr int RPW = DRC / NW;   // gathers per wave per chunk
  constexpr int DPW4 = 8 / NW + 4 / NW;   // DMA instructions per wave per FP4 chunk
  constexpr int DPW8 = 16 / NW;           // DMA instructions per wave per FP8 window chunk
  __shared__ __attribute__((aligned(16))) unsigned char ring[DNS * DRC * PRS];
  __shared__ int rowlist[MAX_ROWS];
  __shared__ int n_sel_s;
  static_assert(!FP4 || 2 * DRC * PRS + DNS * RAW4 <= DNS * DRC * PRS, "FP4 buffers fit in the ring");
  static_assert(!W8 || 2 * DRC * PRS + DNS * DRC * 512 <= DNS * DRC * PRS, "FP8 window buffers fit in the ring");

  const int qi = blockIdx.x / n_splits, split = blockIdx.x % n_splits;
  const int b = qi / T_len;
  const int bt = qi;
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // the query fragments are requested right after the first row ids (in wave 0,
  // which builds the row list), so they arrive while the list is built
  const int head = wave * 16 + lr;
  bf16x8 qf[16];
  const bf16* qrow = q + ((size_t)bt * H + head) * 512;
  int pos0 = swa_pos0[b];
  if constexpr (W8) {   // the ring's first position: from the sequence's newest query
    int nw = -2147483647 - 1;
    for (int t = lane; t < T_len; t += 64) nw = max(nw, q_pos[(size_t)b * T_len + t]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) nw = max(nw, __shfl_xor(nw, off, 64));
    pos0 = max(pos0, __builtin_amdgcn_readfirstlane(nw) - L_w + 1);   // every lane holds the maximum
  }
  const int n_rows = build_rowlist(rowlist, &n_sel_s, topk + (size_t)bt * k, k, N_cap, q_pos[bt], pos0, L_w, W,
                                   [&]() {
#pragma unroll
                                     for (int ks = 0; ks < 16; ++ks) {
                                       if (head < H) qf[ks] = load_frag(qrow + ks * 32 + 8 * lg);
                                       else zero_frag(qf[ks]);
                                     }
                                   },
                                   W8);
  // rows [rb, rb + nr) of the row list belong to this workgroup's kind of split
  int rb = 0, nr = n_rows, sp = split, nsp = n_splits;
  bool fp4_rows = false, fp8_rows = false;
  if constexpr (FP4 || W8) {
    const int n_sel = n_sel_s;
    if (split < n_fp4) {
      nr = n_sel; nsp = n_fp4; fp4_rows = FP4;
    } else {
      rb = n_sel; nr = n_rows - n_sel; sp = split - n_fp4; nsp = n_splits - n_fp4; fp8_rows = W8;
    }
  }
  const bf16* kvb = static_cast<const bf16*>(kv) + (size_t)b * N_cap * 512;   // bf16 rows (not read by FP4 splits)
  const bf16* swb = static_cast<const bf16*>(swa) + (size_t)b * L_w * 512;    // dense bf16 window (not with W8)
  f32x4 oacc[32];
#pragma unroll
  for (int dt = 0; dt < 32; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  WAIT_VMCNT(0);   // the query is in registers; from here on only the gathers use the counter

  const int nch_all = (nr + DRC - 1) / DRC;
  const int c0 = (int)(((long long)nch_all * sp) / nsp);
  const int c1 = (int)(((long long)nch_all * (sp + 1)) / nsp);
  const int* rl = rowlist + rb;
  // swizzled unit offsets of the S reads and the transposed PV reads
  int soff[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) soff[u] = ((4 * u + lg) ^ swz(lr)) << 4;
  const int tsw = swz(4 * lg + (lr >> 2)), th = (lr & 3) >> 1;
  int toff[8];
#pragma unroll
  for (int d8 = 0; d8 < 8; ++d8) toff[d8] = (((2 * d8 + th) ^ tsw) << 4) + (4 * lg + (lr >> 2)) * PRS + 8 * (lr & 1);

  // one 32-row chunk c in LDS (bf16, swizzled): scores, online softmax, PV
  // mid(0) and mid(1) run between S's MFMAs (the FP4 and FP8 splits widen the next
  // chunk there, so its VALU work overlaps the MFMAs in flight)
  auto attend = [&](const unsigned char* cur, int c, auto&& mid) __attribute__((always_inline)) {
    // ---- S^T = R Q^T: 32 rows (two row tiles) x this wave's 16 heads
    f32x4 s[2];
    s[0] = f32x4{0.f, 0.f, 0.f, 0.f};
    s[1] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto rd = [&](int f) -> bf16x8 {   // fragment f = (row tile f / 16, k-step f % 16)
      return *reinterpret_cast<const bf16x8*>(cur + ((f >> 4) * 16 + lr) * PRS + soff[f & 3] + ((f & 15) >> 2) * 256);
    };
    bf16x8 a0 = rd(0), a1 = rd(1);
#pragma unroll
    for (int f = 0; f < 32; ++f) {
      bf16x8 a2;
      if (f + 2 < 32) a2 = rd(f + 2);
      __builtin_amdgcn_sched_barrier(0);
      s[f >> 4] = mma16(a0, qf[f & 15], s[f >> 4]);
      __builtin_amdgcn_sched_barrier(0);
      if (f == 7) mid(0);
      if (f == 23) mid(1);
      a0 = a1;
      if (f + 2 < 32) a1 = a2;
    }

    // ---- online softmax (base 2, lazy rescale); rows past the list are masked
    float x[8];
    float cmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = c * DRC + (i >> 2) * 16 + 4 * lg + (i & 3);
      x[i] = row < nr ? s[i >> 2][i & 3] * scale_log2 : -INFINITY;
      cmax = fmaxf(cmax, x[i]);
    }
    cmax = max_lane_groups(cmax);   // every chunk holds a valid row, so cmax is finite
    const bool grow = cmax > m_run + RESCALE_SLACK;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float m_new = grow ? cmax : m_run;
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;   // 0 on the first rows
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 32; ++dt) oacc[dt] *= alpha;
      m_run = m_new;
    }
    bf16x8 pf;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float pv = __builtin_amdgcn_exp2f(x[i] - m_run);
      psum += pv;
      pf[i] = (bf16)pv;
    }
    l_run += psum;

    // ---- O^T += R^T P^T over the 512 dims (k-slots: rows 4g+i of tile 0, then of tile 1)
    const lds_u8* lcur = (const lds_u8*)cur;
    auto rdt = [&](int dt) -> bf16x8 {
      const v4s lo4 = tr_read(lcur + toff[dt & 7] + (dt >> 3) * 256);
      const v4s hi4 = tr_read(lcur + toff[dt & 7] + (dt >> 3) * 256 + 16 * PRS);
      bf16x8 a;
      __builtin_memcpy(&a, &lo4, 8);
      __builtin_memcpy(reinterpret_cast<char*>(&a) + 8, &hi4, 8);
      return a;
    };
    bf16x8 v0 = rdt(0), v1 = rdt(1);
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) {
      bf16x8 v2;
      if (dt + 2 < 32) v2 = rdt(dt + 2);
      __builtin_amdgcn_sched_barrier(0);
      oacc[dt] = mma16(v0, pf, oacc[dt]);
      __builtin_amdgcn_sched_barrier(0);
      v0 = v1;
      if (dt + 2 < 32) v1 = v2;
    }
    WAIT_LGKM0();
    COMPILER_FENCE();
  };

  // two dequantised chunks (chunk c in buffer c & 1), then a raw ring of 4 stages.
  // Chunk c + 1 is dequantised while chunk c is attended, so one barrier per
  // chunk: it finds raw chunk c + 1 landed, chunk c dequantised by every wave and
  // chunk c - 1 (whose buffer chunk c + 1 takes) no longer read.  DPW = DMA
  // instructions per wave per raw chunk.
  auto dqb = [&](int c) -> unsigned char* { return ring + (c & 1) * (DRC * PRS); };
  typedef float v2f __attribute__((ext_vector_type(2)));
  auto bf16_pair = [](float lo, float hi) -> uint32_t {
    return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
  };
  auto dq_loop = [&](auto dpw_c, auto issue_raw, auto dequant) {
    constexpr int DPW = decltype(dpw_c)::value;
    for (int c = c0; c < c0 + DNS - 1 && c < c1; ++c) issue_raw(c);
    if (c0 < c1) {
      if (c1 - c0 >= 3) WAIT_VMCNT(2 * DPW);
      else if (c1 - c0 == 2) WAIT_VMCNT(DPW);
      else WAIT_VMCNT(0);
      __builtin_amdgcn_s_barrier();   // raw chunk c0 is in LDS
      COMPILER_FENCE();
      dequant(c0, 0);
      dequant(c0, 1);
    }
    for (int c = c0; c < c1; ++c) {
      const int younger = min(c1 - 2 - c, DNS - 3);   // chunks issued after c + 1
      if (younger >= 1) WAIT_VMCNT(DPW);
      else WAIT_VMCNT(0);
      WAIT_LGKM0();
      __builtin_amdgcn_s_barrier();
      COMPILER_FENCE();
      if (c + DNS - 1 < c1) issue_raw(c + DNS - 1);
      attend(dqb(c), c, [&](int h) {
        if (c + 1 < c1) dequant(c + 1, h);
      });
    }
  };

  if (!fp4_rows && !fp8_rows) {
    auto stage = [&](int c) -> unsigned char* { return ring + (c & (DNS - 1)) * (DRC * PRS); };
    auto issue = [&](int c) {
      unsigned char* buf = stage(c);
#pragma unroll
      for (int j = 0; j < RPW; ++j) {
        const int rr = wave + NW * j;
        const int r = c * DRC + rr;
        const int rid = rl[r < nr ? r : 0];
        const unsigned char* src = reinterpret_cast<const unsigned char*>(row_ptr(rid, kvb, swb));
        dma16_asm(src + ((lane ^ swz(rr & 15)) << 4), (const lds_u8*)(buf + rr * PRS));
      }
    };
    for (int c = c0; c < c0 + DNS - 1 && c < c1; ++c) issue(c);
    for (int c = c0; c < c1; ++c) {
      const int younger = min(c1 - 1 - c, DNS - 2);   // chunks issued after c
      if (younger >= 2) WAIT_VMCNT(2 * RPW < 63 ? 2 * RPW : 63);
      else if (younger == 1) WAIT_VMCNT(RPW < 63 ? RPW : 63);
      else WAIT_VMCNT(0);
      __builtin_amdgcn_s_barrier();   // chunk c is in LDS; every wave is done with chunk c - 1
      COMPILER_FENCE();
      if (c + DNS - 1 < c1) issue(c + DNS - 1);
      attend(stage(c), c, [](int) {});
    }
  } else if (fp4_rows) {
   if constexpr (FP4) {
    const uint8_t* codes_b = static_cast<const uint8_t*>(kv) + (size_t)b * N_cap * 256;
    const uint8_t* scales_b = kv_scales + (size_t)b * N_cap * 32;
    auto raw = [&](int c) -> unsigned char* { return ring + 2 * DRC * PRS + (c & (DNS - 1)) * RAW4; };
    auto issue4 = [&](int c) {
      unsigned char* st = raw(c);
#pragma unroll
      for (int jj = 0; jj < 8 / NW; ++jj) {   // codes: one instruction moves 4 rows x 256 B
        const int j = wave + NW * jj;
        const int r = c * DRC + 4 * j + (lane >> 4);
        const int rid = rl[r < nr ? r : 0];
        dma16_asm(codes_b + (size_t)rid * 256 + (lane & 15) * 16, (const lds_u8*)(st + j * 1024));
      }
#pragma unroll
      for (int jj = 0; jj < 4 / NW; ++jj) {   // scales: one instruction moves 8 rows x 32 B
        const int j = wave + NW * jj;
        const int r = c * DRC + 8 * j + (lane >> 3);
        const int rid = rl[r < nr ? r : 0];
        dma4_asm(scales_b + (size_t)rid * 32 + (lane & 7) * 4, (const lds_u8*)(st + DRC * 256 + j * 256));
      }
    };
    // A code word holds 8 dims.  Its nibbles become E4M3 bytes of the same value
    // (E2M1 magnitude k -> byte via an 8-entry v_perm table, sign to bit 7), the
    // hardware FP8 conversion yields float32, the block scale multiplies, and the
    // upper halves are the exact bf16 values.
    auto to_e4m3 = [](uint32_t nib4) -> uint32_t {   // 4 nibbles, one per byte
      return __builtin_amdgcn_perm(0x4C484440u, 0x3C383000u, nib4 & 0x07070707u) | ((nib4 & 0x08080808u) << 4);
    };
    // 16 threads per row, thread l of a row takes units l, l + 16, l + 32, l + 48
    // (16-B units of the bf16 row = 8 dims = one code word): the 16 stores of a row
    // land on 16 distinct slots of the swizzled row, so they are free of bank
    // conflicts (rows of 8 threads x 8 consecutive units conflicted 4 ways).
    auto dequant = [&](int c, int h) {   // half h of the chunk's rows
      const unsigned char* st = raw(c);
      for (int x = threadIdx.x + h * (DRC * 8); x < (h + 1) * (DRC * 8); x += 64 * NW) {
        const int rr = x >> 4, l = x & 15;
        const uint32_t* crow = reinterpret_cast<const uint32_t*>(st + rr * 256);
        const unsigned char* srow = st + DRC * 256 + rr * 32;
        unsigned char* drow = dqb(c) + rr * PRS;
        const int sz = swz(rr & 15);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int unit = 16 * j + l;
          const uint32_t w = crow[unit];
          const float sc = e4m3_decode(srow[unit >> 1]);
          const uint32_t ev = to_e4m3(w & 0x0F0F0F0Fu);          // dims 0, 2, 4, 6
          const uint32_t od = to_e4m3((w >> 4) & 0x0F0F0F0Fu);   // dims 1, 3, 5, 7
          const v2f e0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)ev, false), e1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)ev, true);
          const v2f o0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)od, false), o1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)od, true);
          const uint4 h = make_uint4(bf16_pair(e0.x * sc, o0.x * sc), bf16_pair(e0.y * sc, o0.y * sc),
                                     bf16_pair(e1.x * sc, o1.x * sc), bf16_pair(e1.y * sc, o1.y * sc));
          *reinterpret_cast<uint4*>(drow + ((unit ^ sz) << 4)) = h;
        }
      }
    };
    dq_loop(std::integral_constant<int, DPW4>{}, issue4, dequant);
   }
  } else {
   if constexpr (W8) {
    const uint8_t* ring8 = static_cast<const uint8_t*>(swa) + (size_t)b * L_w * 512;
    auto raw = [&](int c) -> unsigned char* { return ring + 2 * DRC * PRS + (c & (DNS - 1)) * (DRC * 512); };
    auto issue8 = [&](int c) {   // one instruction moves 2 rows x 512 B; window rows are -(slot + 1)
      unsigned char* st = raw(c);
#pragma unroll
      for (int jj = 0; jj < 16 / NW; ++jj) {
        const int j = wave + NW * jj;
        const int r = c * DRC + 2 * j + (lane >> 5);
        const int rid = rl[r < nr ? r : 0];
        dma16_asm(ring8 + (size_t)(-rid - 1) * 512 + (lane & 31) * 16, (const lds_u8*)(st + j * 1024));
      }
    };
    // 16 threads per row, thread l of a row widening units l, l + 16, l + 32, l + 48
    // (8 dims each) into their swizzled slots, as for an FP4 chunk
    auto widen = [&](int c, int h) {   // half h of the chunk's rows
      const unsigned char* st = raw(c);
      for (int x = threadIdx.x + h * (DRC * 8); x < (h + 1) * (DRC * 8); x += 64 * NW) {
        const int rr = x >> 4, l = x & 15;
        const unsigned char* srow = st + rr * 512;
        unsigned char* drow = dqb(c) + rr * PRS;
        const int sz = swz(rr & 15);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int unit = 16 * j + l;
          const uint2 w = *reinterpret_cast<const uint2*>(srow + unit * 8);
          const v2f a0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, false), a1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, true);
          const v2f b0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, false), b1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, true);
          const uint4 h = make_uint4(bf16_pair(a0.x, a0.y), bf16_pair(a1.x, a1.y), bf16_pair(b0.x, b0.y),
                                     bf16_pair(b1.x, b1.y));
          *reinterpret_cast<uint4*>(drow + ((unit ^ sz) << 4)) = h;
        }
      }
    };
    dq_loop(std::integral_constant<int, DPW8>{}, issue8, widen);
   }
  }

  // ---- this split's normalised output and log-sum-exp (base 2) per head; the
  // sink enters once, here for a single split, else in attn_combine
  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  float lse2;
  const float inv = softmax_norm(m_run, l_tot, n_splits == 1 ? sink_log2(sink, head, H) : -INFINITY, lse2);
  typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
  if (n_splits == 1) {
    if (head < H) {
      bf16* orow = o + ((size_t)bt * H + head) * 512;
#pragma unroll
      for (int dt = 0; dt < 32; ++dt) {
        bf16x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = (bf16)(oacc[dt][i] * inv);
        *reinterpret_cast<bf16x4*>(orow + dt * 16 + 4 * lg) = v;
      }
      if (lse != nullptr && lg == 0) lse[(size_t)bt * H + head] = lse2 * 0.69314718055994531f;
    }
    return;
  }
  // A split's partial: the heads' bf16 rows go through LDS (the ring is free once
  // every wave has passed the barrier) so that the workgroup stores them as one
  // contiguous run of H KB.  Staging stride 1040 B: the 8-byte writes of a
  // half-wave (16 heads x 2 dim quads) then fall on 64 distinct banks.
  constexpr int OST = 1040;
  static_assert(OST * 16 * NW <= DNS * DRC * PRS, "staging fits in the ring");
  __syncthreads();
  unsigned char* srow = ring + (wave * 16 + lr) * OST + 8 * lg;
#pragma unroll
  for (int dt = 0; dt < 32; ++dt) {
    bf16x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (bf16)(oacc[dt][i] * inv);
    *reinterpret_cast<bf16x4*>(srow + dt * 32) = v;
  }
  const size_t prow0 = ((size_t)bt * n_splits + split) * H;
  if (head < H && lg == 0) part_lse[prow0 + head] = lse2;
  __syncthreads();
  const int nh = H < 16 * NW ? H : 16 * NW;
  uint4* pdst = reinterpret_cast<uint4*>(part_o + prow0 * 512);
  for (int u = threadIdx.x; u < nh * 64; u += 64 * NW)
    pdst[u] = *reinterpret_cast<const uint4*>(ring + (u >> 6) * OST + (u & 63) * 16);
}

// Merge of row-split partials: one thread per (query, head, 8 dims).
__global__ __launch_bounds__(256) void attn_combine_bf16(const bf16* __restrict__ part_o,
                                                         const float* __restrict__ part_lse, bf16* __restrict__ o,
                                                         float* __restrict__ lse, const float* __restrict__ sink, int Q,
                                                         int H, int n_splits) {
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long total = (long long)Q * H * 64;
  if (gid >= total) return;
  const int d0 = (int)(gid & 63) * 8;
  const long long qh = gid >> 6;
  const int h = (int)(qh % H);
  const long long qi = qh / H;
  const float* ls_q = part_lse + qi * n_splits * H + h;                    // split s at s * H
  const bf16* po_q = part_o + (qi * n_splits * H + h) * 512 + d0;          // split s at s * H * 512
  const float s2 = sink_log2(sink, h, H);   // the head's sink logit, counted once here
  // online merge, eight splits at a time: their log-sum-exps and partial rows are
  // loaded together, then the running maximum (which starts at the sink) is raised
  // to theirs and the sums rescaled, so a call costs one load round per eight
  // splits (an empty split's row is read but not used: its log-sum-exp is -inf)
  float mx = s2;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0}, den = 0.f;
  constexpr int CB = 8;
  for (int s = 0; s < n_splits; s += CB) {
    float ls[CB];
    uint4 a[CB];
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      const bool in = s + u < n_splits;
      ls[u] = in ? ls_q[(size_t)(s + u) * H] : -INFINITY;
      a[u] = in ? *reinterpret_cast<const uint4*>(po_q + (size_t)(s + u) * H * 512) : make_uint4(0, 0, 0, 0);
    }
    float cm = ls[0];
#pragma unroll
    for (int u = 1; u < CB; ++u) cm = fmaxf(cm, ls[u]);
    if (cm > mx) {   // mx = -inf (nothing yet) gives the factor 0 on the zero sums
      const float f = exp2f(mx - cm);
      den *= f;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] *= f;
      mx = cm;
    }
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      if (ls[u] == -INFINITY) continue;
      const float wgt = exp2f(ls[u] - mx);
      den += wgt;
      const uint32_t w[4] = {a[u].x, a[u].y, a[u].z, a[u].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += wgt * __uint_as_float(w[i] << 16);
        acc[2 * i + 1] += wgt * __uint_as_float(w[i] & 0xFFFF0000u);
      }
    }
  }
  if (s2 != -INFINITY) den += exp2f(s2 - mx);
  const float inv = den > 0.f ? 1.0f / den : 0.f;
  bf16x8 ov;
#pragma unroll
  for (int i = 0; i < 8; ++i) ov[i] = (bf16)(acc[i] * inv);
  *reinterpret_cast<bf16x8*>(o + (qi * H + h) * 512 + d0) = ov;
  if (lse != nullptr && d0 == 0) lse[qi * H + h] = den > 0.f ? (mx + log2f(den)) * 0.69314718055994531f : -INFINITY;
}

// ----------------------------------------------------------------- float32
// Generic path (row-major LDS chunk, scalar transposed reads); used for fp32
// tensors, whose workloads are small.

constexpr int FRC = 32;

__global__ __launch_bounds__(256) void attn_f32(const float* __restrict__ q, const float* __restrict__ kv,
                                                const int32_t* __restrict__ topk, const float* __restrict__ swa,
                                                const int32_t* __restrict__ swa_pos0, const int32_t* __restrict__ q_pos,
                                                float* __restrict__ o, float* __restrict__ lse,
                                                const float* __restrict__ sink, int T_len, int H, int N_cap, int k,
                                                int L_w, int W, float scale_log2) {
  constexpr int RSF = 512 + 4;  // floats
  __shared__ __attribute__((aligned(16))) float buf[FRC * RSF];
  __shared__ int rowlist[MAX_ROWS];
  __shared__ int n_sel_s;
  const int t = blockIdx.x, b = blockIdx.y;
  const int bt = b * T_len + t;
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int n_rows = build_rowlist(rowlist, &n_sel_s, topk + (size_t)bt * k, k, N_cap, q_pos[bt], swa_pos0[b],
                                   L_w, W, []() {});
  const float* kvb = kv + (size_t)b * N_cap * 512;
  const float* swb = swa + (size_t)b * L_w * 512;
  const int head = wave * 16 + lr;
  f32x8 qf[16];
  const float* qrow = q + ((size_t)bt * H + head) * 512;
  for (int ks = 0; ks < 16; ++ks) {
    if (head < H) qf[ks] = load_frag(qrow + ks * 32 + 8 * lg);
    else zero_frag(qf[ks]);
  }
  f32x4 oacc[32];
  for (int dt = 0; dt < 32; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  for (int r0 = 0; r0 < n_rows; r0 += FRC) {
    for (int qd = threadIdx.x; qd < FRC * 128; qd += blockDim.x) {
      const int r = qd / 128, cc = qd % 128;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (r0 + r < n_rows) v = *reinterpret_cast<const float4*>(row_ptr(rowlist[r0 + r], kvb, swb) + cc * 4);
      *reinterpret_cast<float4*>(&buf[r * RSF + cc * 4]) = v;
    }
    __syncthreads();
    f32x4 s[2];
    for (int mt = 0; mt < 2; ++mt) {
      s[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int ks = 0; ks < 16; ++ks) s[mt] = mma16(load_frag(&buf[(mt * 16 + lr) * RSF + ks * 32 + 8 * lg]), qf[ks], s[mt]);
    }
    float x[8];
    float cmax = -INFINITY;
    for (int mt = 0; mt < 2; ++mt)
      for (int i = 0; i < 4; ++i) {
        const int row = r0 + mt * 16 + 4 * lg + i;
        x[mt * 4 + i] = row < n_rows ? s[mt][i] * scale_log2 : -INFINITY;
        cmax = fmaxf(cmax, x[mt * 4 + i]);
      }
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
    const float m_new = fmaxf(m_run, cmax);
    const float alpha = exp2f(m_run - m_new);
    float psum = 0.f;
    f32x8 pf;
    for (int i = 0; i < 8; ++i) {
      pf.v[i] = exp2f(x[i] - m_new);
      psum += pf.v[i];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    for (int dt = 0; dt < 32; ++dt) {
      f32x8 a;
      const int d = dt * 16 + lr;
      for (int i = 0; i < 4; ++i) {
        a.v[i] = buf[(4 * lg + i) * RSF + d];
        a.v[4 + i] = buf[(16 + 4 * lg + i) * RSF + d];
      }
      oacc[dt] = mma16(a, pf, oacc[dt] * alpha);
    }
    __syncthreads();
  }
  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  float lse2;
  const float inv = softmax_norm(m_run, l_tot, sink_log2(sink, head, H), lse2);
  if (head < H) {
    float* orow = o + ((size_t)bt * H + head) * 512;
    for (int dt = 0; dt < 32; ++dt) {
      const int d = dt * 16 + 4 * lg;
      *reinterpret_cast<float4*>(orow + d) =
          make_float4(oacc[dt][0] * inv, oacc[dt][1] * inv, oacc[dt][2] * inv, oacc[dt][3] * inv);
    }
    if (lse != nullptr && lg == 0) lse[(size_t)bt * H + head] = lse2 * 0.69314718055994531f;
  }
}

}  // namespace

AttnPlan plan_attn(int dtype, int B, int T, int H, int k, int W, bool kv_fp4, int N_cap, bool swa_fp8, int L_w) {
  AttnPlan p{};
  const long long Q = (long long)B * T;
  p.decode = (dtype == 1) && Q < 512;
  p.kv_fp4 = kv_fp4;
  p.n_splits = 1;
  if (p.decode) {
    // A workgroup per (query, row split) keeps three 32-row chunks in flight; the
    // splits give the GPU about 256 workgroups (one per CU) and cost a partial
    // (512 bf16 + a float32 log-sum-exp) per query, split and head, merged by
    // attn_combine.
    const int max_chunks = (k + W + DRC - 1) / DRC;
    int ns = (int)((256 + Q - 1) / Q);
    if (ns > max_chunks) ns = max_chunks;
    if (ns < 1) ns = 1;
    // An FP8 window ring is read by the kernel itself when the query has two or more
    // splits anyway (with one, it is widened into a dense window first)
    p.ring_direct = swa_fp8 && (kv_fp4 || ns >= 2);
    if (kv_fp4 || p.ring_direct) {
      // selected rows (FP4 or bf16) and window rows (bf16, or FP8 from the ring) go
      // to different splits, in proportion to their chunk counts; at least one of each
      const int c4 = (k + DRC - 1) / DRC, cw = (W + DRC - 1) / DRC;
      if (ns < 2) ns = 2;
      int nw = (int)(((long long)ns * cw + (c4 + cw) / 2) / (c4 + cw));
      if (nw < 1) nw = 1;
      if (nw > ns - 1) nw = ns - 1;
      p.n_fp4 = ns - nw;
    }
    p.n_splits = ns;
  }
  if (p.decode && p.n_splits > 1)
    p.ws_bytes = (size_t)Q * p.n_splits * H * (512 * 2 + 4) + 256;
  else if (kv_fp4 && !p.decode)
    p.ws_bytes = (size_t)B * N_cap * 512 * (dtype == 1 ? 2 : 4) + 256;
  if (swa_fp8 && !p.ring_direct) {   // the ring's dense rows, then each sequence's first dense position
    p.swa_off = (p.ws_bytes + 255) / 256 * 256;
    p.ws_bytes = p.swa_off + (size_t)B * L_w * 512 * (dtype == 1 ? 2 : 4) + (size_t)B * 4 + 256;
  }
  return p;
}

hipError_t launch_sparse_attn(int dtype, const void* q, const void* kv, const uint8_t* kv_scales, const int32_t* topk,
                              const void* swa_kv, const int32_t* swa_pos0, const int32_t* q_pos, void* o, float* lse,
                              const float* sink, int B, int T, int H, int N_cap, int k, int L_w, int W, float scale,
                              void* workspace, const AttnPlan& p, hipStream_t st, bool swa_fp8) {
  if (B == 0 || T == 0) return hipSuccess;
  if (swa_fp8 && !p.ring_direct) {
    // the ring's rows of each sequence's last L_w positions, in position order, as
    // dense rows of the dtype; the attention below reads them as a dense window
    unsigned char* wb = static_cast<unsigned char*>(workspace) + p.swa_off;
    int32_t* pos0_d = reinterpret_cast<int32_t*>(wb + (size_t)B * L_w * 512 * (dtype == 1 ? 2 : 4));
    hipError_t e = launch_swa_window(dtype, static_cast<const uint8_t*>(swa_kv), q_pos, swa_pos0, wb, pos0_d, B, T,
                                     L_w, st);
    if (e != hipSuccess) return e;
    swa_kv = wb;
    swa_pos0 = pos0_d;
  }
  const float sl2 = scale * 1.4426950408889634f;
  const int nw = (H + 15) / 16;
  if (p.kv_fp4 && !p.decode) {
    // every row is read by many queries: dequantise the cache once into the workspace
    hipError_t e = launch_kv_fp4_dequant(dtype, static_cast<const uint8_t*>(kv), kv_scales, (int64_t)B * N_cap,
                                         workspace, st);
    if (e != hipSuccess) return e;
    kv = workspace;
  }
  if (dtype == 0) {
    hipLaunchKernelGGL(attn_f32, dim3(T, B), dim3(64 * nw), 0, st, static_cast<const float*>(q),
                       static_cast<const float*>(kv), topk, static_cast<const float*>(swa_kv), swa_pos0, q_pos,
                       static_cast<float*>(o), lse, sink, T, H, N_cap, k, L_w, W, sl2);
    return hipGetLastError();
  }
  const bf16* qq = static_cast<const bf16*>(q);
  const bf16* kk = static_cast<const bf16*>(kv);
  bf16* oo = static_cast<bf16*>(o);
  if (!p.decode) {
    const bf16* ss = static_cast<const bf16*>(swa_kv);
    // head pairs of 32 heads; two waves (dim halves) each
    const int tbl = std::max(1, std::min(128, (T + 7) / 8));   // tokens per run dealt to one XCD
    const dim3 grid(8 * tbl * ((T + 8 * tbl - 1) / (8 * tbl)), B);
    if (H > 32)
      hipLaunchKernelGGL(attn_prefill_bf16<4>, grid, dim3(256), 0, st, qq, kk, topk, ss, swa_pos0, q_pos,
                         oo, lse, sink, T, H, N_cap, k, L_w, W, sl2, tbl);
    else
      hipLaunchKernelGGL(attn_prefill_bf16<2>, grid, dim3(128), 0, st, qq, kk, topk, ss, swa_pos0, q_pos,
                         oo, lse, sink, T, H, N_cap, k, L_w, W, sl2, tbl);
    return hipGetLastError();
  }
  const int Q = B * T;
  const int groups = Q * p.n_splits;
  bf16* part_o = static_cast<bf16*>(workspace);
  float* part_lse = reinterpret_cast<float*>(part_o + (size_t)Q * p.n_splits * H * 512);
#define CSA2_DECODE(NWV, F4, W8)                                                                                   \
  hipLaunchKernelGGL((attn_decode_bf16<NWV, F4, W8>), dim3(groups), dim3(64 * NWV), 0, st, qq, kv, kv_scales, topk, \
                     swa_kv, swa_pos0, q_pos, oo, lse, sink, part_o, part_lse, T, H, N_cap, k, L_w, W, sl2,           \
                     p.n_splits, p.n_fp4)
#define CSA2_DECODE_NW(F4, W8)              \
  do {                                      \
    if (H > 32) CSA2_DECODE(4, F4, W8);     \
    else if (H > 16) CSA2_DECODE(2, F4, W8); \
    else CSA2_DECODE(1, F4, W8);            \
  } while (0)
  if (p.kv_fp4) {
    if (p.ring_direct) CSA2_DECODE_NW(true, true);
    else CSA2_DECODE_NW(true, false);
  } else {
    if (p.ring_direct) CSA2_DECODE_NW(false, true);
    else CSA2_DECODE_NW(false, false);
  }
#undef CSA2_DECODE_NW
#undef CSA2_DECODE
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_splits == 1) return e;
  const long long total = (long long)Q * H * 64;
  hipLaunchKernelGGL(attn_combine_bf16, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, part_o, part_lse, oo,
                     lse, sink, Q, H, p.n_splits);
  return hipGetLastError();
}

}  // namespace csa2
