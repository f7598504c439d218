// (e) Sparse attention of one query token over its selected cache entries plus
// its sliding window, with key = value = the 512-d latent row.
//
// Method ([P1] "DeepSeek-V4.1 模型结构（2）…", section "一层全局注意力算四样东西":
// the layer's own query reads the k selected entries and the 128 rows of its
// sliding window; [P2] "DeepSeek v4.1 Flash技术剖析——架构篇", CSA2-FULL: one vector
// serves as key and value; [P3] "…分级缓存", section four: p_j proportional to
// exp(c_j . q / sqrt(d)), o = sum_j p_j c_j).
//
// Both kernels list the token's rows once (selected entries, then window
// positions) and stream them through LDS with direct global->LDS loads
// (global_load_lds_dwordx4: one wave instruction moves one 1 KB bf16 row),
// double-buffered so the next chunk is in flight while the current one is used.
// S^T = R Q^T has cache rows as MFMA rows and 16 heads as columns; its
// accumulator already is the P^T operand of O^T = R^T P^T once the k-slots of
// the PV step are numbered (row 4g+i of tile 0, row 4g+i of tile 1) for lane
// group g.  The R^T operand is read from the row-major LDS copy with
// ds_read_b64_tr_b16 (each 16-lane group transposes 4 rows x 16 dims), so no
// transposed copy is stored.  Online softmax in base 2, float32 throughout; each
// lane owns one head, so running max, sum and rescale are per-lane scalars.
//
// attn_prefill: one workgroup per token, wave w = heads 16w..16w+15, 32-row
//   chunks shared by the waves.
// attn_decode: one workgroup per (token, row split, head group); its 4 waves take
//   interleaved 16-row chunks with private double buffers and are merged through
//   LDS at the end.  The 4 head-group workgroups of a token are numbered so they
//   land on the same XCD (block id mod 8), so its rows come from HBM once and are
//   re-read from that XCD's L2.  Row splits, when used, write float32 partials
//   (normalised output + log-sum-exp) that attn_combine merges.
#include "csa2_internal.h"
#include "device_common.h"

namespace csa2 {

namespace {

constexpr int MAX_ROWS = 2048;   // selected + window rows per query (host-checked)

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

// s_waitcnt immediates (gfx9 encoding): wait until at most n vector-memory ops
// of this wave are outstanding / until all LDS ops are done.
#define WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | 0x70 | 0xF00)
#define WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(0xC07F)

__device__ __forceinline__ void dma16(const void* gsrc, lds_u8* ldst) {
  __builtin_amdgcn_global_load_lds(gsrc, (lds_void*)ldst, 16, 0, 0);
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
// encoded as -(j+1) for swa row j.  Returns the number of rows.  Needs a
// __syncthreads() before use by other waves (done by the callers).
__device__ __forceinline__ int build_rowlist(int* rowlist, int* n_sel_s, const int32_t* tk, int k, int N_cap, int p,
                                             int pos0, int L_w, int W) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (wave == 0) {
    int cnt = 0;
    for (int j0 = 0; j0 < k; j0 += 64) {
      const int j = j0 + lane;
      const int g = j < k ? tk[j] : -1;
      const bool ok = g >= 0 && g < N_cap;
      const unsigned long long bal = __ballot(ok);
      const int before = __popcll(bal & ((1ull << lane) - 1ull));
      if (ok) rowlist[cnt + before] = g;
      cnt += __popcll(bal);
    }
    if (lane == 0) *n_sel_s = cnt;
  }
  __syncthreads();
  const int n_sel = *n_sel_s;
  int lo = p - W + 1;
  if (lo < 0) lo = 0;
  if (lo < pos0) lo = pos0;
  int hi = p;
  if (hi > pos0 + L_w - 1) hi = pos0 + L_w - 1;
  const int n_win = hi >= lo ? hi - lo + 1 : 0;
  for (int j = threadIdx.x; j < n_win; j += blockDim.x) rowlist[n_sel + j] = -(lo - pos0 + j) - 1;
  __syncthreads();
  return n_sel + n_win;
}

template <typename T>
__device__ __forceinline__ const T* row_ptr(int id, const T* kvb, const T* swb) {
  return id >= 0 ? kvb + (size_t)id * 512 : swb + (size_t)(-id - 1) * 512;
}

// ----------------------------------------------------------------- prefill

constexpr int PRC = 32;                 // rows per chunk
constexpr int PRS = 1024;               // LDS row stride (bytes) for bf16 rows (swizzled, no padding)
constexpr float RESCALE_SLACK = 8.0f;   // log2 units the running max may lag behind before rescaling

__global__ __launch_bounds__(256, 2) void attn_prefill_bf16(
    const bf16* __restrict__ q, const bf16* __restrict__ kv, const int32_t* __restrict__ topk,
    const bf16* __restrict__ swa, const int32_t* __restrict__ swa_pos0, const int32_t* __restrict__ q_pos,
    bf16* __restrict__ o, float* __restrict__ lse, int T_len, int H, int N_cap, int k, int L_w, int W,
    float scale_log2) {
  __shared__ __attribute__((aligned(16))) unsigned char buf0[PRC * PRS];
  __shared__ __attribute__((aligned(16))) unsigned char buf1[PRC * PRS];
  __shared__ int rowlist[MAX_ROWS];
  __shared__ int n_sel_s;

  const int t = blockIdx.x, b = blockIdx.y;
  const int bt = b * T_len + t;
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int nw = blockDim.x >> 6;
  const int n_rows = build_rowlist(rowlist, &n_sel_s, topk + (size_t)bt * k, k, N_cap, q_pos[bt], swa_pos0[b],
                                   L_w, W);
  const bf16* kvb = kv + (size_t)b * N_cap * 512;
  const bf16* swb = swa + (size_t)b * L_w * 512;

  const int head = wave * 16 + lr;
  bf16x8 qf[16];
  const bf16* qrow = q + ((size_t)bt * H + head) * 512;
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) {
    if (head < H) qf[ks] = load_frag(qrow + ks * 32 + 8 * lg);
    else zero_frag(qf[ks]);
  }
  f32x4 oacc[32];
#pragma unroll
  for (int dt = 0; dt < 32; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // per-lane swizzled byte offsets (within a 256-B group of 16 units)
  int soff[4], toff[8];
#pragma unroll
  for (int b = 0; b < 4; ++b) soff[b] = ((4 * b + lg) ^ swz(lr)) << 4;
#pragma unroll
  for (int b = 0; b < 8; ++b) toff[b] = ((2 * b + ((lr & 3) >> 1)) ^ swz(4 * lg + (lr >> 2))) << 4;

  const int nch = (n_rows + PRC - 1) / PRC;
  const int rows_per_wave = PRC / nw;   // nw in {1, 2, 4}: 32, 16, 8 loads per wave per chunk
  // every wave issues exactly rows_per_wave loads per chunk; rows past the end
  // repeat row 0 (finite data, masked to probability 0)
  auto issue = [&](int c, unsigned char* buf) {
    for (int j = 0; j < rows_per_wave; ++j) {
      const int rr = wave + j * nw;
      const int r = c * PRC + rr;
      const int id = rowlist[r < n_rows ? r : 0];
      const bf16* src = row_ptr(id, kvb, swb);
      dma16(reinterpret_cast<const unsigned char*>(src) + ((lane ^ swz(rr & 15)) << 4), (lds_u8*)(buf + rr * PRS));
    }
  };
  auto step = [&](int c, unsigned char* cur, unsigned char* nxt) {
    if (c + 1 < nch) {
      issue(c + 1, nxt);
      if (rows_per_wave == 8) WAIT_VMCNT(8);
      else if (rows_per_wave == 16) WAIT_VMCNT(16);
      else WAIT_VMCNT(32);
    } else {
      WAIT_VMCNT(0);
    }
    __builtin_amdgcn_s_barrier();
    const lds_u8* lcur = (const lds_u8*)cur;

    // ---- S^T = R Q^T; k-step ks = 4a + b reads unit 16a + ((4b + lg) ^ swz(lr))
    f32x4 s[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      s[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const unsigned char* srow = cur + (mt * 16 + lr) * PRS;
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(srow + soff[ks & 3] + (ks >> 2) * 256);
        s[mt] = mma16(a, qf[ks], s[mt]);
      }
    }
    // ---- online softmax; the running max is only moved (and the output
    // rescaled) when it would grow by more than RESCALE_SLACK, so exp2 values stay
    // below 2^RESCALE_SLACK and most chunks skip the rescale
    float x[8];
    float cmax = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = c * PRC + mt * 16 + 4 * lg + i;
        const float v = row < n_rows ? s[mt][i] * scale_log2 : -INFINITY;
        x[mt * 4 + i] = v;
        cmax = fmaxf(cmax, v);
      }
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
    const bool grow = cmax > m_run + RESCALE_SLACK;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float m_new = grow ? cmax : m_run;
      const float alpha = grow ? exp2f(m_run - m_new) : 1.0f;  // 0 on the first chunk
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 32; ++dt) oacc[dt] *= alpha;
      m_run = m_new;
    }
    float psum = 0.f;
    bf16x8 pf;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float pv = exp2f(x[i] - m_run);
      psum += pv;
      pf[i] = (bf16)pv;
    }
    l_run += psum;
    // ---- O^T += R^T P^T: A operand via transposed reads of rows 4g.. and 16+4g..
    // lane's rows 4g + lr/4 (and +16; same swizzle); dim tile dt = 8a + b reads
    // unit 16a + ((2b + (lr&3)/2) ^ swz(row)), half lr&1
    const lds_u8* tb = lcur + (4 * lg + (lr >> 2)) * PRS + 8 * (lr & 1);
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) {
      const int unit = toff[dt & 7] + (dt >> 3) * 256;
      const v4s lo = tr_read(tb + unit);
      const v4s hi = tr_read(tb + 16 * PRS + unit);
      bf16x8 a;
      __builtin_memcpy(&a, &lo, 8);
      __builtin_memcpy(reinterpret_cast<char*>(&a) + 8, &hi, 8);
      oacc[dt] = mma16(a, pf, oacc[dt]);
    }
    WAIT_LGKM0();
    __builtin_amdgcn_s_barrier();
  };
  if (nch > 0) issue(0, buf0);
  for (int c = 0; c < nch; c += 2) {
    step(c, buf0, buf1);
    if (c + 1 < nch) step(c + 1, buf1, buf0);
  }

  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (head < H) {
    bf16* orow = o + ((size_t)bt * H + head) * 512;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) {
      const int d = dt * 16 + 4 * lg;
      bf16x2 p0, p1;
      p0[0] = (bf16)(oacc[dt][0] * inv); p0[1] = (bf16)(oacc[dt][1] * inv);
      p1[0] = (bf16)(oacc[dt][2] * inv); p1[1] = (bf16)(oacc[dt][3] * inv);
      uint2 u;
      __builtin_memcpy(&u.x, &p0, 4);
      __builtin_memcpy(&u.y, &p1, 4);
      *reinterpret_cast<uint2*>(orow + d) = u;
    }
    if (lse != nullptr && lg == 0)
      lse[(size_t)bt * H + head] = (l_tot > 0.f) ? (m_run + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
  }
}

// ----------------------------------------------------------------- decode

constexpr int DRC = 16;                 // rows per chunk (per wave)
constexpr int DRS = 1024;               // swizzled rows, no padding

// grid.x = 32 * ceil(groups / 8), group = (query, split); block id ->
// (group, head group) so that the 4 head groups of a group share block id mod 8.
__global__ __launch_bounds__(256, 1) void attn_decode_bf16(
    const bf16* __restrict__ q, const bf16* __restrict__ kv, const int32_t* __restrict__ topk,
    const bf16* __restrict__ swa, const int32_t* __restrict__ swa_pos0, const int32_t* __restrict__ q_pos,
    bf16* __restrict__ o, float* __restrict__ lse, float* __restrict__ part_o, float* __restrict__ part_lse,
    int Q, int T_len, int H, int N_cap, int k, int L_w, int W, float scale_log2, int n_splits) {
  __shared__ __attribute__((aligned(16))) unsigned char bufA[4 * DRC * DRS];   // per-wave buffer 0
  __shared__ __attribute__((aligned(16))) unsigned char bufB[4 * DRC * DRS];   // per-wave buffer 1
  __shared__ int rowlist[MAX_ROWS];
  __shared__ int n_sel_s;
  __shared__ float wm[4][16], wl[4][16];

  const int id = blockIdx.x;
  const int hg = (id >> 3) & 3;
  const int group = (id >> 5) * 8 + (id & 7);
  if (group >= Q * n_splits) return;
  const int qi = group / n_splits, split = group % n_splits;
  const int b = qi / T_len, t = qi % T_len;
  const int bt = qi;
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int n_rows = build_rowlist(rowlist, &n_sel_s, topk + (size_t)bt * k, k, N_cap, q_pos[bt], swa_pos0[b],
                                   L_w, W);
  const bf16* kvb = kv + (size_t)b * N_cap * 512;
  const bf16* swb = swa + (size_t)b * L_w * 512;

  const int head = hg * 16 + lr;
  bf16x8 qf[16];
  const bf16* qrow = q + ((size_t)bt * H + head) * 512;
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) {
    if (head < H) qf[ks] = load_frag(qrow + ks * 32 + 8 * lg);
    else zero_frag(qf[ks]);
  }
  f32x4 oacc[32];
#pragma unroll
  for (int dt = 0; dt < 32; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  int soff[4], toff[8];
#pragma unroll
  for (int b = 0; b < 4; ++b) soff[b] = ((4 * b + lg) ^ swz(lr)) << 4;
#pragma unroll
  for (int b = 0; b < 8; ++b) toff[b] = ((2 * b + ((lr & 3) >> 1)) ^ swz(4 * lg + (lr >> 2))) << 4;
  // this split's range of 64-row chunks; wave w owns rows 16w..16w+15 of each
  const int nch_all = (n_rows + 4 * DRC - 1) / (4 * DRC);
  const int c0 = (int)(((long long)nch_all * split) / n_splits);
  const int c1 = (int)(((long long)nch_all * (split + 1)) / n_splits);
  unsigned char* myA = bufA + wave * DRC * DRS;
  unsigned char* myB = bufB + wave * DRC * DRS;
  // (the trip count is read from blockDim so that the compiler leaves the
  // vector-memory wait counts to the explicit waits below)
  const int drc_rt = (int)(blockDim.x >> 4);   // == DRC for the 256-thread launch
  auto issue = [&](int c, unsigned char* buf) {
    for (int rr = 0; rr < drc_rt; ++rr) {
      const int r = c * 4 * DRC + wave * DRC + rr;
      const int rid = rowlist[r < n_rows ? r : 0];
      dma16(reinterpret_cast<const unsigned char*>(row_ptr(rid, kvb, swb)) + ((lane ^ swz(rr)) << 4),
            (lds_u8*)(buf + rr * DRS));
    }
  };
  auto step = [&](int c, unsigned char* cur, unsigned char* nxt) {
    if (c + 1 < c1) {
      issue(c + 1, nxt);
      WAIT_VMCNT(DRC);
    } else {
      WAIT_VMCNT(0);
    }
    __builtin_amdgcn_s_barrier();
    // S^T: 16 rows x 16 heads
    f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(cur + lr * DRS + soff[ks & 3] + (ks >> 2) * 256);
      s = mma16(a, qf[ks], s);
    }
    float x[4];
    float cmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = c * 4 * DRC + wave * DRC + 4 * lg + i;
      x[i] = row < n_rows ? s[i] * scale_log2 : -INFINITY;
      cmax = fmaxf(cmax, x[i]);
    }
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
    const bool grow = cmax > m_run + RESCALE_SLACK;   // false while cmax = -inf
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float m_new = grow ? cmax : m_run;
      const float alpha = grow ? exp2f(m_run - m_new) : 1.0f;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 32; ++dt) oacc[dt] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.0f : m_run;
    float psum = 0.f;
    v4s pf;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pv = exp2f(x[i] - m_use);
      psum += pv;
      bf16 hb = (bf16)pv;
      __builtin_memcpy(reinterpret_cast<char*>(&pf) + 2 * i, &hb, 2);
    }
    l_run += psum;
    const lds_u8* tb = (const lds_u8*)cur + (4 * lg + (lr >> 2)) * DRS + 8 * (lr & 1);
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) {
      const v4s a = tr_read(tb + toff[dt & 7] + (dt >> 3) * 256);
      oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pf, oacc[dt], 0, 0, 0);
    }
    WAIT_LGKM0();
  };
  if (c0 < c1) issue(c0, myA);
  for (int c = c0; c < c1; c += 2) {
    step(c, myA, myB);
    if (c + 1 < c1) step(c + 1, myB, myA);
  }

  // ---- merge the 4 waves through LDS (reusing the row buffers)
  float l_w = l_run + __shfl_xor(l_run, 16, 64);
  l_w += __shfl_xor(l_w, 32, 64);
  __syncthreads();
  if (lg == 0) {
    wm[wave][lr] = m_run;
    wl[wave][lr] = l_w;
  }
  // per-wave [16 heads][512] float32 blocks: waves 0,1 in bufA, waves 2,3 in bufB
  auto wave_block = [&](int w) -> float* {
    return reinterpret_cast<float*>((w < 2 ? bufA : bufB) + (w & 1) * (16 * 512 * 4));
  };
  {
    float* mine = wave_block(wave);
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) *reinterpret_cast<f32x4*>(&mine[lr * 512 + dt * 16 + 4 * lg]) = oacc[dt];
  }
  __syncthreads();
  {
    const int h = threadIdx.x >> 4;          // head within the group
    const int d0 = (threadIdx.x & 15) * 32;  // 32 dims per thread
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) mx = fmaxf(mx, wm[w][h]);
    float sc[4], den = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      sc[w] = (wm[w][h] == -INFINITY) ? 0.f : exp2f(wm[w][h] - mx);
      den += sc[w] * wl[w][h];
    }
    const float inv = den > 0.f ? 1.0f / den : 0.f;
    const int hh = hg * 16 + h;
    if (hh < H) {
      if (n_splits == 1) {
        bf16* orow = o + ((size_t)bt * H + hh) * 512 + d0;
        for (int d = 0; d < 32; d += 2) {
          float v0 = 0.f, v1 = 0.f;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            v0 += sc[w] * wave_block(w)[h * 512 + d0 + d];
            v1 += sc[w] * wave_block(w)[h * 512 + d0 + d + 1];
          }
          bf16x2 pr;
          pr[0] = (bf16)(v0 * inv);
          pr[1] = (bf16)(v1 * inv);
          *reinterpret_cast<bf16x2*>(orow + d) = pr;
        }
        if (lse != nullptr && (threadIdx.x & 15) == 0)
          lse[(size_t)bt * H + hh] = den > 0.f ? (mx + log2f(den)) * 0.69314718055994531f : -INFINITY;
      } else {
        float* prow = part_o + (((size_t)bt * n_splits + split) * H + hh) * 512 + d0;
        for (int d = 0; d < 32; ++d) {
          float v = 0.f;
#pragma unroll
          for (int w = 0; w < 4; ++w) v += sc[w] * wave_block(w)[h * 512 + d0 + d];
          prow[d] = v * inv;
        }
        if ((threadIdx.x & 15) == 0)
          part_lse[((size_t)bt * n_splits + split) * H + hh] = den > 0.f ? mx + log2f(den) : -INFINITY;
      }
    }
  }
}

// Merge of row-split partials: one thread per (query, head, 8 dims).
__global__ __launch_bounds__(256) void attn_combine_bf16(const float* __restrict__ part_o,
                                                         const float* __restrict__ part_lse, bf16* __restrict__ o,
                                                         float* __restrict__ lse, int Q, int H, int n_splits) {
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long total = (long long)Q * H * 64;
  if (gid >= total) return;
  const int d0 = (int)(gid & 63) * 8;
  const long long qh = gid >> 6;
  const int h = (int)(qh % H);
  const long long qi = qh / H;
  float mx = -INFINITY;
  for (int s = 0; s < n_splits; ++s) mx = fmaxf(mx, part_lse[(qi * n_splits + s) * H + h]);
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0}, den = 0.f;
  for (int s = 0; s < n_splits; ++s) {
    const float ls = part_lse[(qi * n_splits + s) * H + h];
    if (ls == -INFINITY) continue;
    const float wgt = exp2f(ls - mx);
    den += wgt;
    const float* pr = part_o + ((qi * n_splits + s) * H + h) * 512 + d0;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += wgt * pr[i];
  }
  const float inv = den > 0.f ? 1.0f / den : 0.f;
  bf16* orow = o + (qi * H + h) * 512 + d0;
#pragma unroll
  for (int i = 0; i < 8; ++i) orow[i] = (bf16)(acc[i] * inv);
  if (lse != nullptr && d0 == 0) lse[qi * H + h] = den > 0.f ? (mx + log2f(den)) * 0.69314718055994531f : -INFINITY;
}

// ----------------------------------------------------------------- float32
// Generic path (row-major LDS chunk, scalar transposed reads); used for fp32
// tensors, whose workloads are small.

constexpr int FRC = 32;

__global__ __launch_bounds__(256) void attn_f32(const float* __restrict__ q, const float* __restrict__ kv,
                                                const int32_t* __restrict__ topk, const float* __restrict__ swa,
                                                const int32_t* __restrict__ swa_pos0, const int32_t* __restrict__ q_pos,
                                                float* __restrict__ o, float* __restrict__ lse, int T_len, int H,
                                                int N_cap, int k, int L_w, int W, float scale_log2) {
  constexpr int RSF = 512 + 4;  // floats
  __shared__ __attribute__((aligned(16))) float buf[FRC * RSF];
  __shared__ int rowlist[MAX_ROWS];
  __shared__ int n_sel_s;
  const int t = blockIdx.x, b = blockIdx.y;
  const int bt = b * T_len + t;
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int n_rows = build_rowlist(rowlist, &n_sel_s, topk + (size_t)bt * k, k, N_cap, q_pos[bt], swa_pos0[b],
                                   L_w, W);
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
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (head < H) {
    float* orow = o + ((size_t)bt * H + head) * 512;
    for (int dt = 0; dt < 32; ++dt) {
      const int d = dt * 16 + 4 * lg;
      *reinterpret_cast<float4*>(orow + d) =
          make_float4(oacc[dt][0] * inv, oacc[dt][1] * inv, oacc[dt][2] * inv, oacc[dt][3] * inv);
    }
    if (lse != nullptr && lg == 0)
      lse[(size_t)bt * H + head] = (l_tot > 0.f) ? (m_run + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
  }
}

}  // namespace

AttnPlan plan_attn(int dtype, int B, int T, int H, int k, int W) {
  AttnPlan p{};
  const long long Q = (long long)B * T;
  p.decode = (dtype == 1) && Q < 512;
  p.n_splits = 1;
  if (p.decode) {
    // Each (query, head group) workgroup streams all of the query's rows, so the
    // time of one call is about that of one workgroup; row splits only pay for
    // their float32 partials (128 KB per query and split) when the batch is too
    // small to give each CU a workgroup.
    const int max_chunks = (k + W + 4 * DRC - 1) / (4 * DRC);
    int ns = 1;
    if (Q * 4 < 128) {
      ns = (int)(256 / (Q * 4));
      if (ns > max_chunks) ns = max_chunks;
      if (ns < 1) ns = 1;
    }
    p.n_splits = ns;
  }
  p.ws_bytes = (p.decode && p.n_splits > 1) ? (size_t)Q * p.n_splits * H * (512 + 1) * 4 + 256 : 0;
  return p;
}

hipError_t launch_sparse_attn(int dtype, const void* q, const void* kv, const int32_t* topk, const void* swa_kv,
                              const int32_t* swa_pos0, const int32_t* q_pos, void* o, float* lse, int B, int T, int H,
                              int N_cap, int k, int L_w, int W, float scale, void* workspace, const AttnPlan& p,
                              hipStream_t st) {
  if (B == 0 || T == 0) return hipSuccess;
  const float sl2 = scale * 1.4426950408889634f;
  const int nw = (H + 15) / 16;
  if (dtype == 0) {
    hipLaunchKernelGGL(attn_f32, dim3(T, B), dim3(64 * nw), 0, st, static_cast<const float*>(q),
                       static_cast<const float*>(kv), topk, static_cast<const float*>(swa_kv), swa_pos0, q_pos,
                       static_cast<float*>(o), lse, T, H, N_cap, k, L_w, W, sl2);
    return hipGetLastError();
  }
  const bf16* qq = static_cast<const bf16*>(q);
  const bf16* kk = static_cast<const bf16*>(kv);
  const bf16* ss = static_cast<const bf16*>(swa_kv);
  bf16* oo = static_cast<bf16*>(o);
  if (!p.decode) {
    const int nwp = nw == 3 ? 4 : nw;   // 1, 2 or 4 waves (32 rows split evenly)
    hipLaunchKernelGGL(attn_prefill_bf16, dim3(T, B), dim3(64 * nwp), 0, st, qq, kk, topk, ss, swa_pos0, q_pos, oo,
                       lse, T, H, N_cap, k, L_w, W, sl2);
    return hipGetLastError();
  }
  const int Q = B * T;
  const int groups = Q * p.n_splits;
  float* part_o = static_cast<float*>(workspace);
  float* part_lse = part_o + (size_t)Q * p.n_splits * H * 512;
  hipLaunchKernelGGL(attn_decode_bf16, dim3(32 * ((groups + 7) / 8)), dim3(256), 0, st, qq, kk, topk, ss, swa_pos0,
                     q_pos, oo, lse, part_o, part_lse, Q, T, H, N_cap, k, L_w, W, sl2, p.n_splits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_splits == 1) return e;
  const long long total = (long long)Q * H * 64;
  hipLaunchKernelGGL(attn_combine_bf16, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, part_o, part_lse, oo,
                     lse, Q, H, p.n_splits);
  return hipGetLastError();
}

}  // namespace csa2
