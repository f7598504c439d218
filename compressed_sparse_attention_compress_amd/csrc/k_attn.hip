// (e) Sparse attention of one query token over its selected cache entries plus
// its sliding window, with key = value = the 512-d latent row.
//
// Method ([P1] "DeepSeek-V4.1 模型结构（2）…", section "一层全局注意力算四样东西":
// the layer's own query reads the k selected entries and the 128 rows of its
// sliding window; [P2] "DeepSeek v4.1 Flash技术剖析——架构篇", CSA2-FULL: one vector
// serves as key and value; [P3] "…分级缓存", section four: p_j proportional to
// exp(c_j . q / sqrt(d)), o = sum_j p_j c_j).
//
// Kernel: one workgroup per (sequence, query token); wave w owns heads 16w..16w+15.
// The token's rows (selected entries, then window positions) are listed once,
// then streamed in chunks of 32 rows through LDS, stored both row-major (for
// S^T = R Q^T, MFMA rows = cache rows, columns = heads) and transposed (for
// O^T = R^T P^T, MFMA rows = latent dims).  The S^T accumulator already has the
// layout of the P^T operand when the 32 k-slots of the PV step are numbered
// (row 4g+i of tile 0, row 4g+i of tile 1) for lane group g, so P never leaves
// registers.  Online softmax in base 2, float32 throughout; each lane owns one
// head, so the running max, sum and output rescale are per-lane scalars.
#include "csa2_internal.h"
#include "device_common.h"

namespace csa2 {

namespace {

constexpr int RC = 32;           // rows per chunk
constexpr int MAX_ROWS = 2048;   // selected + window rows per query (host-checked)

template <typename T>
struct AttnLds {
  static constexpr int KSTRIDE = 512 + 16 / (int)sizeof(T);   // row-major row stride (elements)
  static constexpr int VSTRIDE = RC + 16 / (int)sizeof(T);    // transposed row stride (elements)
};

template <typename T>
__global__ __launch_bounds__(256) void sparse_attn_kernel(
    const T* __restrict__ q, const T* __restrict__ kv, const int32_t* __restrict__ topk, const T* __restrict__ swa,
    const int32_t* __restrict__ swa_pos0, const int32_t* __restrict__ q_pos, T* __restrict__ o, float* __restrict__ lse,
    int T_len, int H, int N_cap, int k, int L_w, int W, float scale_log2) {
  typedef typename Frag<T>::type FragT;
  typedef AttnLds<T> L;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  T* Ks = reinterpret_cast<T*>(smem_raw);                       // [RC][KSTRIDE]
  T* Vt = Ks + RC * L::KSTRIDE;                                  // [512][VSTRIDE]
  int* rowlist = reinterpret_cast<int*>(Vt + 512 * L::VSTRIDE);  // [MAX_ROWS]
  __shared__ int n_sel_s;

  const int t = blockIdx.x, b = blockIdx.y;
  const int bt = b * T_len + t;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, lr = lane & 15, lg = lane >> 4;
  const int nthreads = blockDim.x;
  const int p = q_pos[bt];
  const int pos0 = swa_pos0[b];

  // ---- row list: valid selected entries (order kept), then window positions
  if (wave == 0) {
    const int32_t* tk = topk + (size_t)bt * k;
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
    if (lane == 0) n_sel_s = cnt;
  }
  __syncthreads();
  const int n_sel = n_sel_s;
  int lo = p - W + 1;
  if (lo < 0) lo = 0;
  if (lo < pos0) lo = pos0;
  int hi = p;
  if (hi > pos0 + L_w - 1) hi = pos0 + L_w - 1;
  const int n_win = hi >= lo ? hi - lo + 1 : 0;
  for (int j = threadIdx.x; j < n_win; j += nthreads) rowlist[n_sel + j] = -(lo - pos0 + j) - 1;
  const int n_rows = n_sel + n_win;
  __syncthreads();

  // ---- query fragments (B operand of S^T): head 16*wave + lr, dims 32ks + 8lg ..
  const int head = wave * 16 + lr;
  FragT qf[16];
  const T* qrow = q + ((size_t)bt * H + head) * 512;
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) {
    if (head < H) qf[ks] = load_frag(qrow + ks * 32 + 8 * lg);
    else zero_frag(qf[ks]);
  }

  f32x4 oacc[32];
#pragma unroll
  for (int dt = 0; dt < 32; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const T* kvb = kv + (size_t)b * N_cap * 512;
  const T* swb = swa + (size_t)b * L_w * 512;
  constexpr int CH = 16 / (int)sizeof(T);           // elements per 16-B chunk
  constexpr int CPR = 512 / CH;                     // chunks per row

  for (int r0 = 0; r0 < n_rows; r0 += RC) {
    // ---- stage 32 rows: row-major and transposed
    for (int qd = threadIdx.x; qd < RC * CPR; qd += nthreads) {
      const int r = qd % RC, cc = qd / RC;  // consecutive threads: consecutive rows
      uint4 v = make_uint4(0, 0, 0, 0);
      if (r0 + r < n_rows) {
        const int id = rowlist[r0 + r];
        const T* src = id >= 0 ? kvb + (size_t)id * 512 : swb + (size_t)(-id - 1) * 512;
        v = *reinterpret_cast<const uint4*>(src + cc * CH);
      }
      *reinterpret_cast<uint4*>(&Ks[r * L::KSTRIDE + cc * CH]) = v;
      const T* ve = reinterpret_cast<const T*>(&v);
#pragma unroll
      for (int e = 0; e < CH; ++e) Vt[(cc * CH + e) * L::VSTRIDE + r] = ve[e];
    }
    __syncthreads();

    // ---- S^T = R Q^T: 2 row tiles x 16 k-steps
    f32x4 s[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      s[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        FragT a = load_frag(&Ks[(mt * 16 + lr) * L::KSTRIDE + ks * 32 + 8 * lg]);
        s[mt] = mma16(a, qf[ks], s[mt]);
      }
    }
    // ---- online softmax (base 2); lane's head = lr, rows 16mt + 4lg + i
    float x[8];
    float cmax = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = r0 + mt * 16 + 4 * lg + i;
        const float v = row < n_rows ? s[mt][i] * scale_log2 : -INFINITY;
        x[mt * 4 + i] = v;
        cmax = fmaxf(cmax, v);
      }
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
    const float m_new = fmaxf(m_run, cmax);
    const float alpha = exp2f(m_run - m_new);  // m_run = -inf on the first chunk -> 0
    float psum = 0.f;
    FragT pf;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float pv = exp2f(x[i] - m_new);
      psum += pv;
      if constexpr (sizeof(T) == 2) pf[i] = (bf16)pv;
      else pf.v[i] = pv;
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) oacc[dt] *= alpha;
    // ---- O^T += R^T P^T: 32 dim tiles, one 32-row k-step
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) {
      const T* vrow = &Vt[(dt * 16 + lr) * L::VSTRIDE];
      FragT a;
      if constexpr (sizeof(T) == 2) {
        const uint2 u0 = *reinterpret_cast<const uint2*>(vrow + 4 * lg);
        const uint2 u1 = *reinterpret_cast<const uint2*>(vrow + 16 + 4 * lg);
        uint4 u = make_uint4(u0.x, u0.y, u1.x, u1.y);
        a = *reinterpret_cast<const bf16x8*>(&u);
      } else {
        const float4 u0 = *reinterpret_cast<const float4*>(vrow + 4 * lg);
        const float4 u1 = *reinterpret_cast<const float4*>(vrow + 16 + 4 * lg);
        a.v[0] = u0.x; a.v[1] = u0.y; a.v[2] = u0.z; a.v[3] = u0.w;
        a.v[4] = u1.x; a.v[5] = u1.y; a.v[6] = u1.z; a.v[7] = u1.w;
      }
      oacc[dt] = mma16(a, pf, oacc[dt]);
    }
    __syncthreads();
  }

  // ---- finish: full sum over the lane group, normalise, write
  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (head < H) {
    T* orow = o + ((size_t)bt * H + head) * 512;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) {
      const int d = dt * 16 + 4 * lg;
#pragma unroll
      for (int i = 0; i < 4; ++i) orow[d + i] = from_f32<T>(oacc[dt][i] * inv);
    }
    if (lse != nullptr && lg == 0)
      lse[(size_t)bt * H + head] = (l_tot > 0.f) ? (m_run + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
  }
}

template <typename T>
size_t attn_smem_bytes() {
  typedef AttnLds<T> L;
  return (size_t)(RC * L::KSTRIDE + 512 * L::VSTRIDE) * sizeof(T) + MAX_ROWS * sizeof(int);
}

template <typename T>
hipError_t launch_t(const void* q, const void* kv, const int32_t* topk, const void* swa, const int32_t* swa_pos0,
                    const int32_t* q_pos, void* o, float* lse, int B, int T_len, int H, int N_cap, int k, int L_w,
                    int W, float scale, hipStream_t st) {
  const int nw = (H + 15) / 16;
  const size_t smem = attn_smem_bytes<T>();
  static bool attr_set = false;
  if (!attr_set) {
    hipFuncSetAttribute(reinterpret_cast<const void*>(&sparse_attn_kernel<T>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    attr_set = true;
  }
  dim3 grid(T_len, B), blk(64 * nw);
  hipLaunchKernelGGL((sparse_attn_kernel<T>), grid, blk, smem, st, static_cast<const T*>(q),
                     static_cast<const T*>(kv), topk, static_cast<const T*>(swa), swa_pos0, q_pos,
                     static_cast<T*>(o), lse, T_len, H, N_cap, k, L_w, W, scale * 1.4426950408889634f);
  return hipGetLastError();
}

}  // namespace

size_t attn_workspace_bytes(int, int, int) { return 0; }

hipError_t launch_sparse_attn(int dtype, const void* q, const void* kv, const int32_t* topk, const void* swa_kv,
                              const int32_t* swa_pos0, const int32_t* q_pos, void* o, float* lse, int B, int T, int H,
                              int N_cap, int k, int L_w, int W, float scale, void*, hipStream_t stream) {
  if (B == 0 || T == 0) return hipSuccess;
  if (dtype == 1)
    return launch_t<bf16>(q, kv, topk, swa_kv, swa_pos0, q_pos, o, lse, B, T, H, N_cap, k, L_w, W, scale, stream);
  return launch_t<float>(q, kv, topk, swa_kv, swa_pos0, q_pos, o, lse, B, T, H, N_cap, k, L_w, W, scale, stream);
}

}  // namespace csa2
