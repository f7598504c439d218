// Host side of the CSA2 C ABI: argument validation, the shared runtime slots,
// mode dispatch and workspace sizing.  No device memory is allocated here.
//
// Slots follow [P1] "DeepSeek-V4.1 模型结构（2）…", section "共享池里有四样东西":
// one position per slot, no per-layer numbering, only borrowed pointers; a Full
// layer publishes main KV (and index K, which Reindex layers read, [P2] mode
// table), Full and Reindex layers publish top-k indices, and a Full layer that
// builds the hierarchical pool publishes the candidates ([P2] CSA2-ReIndex).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>

#include "csa2.h"
#include "csa2_internal.h"

struct csa2_runtime {
  struct Slot {
    int filled = 0;
    uint64_t generation = 0;
    const void* ptr = nullptr;
    const void* ptr2 = nullptr;
    int dtype = 0, B = 0, rows = 0, cols = 0, extra = 0, kv_fmt = 0;
  } slot[4];
};

namespace {

thread_local char g_err[512] = "";

csa2_status fail(csa2_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}
csa2_status ok() {
  g_err[0] = 0;
  return CSA2_OK;
}
csa2_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(CSA2_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}
bool dtype_ok(int d) { return d == CSA2_F32 || d == CSA2_BF16; }
hipStream_t st(csa2_stream s) { return reinterpret_cast<hipStream_t>(s); }

void publish(csa2_runtime* rt, csa2_slot which, const void* p, const void* p2, int dtype, int B, int rows, int cols,
             int extra, int kv_fmt = CSA2_KV_DENSE) {
  if (!rt) return;
  auto& s = rt->slot[which];
  s.kv_fmt = kv_fmt;
  s.filled = 1;
  s.generation += 1;
  s.ptr = p;
  s.ptr2 = p2;
  s.dtype = dtype;
  s.B = B;
  s.rows = rows;
  s.cols = cols;
  s.extra = extra;
}

#define REQ(cond, code, ...) \
  do {                       \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

csa2_status check_compress(const csa2_compress_args* a) {
  REQ(a, CSA2_ERR_INVALID_ARG, "csa2_compress: args is NULL");
  REQ(dtype_ok(a->dtype), CSA2_ERR_DTYPE, "csa2_compress: unsupported dtype %d", a->dtype);
  REQ(a->m == 1 || a->m == 2 || a->m == 4, CSA2_ERR_INVALID_ARG, "csa2_compress: m must be 1, 2 or 4 (got %d)", a->m);
  REQ(a->m == 1 || a->w_gate != nullptr, CSA2_ERR_INVALID_ARG, "csa2_compress: m > 1 needs w_gate");
  REQ(a->m > 1 || a->w_gate == nullptr, CSA2_ERR_INVALID_ARG, "csa2_compress: m == 1 has no gate; w_gate must be NULL");
  REQ(a->B >= 0 && a->T >= 0 && a->D > 0, CSA2_ERR_SHAPE, "csa2_compress: bad B/T/D");
  REQ(a->T % a->m == 0, CSA2_ERR_SHAPE, "csa2_compress: T (%d) must be a multiple of m (%d)", a->T, a->m);
  REQ(a->D % 64 == 0, CSA2_ERR_SHAPE, "csa2_compress: D (%d) must be a multiple of 64", a->D);
  REQ(a->start_pos >= 0 && a->start_pos % a->m == 0, CSA2_ERR_SHAPE, "csa2_compress: start_pos must be >= 0 and a multiple of m");
  REQ((long long)a->start_pos / a->m + a->T / a->m <= a->N_cap, CSA2_ERR_SHAPE,
      "csa2_compress: cache too small (N_cap %d < %d)", a->N_cap, a->start_pos / a->m + a->T / a->m);
  REQ(a->x && a->w_kv && a->gamma && a->latent_pre && a->kv_cache, CSA2_ERR_INVALID_ARG, "csa2_compress: NULL tensor");
  REQ(a->kv_fmt == CSA2_KV_DENSE || a->kv_fmt == CSA2_KV_FP4, CSA2_ERR_INVALID_ARG, "csa2_compress: bad kv_fmt %d",
      a->kv_fmt);
  REQ(a->kv_fmt != CSA2_KV_FP4 || a->kv_scales != nullptr, CSA2_ERR_INVALID_ARG,
      "csa2_compress: FP4 main KV needs kv_scales");
  REQ(a->kv_fmt != CSA2_KV_FP4 || ((uintptr_t)a->kv_cache & 15u) == 0, CSA2_ERR_INVALID_ARG,
      "csa2_compress: FP4 codes must be 16-byte aligned");
  REQ(a->eps >= 0.f && a->rope_base > 0.f, CSA2_ERR_INVALID_ARG, "csa2_compress: bad eps/rope_base");
  return CSA2_OK;
}

csa2_status check_compress_step(const csa2_compress_step_args* a) {
  REQ(a, CSA2_ERR_INVALID_ARG, "csa2_compress_step: args is NULL");
  REQ(dtype_ok(a->dtype), CSA2_ERR_DTYPE, "csa2_compress_step: unsupported dtype %d", a->dtype);
  REQ(a->m == 1 || a->m == 2 || a->m == 4, CSA2_ERR_INVALID_ARG, "csa2_compress_step: m must be 1, 2 or 4 (got %d)",
      a->m);
  REQ(a->m == 1 || (a->w_gate != nullptr && a->state != nullptr), CSA2_ERR_INVALID_ARG,
      "csa2_compress_step: m > 1 needs w_gate and state");
  REQ(a->m > 1 || a->w_gate == nullptr, CSA2_ERR_INVALID_ARG,
      "csa2_compress_step: m == 1 has no gate; w_gate must be NULL");
  REQ(a->B >= 0 && a->D > 0 && a->D % 64 == 0, CSA2_ERR_SHAPE, "csa2_compress_step: bad B/D (D %% 64 == 0)");
  REQ(a->N_cap >= 0, CSA2_ERR_SHAPE, "csa2_compress_step: bad N_cap");
  REQ(a->x && a->pos && a->w_kv && a->gamma && a->w_ik && a->kv_cache && a->ik_codes && a->ik_scales,
      CSA2_ERR_INVALID_ARG, "csa2_compress_step: NULL tensor");
  REQ(a->eps >= 0.f && a->rope_base > 0.f, CSA2_ERR_INVALID_ARG, "csa2_compress_step: bad eps/rope_base");
  REQ(a->kv_fmt == CSA2_KV_DENSE || a->kv_fmt == CSA2_KV_FP4, CSA2_ERR_INVALID_ARG,
      "csa2_compress_step: bad kv_fmt %d", a->kv_fmt);
  REQ(a->kv_fmt != CSA2_KV_FP4 || a->kv_scales != nullptr, CSA2_ERR_INVALID_ARG,
      "csa2_compress_step: FP4 main KV needs kv_scales");
  REQ(a->scale_fmt == CSA2_SCALE_E4M3 || a->scale_fmt == CSA2_SCALE_UE8M0, CSA2_ERR_INVALID_ARG,
      "csa2_compress_step: bad scale_fmt %d", a->scale_fmt);
  const size_t need = (size_t)a->B * 1024 * 4 * 4;   // C and Z partials of 4 K quarters
  REQ(a->B == 0 || (a->workspace != nullptr && a->workspace_bytes >= need), CSA2_ERR_WORKSPACE,
      "csa2_compress_step: workspace of %zu bytes needed (got %zu)", need, a->workspace_bytes);
  REQ(a->B == 0 || ((uintptr_t)a->workspace & 15u) == 0, CSA2_ERR_WORKSPACE,
      "csa2_compress_step: workspace not 16-byte aligned");
  return CSA2_OK;
}

csa2_status check_index_k(const csa2_index_k_args* a) {
  REQ(a, CSA2_ERR_INVALID_ARG, "csa2_index_k: args is NULL");
  REQ(dtype_ok(a->dtype), CSA2_ERR_DTYPE, "csa2_index_k: unsupported dtype %d", a->dtype);
  REQ(a->B >= 0 && a->N >= 0 && a->m >= 1 && a->entry0 >= 0, CSA2_ERR_SHAPE, "csa2_index_k: bad B/N/m/entry0");
  REQ((long long)a->entry0 + a->N <= a->N_cap, CSA2_ERR_SHAPE, "csa2_index_k: cache too small");
  REQ(a->latent_pre && a->w_ik && a->codes && a->scales, CSA2_ERR_INVALID_ARG, "csa2_index_k: NULL tensor");
  REQ(a->rope_base > 0.f, CSA2_ERR_INVALID_ARG, "csa2_index_k: bad rope_base");
  REQ(a->scale_fmt == CSA2_SCALE_E4M3 || a->scale_fmt == CSA2_SCALE_UE8M0, CSA2_ERR_INVALID_ARG,
      "csa2_index_k: bad scale_fmt %d", a->scale_fmt);
  return CSA2_OK;
}

bool pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

// Fills codes/scales/candidates from the runtime when NULL and validates.
csa2_status resolve_score(const csa2_runtime* rt, csa2_score_topk_args& a) {
  REQ(dtype_ok(a.dtype), CSA2_ERR_DTYPE, "csa2_score_topk: unsupported dtype %d", a.dtype);
  REQ(a.B >= 0 && a.T >= 0, CSA2_ERR_SHAPE, "csa2_score_topk: bad B/T");
  REQ(a.H_I >= 1 && a.H_I <= 32, CSA2_ERR_SHAPE, "csa2_score_topk: H_I must be in [1, 32] (got %d)", a.H_I);
  REQ(a.m >= 1, CSA2_ERR_INVALID_ARG, "csa2_score_topk: m must be >= 1");
  REQ(a.N_cap >= 1, CSA2_ERR_SHAPE, "csa2_score_topk: N_cap must be >= 1");
  REQ(a.k >= 1 && a.k <= CSA2_MAX_TOPK, CSA2_ERR_SHAPE, "csa2_score_topk: k must be in [1, %d]", CSA2_MAX_TOPK);
  REQ(a.hsi >= CSA2_HSI_NONE && a.hsi <= CSA2_HSI_USE, CSA2_ERR_INVALID_ARG, "csa2_score_topk: bad hsi mode");
  if (a.hsi != CSA2_HSI_NONE) {
    REQ(pow2(a.hsi_s) && a.hsi_s <= 8192, CSA2_ERR_SHAPE, "csa2_score_topk: hsi_s must be a power of two <= 8192");
    REQ(a.hsi_nb >= 1 && a.hsi_nb <= 1024, CSA2_ERR_SHAPE, "csa2_score_topk: hsi_nb must be in [1, 1024]");
  }
  if (a.codes == nullptr && a.scales == nullptr) {
    REQ(rt != nullptr, CSA2_ERR_INVALID_ARG, "csa2_score_topk: no index K given and no runtime");
    const auto& s = rt->slot[CSA2_SLOT_INDEX_K];
    REQ(s.filled, CSA2_ERR_SLOT_EMPTY, "csa2_score_topk: index_k slot is empty (no Full layer ran)");
    REQ(s.B == a.B && s.rows == a.N_cap, CSA2_ERR_SLOT_MISMATCH,
        "csa2_score_topk: index_k slot is [B=%d, N_cap=%d], call has [B=%d, N_cap=%d]", s.B, s.rows, a.B, a.N_cap);
    REQ(a.n_entries <= s.cols, CSA2_ERR_SLOT_MISMATCH, "csa2_score_topk: n_entries %d exceeds the slot's %d",
        a.n_entries, s.cols);
    a.codes = static_cast<const uint8_t*>(s.ptr);
    a.scales = static_cast<const uint8_t*>(s.ptr2);
    a.scale_fmt = s.kv_fmt;   // the index_k slot records its scale format
  }
  REQ(a.scale_fmt == CSA2_SCALE_E4M3 || a.scale_fmt == CSA2_SCALE_UE8M0, CSA2_ERR_INVALID_ARG,
      "csa2_score_topk: bad scale_fmt %d", a.scale_fmt);
  REQ(a.codes && a.scales, CSA2_ERR_INVALID_ARG, "csa2_score_topk: codes and scales must both be given or both NULL");
  REQ(a.n_entries >= 0 && a.n_entries <= a.N_cap, CSA2_ERR_SHAPE, "csa2_score_topk: n_entries must be in [0, N_cap]");
  if (a.hsi == CSA2_HSI_USE && a.candidates == nullptr) {
    REQ(rt != nullptr, CSA2_ERR_INVALID_ARG, "csa2_score_topk: HSI USE without candidates and no runtime");
    const auto& s = rt->slot[CSA2_SLOT_CANDIDATES];
    REQ(s.filled, CSA2_ERR_SLOT_EMPTY, "csa2_score_topk: candidates slot is empty (no Full layer built a pool)");
    REQ(s.B == a.B && s.rows == a.T && s.cols == a.hsi_nb && s.extra == a.hsi_s, CSA2_ERR_SLOT_MISMATCH,
        "csa2_score_topk: candidates slot [B=%d,T=%d,n_b=%d,s=%d] does not fit [B=%d,T=%d,n_b=%d,s=%d]", s.B, s.rows,
        s.cols, s.extra, a.B, a.T, a.hsi_nb, a.hsi_s);
    a.candidates = const_cast<int32_t*>(static_cast<const int32_t*>(s.ptr));
  }
  REQ(a.q_idx && a.w && a.q_pos && a.topk, CSA2_ERR_INVALID_ARG, "csa2_score_topk: NULL tensor");
  REQ(a.hsi == CSA2_HSI_NONE || a.candidates != nullptr, CSA2_ERR_INVALID_ARG, "csa2_score_topk: candidates is NULL");
  REQ(((uintptr_t)a.scores & 3u) == 0, CSA2_ERR_INVALID_ARG, "csa2_score_topk: scores must be 4-byte aligned");
  return CSA2_OK;
}

int score_scan(const csa2_score_topk_args& a) {
  return a.hsi == CSA2_HSI_USE ? a.hsi_nb * a.hsi_s : a.n_entries;
}

csa2_status resolve_attn(const csa2_runtime* rt, csa2_sparse_attn_args& a) {
  REQ(dtype_ok(a.dtype), CSA2_ERR_DTYPE, "csa2_sparse_attn: unsupported dtype %d", a.dtype);
  REQ(a.B >= 0 && a.T >= 0 && a.H >= 1 && a.H <= 64, CSA2_ERR_SHAPE, "csa2_sparse_attn: H must be in [1, 64]");
  REQ(a.k >= 0 && a.k <= CSA2_MAX_TOPK, CSA2_ERR_SHAPE, "csa2_sparse_attn: k must be in [0, %d]", CSA2_MAX_TOPK);
  REQ(a.W >= 1 && a.k + a.W <= 2048, CSA2_ERR_SHAPE, "csa2_sparse_attn: need W >= 1 and k + W <= 2048");
  REQ(a.L_w >= 1, CSA2_ERR_SHAPE, "csa2_sparse_attn: L_w must be >= 1");
  if (a.kv == nullptr) {
    REQ(rt != nullptr, CSA2_ERR_INVALID_ARG, "csa2_sparse_attn: no kv given and no runtime");
    const auto& s = rt->slot[CSA2_SLOT_COMPRESS_KV];
    REQ(s.filled, CSA2_ERR_SLOT_EMPTY, "csa2_sparse_attn: compress_kv slot is empty (no Full layer ran)");
    REQ(s.B == a.B && s.dtype == a.dtype, CSA2_ERR_SLOT_MISMATCH, "csa2_sparse_attn: compress_kv slot does not fit");
    a.kv = s.ptr;
    a.N_cap = s.rows;
    a.kv_fmt = s.kv_fmt;
    a.kv_scales = static_cast<const uint8_t*>(s.ptr2);
  }
  REQ(a.kv_fmt == CSA2_KV_DENSE || a.kv_fmt == CSA2_KV_FP4, CSA2_ERR_INVALID_ARG, "csa2_sparse_attn: bad kv_fmt %d",
      a.kv_fmt);
  REQ(a.kv_fmt != CSA2_KV_FP4 || a.kv_scales != nullptr, CSA2_ERR_INVALID_ARG,
      "csa2_sparse_attn: FP4 main KV needs kv_scales");
  REQ(a.kv_fmt != CSA2_KV_FP4 || (((uintptr_t)a.kv & 15u) == 0 && ((uintptr_t)a.kv_scales & 3u) == 0),
      CSA2_ERR_INVALID_ARG, "csa2_sparse_attn: FP4 codes must be 16-byte and scales 4-byte aligned");
  if (a.topk == nullptr) {
    REQ(rt != nullptr, CSA2_ERR_INVALID_ARG, "csa2_sparse_attn: no topk given and no runtime");
    const auto& s = rt->slot[CSA2_SLOT_TOPK_IDXS];
    REQ(s.filled, CSA2_ERR_SLOT_EMPTY, "csa2_sparse_attn: topk_idxs slot is empty (no Full or Reindex layer ran)");
    REQ(s.B == a.B && s.rows == a.T && s.cols == a.k, CSA2_ERR_SLOT_MISMATCH,
        "csa2_sparse_attn: topk_idxs slot [B=%d,T=%d,k=%d] does not fit [B=%d,T=%d,k=%d]", s.B, s.rows, s.cols, a.B,
        a.T, a.k);
    a.topk = static_cast<const int32_t*>(s.ptr);
  }
  REQ(a.N_cap >= 0, CSA2_ERR_SHAPE, "csa2_sparse_attn: bad N_cap");
  REQ(a.q && a.kv && a.topk && a.swa_kv && a.swa_pos0 && a.q_pos && a.o, CSA2_ERR_INVALID_ARG,
      "csa2_sparse_attn: NULL tensor");
  REQ(a.swa_fmt == CSA2_SWA_DENSE || a.swa_fmt == CSA2_SWA_FP8_RING, CSA2_ERR_INVALID_ARG,
      "csa2_sparse_attn: bad swa_fmt %d", a.swa_fmt);
  REQ(a.swa_fmt != CSA2_SWA_FP8_RING || a.W <= a.L_w, CSA2_ERR_SHAPE,
      "csa2_sparse_attn: an FP8 window ring of L_w = %d rows cannot serve a window of W = %d", a.L_w, a.W);
  REQ(a.swa_fmt != CSA2_SWA_FP8_RING || ((uintptr_t)a.swa_kv & 15u) == 0, CSA2_ERR_INVALID_ARG,
      "csa2_sparse_attn: the FP8 window ring must be 16-byte aligned");
  REQ((((uintptr_t)a.q | (uintptr_t)a.o) & 15u) == 0 && (a.kv_fmt == CSA2_KV_FP4 || ((uintptr_t)a.kv & 15u) == 0) &&
          (a.swa_fmt == CSA2_SWA_FP8_RING || ((uintptr_t)a.swa_kv & 15u) == 0),
      CSA2_ERR_INVALID_ARG, "csa2_sparse_attn: q, o and dense kv and window rows must be 16-byte aligned");
  return CSA2_OK;
}

csa2::AttnPlan attn_plan(const csa2_sparse_attn_args& a) {
  return csa2::plan_attn(a.dtype, a.B, a.T, a.H, a.k, a.W, a.kv_fmt == CSA2_KV_FP4, a.N_cap,
                         a.swa_fmt == CSA2_SWA_FP8_RING, a.L_w);
}

}  // namespace

extern "C" {

const char* csa2_version(void) { return "csa2-mi355x 0.1 gfx950"; }

const char* csa2_status_string(csa2_status s) {
  switch (s) {
    case CSA2_OK: return "ok";
    case CSA2_ERR_INVALID_ARG: return "invalid argument";
    case CSA2_ERR_SHAPE: return "bad shape";
    case CSA2_ERR_DTYPE: return "unsupported dtype";
    case CSA2_ERR_SLOT_EMPTY: return "runtime slot empty";
    case CSA2_ERR_SLOT_MISMATCH: return "runtime slot mismatch";
    case CSA2_ERR_WORKSPACE: return "workspace too small";
    case CSA2_ERR_HIP: return "HIP error";
    case CSA2_ERR_UNSUPPORTED: return "unsupported";
  }
  return "unknown status";
}

const char* csa2_last_error(void) { return g_err; }

csa2_status csa2_runtime_create(csa2_runtime** out) {
  REQ(out, CSA2_ERR_INVALID_ARG, "csa2_runtime_create: out is NULL");
  *out = new (std::nothrow) csa2_runtime();
  REQ(*out, CSA2_ERR_INVALID_ARG, "csa2_runtime_create: out of host memory");
  return ok();
}

csa2_status csa2_runtime_destroy(csa2_runtime* rt) {
  delete rt;
  return ok();
}

csa2_status csa2_runtime_reset(csa2_runtime* rt) {
  REQ(rt, CSA2_ERR_INVALID_ARG, "csa2_runtime_reset: rt is NULL");
  for (auto& s : rt->slot) {
    uint64_t g = s.generation;
    s = csa2_runtime::Slot();
    s.generation = g;
  }
  return ok();
}

csa2_status csa2_runtime_slot(const csa2_runtime* rt, csa2_slot slot, csa2_slot_info* out) {
  REQ(rt && out, CSA2_ERR_INVALID_ARG, "csa2_runtime_slot: NULL argument");
  REQ(slot >= 0 && slot < 4, CSA2_ERR_INVALID_ARG, "csa2_runtime_slot: bad slot %d", (int)slot);
  const auto& s = rt->slot[slot];
  out->filled = s.filled;
  out->generation = s.generation;
  out->ptr = s.ptr;
  out->ptr2 = s.ptr2;
  out->dtype = s.dtype;
  out->B = s.B;
  out->rows = s.rows;
  out->cols = s.cols;
  out->extra = s.extra;
  out->kv_fmt = s.kv_fmt;
  return ok();
}

csa2_status csa2_compress(csa2_runtime* rt, const csa2_compress_args* a, csa2_stream stream) {
  csa2_status s = check_compress(a);
  if (s != CSA2_OK) return s;
  uint8_t* ksc = a->kv_fmt == CSA2_KV_FP4 ? a->kv_scales : nullptr;
  hipError_t e = csa2::launch_compress(a->dtype, a->x, a->w_kv, a->w_gate, a->gamma, a->latent_pre, a->kv_cache, ksc,
                                       a->B, a->T, a->D, a->m, a->start_pos, a->N_cap, a->eps, a->rope_base,
                                       st(stream));
  if (e != hipSuccess) return hip_status(e, "csa2_compress launch");
  publish(rt, CSA2_SLOT_COMPRESS_KV, a->kv_cache, ksc, a->dtype, a->B, a->N_cap,
          a->start_pos / a->m + a->T / a->m, a->m, a->kv_fmt);
  return ok();
}

csa2_status csa2_compress_step(csa2_runtime* rt, const csa2_compress_step_args* a, csa2_stream stream) {
  csa2_status s = check_compress_step(a);
  if (s != CSA2_OK) return s;
  REQ(rt == nullptr || (a->n_entries >= 0 && a->n_entries <= a->N_cap), CSA2_ERR_SHAPE,
      "csa2_compress_step: n_entries (%d) must be in [0, N_cap = %d]", a->n_entries, a->N_cap);
  hipError_t e = csa2::launch_compress_step(a->dtype, a->x, a->pos, a->w_kv, a->w_gate, a->gamma, a->w_ik, a->state,
                                            a->kv_cache, a->kv_fmt == CSA2_KV_FP4 ? a->kv_scales : nullptr,
                                            a->ik_codes, a->ik_scales, a->latent_pre,
                                            static_cast<float*>(a->workspace), a->B, a->D, a->m, a->N_cap, a->eps,
                                            a->rope_base, st(stream), a->scale_fmt);
  if (e != hipSuccess) return hip_status(e, "csa2_compress_step launch");
  // the Full layer's caches as they stand after this step, for the layers that borrow them
  publish(rt, CSA2_SLOT_COMPRESS_KV, a->kv_cache, a->kv_fmt == CSA2_KV_FP4 ? a->kv_scales : nullptr, a->dtype, a->B,
          a->N_cap, a->n_entries, a->m, a->kv_fmt);
  publish(rt, CSA2_SLOT_INDEX_K, a->ik_codes, a->ik_scales, 0, a->B, a->N_cap, a->n_entries, a->m, a->scale_fmt);
  return ok();
}

csa2_status csa2_index_k(csa2_runtime* rt, const csa2_index_k_args* a, csa2_stream stream) {
  csa2_status s = check_index_k(a);
  if (s != CSA2_OK) return s;
  hipError_t e = csa2::launch_index_k(a->dtype, a->latent_pre, a->w_ik, a->codes, a->scales, a->B, a->N, a->m,
                                      a->entry0, a->N_cap, a->rope_base, st(stream), a->scale_fmt);
  if (e != hipSuccess) return hip_status(e, "csa2_index_k launch");
  publish(rt, CSA2_SLOT_INDEX_K, a->codes, a->scales, 0, a->B, a->N_cap, a->entry0 + a->N, a->m, a->scale_fmt);
  return ok();
}

}  // extern "C"

namespace csa2 {

csa2_status set_error(csa2_status s, const char* msg) { return fail(s, "%s", msg); }

csa2_status score_topk_plan(const csa2_runtime* rt, const csa2_score_topk_args* in, size_t* bytes) {
  REQ(in && bytes, CSA2_ERR_INVALID_ARG, "csa2_score_topk: args is NULL");
  csa2_score_topk_args a = *in;
  csa2_status s = resolve_score(rt, a);
  if (s != CSA2_OK) return s;
  *bytes = plan_score(a.dtype, a.B, a.T, score_scan(a), a.k, a.hsi, a.hsi_s, a.hsi_nb).total_bytes;
  return ok();
}

}  // namespace csa2

extern "C" {

csa2_status csa2_score_topk(csa2_runtime* rt, const csa2_score_topk_args* in, csa2_stream stream) {
  REQ(in, CSA2_ERR_INVALID_ARG, "csa2_score_topk: args is NULL");
  csa2_score_topk_args a = *in;
  csa2_status s = resolve_score(rt, a);
  if (s != CSA2_OK) return s;
  const csa2::ScorePlan plan = csa2::plan_score(a.dtype, a.B, a.T, score_scan(a), a.k, a.hsi, a.hsi_s, a.hsi_nb);
  REQ(a.workspace != nullptr && a.workspace_bytes >= plan.total_bytes, CSA2_ERR_WORKSPACE,
      "csa2_score_topk: workspace of %zu bytes needed (got %zu)", plan.total_bytes, a.workspace_bytes);
  REQ(((uintptr_t)a.workspace & 15u) == 0, CSA2_ERR_WORKSPACE, "csa2_score_topk: workspace not 16-byte aligned");
  hipError_t e = csa2::launch_score_topk(a.dtype, a.q_idx, a.w, a.codes, a.scales, a.q_pos, a.topk, a.candidates, a.B,
                                         a.T, a.H_I, a.N_cap, a.n_entries, a.m, a.k, a.hsi, a.hsi_s, a.hsi_nb,
                                         a.workspace, plan, st(stream), a.scores, a.scale_fmt);
  if (e != hipSuccess) return hip_status(e, "csa2_score_topk launch");
  publish(rt, CSA2_SLOT_TOPK_IDXS, a.topk, nullptr, 0, a.B, a.T, a.k, 0);
  if (a.hsi == CSA2_HSI_BUILD) publish(rt, CSA2_SLOT_CANDIDATES, a.candidates, nullptr, 0, a.B, a.T, a.hsi_nb, a.hsi_s);
  return ok();
}

csa2_status csa2_sparse_attn(csa2_runtime* rt, const csa2_sparse_attn_args* in, csa2_stream stream) {
  REQ(in, CSA2_ERR_INVALID_ARG, "csa2_sparse_attn: args is NULL");
  csa2_sparse_attn_args a = *in;
  csa2_status s = resolve_attn(rt, a);
  if (s != CSA2_OK) return s;
  const float scale = a.scale > 0.f ? a.scale : 1.0f / std::sqrt(512.0f);
  const csa2::AttnPlan plan = attn_plan(a);
  REQ(plan.ws_bytes == 0 || (a.workspace != nullptr && a.workspace_bytes >= plan.ws_bytes), CSA2_ERR_WORKSPACE,
      "csa2_sparse_attn: workspace of %zu bytes needed (got %zu)", plan.ws_bytes, a.workspace_bytes);
  REQ(plan.ws_bytes == 0 || ((uintptr_t)a.workspace & 15u) == 0, CSA2_ERR_WORKSPACE,
      "csa2_sparse_attn: workspace not 16-byte aligned");
  hipError_t e = csa2::launch_sparse_attn(a.dtype, a.q, a.kv, a.kv_fmt == CSA2_KV_FP4 ? a.kv_scales : nullptr,
                                          a.topk, a.swa_kv, a.swa_pos0, a.q_pos, a.o, a.lse,
                                          a.sink, a.B, a.T, a.H, a.N_cap, a.k, a.L_w, a.W, scale, a.workspace, plan,
                                          st(stream), a.swa_fmt == CSA2_SWA_FP8_RING);
  if (e != hipSuccess) return hip_status(e, "csa2_sparse_attn launch");
  return ok();
}

csa2_status csa2_swa_append(const csa2_swa_append_args* a, csa2_stream stream) {
  REQ(a, CSA2_ERR_INVALID_ARG, "csa2_swa_append: args is NULL");
  REQ(dtype_ok(a->dtype), CSA2_ERR_DTYPE, "csa2_swa_append: unsupported dtype %d", a->dtype);
  REQ(a->B >= 0 && a->T >= 0 && a->L_w >= 1, CSA2_ERR_SHAPE, "csa2_swa_append: need B, T >= 0 and L_w >= 1");
  if (a->B == 0 || a->T == 0) return ok();
  REQ(a->rows && a->pos && a->ring, CSA2_ERR_INVALID_ARG, "csa2_swa_append: NULL tensor");
  REQ(((uintptr_t)a->rows & 15u) == 0 && ((uintptr_t)a->ring & 7u) == 0, CSA2_ERR_INVALID_ARG,
      "csa2_swa_append: rows must be 16-byte and the ring 8-byte aligned");
  hipError_t e = csa2::launch_swa_append(a->dtype, a->rows, a->pos, a->ring, a->B, a->T, a->L_w, st(stream));
  if (e != hipSuccess) return hip_status(e, "csa2_swa_append launch");
  return ok();
}

csa2_status csa2_workspace_size(int32_t op, const void* args, const csa2_layer_cfg* cfg, size_t* bytes) {
  REQ(bytes && args, CSA2_ERR_INVALID_ARG, "csa2_workspace_size: NULL argument");
  if (op == CSA2_OP_SCORE_TOPK) {
    const csa2_score_topk_args* a = static_cast<const csa2_score_topk_args*>(args);
    *bytes = csa2::plan_score(a->dtype, a->B, a->T, score_scan(*a), a->k, a->hsi, a->hsi_s, a->hsi_nb).total_bytes;
    return ok();
  }
  if (op == CSA2_OP_SPARSE_ATTN) {
    const csa2_sparse_attn_args* a = static_cast<const csa2_sparse_attn_args*>(args);
    // with kv NULL the slot decides the format; size for FP4 when the caller says so
    *bytes = attn_plan(*a).ws_bytes;
    return ok();
  }
  if (op == CSA2_OP_COMPRESS_STEP) {
    const csa2_compress_step_args* a = static_cast<const csa2_compress_step_args*>(args);
    *bytes = a->B > 0 ? (size_t)a->B * 1024 * 4 * 4 : 0;
    return ok();
  }
  if (op == CSA2_OP_LAYER) {
    REQ(cfg, CSA2_ERR_INVALID_ARG, "csa2_workspace_size: layer op needs cfg");
    const csa2_layer_io* io = static_cast<const csa2_layer_io*>(args);
    size_t need = csa2::plan_attn(cfg->dtype, io->B, io->T, cfg->H, cfg->k, cfg->W, cfg->kv_fmt == CSA2_KV_FP4,
                                  io->N_cap, cfg->swa_fmt == CSA2_SWA_FP8_RING, io->L_w).ws_bytes;
    if (cfg->mode != CSA2_REUSE) {
      const int n_entries = io->N_cap;  // upper bound
      const int scan = cfg->hsi == CSA2_HSI_USE ? cfg->hsi_nb * cfg->hsi_s : n_entries;
      const size_t sb = csa2::plan_score(cfg->dtype, io->B, io->T, scan, cfg->k, cfg->hsi, cfg->hsi_s, cfg->hsi_nb).total_bytes;
      if (sb > need) need = sb;
    }
    *bytes = need;
    return ok();
  }
  return fail(CSA2_ERR_INVALID_ARG, "csa2_workspace_size: unknown op %d", op);
}

csa2_status csa2_layer_forward(csa2_runtime* rt, const csa2_layer_cfg* cfg, const csa2_layer_io* io,
                               csa2_stream stream) {
  REQ(rt && cfg && io, CSA2_ERR_INVALID_ARG, "csa2_layer_forward: NULL argument");
  REQ(cfg->mode >= CSA2_FULL && cfg->mode <= CSA2_REUSE, CSA2_ERR_INVALID_ARG, "csa2_layer_forward: bad mode");
  REQ(io->T_x >= 0, CSA2_ERR_SHAPE, "csa2_layer_forward: T_x must be >= 0");
  const int T_x = io->T_x > 0 ? io->T_x : io->T;   // hidden-state tokens a Full layer compresses
  csa2_status s;
  int n_entries = 0;
  if (cfg->mode == CSA2_FULL) {
    REQ(cfg->hsi != CSA2_HSI_USE, CSA2_ERR_INVALID_ARG, "csa2_layer_forward: a Full layer cannot use a pool");
    csa2_compress_args ca{};
    ca.dtype = cfg->dtype; ca.B = io->B; ca.T = T_x; ca.D = io->D; ca.m = cfg->m; ca.start_pos = io->start_pos;
    ca.N_cap = io->N_cap; ca.eps = cfg->eps; ca.rope_base = cfg->rope_base; ca.x = io->x; ca.w_kv = io->w_kv;
    ca.w_gate = io->w_gate; ca.gamma = io->gamma; ca.latent_pre = io->latent_pre; ca.kv_cache = io->kv_cache;
    ca.kv_fmt = cfg->kv_fmt; ca.kv_scales = io->kv_scales;
    s = check_compress(&ca);
    if (s != CSA2_OK) return s;
    csa2_index_k_args ia{};
    ia.dtype = cfg->dtype; ia.B = io->B; ia.N = T_x / cfg->m; ia.m = cfg->m; ia.entry0 = io->start_pos / cfg->m;
    ia.N_cap = io->N_cap; ia.rope_base = cfg->rope_base; ia.latent_pre = io->latent_pre; ia.w_ik = io->w_ik;
    ia.codes = io->ik_codes; ia.scales = io->ik_scales; ia.scale_fmt = cfg->scale_fmt;
    s = check_index_k(&ia);
    if (s != CSA2_OK) return s;
    n_entries = ia.entry0 + ia.N;
  } else {
    REQ(rt->slot[CSA2_SLOT_COMPRESS_KV].filled, CSA2_ERR_SLOT_EMPTY,
        "csa2_layer_forward: compress_kv slot is empty (no Full layer ran)");
    if (cfg->mode == CSA2_REINDEX) {
      REQ(cfg->hsi != CSA2_HSI_BUILD, CSA2_ERR_INVALID_ARG, "csa2_layer_forward: only a Full layer builds a pool");
      REQ(rt->slot[CSA2_SLOT_INDEX_K].filled, CSA2_ERR_SLOT_EMPTY, "csa2_layer_forward: index_k slot is empty");
      n_entries = rt->slot[CSA2_SLOT_INDEX_K].cols;
    }
  }
  csa2_score_topk_args sa{};
  if (cfg->mode != CSA2_REUSE) {
    sa.dtype = cfg->dtype; sa.B = io->B; sa.T = io->T; sa.H_I = cfg->H_I; sa.N_cap = io->N_cap;
    sa.n_entries = n_entries; sa.m = cfg->m; sa.k = cfg->k; sa.hsi = cfg->hsi; sa.hsi_s = cfg->hsi_s;
    sa.hsi_nb = cfg->hsi_nb; sa.q_idx = io->q_idx; sa.w = io->w; sa.q_pos = io->q_pos; sa.topk = io->topk;
    sa.candidates = io->candidates; sa.workspace = io->workspace; sa.workspace_bytes = io->workspace_bytes;
    if (cfg->mode == CSA2_FULL) {
      sa.codes = io->ik_codes;
      sa.scales = io->ik_scales;
      sa.scale_fmt = cfg->scale_fmt;
    } else {
      sa.N_cap = rt->slot[CSA2_SLOT_INDEX_K].rows;
    }
    s = resolve_score(rt, sa);
    if (s != CSA2_OK) return s;
    const csa2::ScorePlan plan = csa2::plan_score(sa.dtype, sa.B, sa.T, score_scan(sa), sa.k, sa.hsi, sa.hsi_s, sa.hsi_nb);
    REQ(sa.workspace != nullptr && sa.workspace_bytes >= plan.total_bytes, CSA2_ERR_WORKSPACE,
        "csa2_layer_forward: workspace of %zu bytes needed (got %zu)", plan.total_bytes, sa.workspace_bytes);
    REQ(((uintptr_t)sa.workspace & 15u) == 0, CSA2_ERR_WORKSPACE, "csa2_layer_forward: workspace not 16-byte aligned");
  }
  csa2_sparse_attn_args aa{};
  aa.dtype = cfg->dtype; aa.B = io->B; aa.T = io->T; aa.H = cfg->H; aa.k = cfg->k; aa.L_w = io->L_w; aa.W = cfg->W;
  aa.scale = cfg->scale; aa.q = io->q; aa.swa_kv = io->swa_kv; aa.swa_pos0 = io->swa_pos0; aa.q_pos = io->q_pos;
  aa.o = io->o; aa.workspace = io->workspace; aa.workspace_bytes = io->workspace_bytes; aa.sink = io->sink;
  aa.swa_fmt = cfg->swa_fmt;
  if (cfg->mode == CSA2_FULL) {
    aa.kv = io->kv_cache;
    aa.kv_fmt = cfg->kv_fmt;
    aa.kv_scales = io->kv_scales;
    aa.N_cap = io->N_cap;
    aa.topk = io->topk;
  } else if (cfg->mode == CSA2_REINDEX) {
    aa.topk = io->topk;  // kv from the slot
  }
  // validate attention against the slots as they will be after this layer's writes
  {
    csa2_sparse_attn_args probe = aa;
    if (probe.kv == nullptr) {
      REQ(rt->slot[CSA2_SLOT_COMPRESS_KV].dtype == cfg->dtype && rt->slot[CSA2_SLOT_COMPRESS_KV].B == io->B,
          CSA2_ERR_SLOT_MISMATCH, "csa2_layer_forward: compress_kv slot does not fit this layer");
      probe.kv = rt->slot[CSA2_SLOT_COMPRESS_KV].ptr;
      probe.N_cap = rt->slot[CSA2_SLOT_COMPRESS_KV].rows;
      probe.kv_fmt = rt->slot[CSA2_SLOT_COMPRESS_KV].kv_fmt;
      probe.kv_scales = static_cast<const uint8_t*>(rt->slot[CSA2_SLOT_COMPRESS_KV].ptr2);
    }
    if (probe.topk == nullptr) {
      const auto& ts = rt->slot[CSA2_SLOT_TOPK_IDXS];
      REQ(ts.filled, CSA2_ERR_SLOT_EMPTY, "csa2_layer_forward: topk_idxs slot is empty (no Full or Reindex layer ran)");
      REQ(ts.B == io->B && ts.rows == io->T && ts.cols == cfg->k, CSA2_ERR_SLOT_MISMATCH,
          "csa2_layer_forward: topk_idxs slot does not fit this layer");
      probe.topk = static_cast<const int32_t*>(ts.ptr);
    }
    s = resolve_attn(rt, probe);
    if (s != CSA2_OK) return s;
    // the attention workspace, for the main KV actually attended (a borrowed FP4
    // cache may be dequantised whole), before anything is enqueued
    const csa2::AttnPlan ap = attn_plan(probe);
    REQ(ap.ws_bytes == 0 || (io->workspace != nullptr && io->workspace_bytes >= ap.ws_bytes), CSA2_ERR_WORKSPACE,
        "csa2_layer_forward: attention needs a workspace of %zu bytes (got %zu)", ap.ws_bytes, io->workspace_bytes);
    REQ(ap.ws_bytes == 0 || ((uintptr_t)io->workspace & 15u) == 0, CSA2_ERR_WORKSPACE,
        "csa2_layer_forward: workspace not 16-byte aligned");
  }
  // ---- enqueue
  if (cfg->mode == CSA2_FULL) {
    csa2_compress_args ca{};
    ca.dtype = cfg->dtype; ca.B = io->B; ca.T = T_x; ca.D = io->D; ca.m = cfg->m; ca.start_pos = io->start_pos;
    ca.N_cap = io->N_cap; ca.eps = cfg->eps; ca.rope_base = cfg->rope_base; ca.x = io->x; ca.w_kv = io->w_kv;
    ca.w_gate = io->w_gate; ca.gamma = io->gamma; ca.latent_pre = io->latent_pre; ca.kv_cache = io->kv_cache;
    ca.kv_fmt = cfg->kv_fmt; ca.kv_scales = io->kv_scales;
    csa2_index_k_args ia{};
    ia.dtype = cfg->dtype; ia.B = io->B; ia.N = T_x / cfg->m; ia.m = cfg->m; ia.entry0 = io->start_pos / cfg->m;
    ia.N_cap = io->N_cap; ia.rope_base = cfg->rope_base; ia.latent_pre = io->latent_pre; ia.w_ik = io->w_ik;
    ia.codes = io->ik_codes; ia.scales = io->ik_scales; ia.scale_fmt = cfg->scale_fmt;
    if (csa2::compress_makes_index_k(cfg->dtype, cfg->m, cfg->kv_fmt == CSA2_KV_FP4)) {
      // one kernel writes the cache rows, the pre-RoPE latent and the index K
      // (both argument sets were checked above)
      hipError_t e = csa2::launch_compress_index_k(ca.x, ca.w_kv, ca.gamma, ca.latent_pre, ca.kv_cache, ia.w_ik,
                                                   ia.codes, ia.scales, ca.B, ca.T, ca.D, ca.start_pos, ca.N_cap,
                                                   ca.eps, ca.rope_base, st(stream), ia.scale_fmt);
      if (e != hipSuccess) return hip_status(e, "csa2_layer_forward: compress launch");
      publish(rt, CSA2_SLOT_COMPRESS_KV, ca.kv_cache, nullptr, ca.dtype, ca.B, ca.N_cap, ca.start_pos + ca.T, 1,
              ca.kv_fmt);
      publish(rt, CSA2_SLOT_INDEX_K, ia.codes, ia.scales, 0, ia.B, ia.N_cap, ia.entry0 + ia.N, 1, ia.scale_fmt);
    } else {
      if ((s = csa2_compress(rt, &ca, stream)) != CSA2_OK) return s;
      if ((s = csa2_index_k(rt, &ia, stream)) != CSA2_OK) return s;
    }
  }
  if (cfg->mode != CSA2_REUSE) {
    if ((s = csa2_score_topk(rt, &sa, stream)) != CSA2_OK) return s;
  }
  return csa2_sparse_attn(rt, &aa, stream);
}

csa2_status csa2_kv_fp4_pack(const float* rows, int64_t n_rows, uint8_t* codes, uint8_t* scales, csa2_stream stream) {
  REQ(n_rows >= 0, CSA2_ERR_SHAPE, "csa2_kv_fp4_pack: n_rows < 0");
  REQ(n_rows == 0 || (rows && codes && scales), CSA2_ERR_INVALID_ARG, "csa2_kv_fp4_pack: NULL tensor");
  REQ(n_rows == 0 || ((uintptr_t)rows & 15u) == 0, CSA2_ERR_INVALID_ARG, "csa2_kv_fp4_pack: rows not 16-byte aligned");
  hipError_t e = csa2::launch_kv_fp4_pack(rows, n_rows, codes, scales, st(stream));
  if (e != hipSuccess) return hip_status(e, "csa2_kv_fp4_pack launch");
  return ok();
}

csa2_status csa2_fp4_pack(const float* rows, int64_t n_rows, uint8_t* codes, uint8_t* scales, csa2_stream stream) {
  REQ(n_rows >= 0, CSA2_ERR_SHAPE, "csa2_fp4_pack: n_rows < 0");
  REQ(n_rows == 0 || (rows && codes && scales), CSA2_ERR_INVALID_ARG, "csa2_fp4_pack: NULL tensor");
  hipError_t e = csa2::launch_fp4_pack(rows, n_rows, codes, scales, st(stream));
  if (e != hipSuccess) return hip_status(e, "csa2_fp4_pack launch");
  return ok();
}

}  // extern "C"
