// Internal launcher interface between the host API (csa2_api.cpp) and the HIP
// kernel translation units.  Every launcher assumes its arguments were validated
// by the caller and returns the hipError_t of the launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa2 {

// ---- compressor (k_compress.hip)
// kv_scales != nullptr: the cache is FP4 main KV (kv_cache = codes [B, N_cap, 256],
// kv_scales = E4M3 scales [B, N_cap, 32]); otherwise rows of the dtype
hipError_t launch_compress(int dtype, const void* x, const void* w_kv, const void* w_gate,
                           const float* gamma, float* latent_pre, void* kv_cache, uint8_t* kv_scales, int B, int T,
                           int D, int m, int start_pos, int N_cap, float eps, float rope_base,
                           hipStream_t stream);

// Full layer with m == 1, bf16 and a bf16 cache: the compressor kernel also writes
// the index-K codes and scales (what launch_index_k would write from latent_pre)
bool compress_makes_index_k(int dtype, int m, bool kv_fp4);
hipError_t launch_compress_index_k(const void* x, const void* w_kv, const float* gamma, float* latent_pre,
                                   void* kv_cache, const void* w_ik, uint8_t* codes, uint8_t* scales, int B, int T,
                                   int D, int start_pos, int N_cap, float eps, float rope_base, hipStream_t stream,
                                   int scale_fmt);

// decode append: C and Z of one token per sequence into cz [B, 1024] (float32), then
// the group pool / entry / index-K row per sequence
hipError_t launch_compress_step(int dtype, const void* x, const int32_t* pos, const void* w_kv,
                                const void* w_gate, const float* gamma, const void* w_ik, float* state,
                                void* kv_cache, uint8_t* kv_scales, uint8_t* codes, uint8_t* scales, float* latent_pre,
                                float* cz, int B, int D, int m, int N_cap, float eps, float rope_base,
                                hipStream_t stream, int scale_fmt);

// ---- index K and FP4 packing (k_index_k.hip)
hipError_t launch_index_k(int dtype, const float* latent_pre, const void* w_ik, uint8_t* codes,
                          uint8_t* scales, int B, int N, int m, int entry0, int N_cap,
                          float rope_base, hipStream_t stream, int scale_fmt);
hipError_t launch_fp4_pack(const float* rows, int64_t n_rows, uint8_t* codes, uint8_t* scales,
                           hipStream_t stream);
// FP4 main KV: 512-d float32 rows -> codes [n, 256] + E4M3 scales [n, 32], and back
// to dense rows of the dtype
hipError_t launch_kv_fp4_pack(const float* rows, int64_t n_rows, uint8_t* codes, uint8_t* scales,
                              hipStream_t stream);
hipError_t launch_kv_fp4_dequant(int dtype, const uint8_t* codes, const uint8_t* scales, int64_t n_rows, void* out,
                                 hipStream_t stream);

// ---- window KV in FP8 (k_swa.hip)
hipError_t launch_swa_append(int dtype, const void* rows, const int32_t* pos, uint8_t* ring, int B, int T_len,
                             int L_w, hipStream_t stream);
// ring -> dense rows [B, L_w, 512] of the dtype, row j = position (newest_b - L_w + 1 + j);
// pos0_out[b] = max(swa_pos0[b], newest_b - L_w + 1)
hipError_t launch_swa_window(int dtype, const uint8_t* ring, const int32_t* q_pos, const int32_t* swa_pos0,
                             void* dense, int32_t* pos0_out, int B, int T_len, int L_w, hipStream_t stream);

// ---- indexer score + top-k (k_score.hip)
struct ScorePlan {
  bool tiled;       // two-phase path: query-tiled scoring into a key matrix, then one select per query
  bool stream;      // streaming path: filtered scoring over parts of `chunk` entries, then a merge
  int chunk;        // entries per chunk (a power of two), or per part on the streaming path
  int n_chunks;     // chunks per query
  int k_chunk;      // candidates kept per chunk = min(k, chunk)
  int pf_cpg;       // chunks per pre-filter group before the merge (0: no pre-filter)
  int pf_groups;    // pre-filter groups per query
  size_t cand_bytes, lb_bytes, blk_bytes, seg_bytes, key_bytes, total_bytes;
};
ScorePlan plan_score(int dtype, int B, int T, int n_scan, int k, int hsi, int hsi_s, int hsi_nb);
hipError_t launch_score_topk(int dtype, const void* q_idx, const float* w, const uint8_t* codes,
                             const uint8_t* scales, const int32_t* q_pos, int32_t* topk,
                             int32_t* candidates, int B, int T, int H_I, int N_cap, int n_entries,
                             int m, int k, int hsi, int hsi_s, int hsi_nb, void* workspace,
                             const ScorePlan& plan, hipStream_t stream, float* scores_out = nullptr,
                             int scale_fmt = 0);

// ---- host API (csa2_api.cpp)
// Validates a score/top-k call (resolving slots) and gives the workspace bytes it
// needs; returns a csa2_status (int) and sets the thread's last error on failure.
}  // namespace csa2
#include "csa2.h"
namespace csa2 {
csa2_status score_topk_plan(const csa2_runtime* rt, const csa2_score_topk_args* a, size_t* bytes);
// Sets the thread's last error message and returns s.
csa2_status set_error(csa2_status s, const char* msg);

// ---- sparse attention (k_attn.hip)
struct AttnPlan {
  bool decode;      // few queries: workgroup per (query, split, head group)
  bool kv_fp4;      // main KV stored as FP4
  int n_splits;     // row splits per query (decode only)
  int n_fp4;        // decode with FP4 KV or an FP8 window ring: the first n_fp4 splits take the selected rows, the rest the window
  size_t ws_bytes;  // decode: split partials (bf16 rows, float32 log-sum-exp) when n_splits > 1;
                    // FP4 KV outside decode: the dequantised cache rows [B, N_cap, 512];
                    // then, with an FP8 window ring, its dense rows [B, L_w, 512] and B int32
  bool ring_direct; // FP8 window ring read by the decode kernel itself (window rows in splits of their own)
  size_t swa_off;   // byte offset of the dense window rows in the workspace (FP8 ring, when not ring_direct)
};
AttnPlan plan_attn(int dtype, int B, int T, int H, int k, int W, bool kv_fp4, int N_cap, bool swa_fp8 = false,
                   int L_w = 0);
hipError_t launch_sparse_attn(int dtype, const void* q, const void* kv, const uint8_t* kv_scales, const int32_t* topk,
                              const void* swa_kv, const int32_t* swa_pos0, const int32_t* q_pos,
                              void* o, float* lse, const float* sink, int B, int T, int H, int N_cap, int k,
                              int L_w, int W, float scale, void* workspace, const AttnPlan& plan, hipStream_t stream,
                              bool swa_fp8 = false);

}  // namespace csa2
