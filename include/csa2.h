/*
 * csa2.h -- C ABI of the CSA2 (Compressed Sparse Attention 2) layer hot path
 * for AMD Instinct MI355X (gfx950).
 *
 * Pages cited (titles as published):
 *   [P1] "DeepSeek-V4.1 模型结构（2）：序列维度（中），CSA2 的三种模式" (blog.javazero.top)
 *   [P2] "DeepSeek v4.1 Flash技术剖析——架构篇" (myhz0606.com)
 *   [P3] "DeepSeek-V4.1-Flash：把百万 Token 的记忆，压缩成一套分级缓存" (junki.cn)
 *   [P4] "CSA2 — l'attention creuse compressée de seconde génération" (mkdocs.reaper.mx)
 *
 * Conventions shared by every entry point
 *   - All tensor arguments are DEVICE pointers to dense row-major arrays that the
 *     caller allocates, owns and keeps alive until the enqueued work has finished.
 *     The library never allocates, frees or copies device memory on these paths.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     asynchronously; nothing synchronises.  A fault inside a kernel surfaces at
 *     the caller's next synchronisation with that stream.
 *   - Every call validates its arguments on the host and returns a csa2_status
 *     BEFORE enqueuing anything; on error nothing is enqueued and
 *     csa2_last_error() (thread-local) describes the problem.  No C++ exception
 *     crosses this interface.
 *   - Index K storage ("FP4 with one scale per 32 dims", [P1] indexer-K section;
 *     68 B per entry, [P3] section six): per entry 64 code bytes (E2M1, the code
 *     of dim 2j in the low nibble of byte j, dim 2j+1 in the high nibble) and 4
 *     scale bytes (E4M3FN, one per 32 dims).  value = e2m1(code) * e4m3(scale).
 *   - Latent rows are 512 wide; RoPE turns the last 64 dims of a row as
 *     interleaved pairs (2i, 2i+1) by pos * rope_base^(-2i/64).
 *   - Inputs must be finite.
 */
#ifndef CSA2_H_
#define CSA2_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA2_LATENT_DIM 512
#define CSA2_INDEX_DIM 128
#define CSA2_ROPE_DIMS 64
#define CSA2_FP4_BLOCK 32
#define CSA2_MAX_TOPK 1024

typedef enum csa2_status {
  CSA2_OK = 0,
  CSA2_ERR_INVALID_ARG = 1,   /* NULL pointer, bad enum, m not in {1,2,4}, w_gate given with m == 1 ... */
  CSA2_ERR_SHAPE = 2,         /* sizes inconsistent or unsupported */
  CSA2_ERR_DTYPE = 3,         /* dtype not supported for this argument */
  CSA2_ERR_SLOT_EMPTY = 4,    /* a runtime slot was read before any layer wrote it */
  CSA2_ERR_SLOT_MISMATCH = 5, /* a runtime slot does not fit the consumer's shapes */
  CSA2_ERR_WORKSPACE = 6,     /* workspace missing, smaller than csa2_workspace_size() or not 16-byte aligned */
  CSA2_ERR_HIP = 7,           /* a HIP launch failed */
  CSA2_ERR_UNSUPPORTED = 8    /* valid request this build does not implement */
} csa2_status;

typedef enum csa2_dtype { CSA2_F32 = 0, CSA2_BF16 = 1 } csa2_dtype;

/* Storage of the main KV cache rows.  DENSE: 512 values of the layer dtype per
 * row.  FP4 ([P3] section seven, FP4 main KV: E2M1 data with an E4M3 scale shared
 * by a group of channels, dequantised to a wider type before attention; [P3]
 * section six: 288 B per entry, hence one scale per 16 channels): per row 256
 * code bytes (E2M1, dim 2j in the low nibble of byte j) in the cache tensor and
 * 32 E4M3FN scale bytes in a second tensor.  Each 16-dim block is quantised as
 * the index K is: s = E4M3(amax / 6) (float32 divide, nearest-even, saturating at
 * 448), codes E2M1(u / s) (nearest-even, saturating at 6, sign kept), all zero
 * when s is 0.  The rows quantised are the float32 post-RoPE latents.         */
typedef enum csa2_kv_fmt { CSA2_KV_DENSE = 0, CSA2_KV_FP4 = 1 } csa2_kv_fmt;

/* Storage of a layer's sliding-window KV.  DENSE: [B, L_w, 512] of the layer dtype,
 * row j holding position swa_pos0[b] + j.  FP8_RING ([P3] section seven: the local
 * window KV is more sensitive to quantisation and is kept in FP8): uint8
 * [B, L_w, 512] E4M3FN bytes, one per dimension, no scale (round to nearest
 * even, saturating at +-448), in a ring: the row of position u sits in slot
 * u mod L_w (written by csa2_swa_append).  Attention with a ring needs W <= L_w
 * and a 16-byte aligned ring; for each sequence the ring must hold the positions
 * newest - L_w + 1 .. newest, newest being the largest q_pos of that sequence in
 * the call, and swa_pos0[b] is the first position ever written (earlier positions
 * are absent).  A query's window is clipped at newest - L_w + 1, so the query
 * positions of one sequence in one call should lie within L_w - W of newest
 * (decode: one query per sequence); a prefill attends its dense window rows and
 * then appends the last L_w of them.  The rows are attended as their exact values
 * (E4M3 values are exact in bf16). */
typedef enum csa2_swa_fmt { CSA2_SWA_DENSE = 0, CSA2_SWA_FP8_RING = 1 } csa2_swa_fmt;

/* Layer modes ([P1] section on the four slots and the mode excerpt; [P2] mode
 * tables; [P4] "Les trois modes"): Full computes main KV, index K and top-k;
 * Reindex borrows main KV and index K and selects anew; Reuse borrows main KV and
 * the latest top-k and only attends. */
typedef enum csa2_mode { CSA2_FULL = 0, CSA2_REINDEX = 1, CSA2_REUSE = 2 } csa2_mode;

/* Hierarchical candidate pool ([P2] section CSA2-ReIndex; [P3] section five):
 * BUILD (Full layer): also keep the n_b best blocks of s entries per query (block
 * score = max index score, the block of the newest visible entry always kept);
 * USE (Reindex layer): select only inside that pool. */
typedef enum csa2_hsi { CSA2_HSI_NONE = 0, CSA2_HSI_BUILD = 1, CSA2_HSI_USE = 2 } csa2_hsi;

typedef void* csa2_stream; /* hipStream_t */
typedef struct csa2_runtime csa2_runtime;

/* ------------------------------------------------------------------------ */
/* Shared runtime: four single-occupancy slots holding borrowed device views
 * ([P1] section "共享池里有四样东西": main KV, index K, top-k indices and the
 * candidate pool; one position each, no per-layer numbering, only pointers).
 * The runtime object is host memory owned by the caller via create/destroy.  */

csa2_status csa2_runtime_create(csa2_runtime** out);
csa2_status csa2_runtime_destroy(csa2_runtime* rt);
/* Empty all four slots (e.g. between requests). */
csa2_status csa2_runtime_reset(csa2_runtime* rt);

typedef enum csa2_slot {
  CSA2_SLOT_COMPRESS_KV = 0, CSA2_SLOT_INDEX_K = 1, CSA2_SLOT_TOPK_IDXS = 2, CSA2_SLOT_CANDIDATES = 3
} csa2_slot;

typedef struct csa2_slot_info {
  int32_t filled;       /* 0 = empty */
  uint64_t generation;  /* increments on every write of this slot */
  const void* ptr;      /* main KV / codes / top-k / candidates */
  const void* ptr2;     /* index-K scales (INDEX_K only) */
  int32_t dtype;        /* main KV dtype (COMPRESS_KV only) */
  int32_t B, rows, cols;/* COMPRESS_KV: B, N_cap, n_entries; INDEX_K: B, N_cap, n_entries;
                           TOPK_IDXS: B, T, k; CANDIDATES: B, T, n_b */
  int32_t extra;        /* CANDIDATES: block size s; COMPRESS_KV/INDEX_K: m */
  int32_t kv_fmt;       /* COMPRESS_KV: csa2_kv_fmt (FP4: ptr = codes, ptr2 = scales);
                           INDEX_K: csa2_scale_fmt of the scales */
} csa2_slot_info;

csa2_status csa2_runtime_slot(const csa2_runtime* rt, csa2_slot slot, csa2_slot_info* out);

/* ------------------------------------------------------------------------ */
/* (a) Compressor ([P1] section "压缩算子去掉了重叠和位置偏置": C = x W_kv,
 * Z = x W_gate, softmax of Z over each disjoint group of m tokens per channel,
 * no position bias, pooled sum, RMSNorm, RoPE on the last 64 dims at the group's
 * first-token position; m == 1 is norm(x W_kv) with no gate).
 *
 *   x        [B, T, D]   dtype            T % m == 0, D % 64 == 0
 *   w_kv     [512, D]    dtype            (output x input)
 *   w_gate   [512, D]    dtype, NULL iff m == 1
 *   gamma    [512]       float32          RMSNorm gain
 *   latent_pre [B, T/m, 512] float32 out  normalised entries before RoPE (feeds index K)
 *   kv_cache [B, N_cap, 512] dtype out    rows start_pos/m .. start_pos/m + T/m - 1 written
 *   start_pos  absolute position of x[:, 0] (same for all sequences), multiple of m
 *   kv_fmt   CSA2_KV_FP4: kv_cache is uint8 codes [B, N_cap, 256] and kv_scales
 *            uint8 [B, N_cap, 32] receives the scales (see csa2_kv_fmt)
 * With rt != NULL the compress_kv slot is set to kv_cache (and kv_scales) with
 * n_entries = start_pos/m + T/m.                                              */
typedef struct csa2_compress_args {
  int32_t dtype;            /* csa2_dtype of x, w_kv, w_gate, kv_cache */
  int32_t B, T, D, m;
  int32_t start_pos;
  int32_t N_cap;
  float eps;                /* RMSNorm epsilon (e.g. 1e-6) */
  float rope_base;          /* e.g. 10000 */
  const void* x;
  const void* w_kv;
  const void* w_gate;
  const float* gamma;
  float* latent_pre;
  void* kv_cache;
  int32_t kv_fmt;           /* csa2_kv_fmt */
  uint8_t* kv_scales;       /* FP4 only: [B, N_cap, 32] */
} csa2_compress_args;

csa2_status csa2_compress(csa2_runtime* rt, const csa2_compress_args* a, csa2_stream stream);

/* ------------------------------------------------------------------------ */
/* Scale format of the index K ([P1] indexer-K section: FP4 with one scale per 32
 * dims; the pages name no format for it).  E4M3: scale = E4M3FN(amax / 6)
 * (float32 divide, nearest-even, saturating at 448), codes E2M1(u / s), all zero
 * when s is 0.  UE8M0: the byte b of the smallest power of two X = 2^(b - 127) at
 * or above amax / 6 (b clamped to 0 .. 254, 0 also for an all-zero block), codes
 * E2M1(u / X).  Both: E2M1 nearest-even, saturating at 6, sign kept; 68 B per
 * entry.  The FP4 main KV always uses E4M3. */
typedef enum csa2_scale_fmt { CSA2_SCALE_E4M3 = 0, CSA2_SCALE_UE8M0 = 1 } csa2_scale_fmt;

/* ------------------------------------------------------------------------ */
/* (b) Index K ([P1] section "indexer K 改由 main KV 投影": projected 512 -> 128
 * from the main-KV entry before its RoPE, RoPE on its own last 64 dims at the
 * entry position, stored FP4 with one scale per 32 dims, no Hadamard rotation).
 *
 *   latent_pre [B, N, 512] float32        entries entry0 .. entry0 + N - 1
 *   w_ik       [128, 512]  dtype          (output x input)
 *   codes      [B, N_cap, 64]  uint8 out  rows entry0 .. entry0 + N - 1 written
 *   scales     [B, N_cap, 4]   uint8 out
 *   entry position for RoPE = (entry0 + i) * m
 *   scale_fmt  csa2_scale_fmt of the scales written (CSA2_ERR_INVALID_ARG otherwise)
 * With rt != NULL the index_k slot is set to (codes, scales, scale_fmt),
 * n_entries = entry0 + N. */
typedef struct csa2_index_k_args {
  int32_t dtype;            /* csa2_dtype of w_ik */
  int32_t B, N, m;
  int32_t entry0;
  int32_t N_cap;
  float rope_base;
  const float* latent_pre;
  const void* w_ik;
  uint8_t* codes;
  uint8_t* scales;
  int32_t scale_fmt;        /* csa2_scale_fmt */
} csa2_index_k_args;

csa2_status csa2_index_k(csa2_runtime* rt, const csa2_index_k_args* a, csa2_stream stream);

/* ------------------------------------------------------------------------ */
/* Decode append for a Full layer: the compressor (a) and index K (b) for one new
 * token per sequence after the prefill.  Groups are disjoint runs of m tokens
 * ([P1] section "压缩算子去掉了重叠和位置偏置"), so a token becomes part of an
 * entry only at its group's last token; until then the group lives in a
 * caller-owned state.  The entry is then the one csa2_compress and csa2_index_k
 * would have written for the whole group: per-channel softmax of Z over the
 * group, pooled C, RMSNorm, RoPE on the last 64 dims at position g*m, and its
 * index-K row.
 *
 *   x        [B, D]  dtype               the new token of each sequence, D % 64 == 0
 *   pos      [B] int32 (device)          its absolute position; < 0 = no token
 *   w_kv, w_gate, gamma                  as csa2_compress (w_gate NULL iff m == 1)
 *   w_ik     [128, 512] dtype            as csa2_index_k
 *   state    [B, 3, 512] float32 (device, in/out; NULL iff m == 1): the
 *            group's running softmax pool per channel (maximum of Z, sum of
 *            exp(Z - max), sum of exp(Z - max) C).  A group's first token
 *            overwrites it, so it needs no initialisation.
 *   kv_cache [B, N_cap, 512] dtype out   row pos/m, written at a group's last token
 *            (kv_fmt CSA2_KV_FP4: codes [B, N_cap, 256] and kv_scales [B, N_cap, 32])
 *   ik_codes [B, N_cap, 64], ik_scales [B, N_cap, 4] uint8 out: the same row
 *   latent_pre [B, 512] float32 out      that entry's latent before RoPE (NULL: not written)
 *   workspace  csa2_workspace_size(CSA2_OP_COMPRESS_STEP) bytes (B * 16384: C and
 *              Z partial sums of 4 quarters of the hidden dims), 16-byte aligned
 *   n_entries  (host) entries of the longest sequence once this step is done, i.e.
 *              max over b of (pos[b] + 1) / m for the positions reached so far; in
 *              [0, N_cap].  Read only when rt != NULL.
 * Rows pos/m >= N_cap are not written.  With rt != NULL the compress_kv slot is
 * republished as (kv_cache, kv_scales) and the index_k slot as (ik_codes,
 * ik_scales), both with n_entries entries, so that Reindex and Reuse layers that
 * borrow them see the appended entries ([P1] section "共享池里有四样东西": the
 * slot holds the Full layer's cache as it grows; a query at position p still sees
 * only the entries whose group ended at or before p).                        */
typedef struct csa2_compress_step_args {
  int32_t dtype;            /* csa2_dtype of x, w_kv, w_gate, w_ik, kv_cache */
  int32_t B, D, m;
  int32_t N_cap;
  float eps, rope_base;
  const void* x;
  const int32_t* pos;
  const void* w_kv;
  const void* w_gate;
  const float* gamma;
  const void* w_ik;
  float* state;
  void* kv_cache;
  uint8_t* ik_codes;
  uint8_t* ik_scales;
  float* latent_pre;
  void* workspace;
  size_t workspace_bytes;
  int32_t kv_fmt;           /* csa2_kv_fmt */
  uint8_t* kv_scales;       /* FP4 only: [B, N_cap, 32] */
  int32_t n_entries;        /* host; see above (read only with rt != NULL) */
  int32_t scale_fmt;        /* csa2_scale_fmt of the index-K rows written */
} csa2_compress_step_args;

csa2_status csa2_compress_step(csa2_runtime* rt, const csa2_compress_step_args* a, csa2_stream stream);

/* ------------------------------------------------------------------------ */
/* (c)+(d) Indexer score and causal top-k ([P1] indexer-K section: score =
 * sum over the H_I heads of w * ReLU(q^I . k^I); [P2] CSA2-FULL / CSA2-ReIndex:
 * the k best among the causally visible entries, or inside the candidate pool).
 *
 *   q_idx   [B, T, H_I, 128] dtype       indexer queries, RoPE already applied
 *   w       [B, T, H_I]      float32     per-head weights
 *   codes/scales  index K as above [B, N_cap, 64] / [B, N_cap, 4]; both NULL ->
 *                 taken from the runtime's index_k slot (Reindex)
 *   q_pos   [B, T] int32                 absolute query positions
 *   n_entries  valid cache rows (host); query (b,t) sees
 *              n_t = min(n_entries, (q_pos[b,t] + 1) / m) entries
 *   topk    [B, T, k] int32 out          chosen entry ids ascending, then -1
 *   candidates [B, T, n_b] int32         BUILD: out; USE: in (NULL -> slot);
 *                                        block ids ascending, then -1
 *   workspace  device scratch of at least csa2_workspace_size() bytes, 16-byte
 *              aligned (CSA2_ERR_WORKSPACE otherwise)
 *   scores  [B, T, n_scan] float32 out or NULL: a debug dump of every scanned
 *           position's index score (n_scan = n_entries, or hsi_nb * hsi_s for
 *           HSI_USE, whose positions are the pool's: block j / hsi_s of the
 *           candidates, entry j % hsi_s within it), -inf where the position is not
 *           visible to the query or not a valid pool entry.  4-byte aligned
 *           (CSA2_ERR_INVALID_ARG otherwise).  It adds a fill pass and the stores;
 *           the selection does not read it.
 * Ties in score go to the smaller entry id; -0 counts as +0.
 * With rt != NULL the topk_idxs slot (and on BUILD the candidates slot) is set. */
typedef struct csa2_score_topk_args {
  int32_t dtype;            /* csa2_dtype of q_idx */
  int32_t B, T, H_I;
  int32_t N_cap, n_entries, m, k;
  int32_t hsi;              /* csa2_hsi */
  int32_t hsi_s, hsi_nb;
  const void* q_idx;
  const float* w;
  const uint8_t* codes;
  const uint8_t* scales;
  const int32_t* q_pos;
  int32_t* topk;
  int32_t* candidates;
  void* workspace;
  size_t workspace_bytes;
  float* scores;            /* optional debug dump (see above), or NULL */
  int32_t scale_fmt;        /* csa2_scale_fmt of explicit codes/scales; borrowed ones carry the slot's */
} csa2_score_topk_args;

csa2_status csa2_score_topk(csa2_runtime* rt, const csa2_score_topk_args* a, csa2_stream stream);

/* csa2_score_topk for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the same
 * operation, arguments and results, but its scratch is a fixed device array of
 * CSA2_NOALLOC_SCRATCH_BYTES (16 MiB) inside the library, one per GPU, held until
 * the process ends.  a->workspace must be NULL and a->workspace_bytes 0.  A call
 * whose csa2_workspace_size(CSA2_OP_SCORE_TOPK) exceeds the array returns
 * CSA2_ERR_WORKSPACE before anything is enqueued (the decode workloads, e.g. 64
 * queries over 131072 entries, need about 8.4 MB; many-query prefill calls need
 * more and take csa2_score_topk).  The call allocates and frees nothing.  Every
 * call on one GPU uses that GPU's one array: calls that overlap on one GPU
 * (other streams, other host threads) race and must be serialised by the
 * caller.  Nothing in the array has to be cleared between calls. */
#define CSA2_NOALLOC_SCRATCH_BYTES (16u << 20)
csa2_status csa2_score_topk_noalloc(csa2_runtime* rt, const csa2_score_topk_args* a, csa2_stream stream);

/* ------------------------------------------------------------------------ */
/* (e) Sparse attention ([P1] section "一层全局注意力算四样东西": the layer's own
 * query reads the selected entries plus its 128-entry sliding window; [P2]
 * CSA2-FULL: key and value are the same vector; [P3] section four: softmax of
 * c_j . q / sqrt(d) over the rows, output = weighted sum of the same rows).
 *
 *   q        [B, T, H, 512] dtype        RoPE already applied
 *   kv       [B, N_cap, 512] dtype       NULL -> runtime compress_kv slot
 *            (q, o, dense kv and dense swa_kv 16-byte aligned, else CSA2_ERR_INVALID_ARG)
 *   topk     [B, T, k] int32             NULL -> runtime topk_idxs slot; -1 = empty,
 *                                        ids outside [0, N_cap) are skipped
 *   swa_kv   [B, L_w, 512] dtype         the layer's window KV, row j = position swa_pos0[b] + j
 *   swa_pos0 [B] int32, q_pos [B, T] int32
 *   rows of query (b,t): kv[topk[b,t,j]] for valid j, then window positions
 *   max(0, p-W+1, swa_pos0) .. min(p, swa_pos0 + L_w - 1) with p = q_pos[b,t]
 *   o        [B, T, H, 512] dtype out
 *   lse      [B, T, H] float32 out (optional, natural-log sum of exp of scaled logits)
 *   scale    0 -> 1/sqrt(512)
 *   workspace  device scratch of csa2_workspace_size() bytes (may be 0 bytes:
 *              then NULL is accepted), 16-byte aligned
 *   sink     [H] float32 or NULL.  Every layer has one attention sink per head
 *            ([P1] sections "三种模式的参数清单" and "容易混淆的几点"); the pages
 *            give no formula.  Read here as a logit s_h that enters only the
 *            softmax denominator: p_r = exp(l_r) / (exp(s_h) + sum_r' exp(l_r')),
 *            o = sum_r p_r row_r, lse = log(exp(s_h) + sum_r exp(l_r)), with
 *            l_r = scale * q . row_r.  NULL is the plain softmax.
 *   kv_fmt   CSA2_KV_FP4: kv is uint8 codes [B, N_cap, 256] (16-byte aligned)
 *            and kv_scales uint8 [B, N_cap, 32] (4-byte aligned); the rows are
 *            attended as their exact dequantised values (window rows stay
 *            dense).  Few-query bf16 calls dequantise inside the row gather;
 *            other calls dequantise the whole cache once into the workspace
 *            (B * N_cap * 512 elements of the dtype), since there each row is
 *            read by many queries.  With kv == NULL the slot's format is used. */
typedef struct csa2_sparse_attn_args {
  int32_t dtype;            /* csa2_dtype of q, kv, swa_kv, o */
  int32_t B, T, H;
  int32_t N_cap, k, L_w, W;
  float scale;
  const void* q;
  const void* kv;
  const int32_t* topk;
  const void* swa_kv;
  const int32_t* swa_pos0;
  const int32_t* q_pos;
  void* o;
  float* lse;
  void* workspace;
  size_t workspace_bytes;
  const float* sink;        /* [H] float32 per-head sink logits, or NULL (no sink) */
  int32_t kv_fmt;           /* csa2_kv_fmt of kv (ignored when kv is NULL) */
  const uint8_t* kv_scales; /* FP4 only: [B, N_cap, 32] */
  int32_t swa_fmt;          /* csa2_swa_fmt of swa_kv; FP8_RING: bf16 calls of fewer than 512 queries
                               whose rows take two or more splits (FP4 KV, or fewer than 256 queries
                               with more than 32 rows: k + W > 32)
                               read the ring inside the attention kernel; every other call first
                               reads it into the workspace (B * L_w * 512 elements of the dtype +
                               B int32).  csa2_workspace_size gives the bytes either way. */
} csa2_sparse_attn_args;

csa2_status csa2_sparse_attn(csa2_runtime* rt, const csa2_sparse_attn_args* a, csa2_stream stream);

/* ------------------------------------------------------------------------ */
/* Window KV ring in FP8 ([P3] section seven; layout at csa2_swa_fmt): quantise
 * each layer's new window rows into its ring.
 *
 *   rows  [B, T, 512] dtype              the window KV rows of positions pos
 *   pos   [B, T] int32 (device)          absolute positions; < 0 = no row
 *   ring  [B, L_w, 512] uint8 in/out     slot pos mod L_w of sequence b is overwritten
 * Decode appends one row per sequence and step (T = 1); after a prefill the last
 * L_w rows of each sequence are appended at once (two rows of one call must not
 * share a slot, i.e. positions of one sequence in one call span fewer than L_w).
 * Errors: CSA2_ERR_DTYPE; CSA2_ERR_SHAPE for B, T < 0 or L_w < 1;
 * CSA2_ERR_INVALID_ARG for a NULL tensor (with B * T > 0), rows not 16-byte or the
 * ring not 8-byte aligned.  Nothing is written on an error; B * T == 0 is a no-op. */
typedef struct csa2_swa_append_args {
  int32_t dtype;            /* csa2_dtype of rows */
  int32_t B, T, L_w;
  const void* rows;
  const int32_t* pos;
  uint8_t* ring;
} csa2_swa_append_args;

csa2_status csa2_swa_append(const csa2_swa_append_args* a, csa2_stream stream);

/* ------------------------------------------------------------------------ */
/* One layer in its configured mode ([P1] mode excerpt: a KV source compresses
 * and publishes main KV; an index source selects and publishes top-k; a layer
 * that is neither reuses both).  Full: compress -> index_k -> score_topk ->
 * sparse_attn.  Reindex: score_topk on the index_k slot -> sparse_attn on the
 * compress_kv slot.  Reuse: sparse_attn on the compress_kv and topk_idxs slots.
 * Fields a mode does not use are ignored.  A Full layer with m = 1, bf16 and a
 * bf16 cache runs compress and index_k as one kernel; its outputs (cache rows,
 * latent_pre, index-K codes and scales, slot contents) are bit for bit those of
 * csa2_compress followed by csa2_index_k.                                    */
typedef struct csa2_layer_cfg {
  int32_t mode;             /* csa2_mode */
  int32_t dtype;            /* csa2_dtype */
  int32_t m, k, W, H_I, H;
  int32_t hsi, hsi_s, hsi_nb;
  float rope_base, eps, scale;
  int32_t kv_fmt;           /* Full: storage of the main KV it writes (csa2_kv_fmt) */
  int32_t swa_fmt;          /* storage of this layer's window KV io->swa_kv (csa2_swa_fmt) */
  int32_t scale_fmt;        /* Full: csa2_scale_fmt of the index K it writes (others read the slot's) */
} csa2_layer_cfg;

typedef struct csa2_layer_io {
  int32_t B, T, D;
  int32_t start_pos;        /* Full: position of x[:, 0] (= q_pos of its first query) */
  int32_t N_cap;
  /* Full only */
  const void* x; const void* w_kv; const void* w_gate; const float* gamma; const void* w_ik;
  float* latent_pre; void* kv_cache; uint8_t* ik_codes; uint8_t* ik_scales;
  /* Full and Reindex */
  const void* q_idx; const float* w; int32_t* topk; int32_t* candidates;
  /* every mode */
  const int32_t* q_pos; const void* q; const void* swa_kv; int32_t L_w; const int32_t* swa_pos0;
  void* o;
  void* workspace; size_t workspace_bytes;
  const float* sink;        /* [H] float32 per-head attention sink, or NULL (see csa2_sparse_attn_args) */
  uint8_t* kv_scales;       /* Full with kv_fmt CSA2_KV_FP4: [B, N_cap, 32]; kv_cache then holds the codes */
  int32_t T_x;              /* Full: hidden-state tokens compressed, x is [B, T_x, D] at positions start_pos ..
                               start_pos + T_x - 1 (0: T_x = T).  The queries keep their own count T and
                               positions q_pos.  A decoder prefill with bounded replay ([P2] "CED(Causal
                               encoder-decoder)", decoder SWA bounded replay; [P3] section two, "为什么还要重放
                               尾部"; [P4] "L'interaction avec le CED") compresses the encoder output of all
                               L prompt tokens (T_x = L) while only the last R tokens pass through the
                               decoder layers (T = R, q_pos = L-R .. L-1, window KV of the replayed
                               segment only: swa_pos0 = L-R). */
} csa2_layer_io;

csa2_status csa2_layer_forward(csa2_runtime* rt, const csa2_layer_cfg* cfg, const csa2_layer_io* io,
                               csa2_stream stream);

/* ------------------------------------------------------------------------ */
typedef enum csa2_op {
  CSA2_OP_SCORE_TOPK = 0, CSA2_OP_SPARSE_ATTN = 1, CSA2_OP_LAYER = 2, CSA2_OP_COMPRESS_STEP = 3
} csa2_op;

/* Device workspace bytes the op needs for these arguments (args points to the
 * op's argument struct; for CSA2_OP_LAYER a csa2_layer_io with the cfg passed
 * through `cfg`, else NULL).  For a Reindex or Reuse layer, io->N_cap and
 * cfg->kv_fmt are read as those of the main KV the layer borrows (the Full
 * layer's cache), since attention there may dequantise that whole cache. */
csa2_status csa2_workspace_size(int32_t op, const void* args, const csa2_layer_cfg* cfg, size_t* bytes);

/* FP4 index-K packing alone (test hook for bit-exactness): rows [n_rows, 128]
 * float32 -> codes [n_rows, 64], scales [n_rows, 4], as described above. */
csa2_status csa2_fp4_pack(const float* rows, int64_t n_rows, uint8_t* codes, uint8_t* scales,
                          csa2_stream stream);

/* FP4 main-KV packing alone (test hook for bit-exactness): rows [n_rows, 512]
 * float32 (16-byte aligned) -> codes [n_rows, 256], scales [n_rows, 32], as
 * described at csa2_kv_fmt. */
csa2_status csa2_kv_fp4_pack(const float* rows, int64_t n_rows, uint8_t* codes, uint8_t* scales,
                             csa2_stream stream);

const char* csa2_status_string(csa2_status s);
const char* csa2_last_error(void);
/* Library version string, e.g. "csa2-mi355x 0.1 gfx950". */
const char* csa2_version(void);

#ifdef __cplusplus
}
#endif
#endif /* CSA2_H_ */
