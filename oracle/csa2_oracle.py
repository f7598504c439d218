"""Plain CPU oracle of the CSA2 layer hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this module:
only the tests, the smoke check and the benchmark's CPU-baseline leg do.  It
shares no code, table or constant generator with the HIP library; the two meet
only through the seeded inputs of ``synth``.

Arithmetic is float64 (numpy) everywhere except the FP4/FP8 encoder, which works
in float32 on purpose: the stored format is defined by float32 divisions and
round-to-nearest-even, and the GPU must reproduce those bytes exactly.

Pages cited (titles as published):
  [P1] "DeepSeek-V4.1 模型结构（2）：序列维度（中），CSA2 的三种模式" (blog.javazero.top)
  [P2] "DeepSeek v4.1 Flash技术剖析——架构篇" (myhz0606.com)
  [P3] "DeepSeek-V4.1-Flash：把百万 Token 的记忆，压缩成一套分级缓存" (junki.cn)
  [P4] "CSA2 — l'attention creuse compressée de seconde génération" (mkdocs.reaper.mx)

Readings taken where the pages are silent or garbled (each one is listed with its
reason in the design notes of the repository):
  * score has no 1/sqrt(d_I) factor (a positive global factor changes no selection);
  * an entry g is visible to a query at position p iff its whole group ends at or
    before p, i.e. g < floor((p+1)/m);
  * RoPE uses interleaved pairs (2i, 2i+1) of the rotated slice with
    theta_i = base^(-2i/n_rope);                          -- parity unpinned (convention)
  * FP4 main KV (optional storage of the cache rows) uses the same rule with one
    scale per 16 dims (288 B per entry);
  * FP4 = E2M1 codes, one E4M3FN scale per 32 dims, scale = RNE(amax/6), codes =
    RNE(u/scale) saturating at 6, sign kept (a negative value rounding to zero is
    code 0x8), even dimension in the low nibble;          -- parity unpinned (convention)
  * top-k ties go to the smaller entry index, -0 counts as +0, the output is
    ascending and padded with -1;
  * the HSI block holding the newest visible entry gets score +inf;
  * the sliding window of a query at position p is the positions
    [max(0, p-W+1, swa_pos0), p]; the current token is included;
  * attention scale is 1/sqrt(d) with d = 512; no attention sink.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

LATENT_DIM = 512  # [P1] section on the KV size: one 512-d latent, K and V are the same vector
ROPE_DIMS = 64    # [P1] compressor section: RoPE on the last 64 dims
INDEX_DIM = 128   # [P1] indexer-K section: W^IK is 512 x 128
FP4_BLOCK = 32    # [P1] indexer-K section: FP4 with one scale per 32 dims
KV_FP4_BLOCK = 16  # [P3] section six: a main-KV entry is 288 B = 256 B of E2M1 codes for
                   # 512 dims + 32 E4M3 scale bytes, i.e. one scale per 16 dims

# ---------------------------------------------------------------------------
# FP4 (E2M1) and FP8 (E4M3FN) codecs.  The formats themselves come from the OCP
# Microscaling / OCP FP8 definitions; [P1] (indexer-K section) fixes "FP4, one
# scale per 32 dims" and [P3] (section six, the 890 B budget) fixes 68 B per
# index-K entry = 64 B of codes + 4 scale bytes.
# ---------------------------------------------------------------------------

# magnitudes of the 8 E2M1 codes 0..7 (sign is bit 3)
E2M1_MAGNITUDE = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """Value of each 4-bit E2M1 code (bit 3 = sign, bits 0-2 index the magnitude)."""
    codes = np.asarray(codes).astype(np.int64)
    mag = E2M1_MAGNITUDE[codes & 7]
    return np.where((codes >> 3) & 1, -mag, mag)


def e2m1_encode(v: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest E2M1 code, ties to the even code,
    saturating at +-6; the sign bit is kept even when the magnitude rounds to 0."""
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v).astype(np.float64)
    mids = (E2M1_MAGNITUDE[:-1] + E2M1_MAGNITUDE[1:]) / 2.0  # 0.25 0.75 1.25 1.75 2.5 3.5 5
    idx = np.searchsorted(mids, a, side="left")  # number of midpoints strictly below a
    at_mid = np.zeros(a.shape, dtype=bool)
    inb = idx < len(mids)
    at_mid[inb] = a[inb] == mids[idx[inb]]
    # at a midpoint idx is the lower neighbour; move up when the lower one is odd
    idx = np.where(at_mid & (idx % 2 == 1), idx + 1, idx)
    sign = np.signbit(v).astype(np.int64)
    return (idx.astype(np.int64) | (sign << 3)).astype(np.uint8)


def e4m3_decode(b: np.ndarray) -> np.ndarray:
    """Value of each E4M3FN byte (bias 7, no infinities, S.1111.111 is NaN)."""
    b = np.asarray(b).astype(np.int64)
    s = (b >> 7) & 1
    e = (b >> 3) & 15
    mnt = b & 7
    sub = mnt / 8.0 * 2.0 ** -6
    nrm = (1.0 + mnt / 8.0) * np.power(2.0, e - 7)
    val = np.where(e == 0, sub, nrm)
    val = np.where((e == 15) & (mnt == 7), np.nan, val)
    return np.where(s == 1, -val, val)


_E4M3_POS_VALUES = e4m3_decode(np.arange(0x7F))  # bytes 0x00..0x7E, strictly increasing


def e4m3_encode_nonneg(v: np.ndarray) -> np.ndarray:
    """Round non-negative float32 values to the nearest E4M3FN byte, ties to the
    even byte, saturating at 448 (byte 0x7E)."""
    a = np.asarray(v, dtype=np.float32).astype(np.float64)
    assert np.all(a >= 0.0), "scale encoder is only used on amax/6 >= 0"
    mids = (_E4M3_POS_VALUES[:-1] + _E4M3_POS_VALUES[1:]) / 2.0
    idx = np.searchsorted(mids, a, side="left")
    at_mid = np.zeros(a.shape, dtype=bool)
    inb = idx < len(mids)
    at_mid[inb] = a[inb] == mids[idx[inb]]
    idx = np.where(at_mid & (idx % 2 == 1), idx + 1, idx)
    idx = np.minimum(idx, 0x7E)
    return idx.astype(np.uint8)


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest E4M3FN byte, ties to the even byte,
    saturating at +-448; bit 7 is the sign (kept for a value rounding to zero)."""
    v = np.asarray(v, dtype=np.float32)
    mag = e4m3_encode_nonneg(np.abs(v))
    return (mag | (np.signbit(v).astype(np.uint8) << 7)).astype(np.uint8)


SCALE_E4M3, SCALE_UE8M0 = "e4m3", "ue8m0"


def ue8m0_decode(b: np.ndarray) -> np.ndarray:
    """Value of each UE8M0 byte: 2^(b - 127); byte 255 is NaN."""
    b = np.asarray(b).astype(np.int64)
    return np.where(b == 255, np.nan, np.ldexp(1.0, b - 127))


def ue8m0_encode_ceil(sigma: np.ndarray) -> np.ndarray:
    """The UE8M0 byte of the smallest power of two at or above each float32
    sigma >= 0 (clamped to 2^-127 .. 2^127); sigma == 0 gives byte 0."""
    a = np.asarray(sigma, dtype=np.float32).astype(np.float64)
    assert np.all(a >= 0.0)
    mant, ex = np.frexp(a)                       # a = mant * 2^ex, mant in [0.5, 1)
    e = np.where(mant == 0.5, ex - 1, ex)        # exact powers of two keep their exponent
    e = np.where(a == 0.0, -127, e)
    return (np.clip(e, -127, 127) + 127).astype(np.uint8)


def fp4_pack(u: np.ndarray, block: int = FP4_BLOCK, scale_fmt: str = SCALE_E4M3):
    """Quantise rows of 128 values to FP4 index-K storage (``block`` = 32), or
    rows of 512 values to FP4 main-KV storage (``block`` = 16, see kv_fp4_pack).

    [P1] indexer-K section: FP4, one scale per 32 dims; [P3] section six: 68 B per
    entry.  Per 32-dim block: amax in float32, sigma = amax / 6 as a float32 division,
    scale byte = E4M3(sigma), s = its value; code_i = E2M1(u_i / s) (float32
    division), or 0 for the whole block when s == 0.  Code of dim 2j goes to the low
    nibble of byte j.  Returns (codes uint8 [rows, d/2], scales uint8 [rows, d/block]).

    scale_fmt SCALE_UE8M0 (index K only; the pages give no scale format for index
    K): the scale byte is the power of two X = 2^(b - 127) nearest at or above
    sigma, so that |u / X| <= 6 up to sigma's own rounding; code_i = E2M1(u_i / X)
    (exact division, nearest-even, saturating at 6).
    """
    u = np.asarray(u, dtype=np.float32)
    rows, d = u.shape
    assert d % block == 0
    nb = d // block
    blocks = u.reshape(rows, nb, block)
    amax = np.max(np.abs(blocks), axis=2).astype(np.float32)
    sigma = (amax / np.float32(6.0)).astype(np.float32)
    if scale_fmt == SCALE_UE8M0:
        sbytes = ue8m0_encode_ceil(sigma)
        s = ue8m0_decode(sbytes).astype(np.float32)
    else:
        assert scale_fmt == SCALE_E4M3
        sbytes = e4m3_encode_nonneg(sigma)
        s = e4m3_decode(sbytes).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = (blocks / s[:, :, None]).astype(np.float32)
    codes = e2m1_encode(ratio)
    codes = np.where((s == 0)[:, :, None], np.uint8(0), codes).reshape(rows, d)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, sbytes.reshape(rows, nb)


def fp4_unpack(codes: np.ndarray, scales: np.ndarray, block: int = FP4_BLOCK,
               scale_fmt: str = SCALE_E4M3) -> np.ndarray:
    """Dequantise FP4 storage: value(code) * value(scale of its block), float64
    [rows, 2 * codes.shape[1]]."""
    codes = np.asarray(codes, dtype=np.uint8)
    rows = codes.shape[0]
    lo = codes & 0x0F
    hi = codes >> 4
    c = np.empty((rows, codes.shape[1] * 2), dtype=np.uint8)
    c[:, 0::2] = lo
    c[:, 1::2] = hi
    vals = e2m1_decode(c)
    s = ue8m0_decode(np.asarray(scales)) if scale_fmt == SCALE_UE8M0 else e4m3_decode(np.asarray(scales))
    return vals * np.repeat(s, block, axis=1)


def kv_fp4_pack(rows: np.ndarray):
    """Quantise 512-d main-KV rows (the compressor's post-RoPE latents) to FP4.

    [P3] section seven, FP4 main KV: E2M1 data, one E4M3 scale shared by each group
    of channels, dequantised to a wider type before attention; [P3] section six: 288 B
    per entry, which fixes the group at 16 channels (256 B of codes + 32 scale bytes).
    Same per-block rule as the index-K codec.  Returns (codes uint8 [rows, 256],
    scales uint8 [rows, 32]).
    """
    rows = np.asarray(rows, dtype=np.float32)
    assert rows.shape[1] == LATENT_DIM
    return fp4_pack(rows, KV_FP4_BLOCK)


def kv_fp4_unpack(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Dequantise FP4 main-KV storage to float64 [rows, 512] (attention reads these)."""
    return fp4_unpack(codes, scales, KV_FP4_BLOCK)


# ---------------------------------------------------------------------------
# RoPE on the trailing slice ([P1] compressor section: RoPE on the last 64
# dims at the group's first-token position; indexer-K section: index K gets its
# own RoPE on its last 64 dims).
# ---------------------------------------------------------------------------

def rope_last(x: np.ndarray, pos, base: float = 10000.0, n_rope: int = ROPE_DIMS) -> np.ndarray:
    """Rotate the last ``n_rope`` dims of each row of ``x`` at position ``pos``.

    Pairs (2i, 2i+1) of the slice turn by pos * base^(-2i/n_rope).  ``pos`` is a
    scalar or one position per row.
    """
    x = np.array(x, dtype=np.float64, copy=True)
    d = x.shape[-1]
    pos = np.asarray(pos, dtype=np.float64)
    i = np.arange(n_rope // 2, dtype=np.float64)
    theta = np.power(float(base), -2.0 * i / n_rope)
    ang = pos[..., None] * theta if pos.ndim else pos * theta
    c, s = np.cos(ang), np.sin(ang)
    x0 = x[..., d - n_rope::2].copy()
    x1 = x[..., d - n_rope + 1::2].copy()
    x[..., d - n_rope::2] = x0 * c - x1 * s
    x[..., d - n_rope + 1::2] = x0 * s + x1 * c
    return x


def rms_norm(e: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis ([P1] compressor code and text: the pooled entry is normalised)."""
    e = np.asarray(e, dtype=np.float64)
    return e / np.sqrt(np.mean(e * e, axis=-1, keepdims=True) + eps) * np.asarray(gamma, dtype=np.float64)


# ---------------------------------------------------------------------------
# (a) Compressor: [P1] section "压缩算子去掉了重叠和位置偏置" (code excerpt and
# text), [P2] section CSA2-FULL, [P4] "Ce qui change par rapport à V4" (table):
# disjoint groups of m tokens, per-channel softmax of the gate over the group,
# no position bias, then RMSNorm, then RoPE on the last 64 dims at the position
# of the group's first token.  m == 1 is a projection plus norm, no gate.
# ---------------------------------------------------------------------------

def compress(x, w_kv, w_gate, gamma, m: int, start_pos: int = 0, eps: float = 1e-6,
             rope_base: float = 10000.0):
    """One sequence.  x [T, D]; w_kv, w_gate [512, D] (output x input); T and
    start_pos multiples of m.  Returns (latent_pre [T/m, 512], kv [T/m, 512],
    entry_ids [T/m]); latent_pre is the normalised entry before RoPE."""
    x = np.asarray(x, dtype=np.float64)
    T = x.shape[0]
    assert T % m == 0 and start_pos % m == 0
    n = T // m
    C = x @ np.asarray(w_kv, dtype=np.float64).T  # C_t: [T, 512]
    if m == 1:
        if w_gate is not None:
            raise ValueError("m == 1 has no gate projection")
        e = C
    else:
        Z = x @ np.asarray(w_gate, dtype=np.float64).T  # Z_t
        Cg = C.reshape(n, m, -1)
        Zg = Z.reshape(n, m, -1)
        Zmax = Zg.max(axis=1, keepdims=True)
        ez = np.exp(Zg - Zmax)
        a = ez / ez.sum(axis=1, keepdims=True)  # softmax over the m tokens, per channel
        e = (a * Cg).sum(axis=1)
    latent_pre = rms_norm(e, gamma, eps)
    entry_ids = start_pos // m + np.arange(n)
    kv = rope_last(latent_pre, entry_ids * m, rope_base)
    return latent_pre, kv, entry_ids


def compress_step(pending, x_tok, w_kv, w_gate, gamma, pos: int, m: int, eps: float = 1e-6,
                  rope_base: float = 10000.0):
    """Decode append for one sequence: the token at absolute position pos joins
    its group g = pos // m ([P1] compressor section: groups of m consecutive
    tokens, no overlap); `pending` is the list of (C_t, Z_t) rows of the group's
    earlier tokens (the partial-group state; empty at a group's first token).
    Returns (pending', entry) where entry is None until the group's last token
    (pos % m == m - 1), then (g, latent_pre [512], kv [512]) computed by the same
    steps as `compress`: softmax of Z over the group per channel, pooled C,
    RMSNorm, RoPE on the last 64 dims at position g*m."""
    x_tok = np.asarray(x_tok, dtype=np.float64)
    c = x_tok @ np.asarray(w_kv, dtype=np.float64).T
    z = None if m == 1 else x_tok @ np.asarray(w_gate, dtype=np.float64).T
    assert len(pending) == pos % m, "the state must hold the group's earlier tokens"
    rows = list(pending) + [(c, z)]
    if len(rows) < m:
        return rows, None
    if m == 1:
        e = c
    else:
        Cg = np.stack([r[0] for r in rows])
        Zg = np.stack([r[1] for r in rows])
        ez = np.exp(Zg - Zg.max(axis=0, keepdims=True))
        e = ((ez / ez.sum(axis=0, keepdims=True)) * Cg).sum(axis=0)
    g = pos // m
    latent_pre = rms_norm(e[None], gamma, eps)[0]
    kv = rope_last(latent_pre[None], np.array([g * m]), rope_base)[0]
    return [], (g, latent_pre, kv)


# ---------------------------------------------------------------------------
# (b) Index K: [P1] section "indexer K 改由 main KV 投影": projected from the
# main-KV entry BEFORE its RoPE, 512 -> 128, RoPE on its own last 64 dims, FP4
# with one scale per 32 dims, no Hadamard rotation.
# ---------------------------------------------------------------------------

def index_k(latent_pre, w_ik, entry_pos, rope_base: float = 10000.0, scale_fmt: str = SCALE_E4M3):
    """latent_pre [N, 512], w_ik [128, 512] (output x input), entry_pos [N] (= g*m).
    Returns (u float64 [N, 128] before quantisation, codes [N, 64], scales [N, 4])."""
    u = np.asarray(latent_pre, dtype=np.float64) @ np.asarray(w_ik, dtype=np.float64).T
    u = rope_last(u, np.asarray(entry_pos), rope_base)
    codes, scales = fp4_pack(u.astype(np.float32), FP4_BLOCK, scale_fmt)
    return u, codes, scales


# ---------------------------------------------------------------------------
# (c) Indexer score: [P1] indexer-K section (score unchanged from V4: per-head
# weight w, ReLU of the q^I . k^I dot product, summed over H^I = 32 heads of
# 128 dims), [P2] CSA2-FULL (causally visible set).
# ---------------------------------------------------------------------------

def visible_entries(p: int, m: int) -> int:
    """Entries visible at query position p: groups that end at or before p."""
    return (int(p) + 1) // m


def index_scores(q_idx, w, k_deq, n_vis: int) -> np.ndarray:
    """q_idx [H_I, 128], w [H_I], k_deq [N, 128]; scores of entries 0..n_vis-1."""
    q = np.asarray(q_idx, dtype=np.float64)
    k = np.asarray(k_deq, dtype=np.float64)[:n_vis]
    dots = k @ q.T  # [n_vis, H_I]
    return np.maximum(dots, 0.0) @ np.asarray(w, dtype=np.float64)


# ---------------------------------------------------------------------------
# (d) Causal top-k: [P1] "一层全局注意力算四样东西" (top-k positions, recomputed
# per query, never cached), [P2] CSA2-FULL / CSA2-ReIndex.
# ---------------------------------------------------------------------------

def topk_select(scores, k: int, candidates=None) -> np.ndarray:
    """Indices of the k largest scores (ties -> smaller index; -0 == +0), returned
    ascending and padded with -1 to length k.  ``candidates`` restricts the choice
    to the given entry ids (default: all of range(len(scores)))."""
    scores = np.asarray(scores, dtype=np.float64) + 0.0  # -0.0 + 0.0 == +0.0
    if candidates is None:
        candidates = np.arange(scores.shape[0])
    candidates = np.asarray(candidates, dtype=np.int64)
    if candidates.size <= k:
        chosen = candidates
    else:
        s = scores[candidates]
        order = np.lexsort((candidates, -s))  # primary: score descending, then index ascending
        chosen = candidates[order[:k]]
    out = np.full(k, -1, dtype=np.int64)
    chosen = np.sort(chosen)
    out[: chosen.size] = chosen
    return out


# ---------------------------------------------------------------------------
# (c') Hierarchical candidate pool (HSI): [P2] CSA2-ReIndex (blocks of s entry
# positions, block score = max index score inside it, keep the best n_b blocks,
# the block of the newest visible entry is forced in, Reindex masks scores outside
# the pool to -inf), [P3] section five (the Full layer scans everything and forms
# the pool; later Reindex layers choose their own top-512 inside it).
# ---------------------------------------------------------------------------

def hsi_pool(full_scores, n_vis: int, s: int, n_b: int) -> np.ndarray:
    """Block ids of the candidate pool for one query, ascending, padded with -1 to n_b."""
    full_scores = np.asarray(full_scores, dtype=np.float64)[:n_vis] + 0.0
    nblk = (n_vis + s - 1) // s
    out = np.full(n_b, -1, dtype=np.int64)
    if nblk == 0:
        return out
    beta = np.array([full_scores[i * s: min((i + 1) * s, n_vis)].max() for i in range(nblk)])
    beta[nblk - 1] = np.inf  # block holding the newest visible entry is always kept
    if nblk <= n_b:
        keep = np.arange(nblk)
    else:
        order = np.lexsort((np.arange(nblk), -beta))
        keep = np.sort(order[:n_b])
    out[: keep.size] = keep
    return out


def pool_entries(blocks, n_vis: int, s: int) -> np.ndarray:
    """Entry ids covered by the pool blocks (clipped to the visible range)."""
    ids = [np.arange(b * s, min((b + 1) * s, n_vis)) for b in np.asarray(blocks) if b >= 0]
    return np.concatenate(ids) if ids else np.zeros(0, dtype=np.int64)


# ---------------------------------------------------------------------------
# (e) Sparse attention: [P1] "一层全局注意力算四样东西" (attention reads the k
# selected entries plus the 128-entry sliding window of the layer), [P2]
# CSA2-FULL (shared key-value: one vector is both key and value; rows are the
# window plus the selected entries), [P3] section four (p_j and o(q) equations,
# o in the convex hull of the selected contents).
# ---------------------------------------------------------------------------

def window_positions(p: int, W: int, swa_pos0: int = 0) -> np.ndarray:
    """Positions of the sliding window of a query at position p (current token included)."""
    lo = max(0, int(p) - W + 1, int(swa_pos0))
    return np.arange(lo, int(p) + 1)


def sparse_attention(q, kv, sel, swa_kv, swa_pos0: int, p: int, W: int,
                     scale: Optional[float] = None, sink=None):
    """One query token.  q [H, d]; kv [N, d]; sel [k] (entry ids, -1 = empty);
    swa_kv [L_w, d] holding positions swa_pos0.. .  Returns (o [H, d], probs [H, R],
    rows [R, d]).

    sink [H] (optional): every layer has one attention sink per head ([P1]
    sections "三种模式的参数清单" and "容易混淆的几点"), with no formula on the
    pages.  Read as a per-head logit that joins the softmax normalisation but
    carries no value row: p_r = exp(l_r) / (exp(sink_h) + sum_r' exp(l_r')), so
    the probabilities of the rows sum to less than 1 and o lies in the convex
    hull of the rows and the origin."""
    q = np.asarray(q, dtype=np.float64)
    kv = np.asarray(kv, dtype=np.float64)
    d = q.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    sel = np.asarray(sel, dtype=np.int64)
    sel = sel[sel >= 0]
    win = window_positions(p, W, swa_pos0)
    rows = np.concatenate([kv[sel], np.asarray(swa_kv, dtype=np.float64)[win - swa_pos0]], axis=0)
    logits = (q @ rows.T) * scale
    if sink is None:
        logits = logits - logits.max(axis=1, keepdims=True)
        ez = np.exp(logits)
        probs = ez / ez.sum(axis=1, keepdims=True)
        return probs @ rows, probs, rows
    sk = np.asarray(sink, dtype=np.float64).reshape(-1, 1)
    top = np.maximum(logits.max(axis=1, keepdims=True) if rows.shape[0] else -np.inf, sk)
    ez = np.exp(logits - top)
    probs = ez / (ez.sum(axis=1, keepdims=True) + np.exp(sk - top))
    return probs @ rows, probs, rows


def attention_lse(q, rows, scale: Optional[float] = None, sink=None) -> np.ndarray:
    """Natural-log sum of exp over the rows' scaled logits (and the sink logit when
    given), per head: the normaliser of sparse_attention."""
    q = np.asarray(q, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.float64)
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    logits = (q @ rows.T) * scale
    if sink is not None:
        logits = np.concatenate([logits, np.asarray(sink, dtype=np.float64).reshape(-1, 1)], axis=1)
    if logits.shape[1] == 0:
        return np.full(q.shape[0], -np.inf)
    mx = logits.max(axis=1)
    return mx + np.log(np.exp(logits - mx[:, None]).sum(axis=1))


# ---------------------------------------------------------------------------
# Modes and the shared runtime: [P1] section "共享池里有四样东西" (four slots,
# one position each, no per-layer numbering; the two mode tests in the
# attention-layer excerpt), [P2] mode tables, [P4] "Les trois modes".
# ---------------------------------------------------------------------------

FULL, REINDEX, REUSE = "full", "reindex", "reuse"


class SlotEmpty(RuntimeError):
    pass


@dataclass
class Runtime:
    """The four single-occupancy slots.  A slot holds a reference (not a copy)."""
    compress_kv: Optional[np.ndarray] = None   # [B, N, 512]
    index_k: Optional[tuple] = None            # (codes [B, N, 64], scales [B, N, 4])
    index_k_fmt: str = SCALE_E4M3              # scale format of index_k
    topk_idxs: Optional[np.ndarray] = None     # [B, T, k]
    candidates: Optional[np.ndarray] = None    # [B, T, n_b] block ids (+ block size)
    candidates_s: int = 0
    writes: list = field(default_factory=list)

    def get(self, name):
        v = getattr(self, name)
        if v is None:
            raise SlotEmpty(name)
        return v


@dataclass
class LayerInputs:
    """Per-layer inputs of one call: batch of B sequences, T query tokens each."""
    q: np.ndarray                       # [B, T, H, 512] attention queries (RoPE applied)
    swa_kv: np.ndarray                  # [B, L_w, 512] this layer's window KV
    q_pos: np.ndarray                   # [B, T] absolute positions of the queries
    swa_pos0: np.ndarray                # [B] position of swa_kv[:, 0]
    q_idx: Optional[np.ndarray] = None  # [B, T, H_I, 128] indexer queries (Full / Reindex)
    w: Optional[np.ndarray] = None      # [B, T, H_I] per-head indexer weights
    x: Optional[np.ndarray] = None      # [B, L, D] hidden states (Full only)
    start_pos: int = 0


@dataclass
class LayerConfig:
    mode: str
    m: int = 1
    k: int = 512
    W: int = 128
    w_kv: Optional[np.ndarray] = None
    w_gate: Optional[np.ndarray] = None
    gamma: Optional[np.ndarray] = None
    w_ik: Optional[np.ndarray] = None
    eps: float = 1e-6
    rope_base: float = 10000.0
    hsi: str = "none"   # none | build (Full) | use (Reindex)
    hsi_s: int = 64
    hsi_nb: int = 256
    scale: Optional[float] = None
    kv_fp4: bool = False   # Full: store the main KV as FP4 (attention reads it dequantised)
    scale_fmt: str = SCALE_E4M3   # Full: scale format of the index K it writes


def _score_and_select(rt: Runtime, cfg: LayerConfig, inp: LayerInputs, codes, scales, scale_fmt=SCALE_E4M3):
    B, T = inp.q_pos.shape
    topk = np.full((B, T, cfg.k), -1, dtype=np.int64)
    cands = np.full((B, T, cfg.hsi_nb), -1, dtype=np.int64) if cfg.hsi == "build" else None
    for b in range(B):
        kdeq = fp4_unpack(codes[b], scales[b], FP4_BLOCK, scale_fmt)
        for t in range(T):
            n_vis = visible_entries(inp.q_pos[b, t], cfg.m)
            sc = index_scores(inp.q_idx[b, t], inp.w[b, t], kdeq, n_vis)
            if cfg.hsi == "use":
                pool = rt.get("candidates")[b, t]
                if rt.candidates_s != cfg.hsi_s:
                    raise ValueError("candidate pool block size mismatch")
                topk[b, t] = topk_select(sc, cfg.k, pool_entries(pool, n_vis, cfg.hsi_s))
            else:
                topk[b, t] = topk_select(sc, cfg.k)
                if cfg.hsi == "build":
                    cands[b, t] = hsi_pool(sc, n_vis, cfg.hsi_s, cfg.hsi_nb)
    return topk, cands


def layer_forward(rt: Runtime, cfg: LayerConfig, inp: LayerInputs):
    """One CSA2 layer in the configured mode; returns o [B, T, H, 512]."""
    if cfg.mode == FULL:
        B = inp.x.shape[0]
        lat, kvs, cs, ss = [], [], [], []
        for b in range(B):
            latent_pre, kv, ids = compress(inp.x[b], cfg.w_kv, cfg.w_gate, cfg.gamma, cfg.m,
                                           inp.start_pos, cfg.eps, cfg.rope_base)
            _, codes, scales = index_k(latent_pre, cfg.w_ik, ids * cfg.m, cfg.rope_base, cfg.scale_fmt)
            if cfg.kv_fp4:
                # [P3] section seven: the stored main KV is FP4; attention sees its
                # dequantised values
                kv = kv_fp4_unpack(*kv_fp4_pack(kv.astype(np.float32)))
            kvs.append(kv), cs.append(codes), ss.append(scales), lat.append(latent_pre)
        rt.compress_kv = np.stack(kvs)
        rt.index_k = (np.stack(cs), np.stack(ss))
        rt.index_k_fmt = cfg.scale_fmt
        rt.writes += ["compress_kv", "index_k"]
        topk, cands = _score_and_select(rt, cfg, inp, *rt.index_k, rt.index_k_fmt)
        rt.topk_idxs = topk
        rt.writes.append("topk_idxs")
        if cands is not None:
            rt.candidates, rt.candidates_s = cands, cfg.hsi_s
            rt.writes.append("candidates")
    elif cfg.mode == REINDEX:
        codes, scales = rt.get("index_k")
        kv_src = rt.get("compress_kv")
        if cfg.hsi == "build":
            raise ValueError("only a Full layer builds the candidate pool")
        topk, _ = _score_and_select(rt, cfg, inp, codes, scales, rt.index_k_fmt)
        rt.topk_idxs = topk
        rt.writes.append("topk_idxs")
    elif cfg.mode == REUSE:
        rt.get("compress_kv")
        rt.get("topk_idxs")
    else:
        raise ValueError(cfg.mode)
    return _attend(rt, cfg, inp)


def _attend(rt: Runtime, cfg: LayerConfig, inp: LayerInputs):
    kv = rt.compress_kv
    topk = rt.topk_idxs
    B, T = inp.q_pos.shape
    o = np.zeros(inp.q.shape, dtype=np.float64)
    for b in range(B):
        for t in range(T):
            o[b, t] = sparse_attention(inp.q[b, t], kv[b], topk[b, t], inp.swa_kv[b],
                                       int(inp.swa_pos0[b]), int(inp.q_pos[b, t]), cfg.W,
                                       cfg.scale)[0]
    return o


# ---------------------------------------------------------------------------
# Decode: a Full layer appends one token per sequence to the caches it owns and
# publishes, and the layers that borrow them see the grown caches ([P1] section
# "共享池里有四样东西": the slots hold the Full layer's main KV and index K, one
# position each; [P1] compressor section: an entry exists once its group of m
# tokens is complete).
# ---------------------------------------------------------------------------

def layer_append(rt: Runtime, cfg: LayerConfig, pending: list, x_tok, pos):
    """One decode token per sequence for a Full layer.  x_tok [B, D]; pos [B]
    absolute positions (< 0: no token for that sequence); pending[b] is the
    partial-group state of `compress_step`.  A completed group's entry (main-KV
    row and index-K row, computed as `compress` and `index_k` would) is written at
    row g of the runtime's compress_kv / index_k, which grow as needed.  Returns
    the ids of the entries written, per sequence (None where none)."""
    kv = rt.get("compress_kv")
    codes, scales = rt.get("index_k")
    written = []
    for b in range(len(pos)):
        p = int(pos[b])
        if p < 0:
            written.append(None)
            continue
        pending[b], entry = compress_step(pending[b], x_tok[b], cfg.w_kv, cfg.w_gate, cfg.gamma, p, cfg.m,
                                          cfg.eps, cfg.rope_base)
        if entry is None:
            written.append(None)
            continue
        g, latent_pre, row = entry
        _, c, s = index_k(latent_pre[None], cfg.w_ik, np.array([g * cfg.m]), cfg.rope_base, rt.index_k_fmt)
        if cfg.kv_fp4:
            row = kv_fp4_unpack(*kv_fp4_pack(row[None].astype(np.float32)))[0]
        if g >= kv.shape[1]:
            grow = g + 1 - kv.shape[1]
            kv = np.concatenate([kv, np.zeros((kv.shape[0], grow, kv.shape[2]))], axis=1)
            codes = np.concatenate([codes, np.zeros((codes.shape[0], grow, codes.shape[2]), codes.dtype)], axis=1)
            scales = np.concatenate([scales, np.zeros((scales.shape[0], grow, scales.shape[2]), scales.dtype)],
                                    axis=1)
        kv[b, g], codes[b, g], scales[b, g] = row, c[0], s[0]
        written.append(g)
    rt.compress_kv, rt.index_k = kv, (codes, scales)
    rt.writes += ["compress_kv", "index_k"]
    return written


def full_decode_step(rt: Runtime, cfg: LayerConfig, pending: list, x_tok, inp: LayerInputs):
    """A Full layer at decode: append the new tokens (`layer_append`, positions
    inp.q_pos[:, 0]), then select over its index K as it now stands and attend,
    as the Full branch of `layer_forward` does after its compressor."""
    assert cfg.mode == FULL and inp.q_pos.shape[1] == 1
    layer_append(rt, cfg, pending, x_tok, inp.q_pos[:, 0])
    topk, cands = _score_and_select(rt, cfg, inp, *rt.index_k, rt.index_k_fmt)
    rt.topk_idxs = topk
    rt.writes.append("topk_idxs")
    if cands is not None:
        rt.candidates, rt.candidates_s = cands, cfg.hsi_s
        rt.writes.append("candidates")
    return _attend(rt, cfg, inp)


# ---------------------------------------------------------------------------
# Decoder prefill with bounded replay: [P2] "CED(Causal encoder-decoder)" (the
# decoder's global KV is built from the encoder output; only the last positions
# of the prompt go through the decoder layers, whose local window is limited to
# that replayed segment; the truncation never touches the global KV), [P3]
# section two ("为什么还要重放尾部": only a fixed tail passes through the decoder),
# [P4] "L'interaction avec le CED" (the decoder's Full layer compresses H20, the
# encoder output).  The replay length R is lost in extraction and is a parameter.
# ---------------------------------------------------------------------------

def decoder_replay(rt: Runtime, cfgs: list, layer_inputs: list, h20, R: int):
    """Runs the decoder layers `cfgs` (cfgs[0] is the Full layer) over the last R of
    the L prompt positions.  h20 [B, L, D] is the encoder output, compressed in
    full by the Full layer into the shared global KV and index K; each
    layer_inputs[l] gives q, q_idx, w for the R replayed positions ([B, R, ...])
    and the layer's window KV rows for positions L-R .. L-1 ([B, R, 512]).
    Returns the outputs of every layer, [B, R, H, 512] each."""
    h20 = np.asarray(h20, dtype=np.float64)
    B, L = h20.shape[:2]
    assert 0 < R <= L
    q_pos = np.tile(np.arange(L - R, L), (B, 1))
    pos0 = np.full(B, L - R)
    outs = []
    for l, (cfg, li) in enumerate(zip(cfgs, layer_inputs)):
        inp = LayerInputs(q=li.q, swa_kv=li.swa_kv, q_pos=q_pos, swa_pos0=pos0, q_idx=li.q_idx, w=li.w,
                          x=h20 if l == 0 else None, start_pos=0)
        outs.append(layer_forward(rt, cfg, inp))
    return outs


# ---------------------------------------------------------------------------
# Window KV in FP8: [P3] section seven (the local sliding-window KV is more
# sensitive to quantisation than the main KV and is kept in FP8).  Read here as
# E4M3FN values with no scale (none is described), one byte per dimension, in a
# per-layer ring of L_w rows: the row of position u sits in slot u mod L_w.
# ---------------------------------------------------------------------------

def swa_ring_append(ring, rows, pos):
    """Quantise `rows` [n, 512] (positions `pos` [n]) into `ring` [L_w, 512] uint8
    in place: slot u mod L_w takes the E4M3 bytes of position u's row."""
    ring = np.asarray(ring)
    L_w = ring.shape[0]
    for r, u in zip(np.asarray(rows, dtype=np.float64), np.asarray(pos)):
        if u >= 0:
            ring[int(u) % L_w] = e4m3_encode(r.astype(np.float32))
    return ring


def swa_ring_rows(ring, first: int, last: int) -> np.ndarray:
    """Dequantised window rows of positions first .. last (inclusive) read from
    their ring slots, float64 [last - first + 1, 512]; the ring must hold them
    (last - first < L_w)."""
    ring = np.asarray(ring)
    L_w = ring.shape[0]
    assert last - first < L_w
    return e4m3_decode(ring[[u % L_w for u in range(first, last + 1)]])
