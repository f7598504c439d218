"""Comparison rules for HIP-vs-oracle parity (test infrastructure).

* Top-k sets (band rule): with the oracle's float64 scores, s_k the k-th best and
  delta = 1e-3 |s_k| (+1e-6 max|s| so that s_k ~ 0 does not make the band empty),
  the GPU set must hold every entry scoring above s_k + delta, none scoring below
  s_k - delta, and exactly min(k, #candidates) entries; output ascending, -1 padded.
  Where the k-th / (k+1)-th gap exceeds delta this is exact set equality.
* FP4 codes / scale bytes: bit-exact, except that a code may differ where the
  oracle's u/s lies within 1e-3 relative of an E2M1 rounding midpoint, and a scale
  byte where amax/6 lies within 1e-3 relative of an E4M3 midpoint (then the whole
  block is exempt).  Codes 0x0 and 0x8 (zero with either sign) may stand for one
  another only where |u/s| <= 1e-3: the sign of a value that close to zero is
  decided by summation order, and both codes decode to zero.
* Floating-point outputs: per row (token, head), max|gpu - ref| / max|ref|.
"""
from __future__ import annotations

import sys

import numpy as np

from oracle import csa2_oracle as O

E2M1_MIDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
ZERO_BAND = 1e-3   # |u / s| below which codes 0x0 and 0x8 (+0 and -0) are interchangeable
_E4M3_GRID = O.e4m3_decode(np.arange(0x7F))
E4M3_MIDS = (_E4M3_GRID[:-1] + _E4M3_GRID[1:]) / 2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def near_any(x, mids, rel=1e-3):
    x = np.abs(np.asarray(x, dtype=np.float64))
    d = np.min(np.abs(x[..., None] - mids), axis=-1)
    return d <= rel * np.maximum(x, 1e-30)


def check_topk_row(scores, cand_ids, gpu_row, k, tag="", exempt=None):
    """scores: oracle float64 scores of the candidate entries (same order as cand_ids).
    ``exempt``: entry ids whose stored FP4 codes legitimately differ between the GPU
    and the oracle (a code at a rounding midpoint); their score is ambiguous by one
    grid step, so the band rule does not constrain them.
    Returns True when the GPU set equals the oracle's exactly."""
    gpu_row = np.asarray(gpu_row)
    cand_ids = np.asarray(cand_ids, dtype=np.int64)
    n = cand_ids.size
    size = min(k, n)
    sel = gpu_row[gpu_row >= 0]
    assert sel.size == size, f"{tag}: |S| = {sel.size}, expected {size}"
    assert np.all(gpu_row[size:] == -1), f"{tag}: padding is not -1"
    assert np.all(np.diff(sel) > 0), f"{tag}: indices not strictly ascending"
    assert np.all(np.isin(sel, cand_ids)), f"{tag}: selected entries outside the candidates"
    if n <= k:
        return True
    s = np.asarray(scores, dtype=np.float64) + 0.0
    order = np.lexsort((cand_ids, -s))
    exact = set(sel.tolist()) == set(cand_ids[order[:k]].tolist())
    # exempt entries leave both sides: the rest of the GPU set must be a valid
    # top-k' of the remaining candidates (k' = how many non-exempt entries it holds)
    s_r, c_r, sel_r = s, cand_ids, sel
    if exempt is not None and len(exempt):
        keep = ~np.isin(cand_ids, exempt)
        s_r, c_r = s[keep], cand_ids[keep]
        sel_r = np.setdiff1d(sel, exempt)
    kr = sel_r.size
    if kr == 0 or c_r.size <= kr:
        return exact
    o_r = np.lexsort((c_r, -s_r))
    sk = s_r[o_r[kr - 1]]
    delta = 1e-3 * abs(sk) + 1e-6 * np.max(np.abs(s_r))
    must_in = c_r[s_r > sk + delta]
    must_out = c_r[s_r < sk - delta]
    miss = np.setdiff1d(must_in, sel_r)
    extra = np.intersect1d(must_out, sel_r)
    assert miss.size == 0, f"{tag}: {miss.size} clearly-better entries missing, e.g. {miss[:5]}"
    assert extra.size == 0, f"{tag}: {extra.size} clearly-worse entries selected, e.g. {extra[:5]}"
    return exact


def check_fp4(u, codes_gpu, scales_gpu, tag="", block=32, scale_fmt=O.SCALE_E4M3):
    """u: oracle float64 values before quantisation [rows, d] (index K: d = 128,
    block 32; main KV: d = 512, block 16).  Returns (#code mismatches, #scale
    mismatches), all of them inside the rounding bands.  UE8M0 scales (index K)
    round sigma up to a power of two, so their band is sigma within 1e-3 relative
    of a power of two."""
    u32 = np.asarray(u, dtype=np.float64).astype(np.float32)
    codes_o, scales_o = O.fp4_pack(u32, block, scale_fmt)
    rows, d = u32.shape
    nb = d // block
    blocks = u32.reshape(rows, nb, block)
    sigma = (np.max(np.abs(blocks), axis=2).astype(np.float32) / np.float32(6)).astype(np.float64)
    sdiff = scales_gpu != scales_o
    if scale_fmt == O.SCALE_UE8M0:
        sd = sigma[sdiff]
        p2 = np.exp2(np.round(np.log2(np.maximum(sd, 1e-300))))   # nearest power of two
        assert np.all(np.abs(sd - p2) <= 1e-3 * sd), f"{tag}: UE8M0 scale bytes differ away from a power of two"
        s = O.ue8m0_decode(scales_o)
    else:
        assert np.all(near_any(sigma[sdiff], E4M3_MIDS)), f"{tag}: scale bytes differ away from an E4M3 midpoint"
        s = O.e4m3_decode(scales_o)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = blocks / s[:, :, None]
    def unpack(c):
        c = np.asarray(c, dtype=np.uint8)
        out = np.empty((rows, d), dtype=np.uint8)
        out[:, 0::2] = c & 15
        out[:, 1::2] = c >> 4
        return out.reshape(rows, nb, block)
    cg, co = unpack(codes_gpu), unpack(codes_o)
    cdiff = (cg != co) & ~sdiff[:, :, None]
    # codes 0x0 and 0x8 both decode to zero; they may stand for one another only
    # where the value itself is within rounding of zero, i.e. |u / s| <= 1e-3 (the
    # same 1e-3 band as the midpoints, in units of the block scale), so that a
    # wrong sign on a clearly nonzero sub-0.25 s value still fails
    signed_zero = ((cg & 7) == 0) & ((co & 7) == 0) & (np.abs(ratio) <= ZERO_BAND)
    ok = (near_any(ratio[cdiff], E2M1_MIDS) | (s[:, :, None].repeat(block, 2)[cdiff] == 0)
          | signed_zero[cdiff])
    assert np.all(ok), f"{tag}: {np.count_nonzero(~ok)} codes differ away from an E2M1 midpoint"
    return int(np.count_nonzero(cdiff)), int(np.count_nonzero(sdiff))


def row_rel_err(gpu, ref):
    """max over rows of max|gpu-ref| / max|ref| (rows = all leading axes)."""
    g = np.asarray(gpu, dtype=np.float64).reshape(-1, np.shape(gpu)[-1])
    r = np.asarray(ref, dtype=np.float64).reshape(-1, np.shape(ref)[-1])
    num = np.max(np.abs(g - r), axis=1)
    den = np.maximum(np.max(np.abs(r), axis=1), 1e-30)
    return float(np.max(num / den)) if len(num) else 0.0
