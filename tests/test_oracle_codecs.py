"""Pins of the oracle's FP4/FP8 codecs and FP4 index-K packing (CPU only)."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import csa2_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _e2m1_table():
    rows = []
    with open(os.path.join(GOLD, "e2m1_codes.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                c, v = line.split()
                rows.append((int(c, 16), float(v)))
    return rows


def test_e2m1_decode_matches_ocp_table():
    rows = _e2m1_table()
    assert len(rows) == 16
    for code, val in rows:
        got = O.e2m1_decode(np.array([code]))[0]
        assert got == val and np.signbit(got) == np.signbit(val), (code, got, val)


def test_e2m1_encode_exact_values_roundtrip():
    for code, val in _e2m1_table():
        enc = O.e2m1_encode(np.array([val], dtype=np.float32))[0]
        assert enc == code, (code, val, enc)


@pytest.mark.parametrize("v,code", [
    (0.25, 0x0), (0.75, 0x2), (1.25, 0x2), (1.75, 0x4), (2.5, 0x4), (3.5, 0x6), (5.0, 0x6),
    (-0.25, 0x8), (-0.75, 0xA), (-5.0, 0xE), (0.2499, 0x0), (0.2501, 0x1), (7.0, 0x7),
    (1e9, 0x7), (-1e9, 0xF), (-1e-7, 0x8),
])
def test_e2m1_encode_ties_to_even_and_saturates(v, code):
    assert O.e2m1_encode(np.array([v], dtype=np.float32))[0] == code


def test_e2m1_encode_is_nearest_brute_force():
    # brute force over the 16 code values: nearest, ties to the even code
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.uniform(-7, 7, 4000), np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])])
    v = v.astype(np.float32)
    enc = O.e2m1_encode(v)
    table = _e2m1_table()
    for x, c in zip(v, enc):
        best = None
        for code, val in table[:8]:
            dist = abs(abs(float(x)) - val)
            key = (dist, code % 2)  # smaller distance, then even code
            if best is None or key < best[0]:
                best = (key, code)
        expect = best[1] | (8 if np.signbit(x) else 0)
        assert c == expect, (x, c, expect)


def test_e4m3_decode_matches_torch_for_all_bytes():
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = O.e4m3_decode(b)
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.all(both_nan | (ref == got))
    assert O.e4m3_decode(np.array([0x7E]))[0] == 448.0


def test_e4m3_encode_matches_torch_cast():
    rng = np.random.default_rng(2)
    grid = O.e4m3_decode(np.arange(0x7F))
    mids = (grid[:-1] + grid[1:]) / 2
    v = np.concatenate([
        rng.uniform(0, 460, 3000), np.exp(rng.uniform(-14, 6, 3000)), grid, mids,
        np.array([0.0, 2.0 ** -10, 1.5 * 2.0 ** -10, 447.9, 449.0, 463.9]),
    ]).astype(np.float32)
    v = v[v < 464]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = O.e4m3_encode_nonneg(v)
    assert np.array_equal(ref, got)
    # saturation above the largest finite value
    assert O.e4m3_encode_nonneg(np.array([500.0, 1e6], dtype=np.float32)).tolist() == [0x7E, 0x7E]


def test_fp4_entry_size_matches_page():
    facts = json.load(open(os.path.join(GOLD, "page_facts.json")))
    u = np.random.default_rng(3).standard_normal((5, 128)).astype(np.float32)
    codes, scales = O.fp4_pack(u)
    assert codes.shape == (5, 64) and scales.shape == (5, 4)
    assert codes.dtype == np.uint8 and scales.dtype == np.uint8
    assert codes.shape[1] + scales.shape[1] == facts["index_k_entry_bytes"]["value"]


def test_fp4_pack_roundtrip_error_bound():
    rng = np.random.default_rng(4)
    u = (rng.standard_normal((300, 128)) * np.exp(rng.uniform(-6, 4, (300, 1)))).astype(np.float32)
    codes, scales = O.fp4_pack(u)
    back = O.fp4_unpack(codes, scales)
    s = np.repeat(O.e4m3_decode(scales), 32, axis=1)
    amax = np.repeat(np.abs(u.reshape(300, 4, 32)).max(axis=2), 32, axis=1)
    # inside the grid the error is at most one grid step (<= s); beyond 6 s the value clips
    err = np.abs(back - u.astype(np.float64))
    assert np.all(err <= s * 1.0 + np.maximum(0.0, amax - 6 * s) + 1e-12)
    # where the scale is non-zero, the largest element of a block keeps at least half
    # its magnitude (the scale is chosen from amax); a zero scale zeroes the block
    sb = O.e4m3_decode(scales)
    bmax = np.abs(back).reshape(300, 4, 32).max(axis=2)
    umax = np.abs(u).reshape(300, 4, 32).max(axis=2)
    assert np.all(bmax[sb > 0] >= 0.5 * umax[sb > 0])
    assert np.all(bmax[sb == 0] == 0) and np.all(umax[sb == 0] <= 6 * 2.0 ** -10)


def test_fp4_pack_special_blocks():
    u = np.zeros((1, 128), dtype=np.float32)
    u[0, 32:64] = -1.0
    u[0, 64] = 6.0
    u[0, 65] = -3.0
    u[0, 66] = -0.1
    codes, scales = O.fp4_pack(u)
    assert scales[0, 0] == 0 and np.all(codes[0, :16] == 0)          # all-zero block
    # block 1: all equal negatives -> each is -6 * s exactly (code 0xF)
    assert np.all(codes[0, 16:32] == 0xFF)
    # block 2: amax 6 -> sigma = 1 -> s = 1; 6 -> 0x7, -3 -> 0xD; -0.1 -> -0 (0x8)
    assert scales[0, 2] == 0x38
    assert codes[0, 32] == (0x7 | (0xD << 4))
    assert (codes[0, 33] & 0xF) == 0x8
    # even dimension in the low nibble
    assert O.fp4_unpack(codes, scales)[0, 64] == 6.0 and O.fp4_unpack(codes, scales)[0, 65] == -3.0


def test_fp4_pack_is_elementwise_brute_force():
    # independent loop implementation of the per-block rule on a few rows
    rng = np.random.default_rng(5)
    u = rng.standard_normal((6, 128)).astype(np.float32)
    codes, scales = O.fp4_pack(u)
    grid = O.e4m3_decode(np.arange(0x7F))
    vals = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for r in range(6):
        for b in range(4):
            blk = u[r, 32 * b: 32 * b + 32]
            sigma = np.float32(np.max(np.abs(blk))) / np.float32(6)
            # nearest e4m3 byte (ties even)
            best = min(range(0x7F), key=lambda i: (abs(grid[i] - float(sigma)), i % 2))
            assert scales[r, b] == best
            s = np.float32(grid[best])
            for i in range(32):
                x = np.float32(blk[i]) / s
                c = min(range(8), key=lambda j: (abs(vals[j] - abs(float(x))), j % 2)) | (8 if x < 0 or np.signbit(x) else 0)
                byte = codes[r, 16 * b + i // 2]
                got = (byte & 0xF) if i % 2 == 0 else (byte >> 4)
                assert got == c, (r, b, i, blk[i], got, c)


# ---- FP4 main KV: same per-block rule, one scale per 16 of the 512 latent dims

def test_kv_fp4_entry_size_matches_page():
    facts = json.load(open(os.path.join(GOLD, "page_facts.json")))
    rows = np.random.default_rng(6).standard_normal((3, 512)).astype(np.float32)
    codes, scales = O.kv_fp4_pack(rows)
    assert codes.shape == (3, 256) and scales.shape == (3, 32)
    assert codes.shape[1] + scales.shape[1] == facts["main_kv_entry_bytes"]["value"]
    assert facts["main_kv_entry_bytes"]["value"] + facts["index_k_entry_bytes"]["value"] == facts["entry_bytes"]["value"]
    enc = facts["encoder_bytes_per_token"]
    assert enc["layers"] * facts["entry_bytes"]["value"] / enc["m"] == enc["value"]


def test_kv_fp4_exact_grid_roundtrip():
    # Rows built on the FP4 grid: per 16-dim block a scale byte and 16 codes, one of
    # them of magnitude 6 (so amax / 6 is exactly that scale).  Encoding must give
    # back exactly those bytes; any slip in block size, nibble order or either
    # rounding rule breaks it.
    rng = np.random.default_rng(7)
    n = 64
    sb = rng.integers(1, 0x7F, (n, 32)).astype(np.uint8)
    c = rng.integers(0, 16, (n, 512)).astype(np.uint8)
    c[c == 8] = 0                                   # -0 and +0 decode alike; keep +0
    c.reshape(n, 32, 16)[:, :, rng.integers(0, 16)] = 0x7 | (8 * rng.integers(0, 2))
    mag = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    val = np.where(c & 8, -1.0, 1.0) * mag[c & 7]
    s = O.e4m3_decode(sb)
    rows = (val * np.repeat(s, 16, axis=1)).astype(np.float32)
    assert np.all(rows.astype(np.float64) == val * np.repeat(s, 16, axis=1))   # exact in float32
    codes, scales = O.kv_fp4_pack(rows)
    assert np.array_equal(scales, sb)
    assert np.array_equal(codes, (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8))
    assert np.array_equal(O.kv_fp4_unpack(codes, scales), rows.astype(np.float64))


def test_kv_fp4_blocks_are_16_dims_and_local():
    rng = np.random.default_rng(8)
    rows = rng.standard_normal((4, 512)).astype(np.float32)
    c0, s0 = O.kv_fp4_pack(rows)
    for d in (0, 15, 16, 250, 511):
        r = rows.copy()
        r[1, d] = 40.0                               # new block maximum
        c1, s1 = O.kv_fp4_pack(r)
        b = d // 16
        changed = np.nonzero(s1[1] != s0[1])[0].tolist()
        assert changed == [b]
        keep = np.ones(256, dtype=bool)
        keep[8 * b: 8 * b + 8] = False
        assert np.array_equal(c1[1, keep], c0[1, keep])
        assert np.array_equal(np.delete(s1, 1, axis=0), np.delete(s0, 1, axis=0))


def test_kv_fp4_roundtrip_error_bound():
    rng = np.random.default_rng(9)
    u = (rng.standard_normal((200, 512)) * np.exp(rng.uniform(-6, 4, (200, 1)))).astype(np.float32)
    codes, scales = O.kv_fp4_pack(u)
    back = O.kv_fp4_unpack(codes, scales)
    s = np.repeat(O.e4m3_decode(scales), 16, axis=1)
    amax = np.repeat(np.abs(u.reshape(200, 32, 16)).max(axis=2), 16, axis=1)
    err = np.abs(back - u.astype(np.float64))
    assert np.all(err <= s + np.maximum(0.0, amax - 6 * s) + 1e-12)
    # a finer block never has a larger scale than the 32-dim block around it
    _, s32 = O.fp4_pack(u, 32)
    assert np.all(O.e4m3_decode(scales).reshape(200, 16, 2).max(axis=2) == O.e4m3_decode(s32).reshape(200, 16))


def test_e4m3_signed_encoder_matches_torch_and_round_trips():
    # all finite E4M3FN values round-trip; values between them round to nearest even
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = O.e4m3_decode(codes).astype(np.float32)
    back = O.e4m3_encode(vals)
    # -0 keeps its sign bit; every other code returns itself
    assert np.array_equal(back, codes)
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(4000) * 3, rng.standard_normal(2000) * 100,
                        rng.standard_normal(2000) * 1e-3]).astype(np.float32)
    x = x[np.abs(x) < 464]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_encode(x), ref)
    # saturation at 448 and the sign of a value rounding to zero
    assert O.e4m3_encode(np.float32([1e4, -1e4, 448.0, -1e-5]))[:4].tolist() == [0x7E, 0xFE, 0x7E, 0x80]


def test_swa_ring_slots_and_wraparound():
    L_w = 8
    ring = np.zeros((L_w, 512), dtype=np.uint8)
    rows = np.arange(20 * 512, dtype=np.float64).reshape(20, 512) % 7 - 3
    O.swa_ring_append(ring, rows[:12], np.arange(12))
    # positions 4..11 are held (slots 4..7, then 0..3)
    got = O.swa_ring_rows(ring, 4, 11)
    assert np.array_equal(got, rows[4:12])   # small integers are exact in E4M3
    O.swa_ring_append(ring, rows[12:15], np.array([12, -1, 14]))
    assert np.array_equal(O.swa_ring_rows(ring, 14, 14), rows[14:15])
    assert np.array_equal(O.swa_ring_rows(ring, 12, 12), rows[12:13])
    assert np.array_equal(O.swa_ring_rows(ring, 7, 11), rows[7:12])  # position 13 was skipped: slot 5 keeps 5
    assert np.array_equal(O.e4m3_decode(ring[5]), rows[5])
    with pytest.raises(AssertionError):
        O.swa_ring_rows(ring, 0, 8)


def test_ue8m0_decode_and_ceil_encoder():
    # UE8M0: a bare biased exponent, 2^(b - 127), 255 is NaN
    assert O.ue8m0_decode(np.array([127, 126, 128, 0, 254])).tolist() == [1.0, 0.5, 2.0, 2.0 ** -127, 2.0 ** 127]
    assert np.isnan(O.ue8m0_decode(np.array([255]))[0])
    # the encoder picks the smallest power of two at or above sigma
    rng = np.random.default_rng(11)
    sig = np.exp(rng.uniform(-60, 60, size=4000)).astype(np.float32)
    x = O.ue8m0_decode(O.ue8m0_encode_ceil(sig))
    assert np.all(x >= sig.astype(np.float64)) and np.all(x / 2 < sig.astype(np.float64))
    p2 = np.float32([0.25, 1.0, 2.0 ** 20, 2.0 ** -100])
    assert np.array_equal(O.ue8m0_decode(O.ue8m0_encode_ceil(p2)), p2.astype(np.float64))
    assert O.ue8m0_encode_ceil(np.float32([0.0]))[0] == 0


def test_fp4_pack_ue8m0_worked_block_and_bounds():
    # amax 3.0: sigma 0.5 is a power of two, X = 0.5 (byte 126): 3.0 -> 6 (code 7), 1.0 -> 2 (code 4);
    # amax 3.1: sigma 0.5167 -> X = 1 (byte 127): 3.1 -> 3 (code 5); a zero block gets byte 0
    u = np.zeros((1, 128), np.float32)
    u[0, 0], u[0, 1:32], u[0, 32] = 3.0, 1.0, 3.1
    codes, scales = O.fp4_pack(u, 32, O.SCALE_UE8M0)
    assert scales[0].tolist() == [126, 127, 0, 0]
    assert codes[0, 0] == 0x47 and codes[0, 1] == 0x44 and codes[0, 16] == 0x05
    # values on the grid round-trip exactly; anything else is within one scale unit
    rng = np.random.default_rng(12)
    vals = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.5, -1, -1.5, -2, -3, -4, -6])
    grid = rng.choice(vals, size=(64, 128)) * np.repeat(np.exp2(rng.integers(-20, 20, size=(64, 4))), 32, axis=1)
    c, s = O.fp4_pack(grid.astype(np.float32), 32, O.SCALE_UE8M0)
    assert np.array_equal(O.fp4_unpack(c, s, 32, O.SCALE_UE8M0), grid)
    x = rng.standard_normal((200, 128)).astype(np.float32) * np.exp2(rng.integers(-8, 8, size=(200, 1)))
    c, s = O.fp4_pack(x, 32, O.SCALE_UE8M0)
    X = np.repeat(O.ue8m0_decode(s), 32, axis=1)
    assert np.all(np.abs(O.fp4_unpack(c, s, 32, O.SCALE_UE8M0) - x) <= X)
    # the same rows through the E4M3 codec keep their layout and size (68 B per entry)
    c4, s4 = O.fp4_pack(x, 32)
    assert c4.shape == c.shape and s4.shape == s.shape and c.shape[1] + s.shape[1] == 68
