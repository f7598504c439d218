"""CPU tests of the comparison rules in parity_utils: each planted difference that
the rules must reject is rejected, and each difference they allow (a rounding
midpoint, a zero whose sign is decided by summation order) is accepted.  The
"GPU" side here is the oracle's own output with the difference planted on the
CPU."""
import numpy as np
import pytest

from oracle import csa2_oracle as O
from parity_utils import check_fp4, check_topk_row


def _block_with(values, block=32):
    """One row of one FP4 block whose amax is 6 (so the scale is exactly 1.0 and
    u/s is the value itself), with the given values in its first slots."""
    u = np.zeros((1, block), dtype=np.float64)
    u[0, -1] = 6.0
    u[0, :len(values)] = values
    return u


def _flip_code(codes, dim, new_code):
    c = codes.copy()
    byte, hi = divmod(dim, 2)
    if hi:
        c[0, byte] = (c[0, byte] & 0x0F) | (new_code << 4)
    else:
        c[0, byte] = (c[0, byte] & 0xF0) | new_code
    return c


def test_exact_codes_pass():
    rng = np.random.default_rng(0)
    u = rng.standard_normal((64, 128))
    codes, scales = O.fp4_pack(u.astype(np.float32))
    assert check_fp4(u, codes, scales) == (0, 0)


def test_signed_zero_allowed_only_near_zero():
    # -1e-5 rounds to code 0x8 (negative zero); the other side may say 0x0
    u = _block_with([-1e-5, -0.2])
    codes, scales = O.fp4_pack(u.astype(np.float32))
    assert O.fp4_pack(np.float32([[-1e-5] + [0.0] * 30 + [6.0]]))[0][0, 0] & 0x0F == 0x8
    assert check_fp4(u, _flip_code(codes, 0, 0x0), scales) == (1, 0)
    # -0.2 also rounds to magnitude 0 but is far from zero: its sign is no
    # rounding accident, so 0x0 against the oracle's 0x8 must fail
    with pytest.raises(AssertionError):
        check_fp4(u, _flip_code(codes, 1, 0x0), scales)


def test_midpoint_flip_allowed_other_flips_rejected():
    u = _block_with([1.25, 1.0])   # 1.25 is the E2M1 midpoint between 1.0 and 1.5
    codes, scales = O.fp4_pack(u.astype(np.float32))
    assert check_fp4(u, _flip_code(codes, 0, 0x3), scales) == (1, 0)   # 1.5 instead of 1.0
    with pytest.raises(AssertionError):
        check_fp4(u, _flip_code(codes, 1, 0x3), scales)                 # 1.0 is no midpoint


def test_scale_byte_flip_away_from_midpoint_rejected():
    u = _block_with([1.0])
    codes, scales = O.fp4_pack(u.astype(np.float32))
    bad = scales.copy()
    bad[0, 0] += 1
    with pytest.raises(AssertionError):
        check_fp4(u, codes, bad)


def test_ue8m0_scale_flip_only_at_a_power_of_two():
    # amax = 6 * 2^3 exactly: sigma = 8 is a power of two, so a GPU whose sigma
    # came out a hair above it may pick the next byte (scale 16), with codes to match
    u = _block_with([1.0]) * 8.0
    codes, scales = O.fp4_pack(u.astype(np.float32), 32, O.SCALE_UE8M0)
    assert scales[0, 0] == 127 + 3
    up = scales.copy()
    up[0, 0] += 1
    codes_up, _ = O.fp4_pack(u.astype(np.float32) / 2.0, 32, O.SCALE_UE8M0)   # the codes under scale 16
    assert check_fp4(u, codes_up, up, scale_fmt=O.SCALE_UE8M0)[1] == 1
    # amax = 6 * 5: sigma = 5 is no power of two, the byte is fixed
    u = _block_with([1.0]) * 5.0
    codes, scales = O.fp4_pack(u.astype(np.float32), 32, O.SCALE_UE8M0)
    bad = scales.copy()
    bad[0, 0] += 1
    with pytest.raises(AssertionError):
        check_fp4(u, codes, bad, scale_fmt=O.SCALE_UE8M0)
    assert check_fp4(u, codes, scales, scale_fmt=O.SCALE_UE8M0) == (0, 0)


def test_topk_band_rule():
    scores = np.array([5.0, 4.0, 3.0, 2.0, 1.0, 0.5])
    ids = np.arange(6)
    assert check_topk_row(scores, ids, np.array([0, 1, 2]), 3)
    with pytest.raises(AssertionError):   # a clearly worse entry instead of a better one
        check_topk_row(scores, ids, np.array([0, 1, 3]), 3)
    with pytest.raises(AssertionError):   # not ascending
        check_topk_row(scores, ids, np.array([1, 0, 2]), 3)
    with pytest.raises(AssertionError):   # padding must be -1
        check_topk_row(scores, ids, np.array([0, 1, 2, 5]), 3)
    # a near tie at the boundary: either side is valid, only the oracle's is exact
    tie = np.array([5.0, 4.0, 3.0, 3.0 * (1 - 1e-5), 1.0])
    assert not check_topk_row(tie, np.arange(5), np.array([0, 1, 3]), 3)
    assert check_topk_row(tie, np.arange(5), np.array([0, 1, 2]), 3)
