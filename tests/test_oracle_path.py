"""Pins of the oracle's compressor, RoPE, index K, scorer, top-k, HSI pool,
sparse attention and the three layer modes (CPU only)."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import csa2_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")
FACTS = json.load(open(os.path.join(GOLD, "page_facts.json")))


def rng(seed=0):
    return np.random.default_rng(seed)


def weights(D=64, seed=0, m=2):
    r = rng(seed)
    w_kv = r.standard_normal((512, D)) / math.sqrt(D)
    w_gate = r.standard_normal((512, D)) / math.sqrt(D) if m > 1 else None
    return w_kv, w_gate, np.ones(512)


# ----------------------------------------------------------------- RoPE ----

def test_rope_leaves_leading_dims_and_is_identity_at_zero():
    x = rng(1).standard_normal((5, 512))
    y = O.rope_last(x, np.array([0, 3, 100, 7, 1 << 20]))
    assert np.array_equal(y[:, :448], x[:, :448])
    assert np.array_equal(y[0], x[0])
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-12)


def test_rope_relative_position_identity():
    r = rng(2)
    x, y = r.standard_normal(128), r.standard_normal(128)
    for a, b in [(5, 2), (1000, 37), (70000, 69999)]:
        lhs = O.rope_last(x, a) @ O.rope_last(y, b)
        rhs = O.rope_last(x, a - b) @ y
        assert abs(lhs - rhs) < 1e-9 * (1 + abs(rhs))


def test_rope_frequencies_and_pairs():
    # a unit vector on the first rotated pair turns by exactly pos radians (theta_0 = 1);
    # on pair i it turns by pos * base^(-2i/64)
    for i in (0, 5, 31):
        x = np.zeros(512)
        x[448 + 2 * i] = 1.0
        y = O.rope_last(x, 3)
        ang = 3 * 10000.0 ** (-2 * i / 64)
        assert np.allclose(y[448 + 2 * i: 450 + 2 * i], [math.cos(ang), math.sin(ang)], atol=1e-14)
        assert np.count_nonzero(np.abs(y) > 1e-15) <= 2


# ----------------------------------------------------------- compressor ----

def test_compressor_m1_is_projection_plus_norm_and_has_no_gate():
    x = rng(3).standard_normal((8, 64))
    w_kv, _, g = weights(64, 3, 1)
    lat, kv, ids = O.compress(x, w_kv, None, g, 1, 0)
    ref = x @ w_kv.T
    ref = ref / np.sqrt((ref ** 2).mean(1, keepdims=True) + 1e-6)
    assert np.allclose(lat, ref, rtol=1e-12, atol=1e-12)
    with pytest.raises(ValueError):
        O.compress(x, w_kv, w_kv, g, 1, 0)


def test_compressor_m1_gate_weight_is_one():
    # a group of two copies of one token pools to that token for every gate: the
    # softmax weights of a group sum to 1, so with one distinct member the weight is 1
    x = rng(4).standard_normal((6, 64))
    w_kv, w_gate, g = weights(64, 4, 2)
    lat1, _, _ = O.compress(x, w_kv, None, g, 1, 0)
    lat2, _, _ = O.compress(np.repeat(x, 2, axis=0), w_kv, w_gate, g, 2, 0)
    assert np.allclose(lat1, lat2, rtol=1e-12, atol=1e-12)


def test_compressor_group_permutation_invariance_and_locality():
    r = rng(5)
    x = r.standard_normal((16, 64))
    w_kv, w_gate, g = weights(64, 5, 4)
    lat, kv, _ = O.compress(x, w_kv, w_gate, g, 4, 0)
    xp = x.copy()
    xp[4:8] = xp[[6, 4, 7, 5]]           # permute inside group 1: no position bias
    latp, kvp, _ = O.compress(xp, w_kv, w_gate, g, 4, 0)
    assert np.allclose(lat, latp, rtol=1e-12, atol=1e-13)
    xq = x.copy()
    xq[9] += 1.0                          # perturb token 9: only entry 2 changes (disjoint groups)
    latq, _, _ = O.compress(xq, w_kv, w_gate, g, 4, 0)
    changed = np.where(np.abs(latq - lat).max(1) > 0)[0]
    assert changed.tolist() == [2]


def test_compressor_zero_gate_is_group_mean_and_dominant_gate_selects():
    r = rng(6)
    x = r.standard_normal((8, 32))
    w_kv = r.standard_normal((512, 32)) / math.sqrt(32)
    g = np.ones(512)
    lat0, _, _ = O.compress(x, w_kv, np.zeros((512, 32)), g, 2, 0)
    C = x @ w_kv.T
    e = C.reshape(4, 2, 512).mean(1)
    assert np.allclose(lat0, O.rms_norm(e, g, 1e-6), rtol=1e-12)
    # gate that is huge for even tokens only (feature 0 = +-1 marks the token)
    x2 = x.copy()
    x2[:, 0] = np.where(np.arange(8) % 2 == 0, 1.0, -1.0)
    wg = np.zeros((512, 32))
    wg[:, 0] = 200.0
    latd, _, _ = O.compress(x2, w_kv, wg, g, 2, 0)
    Cd = x2 @ w_kv.T
    assert np.allclose(latd, O.rms_norm(Cd[0::2], g, 1e-6), rtol=1e-10)


def test_compressor_rms_one_and_rope_at_group_first_token():
    x = rng(7).standard_normal((12, 64))
    w_kv, w_gate, g = weights(64, 7, 2)
    lat, kv, ids = O.compress(x, w_kv, w_gate, g, 2, start_pos=10)
    assert np.allclose(np.sqrt((lat ** 2).mean(1)), 1.0, rtol=1e-5)
    assert ids.tolist() == list(range(5, 11))
    assert np.array_equal(kv[:, :448], lat[:, :448])
    for j in range(6):
        assert np.allclose(kv[j], O.rope_last(lat[j], 10 + 2 * j), rtol=1e-14)


# -------------------------------------------------------------- index K ----

def test_index_k_uses_pre_rope_latent_and_its_own_rope():
    assert 512 * 128 == FACTS["w_ik_params"]["value"]
    r = rng(8)
    lat = r.standard_normal((4, 512))
    w_ik = np.zeros((128, 512))
    w_ik[np.arange(64), 448 + np.arange(64)] = 1.0      # u[:64] copies the latent's RoPE slice
    w_ik[64 + np.arange(64), np.arange(64)] = 1.0       # u[64:] copies latent dims 0..63
    pos = np.array([0, 6, 40, 1000])
    u, codes, scales = O.index_k(lat, w_ik, pos)
    # the first 64 dims of u are the *unrotated* latent slice
    assert np.allclose(u[:, :64], lat[:, 448:], rtol=1e-15)
    # the last 64 dims are rotated at the entry position
    assert np.allclose(u[:, 64:], O.rope_last(lat[:, :64], pos, n_rope=64), rtol=1e-12)
    assert codes.shape == (4, 64) and scales.shape == (4, 4)


# ---------------------------------------------------------------- score ----

def test_score_single_head_is_relu_dot():
    r = rng(9)
    k = r.standard_normal((20, 128))
    q = r.standard_normal((1, 128))
    s = O.index_scores(q, np.array([1.0]), k, 20)
    assert np.allclose(s, np.maximum(k @ q[0], 0))


def test_score_matches_loops_and_respects_visibility():
    r = rng(10)
    k = r.standard_normal((30, 16))
    q = r.standard_normal((3, 16))
    w = r.standard_normal(3)
    s = O.index_scores(q, w, k, 17)
    assert s.shape == (17,)
    for g in range(17):
        tot = 0.0
        for j in range(3):
            d = sum(q[j, i] * k[g, i] for i in range(16))
            tot += w[j] * (d if d > 0 else 0.0)
        assert abs(tot - s[g]) < 1e-12
    assert O.visible_entries(0, 2) == 0 and O.visible_entries(1, 2) == 1 and O.visible_entries(262143, 2) == 131072
    assert O.visible_entries(5, 1) == 6


# ---------------------------------------------------------------- top-k ----

def test_topk_matches_sorting_with_ties():
    r = rng(11)
    for n, k in [(100, 10), (50, 50), (30, 40), (1000, 512), (0, 4)]:
        s = np.round(r.standard_normal(n) * 3) / 2    # many exact ties
        if n:
            s[r.integers(0, n, size=3)] = -0.0
        got = O.topk_select(s, k)
        brute = sorted(range(n), key=lambda g: (-(s[g] + 0.0), g))[:k]
        exp = sorted(brute) + [-1] * (k - min(k, n))
        assert got.tolist() == exp


def test_topk_negative_zero_equals_zero():
    s = np.array([0.0, -0.0, -0.0, 0.0])
    assert O.topk_select(s, 2).tolist() == [0, 1]
    s = np.array([-0.0, 0.0])
    assert O.topk_select(s, 1).tolist() == [0]


# ------------------------------------------------------------------ HSI ----

def test_hsi_pool_forced_block_and_flat_equivalence():
    r = rng(12)
    n, s, nb, k = 300, 8, 5, 16
    sc = r.standard_normal(n)
    pool = O.hsi_pool(sc, n, s, nb)
    nblk = (n + s - 1) // s
    assert (nblk - 1) in pool.tolist()
    # the rest are the best blocks by max score
    beta = np.array([sc[i * s:(i + 1) * s].max() for i in range(nblk)])
    best = sorted(range(nblk - 1), key=lambda i: (-beta[i], i))[:nb - 1]
    assert sorted(pool.tolist()) == sorted(best + [nblk - 1])
    # pool large enough to hold every block -> selection equals flat top-k
    pool_all = O.hsi_pool(sc, n, s, 64)
    assert pool_all[pool_all >= 0].tolist() == list(range(nblk))
    assert np.array_equal(O.topk_select(sc, k, O.pool_entries(pool_all, n, s)), O.topk_select(sc, k))


def test_hsi_block_size_one():
    # s = 1: the pool is the newest entry plus the n_b - 1 best other entries
    r = rng(13)
    sc = r.standard_normal(64)
    pool = O.hsi_pool(sc, 64, 1, 10)
    best = sorted(range(63), key=lambda g: (-sc[g], g))[:9]
    assert pool.tolist() == sorted(best + [63])


def test_hsi_pool_small_and_clipped():
    sc = np.arange(10, dtype=float)
    assert O.hsi_pool(sc, 10, 4, 8).tolist() == [0, 1, 2, -1, -1, -1, -1, -1]
    assert O.pool_entries(np.array([2, -1]), 10, 4).tolist() == [8, 9]
    assert O.hsi_pool(sc, 0, 4, 2).tolist() == [-1, -1]


# ------------------------------------------------------------ attention ----

def test_window_receptive_field_matches_page():
    for case in FACTS["swa_receptive_field"]:
        L, W = case["layers"], case["window"]
        p = 10 ** 6
        reach = {p}
        for _ in range(L):
            reach = set(u for q in reach for u in O.window_positions(q, W).tolist())
        assert len(reach) == case["positions"]


def test_attention_convex_hull_and_special_cases():
    r = rng(14)
    kv = r.standard_normal((40, 512))
    swa = r.standard_normal((20, 512))
    q = r.standard_normal((4, 512))
    sel = np.array([3, 7, 11, 39, -1, -1])
    o, p, rows = O.sparse_attention(q, kv, sel, swa, 100, 110, 8)
    assert rows.shape[0] == 4 + 8
    assert np.all(p >= 0) and np.allclose(p.sum(1), 1)
    assert np.allclose(o, p @ rows)
    lo, hi = rows.min(0), rows.max(0)
    assert np.all(o >= lo - 1e-12) and np.all(o <= hi + 1e-12)
    # q = 0 -> uniform mean of the rows
    o0, _, _ = O.sparse_attention(np.zeros((1, 512)), kv, sel, swa, 100, 110, 8)
    assert np.allclose(o0[0], rows.mean(0))
    # a single row -> o equals that row
    o1, _, _ = O.sparse_attention(q, kv, np.array([5]), swa, 100, 100, 1)
    assert O.window_positions(100, 1, 100).tolist() == [100]
    o1b, _, _ = O.sparse_attention(q, kv, np.array([-1]), swa, 100, 100, 1)
    assert np.allclose(o1b, np.repeat(swa[0][None], 4, 0))


@pytest.mark.parametrize("m", [1, 2, 4])
def test_compress_step_streams_the_prefill_compressor(m):
    """Appending the tokens of a sequence one at a time (the partial-group state
    carries a group's earlier tokens) yields the rows the whole-sequence
    compressor computes: the same group softmax, norm and RoPE at the same entry
    positions, reached by a different route (per-group vs batched)."""
    r = rng(24 + m)
    T, D = 8 * m, 48
    x = r.standard_normal((T, D))
    w_kv = r.standard_normal((512, D)) / math.sqrt(D)
    w_gate = r.standard_normal((512, D)) / math.sqrt(D) if m > 1 else None
    gamma = 1.0 + 0.1 * r.standard_normal(512)
    lat, kv, ids = O.compress(x, w_kv, w_gate, gamma, m, 0)
    pending, got = [], []
    for t in range(T):
        pending, ent = O.compress_step(pending, x[t], w_kv, w_gate, gamma, t, m)
        if t % m == m - 1:
            assert ent is not None and ent[0] == t // m and pending == []
            got.append(ent)
        else:
            assert ent is None and len(pending) == t % m + 1
    assert [g for g, _, _ in got] == list(ids)
    assert np.allclose(np.stack([l for _, l, _ in got]), lat, rtol=1e-12, atol=1e-12)
    assert np.allclose(np.stack([k for _, _, k in got]), kv, rtol=1e-12, atol=1e-12)


def test_attention_sink_special_cases():
    """The sink logit (denominator only): a sink of -inf is the plain softmax; with
    q = 0 every row logit is 0, so o = sum(rows) / (R + exp(sink)) in closed form;
    probabilities stay non-negative and sum to 1 / (1 + exp(sink - lse_rows)); a
    huge sink drives o to 0; the log-sum-exp gains the sink term."""
    r = rng(19)
    kv = r.standard_normal((40, 512))
    swa = r.standard_normal((20, 512))
    q = r.standard_normal((4, 512))
    sel = np.array([3, 7, 11, 39, -1])
    o_plain, p_plain, rows = O.sparse_attention(q, kv, sel, swa, 100, 110, 8)
    o_ninf, p_ninf, _ = O.sparse_attention(q, kv, sel, swa, 100, 110, 8, sink=np.full(4, -np.inf))
    assert np.array_equal(o_ninf, o_plain) or np.allclose(o_ninf, o_plain, rtol=0, atol=1e-15)
    sink = np.array([-3.0, 0.0, 2.5, 7.0])
    R = rows.shape[0]
    o0, p0, _ = O.sparse_attention(np.zeros((4, 512)), kv, sel, swa, 100, 110, 8, sink=sink)
    for h in range(4):
        assert np.allclose(o0[h], rows.sum(0) / (R + math.exp(sink[h])), rtol=1e-12)
        assert np.allclose(p0[h], 1.0 / (R + math.exp(sink[h])), rtol=1e-12)
    o, p, _ = O.sparse_attention(q, kv, sel, swa, 100, 110, 8, sink=sink)
    assert np.all(p >= 0)
    lse_rows = O.attention_lse(q, rows)
    assert np.allclose(p.sum(1), 1.0 / (1.0 + np.exp(sink - lse_rows)), rtol=1e-12)
    assert np.allclose(o, p @ rows)
    # o = (1 - p_sink) * o_plain: the sink only rescales
    assert np.allclose(o, o_plain * p.sum(1, keepdims=True), rtol=1e-10, atol=1e-13)
    big, _, _ = O.sparse_attention(q, kv, sel, swa, 100, 110, 8, sink=np.full(4, 1e3))
    assert np.allclose(big, 0.0, atol=1e-300)
    assert np.allclose(O.attention_lse(q, rows, sink=sink), np.logaddexp(lse_rows, sink), rtol=1e-12)
    # no rows at all: zero output, the sink alone in the normaliser
    assert np.allclose(O.attention_lse(q, rows[:0], sink=sink), sink)


def test_attention_select_all_equals_torch_sdpa():
    r = rng(15)
    kv = r.standard_normal((24, 512))
    swa = r.standard_normal((10, 512))
    q = r.standard_normal((3, 512))
    o, _, rows = O.sparse_attention(q, kv, np.arange(24), swa, 0, 9, 10)
    R = torch.from_numpy(rows)[None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q)[None, :, None], R, R)
    assert np.allclose(o, ref[0, :, 0].numpy(), rtol=1e-10, atol=1e-12)


def test_attention_exponential_tilt():
    # p(q0 + dq) is proportional to p(q0) * exp(c . dq / sqrt(d))
    r = rng(16)
    kv = r.standard_normal((30, 512))
    swa = r.standard_normal((1, 512))
    q0 = r.standard_normal((1, 512))
    dq = r.standard_normal((1, 512)) * 0.3
    sel = np.arange(30)
    _, p0, rows = O.sparse_attention(q0, kv, sel, swa, 0, 0, 1)
    _, p1, _ = O.sparse_attention(q0 + dq, kv, sel, swa, 0, 0, 1)
    t = p0[0] * np.exp(rows @ dq[0] / math.sqrt(512))
    assert np.allclose(p1[0], t / t.sum(), rtol=1e-10)


# ---------------------------------------------------------------- modes ----

def _tiny_layers(B=2, L=16, D=32, m=2, H_I=2, H=2, seed=20):
    r = rng(seed)
    x = r.standard_normal((B, L, D))
    w_kv, w_gate, g = weights(D, seed, m)
    w_ik = r.standard_normal((128, 512)) / math.sqrt(512)
    q_pos = np.tile(np.arange(L), (B, 1))

    def inputs(with_x=True):
        return O.LayerInputs(q=r.standard_normal((B, L, H, 512)), swa_kv=r.standard_normal((B, L, 512)),
                             q_pos=q_pos, swa_pos0=np.zeros(B, int), q_idx=r.standard_normal((B, L, H_I, 128)),
                             w=r.standard_normal((B, L, H_I)), x=x if with_x else None)
    full = O.LayerConfig(O.FULL, m=m, k=3, W=4, w_kv=w_kv, w_gate=w_gate, gamma=g, w_ik=w_ik)
    return full, inputs


def test_modes_reuse_shares_set_and_reindex_rescores():
    full, inputs = _tiny_layers()
    rt = O.Runtime()
    with pytest.raises(O.SlotEmpty):
        O.layer_forward(rt, O.LayerConfig(O.REUSE, m=2, k=3, W=4), inputs(False))
    fin = inputs()
    o_full = O.layer_forward(rt, full, fin)
    kv_full, ik_full, top_full = rt.compress_kv, rt.index_k, rt.topk_idxs.copy()
    # causality of every selected entry, and the set size
    for b in range(2):
        for t in range(16):
            sel = top_full[b, t][top_full[b, t] >= 0]
            assert np.all(sel < O.visible_entries(t, 2))
            assert len(sel) == min(3, O.visible_entries(t, 2))
    # Reuse: same indices bit for bit, its own queries; output = attention over those indices
    rin = inputs(False)
    o_reuse = O.layer_forward(rt, O.LayerConfig(O.REUSE, m=2, k=3, W=4), rin)
    assert rt.topk_idxs is not None and np.array_equal(rt.topk_idxs, top_full)
    ref = O.sparse_attention(rin.q[1, 9], kv_full[1], top_full[1, 9], rin.swa_kv[1], 0, 9, 4)[0]
    assert np.allclose(o_reuse[1, 9], ref)
    # Reuse output does not depend on the index K (poison it)
    rt2 = O.Runtime(compress_kv=kv_full, index_k=(None, None), topk_idxs=top_full)
    assert np.allclose(O.layer_forward(rt2, O.LayerConfig(O.REUSE, m=2, k=3, W=4), rin), o_reuse)
    # Reindex with the Full layer's own indexer queries reproduces its selection,
    # and writes neither the KV nor the index K
    rt.writes.clear()
    rin2 = O.LayerInputs(q=rin.q, swa_kv=rin.swa_kv, q_pos=fin.q_pos, swa_pos0=fin.swa_pos0,
                         q_idx=fin.q_idx, w=fin.w)
    O.layer_forward(rt, O.LayerConfig(O.REINDEX, m=2, k=3, W=4), rin2)
    assert np.array_equal(rt.topk_idxs, top_full)
    assert rt.writes == ["topk_idxs"] and rt.compress_kv is kv_full and rt.index_k is ik_full


def test_modes_hsi_build_and_use():
    full, inputs = _tiny_layers(B=1, L=40, m=1, seed=21)
    full.k, full.hsi, full.hsi_s, full.hsi_nb = 4, "build", 4, 3
    rt = O.Runtime()
    fin = inputs()
    O.layer_forward(rt, full, fin)
    assert rt.candidates.shape == (1, 40, 3) and rt.candidates_s == 4
    rin = inputs(False)
    cfg = O.LayerConfig(O.REINDEX, m=1, k=4, W=4, hsi="use", hsi_s=4, hsi_nb=3)
    O.layer_forward(rt, cfg, rin)
    for t in range(40):
        pool = set(O.pool_entries(rt.candidates[0, t], t + 1, 4).tolist())
        sel = rt.topk_idxs[0, t]
        assert set(sel[sel >= 0].tolist()) <= pool
        assert len(sel[sel >= 0]) == min(4, len(pool))


@pytest.mark.parametrize("m", [1, 2])
def test_decode_append_grows_the_slots_like_a_longer_prefill(m):
    # a Full prefill of P tokens, then S decode appends, leaves the runtime's main KV
    # and index K equal to those of one Full prefill over all P + S tokens (the
    # entries of complete groups; the trailing partial group is not an entry yet)
    B, P, S, D = 2, 8, 2 * m + (1 if m > 1 else 0), 32
    full, inputs = _tiny_layers(B=B, L=P + S, D=D, m=m, seed=30 + m)
    fin = inputs()
    whole = O.Runtime()
    O.layer_forward(whole, full, O.LayerInputs(q=fin.q, swa_kv=fin.swa_kv, q_pos=fin.q_pos, swa_pos0=fin.swa_pos0,
                                               q_idx=fin.q_idx, w=fin.w, x=fin.x[:, :(P + S) // m * m]))
    rt = O.Runtime()
    pre = O.LayerInputs(q=fin.q[:, :P], swa_kv=fin.swa_kv, q_pos=fin.q_pos[:, :P], swa_pos0=fin.swa_pos0,
                        q_idx=fin.q_idx[:, :P], w=fin.w[:, :P], x=fin.x[:, :P])
    O.layer_forward(rt, full, pre)
    pending = [[] for _ in range(B)]
    written = []
    for t in range(P, P + S):
        written.append(O.layer_append(rt, full, pending, fin.x[:, t], np.full(B, t)))
    n = (P + S) // m
    assert rt.compress_kv.shape[1] == n
    assert np.allclose(rt.compress_kv, whole.compress_kv, rtol=1e-12, atol=1e-12)
    assert np.array_equal(rt.index_k[0], whole.index_k[0]) and np.array_equal(rt.index_k[1], whole.index_k[1])
    assert [w[0] for w in written if w[0] is not None] == list(range(P // m, n))
    assert len(pending[0]) == (P + S) % m


def test_full_decode_step_sees_appended_entries_and_reindex_follows():
    # after the appends, a Full decode query selects among all its visible entries
    # (k covers them all, so the appended ones must be in the set), and a Reindex
    # layer reading the slots sees the same grown index K
    B, P, m, k = 1, 8, 2, 16
    full, inputs = _tiny_layers(B=B, L=P + 4, D=32, m=m, seed=40)
    full.k = k
    fin = inputs()
    rt = O.Runtime()
    O.layer_forward(rt, full, O.LayerInputs(q=fin.q[:, :P], swa_kv=fin.swa_kv, q_pos=fin.q_pos[:, :P],
                                            swa_pos0=fin.swa_pos0, q_idx=fin.q_idx[:, :P], w=fin.w[:, :P],
                                            x=fin.x[:, :P]))
    pending = [[]]
    O.layer_append(rt, full, pending, fin.x[:, P], np.array([P]))
    p = P + 1
    step = O.LayerInputs(q=fin.q[:, p:p + 1], swa_kv=fin.swa_kv, q_pos=np.array([[p]]), swa_pos0=fin.swa_pos0,
                         q_idx=fin.q_idx[:, p:p + 1], w=fin.w[:, p:p + 1])
    o = O.full_decode_step(rt, full, pending, fin.x[:, p], step)
    sel = rt.topk_idxs[0, 0]
    assert list(sel[sel >= 0]) == list(range((p + 1) // m))          # 5 entries, the last one just appended
    ref = O.sparse_attention(step.q[0, 0], rt.compress_kv[0], sel, fin.swa_kv[0], 0, p, full.W)[0]
    assert np.allclose(o[0, 0], ref)
    O.layer_forward(rt, O.LayerConfig(O.REINDEX, m=m, k=k, W=full.W), step)
    assert np.array_equal(rt.topk_idxs[0, 0], sel)


def _decoder_stack(B=1, L=48, D=32, H_I=2, H=2, W=6, k=5, seed=50):
    # decoder macro-block: a Full layer at m = 1 (compressing H20), then Reindex, Reuse
    r = rng(seed)
    h20 = r.standard_normal((B, L, D))
    w_kv, _, g = weights(D, seed, 1)
    w_ik = r.standard_normal((128, 512)) / math.sqrt(512)
    cfgs = [O.LayerConfig(O.FULL, m=1, k=k, W=W, w_kv=w_kv, w_gate=None, gamma=g, w_ik=w_ik),
            O.LayerConfig(O.REINDEX, m=1, k=k, W=W), O.LayerConfig(O.REUSE, m=1, k=k, W=W)]
    full_inputs = [O.LayerInputs(q=r.standard_normal((B, L, H, 512)), swa_kv=r.standard_normal((B, L, 512)),
                                 q_pos=np.tile(np.arange(L), (B, 1)), swa_pos0=np.zeros(B, int),
                                 q_idx=r.standard_normal((B, L, H_I, 128)), w=r.standard_normal((B, L, H_I)))
                   for _ in cfgs]
    return h20, cfgs, full_inputs


def _tail(inp, L, R):
    return O.LayerInputs(q=inp.q[:, L - R:], swa_kv=inp.swa_kv[:, L - R:], q_pos=inp.q_pos[:, L - R:],
                         swa_pos0=inp.swa_pos0, q_idx=inp.q_idx[:, L - R:], w=inp.w[:, L - R:])


def test_bounded_replay_keeps_the_global_kv_and_clips_only_the_window():
    h20, cfgs, full_inputs = _decoder_stack()
    L, W = h20.shape[1], cfgs[0].W
    # the un-truncated decoder prefill: every position through every layer
    rt_full = O.Runtime()
    ref = []
    for l, (cfg, inp) in enumerate(zip(cfgs, full_inputs)):
        inp.x = h20 if l == 0 else None
        ref.append(O.layer_forward(rt_full, cfg, inp))
    for R in (L, 17):
        rt = O.Runtime()
        outs = O.decoder_replay(rt, cfgs, [_tail(i, L, R) for i in full_inputs], h20, R)
        # the truncation never touches the global KV or the index K
        assert np.array_equal(rt.compress_kv, rt_full.compress_kv)
        assert np.array_equal(rt.index_k[0], rt_full.index_k[0])
        for l in range(3):
            assert outs[l].shape == (1, R, 2, 512)
            for j in range(R):
                p = L - R + j
                if p >= L - R + W - 1:
                    # the window lies inside the replayed segment: exactly the full prefill
                    assert np.allclose(outs[l][0, j], ref[l][0, p], rtol=1e-12, atol=1e-12), (R, l, p)
        if R < L:
            # the first replayed position sees one window row instead of W
            p = L - R
            assert not np.allclose(outs[2][0, 0], ref[2][0, p])
            tk = rt.topk_idxs[0, 0]
            manual = O.sparse_attention(full_inputs[2].q[0, p], rt.compress_kv[0], tk,
                                        full_inputs[2].swa_kv[0, L - R:], L - R, p, W)[0]
            assert np.allclose(outs[2][0, 0], manual, rtol=1e-12, atol=1e-12)
