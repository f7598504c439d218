"""GPU parity of each CSA2 entry point against the CPU oracle, through the C ABI.

Small seeded cases that span several tiles and ragged tails, plus edge cases
(empty visible range, fewer entries than k, padded / out-of-range top-k ids,
windows clipped by the sequence start or by the window buffer)."""
import math

import numpy as np
import pytest
import torch

from oracle import csa2_oracle as O
from parity_utils import check_fp4, check_topk_row, row_rel_err, say
import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from compressed_sparse_attention_compress_amd import csa2 as K

DEV = "cuda"
TOL = {torch.float32: 1e-3, torch.bfloat16: 2e-2}


def npy(t):
    return t.detach().float().cpu().numpy().astype(np.float64) if t.is_floating_point() else t.cpu().numpy()


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# ------------------------------------------------------------------ FP4 ----

def test_fp4_pack_bitexact():
    say("case: fp4_pack 4096 rows")
    g = torch.Generator().manual_seed(11)
    rows = torch.randn(4096, 128, generator=g) * torch.exp(torch.empty(4096, 1).uniform_(-9, 7, generator=g))
    rows[0] = 0.0
    rows[1, :32] = -1.0
    rows[2, :] = 1e5          # saturating scale
    rows[3, 5] = -1e-30
    rows[4, 64:96] = 6.0
    rows = rows.float()
    codes = torch.empty(4096, 64, dtype=torch.uint8, device=DEV)
    scales = torch.empty(4096, 4, dtype=torch.uint8, device=DEV)
    K.csa2_fp4_pack(rows.to(DEV), codes, scales)
    torch.cuda.synchronize()
    c_o, s_o = O.fp4_pack(rows.numpy())
    assert np.array_equal(scales.cpu().numpy(), s_o)
    assert np.array_equal(codes.cpu().numpy(), c_o)


# -------------------------------------------------------------- index K ----

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_index_k_vs_oracle(dtype):
    B, N, m, entry0, N_cap = 2, 333, 2, 5, 400
    say(f"case: index_k dtype={dtype} B={B} N={N}")
    lat = synth.gaussian((B, N, 512), 1.0, 3, "u", 0, torch.float32, DEV)
    w_ik = synth.linear_weight(128, 512, 3, "w_ik", 0, dtype, DEV)
    codes = torch.zeros(B, N_cap, 64, dtype=torch.uint8, device=DEV)
    scales = torch.zeros(B, N_cap, 4, dtype=torch.uint8, device=DEV)
    K.csa2_index_k(None, lat, w_ik, codes, scales, m=m, entry0=entry0)
    torch.cuda.synchronize()
    cg, sg = codes.cpu().numpy(), scales.cpu().numpy()
    for b in range(B):
        u, _, _ = O.index_k(npy(lat[b]), npy(w_ik), (entry0 + np.arange(N)) * m)
        nc, ns = check_fp4(u, cg[b, entry0:entry0 + N], sg[b, entry0:entry0 + N], f"b{b}")
        say(f"  b={b}: code mismatches in band {nc}, scale mismatches in band {ns}")
        assert nc <= 4 and ns <= 1
    # rows outside [entry0, entry0+N) untouched
    assert codes[:, :entry0].abs().sum().item() == 0 and codes[:, entry0 + N:].sum().item() == 0


# ------------------------------------------------------------ compressor ----

@pytest.mark.parametrize("dtype,m", [(torch.float32, 2), (torch.float32, 1), (torch.bfloat16, 1),
                                     (torch.bfloat16, 2), (torch.bfloat16, 4)])
def test_compress_vs_oracle(dtype, m):
    B, T, D, start = 2, 264, 256 if dtype == torch.float32 else 512, 16
    say(f"case: compress dtype={dtype} m={m} B={B} T={T} D={D}")
    x = synth.gaussian((B, T, D), 1.0, 5, "x", 0, dtype, DEV)
    w_kv = synth.linear_weight(512, D, 5, "w_kv", 0, dtype, DEV)
    w_gate = synth.linear_weight(512, D, 5, "w_gate", 0, dtype, DEV) if m > 1 else None
    gamma = (1.0 + 0.1 * synth.gaussian((512,), 1.0, 5, "w", 0, torch.float32, DEV)).contiguous()
    n = T // m
    N_cap = start // m + n + 3
    lat = torch.empty(B, n, 512, dtype=torch.float32, device=DEV)
    kv = torch.zeros(B, N_cap, 512, dtype=dtype, device=DEV)
    K.csa2_compress(None, x, w_kv, w_gate, gamma, lat, kv, m=m, start_pos=start)
    torch.cuda.synchronize()
    tol = TOL[dtype]
    for b in range(B):
        lp, kvo, ids = O.compress(npy(x[b]), npy(w_kv), None if w_gate is None else npy(w_gate), npy(gamma), m,
                                  start)
        e1 = row_rel_err(npy(lat[b]), lp)
        e2 = row_rel_err(npy(kv[b, start // m:start // m + n]), kvo)
        say(f"  b={b}: latent rel err {e1:.2e}, cache rel err {e2:.2e}")
        assert e1 <= 1e-4 and e2 <= tol
    assert kv[:, :start // m].abs().sum().item() == 0 and kv[:, start // m + n:].abs().sum().item() == 0


# ------------------------------------------------------- score + top-k ----

def _index_cache(B, N_cap, n_fill, seed):
    u = synth.gaussian((B, N_cap, 128), 1.0, seed, "u", 0, torch.float32, "cpu").numpy()
    codes = np.zeros((B, N_cap, 64), np.uint8)
    scales = np.zeros((B, N_cap, 4), np.uint8)
    for b in range(B):
        codes[b, :n_fill], scales[b, :n_fill] = O.fp4_pack(u[b, :n_fill])
    return codes, scales


@pytest.mark.parametrize("dtype,m,k,H_I", [(torch.float32, 2, 32, 4), (torch.bfloat16, 1, 512, 32),
                                           (torch.bfloat16, 2, 100, 32), (torch.bfloat16, 1, 64, 7)])
def test_score_topk_vs_oracle(dtype, m, k, H_I):
    B, N_cap, n_fill = 2, 3000, 2900
    pos = np.array([[0, m - 1, 5, 2 * k * m + 3, 3000 * m], [m * 700 + 1, 1, 9999, 64 * m - 1, 2 * m * 1500 - 1]])
    T = pos.shape[1]
    say(f"case: score_topk dtype={dtype} m={m} k={k} H_I={H_I}")
    codes, scales = _index_cache(B, N_cap, n_fill, 21)
    q_idx = synth.gaussian((B, T, H_I, 128), 1.0, 21, "q_idx", 0, dtype, DEV)
    w = synth.gaussian((B, T, H_I), 1.0, 21, "w", 0, torch.float32, DEV)
    q_pos = torch.tensor(pos, dtype=torch.int32, device=DEV)
    topk = torch.full((B, T, k), -7, dtype=torch.int32, device=DEV)
    K.csa2_score_topk(None, q_idx, w, torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV), q_pos, topk,
                      n_entries=n_fill, m=m, k=k)
    torch.cuda.synchronize()
    tg = topk.cpu().numpy()
    exact = 0
    for b in range(B):
        kd = O.fp4_unpack(codes[b], scales[b])
        for t in range(T):
            nv = min(n_fill, O.visible_entries(pos[b, t], m))
            sc = O.index_scores(npy(q_idx[b, t]), npy(w[b, t]), kd, nv)
            exact += check_topk_row(sc, np.arange(nv), tg[b, t], k, f"b{b} t{t} n_t={nv}")
    say(f"  exact set equality on {exact}/{B * T} queries")
    assert exact >= B * T - 1


@pytest.mark.parametrize("m,k,H_I", [(2, 512, 32), (1, 64, 7)])
def test_score_topk_many_queries_vs_oracle(m, k, H_I):
    """Many bf16 queries over one cache (the query-tiled scorer + per-query select):
    a query count that is not a multiple of the 4-query tile, several 1024-entry
    workgroup chunks, positions before the first entry, inside and past the filled
    cache; every 5th query checked against the oracle."""
    B, T, N_cap, n_fill = 2, 301, 3000, 2900
    say(f"case: score_topk many queries m={m} k={k} H_I={H_I}")
    gen = np.random.default_rng(29)
    pos = gen.integers(-3, n_fill * m + 200, size=(B, T)).astype(np.int32)
    pos[0, :4] = [-1, 0, m - 1, m]
    codes, scales = _index_cache(B, N_cap, n_fill, 29)
    q_idx = synth.gaussian((B, T, H_I, 128), 1.0, 29, "q_idx", 0, torch.bfloat16, DEV)
    w = synth.gaussian((B, T, H_I), 1.0, 29, "w", 0, torch.float32, DEV)
    q_pos = torch.tensor(pos, dtype=torch.int32, device=DEV)
    topk = torch.full((B, T, k), -7, dtype=torch.int32, device=DEV)
    K.csa2_score_topk(None, q_idx, w, torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV), q_pos, topk,
                      n_entries=n_fill, m=m, k=k)
    torch.cuda.synchronize()
    tg = topk.cpu().numpy()
    exact, n = 0, 0
    for b in range(B):
        kd = O.fp4_unpack(codes[b], scales[b])
        for t in list(range(0, T, 5)) + [T - 1]:
            nv = min(n_fill, O.visible_entries(pos[b, t], m)) if pos[b, t] >= 0 else 0
            sc = O.index_scores(npy(q_idx[b, t]), npy(w[b, t]), kd, nv)
            exact += check_topk_row(sc, np.arange(nv), tg[b, t], k, f"b{b} t{t} n_t={nv}")
            n += 1
    say(f"  exact set equality on {exact}/{n} queries")
    assert exact >= n - 1


@pytest.mark.parametrize("dtype,T,n_fill,n_rows", [(torch.bfloat16, 3, 5000, 50), (torch.bfloat16, 300, 5000, 50),
                                                   (torch.bfloat16, 300, 4000, 50), (torch.float32, 3, 5000, 50),
                                                   (torch.bfloat16, 64, 40000, 50), (torch.bfloat16, 8192, 10000, 50),
                                                   (torch.float32, 8192, 10000, 50),
                                                   (torch.bfloat16, 8192, 70000, 50),
                                                   (torch.bfloat16, 4, 100000, 50), (torch.bfloat16, 3, 200000, 8)])
def test_score_topk_exact_ties_vs_oracle(dtype, T, n_fill, n_rows):
    """An index-K cache of n_rows distinct rows repeated: every score value occurs
    n_fill / n_rows times, so the k-th best falls inside a group of equal scores and
    the selection must take that group's smallest positions (ties go to the smaller
    entry id).  Equal rows give bit-identical scores on both sides, and the distinct
    values are kept well apart, so the chosen set is unique and compared exactly:
    T = 3 .. 64 run the chunked scorer and the merge (with 100000 entries and more
    the candidate lists, over 32768 per query, are pre-filtered in groups first;
    with 8 rows over 200000 entries more than the merge's LDS holds survive the
    pre-filter, and it selects straight from the groups' ranges), T = 300 the
    query-tiled scorer and the per-query select (rows of up to 4096 keys held 64
    per lane, longer rows 128), T = 8192 the streaming scorer with its in-part cutbacks to the k
    best (the boundary tie group cut there too), over one part and, with 70000
    entries, two parts and the merge."""
    B, k, H_I, m = 1, 512, 32, 1
    say(f"case: score_topk exact ties dtype={dtype} T={T} n={n_fill} rows={n_rows}")
    u = synth.gaussian((n_rows, 128), 1.0, 31, "u", 0, torch.float32, "cpu").numpy()
    base_c, base_s = O.fp4_pack(u)
    rep = np.random.default_rng(31).integers(0, n_rows, size=n_fill)
    codes = base_c[rep][None].copy()
    scales = base_s[rep][None].copy()
    kd = O.fp4_unpack(codes[0], scales[0])
    q_idx = synth.gaussian((B, T, H_I, 128), 1.0, 31, "q_idx", 0, dtype, DEV)
    w = synth.gaussian((B, T, H_I), 1.0, 31, "w", 0, torch.float32, DEV)
    q_pos = torch.full((B, T), n_fill * m - 1, dtype=torch.int32, device=DEV)
    topk = torch.full((B, T, k), -7, dtype=torch.int32, device=DEV)
    K.csa2_score_topk(None, q_idx, w, torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV), q_pos, topk,
                      n_entries=n_fill, m=m, k=k)
    torch.cuda.synchronize()
    tg = topk.cpu().numpy()
    checked = ties = 0
    for t in sorted(set([0, 1, T - 1] + list(range(0, T, max(37, T // 12))))):
        sc = O.index_scores(npy(q_idx[0, t]), npy(w[0, t]), kd, n_fill)
        vals = np.unique(sc)
        gaps = np.diff(vals) / np.maximum(np.abs(vals[1:]), 1e-30)
        if gaps.size and gaps.min() <= 1e-3:
            continue   # two distinct rows score too close to order them exactly
        order = np.lexsort((np.arange(n_fill), -sc))
        want = np.sort(order[:k])
        assert np.array_equal(tg[0, t], want), f"t={t}: tie-broken top-k differs from the oracle"
        checked += 1
        ties += int(sc[order[k]] == sc[order[k - 1]])   # the k-th best shares its score with the (k+1)-th
    say(f"  {checked} queries compared exactly, {ties} with the boundary inside a tie group")
    assert checked >= 2 and ties >= 1


@pytest.mark.parametrize("dtype,T,n_fill,m", [(torch.bfloat16, 3, 5000, 2), (torch.float32, 3, 5000, 2),
                                              (torch.bfloat16, 300, 3000, 1), (torch.bfloat16, 8192, 10000, 1)])
def test_score_dump_vs_oracle(dtype, T, n_fill, m):
    """The optional debug dump of csa2_score_topk on the chunked (T = 3), tiled
    (T = 300) and streaming (T = 8192) paths: every visible entry's index score
    against the oracle's, -inf past each query's visible range and the cache."""
    B, N_cap, H_I, k = 1, n_fill + 100, 32, 64
    say(f"case: score dump dtype={dtype} T={T} n={n_fill} m={m}")
    codes, scales = _index_cache(B, N_cap, n_fill, 37)
    q_idx = synth.gaussian((B, T, H_I, 128), 1.0, 37, "q_idx", 0, dtype, DEV)
    w = synth.gaussian((B, T, H_I), 1.0, 37, "w", 0, torch.float32, DEV)
    gen = np.random.default_rng(37)
    pos = gen.integers(-2, n_fill * m + 50, size=(B, T)).astype(np.int32)
    pos[0, 0] = n_fill * m - 1
    topk = torch.empty(B, T, k, dtype=torch.int32, device=DEV)
    scores = torch.full((B, T, n_fill), 7.0, dtype=torch.float32, device=DEV)
    K.csa2_score_topk(None, q_idx, w, torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV),
                      torch.from_numpy(pos).to(DEV), topk, n_entries=n_fill, m=m, k=k, scores=scores)
    torch.cuda.synchronize()
    sg = scores.cpu().numpy()
    kd = O.fp4_unpack(codes[0], scales[0])
    for t in sorted(set([0, 1, T - 1] + list(range(0, T, max(1, T // 8))))):
        nv = O.visible_entries(int(pos[0, t]), m) if pos[0, t] >= 0 else 0
        nv = min(nv, n_fill)
        ref = O.index_scores(npy(q_idx[0, t]), npy(w[0, t]), kd, nv)
        got = sg[0, t]
        assert np.all(np.isneginf(got[nv:])), f"t={t}: positions past {nv} not -inf"
        if nv:
            tol = 1e-4 * max(1.0, float(np.abs(ref).max()))
            err = float(np.abs(got[:nv] - ref).max())
            assert err <= tol, f"t={t}: {err:.3e} > {tol:.3e}"
    # the selection is unchanged by the dump
    topk2 = torch.empty_like(topk)
    K.csa2_score_topk(None, q_idx, w, torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV),
                      torch.from_numpy(pos).to(DEV), topk2, n_entries=n_fill, m=m, k=k)
    torch.cuda.synchronize()
    assert torch.equal(topk, topk2)


def test_score_topk_hsi_build_and_use():
    B, N_cap, m, k, s, nb = 2, 4096, 1, 64, 16, 20
    pos = np.array([[4095, 100, 10, 2000], [3000, 319, 4095, 17]])
    T = pos.shape[1]
    say("case: score_topk HSI build/use")
    codes, scales = _index_cache(B, N_cap, N_cap, 23)
    dc, ds = torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV)
    q_pos = torch.tensor(pos, dtype=torch.int32, device=DEV)
    qf = synth.gaussian((B, T, 32, 128), 1.0, 23, "q_idx", 0, torch.bfloat16, DEV)
    wf = synth.gaussian((B, T, 32), 1.0, 23, "w", 0, torch.float32, DEV)
    topk = torch.empty((B, T, k), dtype=torch.int32, device=DEV)
    cand = torch.full((B, T, nb), -5, dtype=torch.int32, device=DEV)
    rt = K.Runtime()
    K.csa2_score_topk(rt, qf, wf, dc, ds, q_pos, topk, n_entries=N_cap, m=m, k=k, hsi=K.HSI_BUILD, hsi_s=s,
                      hsi_nb=nb, candidates=cand)
    torch.cuda.synchronize()
    tg, cg = topk.cpu().numpy(), cand.cpu().numpy()
    pools = np.zeros((B, T, nb), np.int64)
    for b in range(B):
        kd = O.fp4_unpack(codes[b], scales[b])
        for t in range(T):
            nv = O.visible_entries(pos[b, t], m)
            sc = O.index_scores(npy(qf[b, t]), npy(wf[b, t]), kd, nv)
            check_topk_row(sc, np.arange(nv), tg[b, t], k, f"full b{b} t{t}")
            # pool: band rule on block maxima with the newest block forced
            nblk = (nv + s - 1) // s
            beta = np.array([sc[i * s:min((i + 1) * s, nv)].max() for i in range(nblk)])
            beta[-1] = np.inf
            big = np.max(np.abs(beta[:-1])) * 10 + 1 if nblk > 1 else 1.0
            beta_f = np.where(np.isinf(beta), big, beta)
            check_topk_row(beta_f, np.arange(nblk), cg[b, t], nb, f"pool b{b} t{t}")
            assert (nblk - 1) in cg[b, t]
            pools[b, t] = O.hsi_pool(sc, nv, s, nb)
    # USE: a Reindex layer with its own queries, given the oracle's pool as input
    qr = synth.gaussian((B, T, 32, 128), 1.0, 24, "q_idx", 1, torch.bfloat16, DEV)
    wr = synth.gaussian((B, T, 32), 1.0, 24, "w", 1, torch.float32, DEV)
    pool_in = torch.from_numpy(pools.astype(np.int32)).to(DEV)
    topk2 = torch.empty((B, T, k), dtype=torch.int32, device=DEV)
    dump = torch.full((B, T, nb * s), 7.0, dtype=torch.float32, device=DEV)   # debug dump over pool positions
    K.csa2_score_topk(None, qr, wr, dc, ds, q_pos, topk2, n_entries=N_cap, m=m, k=k, hsi=K.HSI_USE, hsi_s=s,
                      hsi_nb=nb, candidates=pool_in, scores=dump)
    torch.cuda.synchronize()
    t2, dg = topk2.cpu().numpy(), dump.cpu().numpy()
    for b in range(B):
        kd = O.fp4_unpack(codes[b], scales[b])
        for t in range(T):
            nv = O.visible_entries(pos[b, t], m)
            sc = O.index_scores(npy(qr[b, t]), npy(wr[b, t]), kd, nv)
            ent = O.pool_entries(pools[b, t], nv, s)
            check_topk_row(sc[ent], ent, t2[b, t], k, f"reindex-in-pool b{b} t{t}")
            # dump position j: entry pool[j // s] * s + j % s, or -inf (empty slot, past n_t)
            for j in range(nb * s):
                blk = int(pools[b, t, j // s])
                e = blk * s + j % s if blk >= 0 else -1
                if 0 <= e < nv:
                    assert abs(dg[b, t, j] - sc[e]) <= 1e-4 * max(1.0, float(np.abs(sc).max())), (b, t, j)
                else:
                    assert np.isneginf(dg[b, t, j]), (b, t, j)
    # slot published by BUILD
    info = rt.slot(K.SLOT_CANDIDATES)
    assert info.filled == 1 and info.extra == s and info.cols == nb and info.ptr == cand.data_ptr()


# ------------------------------------------------------------ attention ----

@pytest.mark.parametrize("H,k,W", [(64, 512, 128), (20, 77, 5), (64, 96, 40)])
def test_sparse_attn_prefill_path_vs_oracle(H, k, W):
    """Many query tokens (the prefill kernel): selected rows with holes (-1 and
    out-of-range ids inside the list, a run of more than one 32-row chunk of holes),
    rows with nothing selected, windows clipped by swa_pos0 and by 0 (a token with
    neither rows nor window gets 0 and lse -inf); two sequences.  Every 13th token
    is checked row by row against the oracle."""
    B, T, N_cap, L_w = 2, 600, 700, 620
    say(f"case: sparse_attn prefill path bf16 H={H} k={k} W={W} T={T}")
    gen = np.random.default_rng(37)
    q = synth.gaussian((B, T, H, 512), 1.0, 37, "q", 0, torch.bfloat16, DEV)
    kv = synth.gaussian((B, N_cap, 512), 1.0, 37, "kv_cache", 0, torch.bfloat16, DEV)
    swa = synth.gaussian((B, L_w, 512), 1.0, 37, "swa_kv", 0, torch.bfloat16, DEV)
    pos0 = np.array([30, 0], np.int32)
    pos = np.stack([np.arange(T) + 25, np.arange(T)]).astype(np.int32)  # b=0: early windows clipped by pos0
    tk = np.full((B, T, k), -1, np.int32)
    for b in range(B):
        for t in range(T):
            n = int(gen.integers(0, k + 1)) if t % 7 else (0 if t % 14 == 0 else k)
            ids = np.sort(gen.choice(N_cap, size=n, replace=False)).astype(np.int32)
            tk[b, t, :n] = ids
            if n > 3 and t % 3 == 0:
                tk[b, t, n // 2] = -1                # hole inside the list
                tk[b, t, n // 3] = N_cap + 9         # out-of-range id inside the list
            if n >= 80 and t % 5 == 0:
                tk[b, t, 5:45] = -1                  # a run of holes longer than one chunk
    o = torch.empty_like(q)
    lse = torch.empty(B, T, H, dtype=torch.float32, device=DEV)
    K.csa2_sparse_attn(None, q, kv, torch.from_numpy(tk).to(DEV), swa, torch.from_numpy(pos0).to(DEV),
                       torch.from_numpy(pos).to(DEV), o, W=W, lse=lse)
    torch.cuda.synchronize()
    og, lg = npy(o), lse.cpu().numpy()
    kvn, swn, qn = npy(kv), npy(swa), npy(q)
    worst, n_checked = 0.0, 0
    for b in range(B):
        for t in list(range(0, T, 13)) + [T - 3, T - 2, T - 1]:
            sel = tk[b, t]
            sel = sel[(sel >= 0) & (sel < N_cap)]
            if len(sel) + len(O.window_positions(int(pos[b, t]), W, int(pos0[b]))) == 0:
                assert np.all(og[b, t] == 0) and np.all(np.isneginf(lg[b, t])), (b, t)
                continue
            ref, p, rows = O.sparse_attention(qn[b, t], kvn[b], sel, swn[b], int(pos0[b]), int(pos[b, t]), W)
            worst = max(worst, row_rel_err(og[b, t], ref))
            logits = (qn[b, t] @ rows.T) / math.sqrt(512)
            mx = logits.max(1)
            lse_ref = mx + np.log(np.exp(logits - mx[:, None]).sum(1))
            assert np.allclose(lg[b, t], lse_ref, rtol=1e-4, atol=1e-3), (b, t)
            n_checked += 1
    say(f"  {n_checked} tokens checked, worst row rel err {worst:.2e}")
    assert worst <= TOL[torch.bfloat16]


@pytest.mark.parametrize("H,k,W", [(64, 512, 128), (16, 96, 40)])
def test_sparse_attn_decode_single_split_vs_oracle(H, k, W):
    """Few-query bf16 attention with one row split per query (256..511 queries: each
    workgroup writes its output directly, no partials), with 4 and 1 waves per
    workgroup; rows with holes, out-of-range ids and no selected entry; every 23rd
    query checked against the oracle."""
    B, T, N_cap, L_w = 3, 100, 1200, 400
    say(f"case: sparse_attn decode single split H={H} k={k} W={W}")
    gen = np.random.default_rng(37)
    q = synth.gaussian((B, T, H, 512), 1.0, 37, "q", 0, torch.bfloat16, DEV)
    kv = synth.gaussian((B, N_cap, 512), 1.0, 37, "kv_cache", 0, torch.bfloat16, DEV)
    swa = synth.gaussian((B, L_w, 512), 1.0, 37, "swa_kv", 0, torch.bfloat16, DEV)
    pos0 = np.array([0, 50, 399], np.int32)
    # positions up to the last row the window buffer holds (some before pos0: empty window)
    pos = np.stack([gen.integers(0, int(pos0[b]) + L_w, size=T) for b in range(B)]).astype(np.int32)
    tk = np.full((B, T, k), -1, np.int32)
    for b in range(B):
        for t in range(T):
            n = int(gen.integers(0, k + 1)) if t % 7 else 0
            tk[b, t, :n] = np.sort(gen.choice(N_cap, size=n, replace=False))
            if n > 3 and t % 3 == 0:
                tk[b, t, 1] = -1            # a hole
                tk[b, t, n - 1] = N_cap + 9  # out of range: skipped
    o = torch.empty_like(q)
    lse = torch.empty(B, T, H, dtype=torch.float32, device=DEV)
    K.csa2_sparse_attn(None, q, kv, torch.from_numpy(tk).to(DEV), swa, torch.from_numpy(pos0).to(DEV),
                       torch.from_numpy(pos).to(DEV), o, W=W, lse=lse)
    torch.cuda.synchronize()
    og, lg = npy(o), lse.cpu().numpy()
    kvn, swn, qn = npy(kv), npy(swa), npy(q)
    worst = 0.0
    for b in range(B):
        for t in list(range(0, T, 23)) + [T - 1]:
            sel = tk[b, t]
            sel = sel[(sel >= 0) & (sel < N_cap)]
            p_t = int(pos[b, t])
            n_win = max(0, min(p_t, int(pos0[b]) + L_w - 1) - max(0, p_t - W + 1, int(pos0[b])) + 1)
            if sel.size + n_win == 0:   # nothing to attend to: zero output, log-sum-exp -inf
                assert np.all(og[b, t] == 0) and np.all(np.isneginf(lg[b, t])), f"b{b} t{t}: empty row"
                continue
            ref, p, rows = O.sparse_attention(qn[b, t], kvn[b], sel, swn[b], int(pos0[b]), p_t, W)
            worst = max(worst, row_rel_err(og[b, t], ref))
            logits = (qn[b, t] @ rows.T) / math.sqrt(512)
            mx = logits.max(1)
            lse_ref = mx + np.log(np.exp(logits - mx[:, None]).sum(1))
            assert np.allclose(lg[b, t], lse_ref, rtol=1e-4, atol=1e-3)
    say(f"  worst row rel err {worst:.2e}")
    assert worst <= TOL[torch.bfloat16]


@pytest.mark.parametrize("dtype,H,k,W", [(torch.float32, 8, 32, 16), (torch.bfloat16, 64, 512, 128),
                                         (torch.bfloat16, 20, 77, 5)])
def test_sparse_attn_vs_oracle(dtype, H, k, W):
    B, T, N_cap, L_w = 2, 4, 900, 300
    say(f"case: sparse_attn dtype={dtype} H={H} k={k} W={W}")
    gen = np.random.default_rng(31)
    q = synth.gaussian((B, T, H, 512), 1.0, 31, "q", 0, dtype, DEV)
    kv = synth.gaussian((B, N_cap, 512), 1.0, 31, "kv_cache", 0, dtype, DEV)
    swa = synth.gaussian((B, L_w, 512), 1.0, 31, "swa_kv", 0, dtype, DEV)
    pos0 = np.array([40, 0], np.int32)
    pos = np.array([[40, 45, 339, 200], [0, 3, 299, 150]], np.int32)  # window clipped by pos0, by 0, by the buffer
    tk = np.full((B, T, k), -1, np.int32)
    for b in range(B):
        for t in range(T):
            n = [k, k // 2, 0, min(k, 7)][t]
            ids = np.sort(gen.choice(N_cap, size=n, replace=False)).astype(np.int32)
            tk[b, t, :n] = ids
    tk[0, 0, -1] = N_cap + 5 if k > 1 else tk[0, 0, -1]   # out-of-range id is skipped
    o = torch.empty_like(q)
    lse = torch.empty(B, T, H, dtype=torch.float32, device=DEV)
    K.csa2_sparse_attn(None, q, kv, torch.from_numpy(tk).to(DEV), swa, torch.from_numpy(pos0).to(DEV),
                       torch.from_numpy(pos).to(DEV), o, W=W, lse=lse)
    torch.cuda.synchronize()
    og, lg = npy(o), lse.cpu().numpy()
    kvn, swn, qn = npy(kv), npy(swa), npy(q)
    worst = 0.0
    for b in range(B):
        for t in range(T):
            sel = tk[b, t]
            sel = sel[(sel >= 0) & (sel < N_cap)]
            ref, p, rows = O.sparse_attention(qn[b, t], kvn[b], sel, swn[b], int(pos0[b]), int(pos[b, t]), W)
            worst = max(worst, row_rel_err(og[b, t], ref))
            logits = (qn[b, t] @ rows.T) / math.sqrt(512)
            mx = logits.max(1)
            lse_ref = mx + np.log(np.exp(logits - mx[:, None]).sum(1))
            assert np.allclose(lg[b, t], lse_ref, rtol=1e-4, atol=1e-3)
    say(f"  worst row rel err {worst:.2e}")
    assert worst <= TOL[dtype]


@pytest.mark.parametrize("H,T", [(64, 4), (64, 150), (16, 4), (64, 300)])
def test_sparse_attn_window_only_decode(H, T):
    """k = 0 (window rows only) on the few-query bf16 path: with row splits (T = 4)
    and with one split per query (B * T = 300); 4 and 1 waves per workgroup; and
    on the many-query path (B * T = 600).  Every wave must still load its query
    fragments although no top-k id is read."""
    B, W, L_w = 2, 128, 400
    say(f"case: sparse_attn window only k=0 H={H} T={T}")
    q = synth.gaussian((B, T, H, 512), 1.0, 41, "q", 0, torch.bfloat16, DEV)
    kv = synth.gaussian((B, 8, 512), 1.0, 41, "kv_cache", 0, torch.bfloat16, DEV)
    swa = synth.gaussian((B, L_w, 512), 1.0, 41, "swa_kv", 0, torch.bfloat16, DEV)
    pos0 = np.array([0, 100], np.int32)
    gen = np.random.default_rng(41)
    pos = np.stack([gen.integers(int(pos0[b]), int(pos0[b]) + L_w, size=T) for b in range(B)]).astype(np.int32)
    tk = torch.full((B, T, 1), 3, dtype=torch.int32, device=DEV)   # never read with k = 0
    o = torch.empty_like(q)
    lse = torch.empty(B, T, H, dtype=torch.float32, device=DEV)
    K.csa2_sparse_attn(None, q, kv, tk, swa, torch.from_numpy(pos0).to(DEV), torch.from_numpy(pos).to(DEV), o,
                       W=W, k=0, lse=lse)
    torch.cuda.synchronize()
    og, lg = npy(o), lse.cpu().numpy()
    swn, qn = npy(swa), npy(q)
    worst = 0.0
    for b in range(B):
        for t in sorted(set([0, 1, 2, T - 1] + list(range(0, T, 37)))):
            ref, _, rows = O.sparse_attention(qn[b, t], np.zeros((0, 512)), np.zeros(0, np.int64), swn[b],
                                              int(pos0[b]), int(pos[b, t]), W)
            worst = max(worst, row_rel_err(og[b, t], ref))
            assert np.allclose(lg[b, t], O.attention_lse(qn[b, t], rows), rtol=1e-4, atol=1e-3), (b, t)
    say(f"  worst row rel err {worst:.2e}")
    assert worst <= TOL[torch.bfloat16]
