"""GPU parity of index K with UE8M0 block scales (a power of two per 32-dim block,
csa2_scale_fmt = CSA2_SCALE_UE8M0) against the oracle: the index-K writer, and
every scorer path (chunked, query-tiled, streaming, HSI pool build and use) on a
cache whose blocks span a wide range of magnitudes inside one entry, so that the
per-entry exponent normalisation of the fp16 scoring operand is exercised."""
import numpy as np
import pytest
import torch

from oracle import csa2_oracle as O
from parity_utils import check_fp4, check_topk_row, say
import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from compressed_sparse_attention_compress_amd import csa2 as K

DEV = "cuda"
UE = O.SCALE_UE8M0


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def npy(t):
    return t.detach().float().cpu().numpy().astype(np.float64) if t.is_floating_point() else t.cpu().numpy()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_index_k_ue8m0_vs_oracle(dtype):
    B, N, m, entry0, N_cap = 2, 333, 2, 5, 400
    say(f"case: index_k UE8M0 dtype={dtype} B={B} N={N}")
    lat = synth.gaussian((B, N, 512), 1.0, 3, "u", 0, torch.float32, DEV)
    w_ik = synth.linear_weight(128, 512, 3, "w_ik", 0, dtype, DEV)
    codes = torch.zeros(B, N_cap, 64, dtype=torch.uint8, device=DEV)
    scales = torch.zeros(B, N_cap, 4, dtype=torch.uint8, device=DEV)
    K.csa2_index_k(None, lat, w_ik, codes, scales, m=m, entry0=entry0, scale_fmt=K.SCALE_UE8M0)
    torch.cuda.synchronize()
    cg, sg = codes.cpu().numpy(), scales.cpu().numpy()
    for b in range(B):
        u, _, _ = O.index_k(npy(lat[b]), npy(w_ik), (entry0 + np.arange(N)) * m)
        nc, ns = check_fp4(u, cg[b, entry0:entry0 + N], sg[b, entry0:entry0 + N], f"b{b}", scale_fmt=UE)
        say(f"  b={b}: code mismatches in band {nc}, scale mismatches in band {ns}")
        assert nc <= 4 and ns <= 1
        # every stored value is within one scale step of the unquantised one
        dq = O.fp4_unpack(cg[b, entry0:entry0 + N], sg[b, entry0:entry0 + N], scale_fmt=UE)
        X = np.repeat(O.ue8m0_decode(sg[b, entry0:entry0 + N]), 32, axis=1)
        assert np.all(np.abs(dq - u) <= X + 1e-6 * np.abs(u))
    assert codes[:, :entry0].abs().sum().item() == 0 and codes[:, entry0 + N:].sum().item() == 0


def _wide_cache(B, N_cap, n_fill, seed):
    """Index-K rows whose four 32-dim blocks are scaled by independent powers of two
    in 2^-14 .. 2^6 (so an entry's scale bytes differ by up to 20), UE8M0-packed."""
    u = synth.gaussian((B, N_cap, 128), 1.0, seed, "u", 0, torch.float32, "cpu").numpy().astype(np.float64)
    e = np.random.default_rng(seed).integers(-14, 7, size=(B, N_cap, 4))
    u = (u.reshape(B, N_cap, 4, 32) * np.ldexp(1.0, e)[..., None]).reshape(B, N_cap, 128).astype(np.float32)
    codes = np.zeros((B, N_cap, 64), np.uint8)
    scales = np.zeros((B, N_cap, 4), np.uint8)
    for b in range(B):
        codes[b, :n_fill], scales[b, :n_fill] = O.fp4_pack(u[b, :n_fill], 32, UE)
    return codes, scales


@pytest.mark.parametrize("dtype,T,n_fill,m", [(torch.bfloat16, 3, 5000, 2), (torch.float32, 3, 5000, 2),
                                              (torch.bfloat16, 300, 3000, 1), (torch.bfloat16, 8192, 10000, 1),
                                              (torch.float32, 8192, 10000, 1)])
def test_score_topk_ue8m0_vs_oracle(dtype, T, n_fill, m):
    """Chunked (T = 3), query-tiled (bf16, T = 300) and streaming (T = 8192)
    scorers over a UE8M0 cache: every dumped index score of the sampled queries
    against the oracle's, and their top-k sets by the band rule."""
    B, N_cap, H_I, k = 1, n_fill + 100, 32, 64
    say(f"case: score_topk UE8M0 dtype={dtype} T={T} n={n_fill} m={m}")
    codes, scales = _wide_cache(B, N_cap, n_fill, 41)
    q_idx = synth.gaussian((B, T, H_I, 128), 1.0, 41, "q_idx", 0, dtype, DEV)
    w = synth.gaussian((B, T, H_I), 1.0, 41, "w", 0, torch.float32, DEV)
    gen = np.random.default_rng(41)
    pos = gen.integers(-2, n_fill * m + 50, size=(B, T)).astype(np.int32)
    pos[0, 0] = n_fill * m - 1
    topk = torch.full((B, T, k), -7, dtype=torch.int32, device=DEV)
    scores = torch.full((B, T, n_fill), 7.0, dtype=torch.float32, device=DEV)
    K.csa2_score_topk(None, q_idx, w, torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV),
                      torch.from_numpy(pos).to(DEV), topk, n_entries=n_fill, m=m, k=k, scores=scores,
                      scale_fmt=K.SCALE_UE8M0)
    torch.cuda.synchronize()
    sg, tg = scores.cpu().numpy(), topk.cpu().numpy()
    kd = O.fp4_unpack(codes[0], scales[0], scale_fmt=UE)
    exact = n = 0
    for t in sorted(set([0, 1, T - 1] + list(range(0, T, max(1, T // 8))))):
        nv = min(O.visible_entries(int(pos[0, t]), m) if pos[0, t] >= 0 else 0, n_fill)
        ref = O.index_scores(npy(q_idx[0, t]), npy(w[0, t]), kd, nv)
        got = sg[0, t]
        assert np.all(np.isneginf(got[nv:])), f"t={t}: positions past {nv} not -inf"
        if nv:
            tol = 1e-4 * max(1.0, float(np.abs(ref).max()))
            err = float(np.abs(got[:nv] - ref).max())
            assert err <= tol, f"t={t}: {err:.3e} > {tol:.3e}"
        exact += check_topk_row(ref, np.arange(nv), tg[0, t], k, f"t={t} n_t={nv}")
        n += 1
    say(f"  exact set equality on {exact}/{n} queries")
    assert exact >= n - 1


def test_score_topk_ue8m0_hsi_build_and_use():
    """HSI pool build (Full scan) and a Reindex scan inside the pool over a UE8M0
    cache: top-k band rule for both, the pool against the block maxima, the
    pool scan's dumped scores against the oracle's."""
    B, N_cap, m, k, s, nb = 2, 4096, 1, 64, 16, 20
    pos = np.array([[4095, 100, 10, 2000], [3000, 319, 4095, 17]])
    T = pos.shape[1]
    say("case: score_topk UE8M0 HSI build/use")
    codes, scales = _wide_cache(B, N_cap, N_cap, 43)
    dc, ds = torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV)
    q_pos = torch.tensor(pos, dtype=torch.int32, device=DEV)
    qf = synth.gaussian((B, T, 32, 128), 1.0, 43, "q_idx", 0, torch.bfloat16, DEV)
    wf = synth.gaussian((B, T, 32), 1.0, 43, "w", 0, torch.float32, DEV)
    topk = torch.empty((B, T, k), dtype=torch.int32, device=DEV)
    cand = torch.full((B, T, nb), -5, dtype=torch.int32, device=DEV)
    K.csa2_score_topk(None, qf, wf, dc, ds, q_pos, topk, n_entries=N_cap, m=m, k=k, hsi=K.HSI_BUILD, hsi_s=s,
                      hsi_nb=nb, candidates=cand, scale_fmt=K.SCALE_UE8M0)
    torch.cuda.synchronize()
    tg, cg = topk.cpu().numpy(), cand.cpu().numpy()
    pools = np.zeros((B, T, nb), np.int64)
    kds = [O.fp4_unpack(codes[b], scales[b], scale_fmt=UE) for b in range(B)]
    for b in range(B):
        for t in range(T):
            nv = O.visible_entries(pos[b, t], m)
            sc = O.index_scores(npy(qf[b, t]), npy(wf[b, t]), kds[b], nv)
            check_topk_row(sc, np.arange(nv), tg[b, t], k, f"full b{b} t{t}")
            nblk = (nv + s - 1) // s
            beta = np.array([sc[i * s:min((i + 1) * s, nv)].max() for i in range(nblk)])
            beta[-1] = np.inf
            big = np.max(np.abs(beta[:-1])) * 10 + 1 if nblk > 1 else 1.0
            check_topk_row(np.where(np.isinf(beta), big, beta), np.arange(nblk), cg[b, t], nb, f"pool b{b} t{t}")
            assert (nblk - 1) in cg[b, t]
            pools[b, t] = O.hsi_pool(sc, nv, s, nb)
    qr = synth.gaussian((B, T, 32, 128), 1.0, 44, "q_idx", 1, torch.bfloat16, DEV)
    wr = synth.gaussian((B, T, 32), 1.0, 44, "w", 1, torch.float32, DEV)
    topk2 = torch.empty((B, T, k), dtype=torch.int32, device=DEV)
    dump = torch.full((B, T, nb * s), 7.0, dtype=torch.float32, device=DEV)
    K.csa2_score_topk(None, qr, wr, dc, ds, q_pos, topk2, n_entries=N_cap, m=m, k=k, hsi=K.HSI_USE, hsi_s=s,
                      hsi_nb=nb, candidates=torch.from_numpy(pools.astype(np.int32)).to(DEV), scores=dump,
                      scale_fmt=K.SCALE_UE8M0)
    torch.cuda.synchronize()
    t2, dg = topk2.cpu().numpy(), dump.cpu().numpy()
    for b in range(B):
        for t in range(T):
            nv = O.visible_entries(pos[b, t], m)
            sc = O.index_scores(npy(qr[b, t]), npy(wr[b, t]), kds[b], nv)
            ent = O.pool_entries(pools[b, t], nv, s)
            check_topk_row(sc[ent], ent, t2[b, t], k, f"reindex-in-pool b{b} t{t}")
            tol = 1e-4 * max(1.0, float(np.abs(sc).max()))
            for j in range(nb * s):
                blk = int(pools[b, t, j // s])
                e = blk * s + j % s if blk >= 0 else -1
                if 0 <= e < nv:
                    assert abs(dg[b, t, j] - sc[e]) <= tol, (b, t, j)
                else:
                    assert np.isneginf(dg[b, t, j]), (b, t, j)


def test_ue8m0_and_e4m3_scorers_differ_only_by_the_scales():
    """The same FP4 codes read with E4M3 and with UE8M0 scale bytes chosen to
    decode to the same powers of two (E4M3 0x38 + 8j = 2^j, UE8M0 127 + j) give
    identical selections and dumped scores on the tiled and chunked paths."""
    B, n, k = 1, 3000, 64
    say("case: E4M3 vs UE8M0 scales of equal value")
    gen = np.random.default_rng(45)
    codes = gen.integers(0, 256, size=(B, n, 64), dtype=np.uint8)
    j = gen.integers(-6, 9, size=(B, n, 4))
    s_e4 = (0x38 + 8 * j).astype(np.uint8)
    s_ue = (127 + j).astype(np.uint8)
    assert np.array_equal(O.e4m3_decode(s_e4), O.ue8m0_decode(s_ue))
    dc = torch.from_numpy(codes).to(DEV)
    for T in (3, 300):
        q = synth.gaussian((B, T, 32, 128), 1.0, 45, "q_idx", T, torch.bfloat16, DEV)
        w = synth.gaussian((B, T, 32), 1.0, 45, "w", T, torch.float32, DEV)
        q_pos = torch.full((B, T), n - 1, dtype=torch.int32, device=DEV)
        out = []
        for sc, fmt in ((s_e4, K.SCALE_E4M3), (s_ue, K.SCALE_UE8M0)):
            topk = torch.empty((B, T, k), dtype=torch.int32, device=DEV)
            dump = torch.empty((B, T, n), dtype=torch.float32, device=DEV)
            K.csa2_score_topk(None, q, w, dc, torch.from_numpy(sc).to(DEV), q_pos, topk, n_entries=n, m=1, k=k,
                              scores=dump, scale_fmt=fmt)
            torch.cuda.synchronize()
            out.append((topk.cpu().numpy(), dump.cpu().numpy()))
        assert np.array_equal(out[0][0], out[1][0]), f"T={T}: selections differ"
        ref = np.abs(out[0][1]).max()
        assert np.abs(out[0][1] - out[1][1]).max() <= 1e-5 * max(1.0, ref), f"T={T}: scores differ"
