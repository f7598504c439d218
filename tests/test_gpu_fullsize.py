"""Parity at the workloads' full sizes, in the launch configuration the benchmark
times: every stage runs on the whole workload on the GPU and a sample of its
outputs (entries, queries, rows) is recomputed one by one by the CPU oracle.

* encoder Full-layer prefill, B=1, L=8192, hidden 4096, m=2 (the benchmark's
  PrefillBench itself);
* decoder macro-block, m=1, L=32768: Full (from one hidden tensor), Reindex, Reuse,
  Reuse;
* batched decode, 64 sequences x 131072 m=2 entries, Reindex + Reuse (the
  benchmark's DecodeBench itself), with bf16 and with FP4 main KV, and with a
  planted top-512 set (entries scoring far above the rest) that must be selected
  exactly;
* 1M-context decode with the HSI candidate pool: 4 sequences x 524288 entries,
  Full layer (flat top-512 + 256 blocks of 64) then Reindex within the pool.

Comparison rules as in parity_utils.  Every oracle input is a seeded input (drawn
again where the workload pre-fills a cache) or the oracle's own output of an
earlier stage: the compressor and index K run over the whole sequence in the
oracle; GPU index-K bytes may differ from the oracle's only at rounding-midpoint
ties (those entries are exempt from the top-k band rule), and attention is
compared over the oracle's own selection wherever the GPU's set equals it.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import synth
from oracle import csa2_oracle as O
from parity_utils import check_fp4, check_topk_row, row_rel_err, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 2e-2


@pytest.fixture(scope="module")
def K():
    from compressed_sparse_attention_compress_amd import csa2 as lib
    lib.lib()
    return lib


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _check_attn(tag, q_tok, kv_seq, sel_row, swa_seq, pos0, p, W, o_tok):
    """swa_seq: the layer's window KV (torch, [L_w, 512], row j = position pos0 + j)."""
    sel = sel_row[sel_row >= 0]
    lo = max(0, p - W + 1, pos0)
    swa_rows = f64(swa_seq[lo - pos0:p - pos0 + 1])
    ref, probs, rows = O.sparse_attention(q_tok, kv_seq, sel, swa_rows, lo, p, W)
    err = row_rel_err(o_tok, ref)
    assert err <= TOL, f"{tag}: attention row rel err {err:.3e}"
    return err


# ---------------------------------------------------------------- prefill C2

def _flips(codes_g, scales_g, codes_o, scales_o):
    """Entries whose stored GPU index-K bytes differ from the oracle's (each such
    difference is a rounding-midpoint tie, checked by check_fp4)."""
    return np.where((codes_g != codes_o).any(1) | (scales_g != scales_o).any(1))[0]


def _selected_attention(tag, sc, nv, k, gpu_row, flips, q_tok, kv_o, swa_seq, pos0, p, W, o_tok):
    """Top-k band check of the GPU row against the oracle's scores, then the GPU
    output against the oracle's attention over the oracle's cache rows: over the
    oracle's own selection where the sets agree exactly, else over the GPU's set
    (which the band rule has just shown to be a valid top-k), so that every sampled
    query has its attention compared.  Returns (exact, err)."""
    exact = check_topk_row(sc, np.arange(nv), gpu_row, k, tag, flips)
    sel = O.topk_select(sc, k) if exact else np.asarray(gpu_row)
    return exact, _check_attn(tag, q_tok, kv_o, sel, swa_seq, pos0, p, W, o_tok)


def test_encoder_prefill_full_size(K):
    import bench
    say("case: encoder Full-layer prefill B=1 L=8192 D=4096 m=2 (benchmark launch configuration)")
    pb = bench.PrefillBench(torch, K, synth)
    pb.step()
    torch.cuda.synchronize()
    s, i = pb.shape, pb.inp
    N = pb.N
    w_kv, w_gate, gamma, w_ik = f64(i["w_kv"]), f64(i["w_gate"]), f64(i["gamma"]), f64(i["w_ik"])
    # the oracle's own compressor and index K over the whole sequence (same seeded inputs)
    lat_o, kv_o, ids = O.compress(f64(i["x"][0]), w_kv, w_gate, gamma, s.m, 0)
    u_o, codes_o, scales_o = O.index_k(lat_o, w_ik, ids * s.m)
    assert row_rel_err(f64(pb.kv[0]), kv_o) <= TOL, "cache rows"
    assert row_rel_err(pb.lat[0].cpu().numpy(), lat_o) <= TOL, "pre-RoPE latents"
    codes, scales = pb.codes[0].cpu().numpy(), pb.scales[0].cpu().numpy()
    nc, ns = check_fp4(u_o, codes, scales, "prefill index K")
    say(f"  FP4 code flips inside the rounding band: {nc} codes, {ns} scales (of {N} entries)")
    flips = _flips(codes, scales, codes_o, scales_o)
    kd = O.fp4_unpack(codes_o, scales_o)
    topk = pb.topk[0].cpu().numpy()
    qi, ww = i["q_idx"][0], i["w"][0]
    # 64 queries spread over the causal range (n_t from 0 to 4096 entries), plus the
    # edges of the k = 512 and chunk boundaries
    sample = sorted(set(np.linspace(0, s.L - 1, 56).astype(int).tolist()
                        + [1, 2, 1022, 1023, 1024, 1025, 4097, s.L - 2]))
    assert len(sample) >= 64
    worst, n_exact = 0.0, 0
    for t in sample:
        nv = O.visible_entries(t, s.m)
        sc = O.index_scores(f64(qi[t]), f64(ww[t]), kd, nv)
        ex, err = _selected_attention(f"prefill t{t}", sc, nv, s.k, topk[t], flips, f64(i["q"][0, t]), kv_o,
                                      i["swa_kv"][0], 0, t, s.W, f64(pb.o[0, t]))
        n_exact += ex
        worst = max(worst, err)
    say(f"  exact sets {n_exact}/{len(sample)}, attention compared for all {len(sample)} queries, "
        f"worst row rel err {worst:.2e}")
    assert n_exact >= len(sample) - 2


# ---------------------------------------------------------- decoder block C3

def test_decoder_macro_block_full_size(K):
    L, D, m, H_I, k, W, H = 32768, 4096, 1, 32, 512, 128, 64
    say(f"case: decoder macro-block Full/Reindex/Reuse/Reuse L={L} m={m}")
    shape = synth.LayerShape(B=1, L=L, D=D, m=m, H_I=H_I, k=k, W=W, H=H)
    bf = torch.bfloat16
    full = synth.full_layer_inputs(shape, 5, bf, DEV, layer=0)
    lay = [full] + [synth.full_layer_inputs(shape, 5, bf, DEV, layer=l, with_x=False) for l in (1, 2, 3)]
    N = L // m
    lat = torch.empty(1, N, 512, dtype=torch.float32, device=DEV)
    kvc = torch.empty(1, N, 512, dtype=bf, device=DEV)
    codes = torch.empty(1, N, 64, dtype=torch.uint8, device=DEV)
    scales = torch.empty(1, N, 4, dtype=torch.uint8, device=DEV)
    rt = K.Runtime()
    modes = [K.FULL, K.REINDEX, K.REUSE, K.REUSE]
    outs, tks = [], []
    for li, mode in enumerate(modes):
        inp = lay[li]
        cfg = K.layer_cfg(mode, K.CSA2_BF16, m=m, k=k, W=W, H_I=H_I, H=H)
        topk = torch.empty(1, L, k, dtype=torch.int32, device=DEV)
        o = torch.empty_like(inp["q"])
        kw = dict(B=1, T=L, q_pos=inp["q_pos"], q=inp["q"], swa_kv=inp["swa_kv"], swa_pos0=inp["swa_pos0"], o=o,
                  N_cap=N)
        if mode == K.FULL:
            kw.update(D=D, x=inp["x"], w_kv=inp["w_kv"], w_gate=None, gamma=inp["gamma"], w_ik=inp["w_ik"],
                      latent_pre=lat, kv_cache=kvc, ik_codes=codes, ik_scales=scales)
        if mode != K.REUSE:
            kw.update(q_idx=inp["q_idx"], w=inp["w"], topk=topk)
        io = K.layer_io(**kw)
        ws = torch.empty(max(K.layer_workspace_bytes(cfg, io), 16), dtype=torch.uint8, device=DEV)
        K.csa2_layer_forward(rt, cfg, K.layer_io(workspace=ws, **kw))
        torch.cuda.synchronize()
        outs.append(o)
        tks.append(topk if mode != K.REUSE else tks[-1])
        del ws
    w_kv, gamma, w_ik = f64(full["w_kv"]), f64(full["gamma"]), f64(full["w_ik"])
    lat_o, kv_o, ids = O.compress(f64(full["x"][0]), w_kv, None, gamma, m, 0)
    u_o, codes_o, scales_o = O.index_k(lat_o, w_ik, ids * m)
    assert row_rel_err(f64(kvc[0]), kv_o) <= TOL, "cache rows"
    cd, sd = codes[0].cpu().numpy(), scales[0].cpu().numpy()
    nc, ns = check_fp4(u_o, cd, sd, "decoder index K")
    say(f"  FP4 code flips inside the rounding band: {nc} codes, {ns} scales (of {N} entries)")
    flips = _flips(cd, sd, codes_o, scales_o)
    kd = O.fp4_unpack(codes_o, scales_o)
    t_full, t_re = tks[0][0].cpu().numpy(), tks[1][0].cpu().numpy()
    # the Reuse layers attend over the Reindex layer's selection
    worst, n_exact, n_all, n_att = 0.0, 0, 0, 0
    for t in [0, 1, 511, 512, 513, 4096, 12345, 20000, 28000, L - 1]:
        nv = O.visible_entries(t, m)
        for li, tk_row in ((0, t_full[t]), (1, t_re[t])):
            inp = lay[li]
            sc = O.index_scores(f64(inp["q_idx"][0, t]), f64(inp["w"][0, t]), kd, nv)
            layers = (0,) if li == 0 else (1, 2, 3)
            ex = check_topk_row(sc, np.arange(nv), tk_row, k, f"decoder layer{li} t{t}", flips)
            n_all += 1
            n_exact += ex
            # over the oracle's selection where the sets agree, else over the GPU's
            # (band-valid) set
            sel_o = O.topk_select(sc, k) if ex else tk_row
            for lj in layers:
                n_att += 1
                worst = max(worst, _check_attn(f"decoder layer{lj} t{t}", f64(lay[lj]["q"][0, t]), kv_o, sel_o,
                                               lay[lj]["swa_kv"][0], 0, t, W, f64(outs[lj][0, t])))
    say(f"  exact sets {n_exact}/{n_all}, {n_att} attention outputs compared, worst row rel err {worst:.2e}")
    assert n_exact >= n_all - 2 and n_att == 40


def test_decoder_bounded_replay_full_size(K):
    """L = 32768 prompt tokens, the last R = 2048 replayed through Full, Reindex,
    Reuse, Reuse (the benchmark's DecoderBench itself); sampled replayed queries
    against the oracle over the oracle's own global KV and index K."""
    import bench
    say("case: decoder bounded replay L=32768 R=2048 (benchmark launch configuration)")
    db = bench.DecoderBench(torch, K, synth, R=2048)
    db.step()
    torch.cuda.synchronize()
    L, R, k, W = db.L, db.R, db.k, db.W
    lat_o, kv_o, ids = O.compress(f64(db.x[0]), f64(db.w_kv), None, f64(db.gamma), 1, 0)
    u_o, codes_o, scales_o = O.index_k(lat_o, f64(db.w_ik), ids)
    assert row_rel_err(f64(db.kv[0]), kv_o) <= TOL, "global KV rows"
    cd, sd = db.codes[0].cpu().numpy(), db.scales[0].cpu().numpy()
    check_fp4(u_o, cd, sd, "replay index K")
    flips = _flips(cd, sd, codes_o, scales_o)
    kd = O.fp4_unpack(codes_o, scales_o)
    tks = [db.layers[l]["topk"][0].cpu().numpy() for l in (0, 1)]
    worst, n_exact, n_att = 0.0, 0, 0
    for j in [0, 1, 63, 126, 127, 128, 1000, R - 1]:
        p = L - R + j
        for li in (0, 1):
            lay = db.layers[li]
            sc = O.index_scores(f64(lay["q_idx"][0, j]), f64(lay["w"][0, j]), kd, p + 1)
            ex = check_topk_row(sc, np.arange(p + 1), tks[li][j], k, f"replay layer{li} j{j}", flips)
            n_exact += ex
            sel = O.topk_select(sc, k) if ex else tks[li][j]
            for lj in ((0,) if li == 0 else (1, 2, 3)):
                ly = db.layers[lj]
                ref, _, _ = O.sparse_attention(f64(ly["q"][0, j]), kv_o, sel, f64(ly["swa_kv"][0]), L - R, p, W)
                err = row_rel_err(f64(ly["o"][0, j]), ref)
                assert err <= TOL, f"replay layer{lj} j{j}: {err:.3e}"
                worst = max(worst, err)
                n_att += 1
    say(f"  exact sets {n_exact}/16, {n_att} attention outputs compared, worst row rel err {worst:.2e}")
    assert n_exact >= 14 and n_att == 32


# -------------------------------------------------------------- decode C4

def test_batched_decode_full_size(K):
    import bench
    say("case: batched decode 64 x 131072 entries, Reindex + Reuse (benchmark launch configuration)")
    db = bench.DecodeBench(torch, K, synth)
    db.step()
    torch.cuda.synchronize()
    topk = db.topk.cpu().numpy()
    p = int(db.q_pos[0, 0].item())
    pos0 = int(db.swa_pos0[0].item())
    worst, n_exact, sample = 0.0, 0, [0, 31, 63]
    for b in sample:
        # the sequence's seeded cache inputs, drawn again; the oracle packs the index K
        u = synth.cache_rows(db.N, 128, db.seed, "u", b, DEV).cpu().numpy()
        codes_o, scales_o = O.fp4_pack(u)
        cg, sg = db.codes[b].cpu().numpy(), db.scales[b].cpu().numpy()
        assert np.array_equal(cg, codes_o) and np.array_equal(sg, scales_o), f"b{b}: index-K bytes"
        kd = O.fp4_unpack(codes_o, scales_o)
        r = db.layers[0]
        sc = O.index_scores(f64(r["q_idx"][b, 0]), f64(r["w"][b, 0]), kd, db.N)
        del kd, u
        ex = check_topk_row(sc, np.arange(db.N), topk[b, 0], db.k, f"decode b{b}")
        n_exact += ex
        sel = O.topk_select(sc, db.k) if ex else topk[b, 0]   # the GPU's set is band-valid
        kv_b = synth.cache_rows(db.N, 512, db.seed, "kv_cache", b, DEV).to(torch.bfloat16)
        rows = f64(kv_b[torch.from_numpy(sel[sel >= 0].astype(np.int64)).to(DEV)])
        del kv_b
        for li in range(2):
            lay = db.layers[li]
            ref, _, _ = O.sparse_attention(f64(lay["q"][b, 0]), rows, np.arange(rows.shape[0]), f64(lay["swa_kv"][b]),
                                           pos0, p, db.W)
            err = row_rel_err(f64(db.o[li][b, 0]), ref)
            assert err <= TOL, f"decode b{b} layer{li}: {err:.3e}"
            worst = max(worst, err)
    say(f"  exact sets {n_exact}/{len(sample)}, attention compared for all, worst row rel err {worst:.2e}")
    assert n_exact >= len(sample) - 1


def test_batched_decode_planted_full_size(K):
    """The batched decode workload (64 x 131072 entries) with 512 entries of 8 of
    the sequences planted: their pre-quantisation index-K rows point along the
    layer's positively weighted indexer heads, so they outscore every other entry
    by far more than the band rule's 1e-3 (checked on the oracle's scores).  The
    GPU's top-512 of those sequences must then be exactly the planted set, and
    their attention outputs match the oracle's over it."""
    import bench
    say("case: batched decode 64 x 131072 entries with planted top-512 sets")
    db = bench.DecodeBench(torch, K, synth)
    gen = np.random.default_rng(97)
    seqs = [0, 9, 18, 27, 36, 45, 54, 63]
    r = db.layers[0]
    planted = {}
    for b in seqs:
        ids = np.sort(gen.choice(db.N, db.k, replace=False))
        qi, wv = f64(r["q_idx"][b, 0]), f64(r["w"][b, 0])
        v = (np.maximum(wv, 0.0)[:, None] * qi).sum(0)
        v /= np.linalg.norm(v)
        rows = (v[None, :] * (8.0 + 4.0 * gen.random((db.k, 1)))
                + 0.05 * gen.standard_normal((db.k, 128))).astype(np.float32)
        c_o, s_o = O.fp4_pack(rows)
        c_g = torch.empty(db.k, 64, dtype=torch.uint8, device=DEV)
        s_g = torch.empty(db.k, 4, dtype=torch.uint8, device=DEV)
        K.csa2_fp4_pack(torch.from_numpy(rows).to(DEV), c_g, s_g)
        torch.cuda.synchronize()
        assert np.array_equal(c_g.cpu().numpy(), c_o) and np.array_equal(s_g.cpu().numpy(), s_o), "planted FP4 rows"
        idx = torch.from_numpy(ids).to(DEV)
        db.codes[b][idx] = c_g
        db.scales[b][idx] = s_g
        planted[b] = (ids, c_o, s_o)
    db.step()
    torch.cuda.synchronize()
    topk = db.topk.cpu().numpy()
    p = int(db.q_pos[0, 0].item())
    pos0 = int(db.swa_pos0[0].item())
    worst = 0.0
    for b in seqs:
        ids, c_o, s_o = planted[b]
        u = synth.cache_rows(db.N, 128, db.seed, "u", b, DEV).cpu().numpy()
        codes_o, scales_o = O.fp4_pack(u)
        codes_o[ids], scales_o[ids] = c_o, s_o
        kd = O.fp4_unpack(codes_o, scales_o)
        sc = O.index_scores(f64(r["q_idx"][b, 0]), f64(r["w"][b, 0]), kd, db.N)
        del kd, u
        others = np.delete(sc, ids)
        margin = sc[ids].min() / max(others.max(), 1e-30) - 1.0
        assert sc[ids].min() > 0 and margin > 1e-2, f"b{b}: planting left a margin of {margin:.2e} only"
        assert np.array_equal(topk[b, 0], ids), f"b{b}: the top-k is not the planted set"
        kv_b = synth.cache_rows(db.N, 512, db.seed, "kv_cache", b, DEV).to(torch.bfloat16)
        rows = f64(kv_b[torch.from_numpy(ids.astype(np.int64)).to(DEV)])
        del kv_b
        for li in range(2):
            lay = db.layers[li]
            ref, _, _ = O.sparse_attention(f64(lay["q"][b, 0]), rows, np.arange(rows.shape[0]), f64(lay["swa_kv"][b]),
                                           pos0, p, db.W)
            err = row_rel_err(f64(db.o[li][b, 0]), ref)
            assert err <= TOL, f"planted decode b{b} layer{li}: {err:.3e}"
            worst = max(worst, err)
        say(f"  b{b}: planted set selected exactly (score margin {margin:.2f})")
    say(f"  {len(seqs)} sequences, worst attention row rel err {worst:.2e}")


def test_batched_decode_fp4_kv_full_size(K):
    import bench
    say("case: batched decode 64 x 131072 entries with FP4 main KV (benchmark launch configuration)")
    db = bench.DecodeBench(torch, K, synth, kv_fp4=True)
    db.step()
    torch.cuda.synchronize()
    topk = db.topk.cpu().numpy()
    p = int(db.q_pos[0, 0].item())
    pos0 = int(db.swa_pos0[0].item())
    worst, n_att = 0.0, 0
    for b in [0, 40, 63]:
        # the oracle's own selection (index K drawn again and packed by the oracle);
        # its rows are drawn again from their seed and quantised by the oracle
        kd = O.fp4_unpack(*O.fp4_pack(synth.cache_rows(db.N, 128, db.seed, "u", b, DEV).cpu().numpy()))
        r = db.layers[0]
        sc = O.index_scores(f64(r["q_idx"][b, 0]), f64(r["w"][b, 0]), kd, db.N)
        del kd
        ex = check_topk_row(sc, np.arange(db.N), topk[b, 0], db.k, f"decode FP4 KV b{b}")
        sel = O.topk_select(sc, db.k) if ex else topk[b, 0]   # the GPU's set is band-valid
        sel = sel[sel >= 0]
        ids = torch.from_numpy(sel.astype(np.int64)).to(DEV)
        r_b = synth.cache_rows(db.N, 512, db.seed, "kv_cache", b, DEV)[ids].cpu().numpy()
        c_o, s_o = O.kv_fp4_pack(r_b)
        assert np.array_equal(db.kv[b][ids].cpu().numpy(), c_o), f"b{b}: FP4 main-KV codes"
        assert np.array_equal(db.kv_scales[b][ids].cpu().numpy(), s_o), f"b{b}: FP4 main-KV scales"
        rows = O.kv_fp4_unpack(c_o, s_o)
        for li in range(2):
            lay = db.layers[li]
            ref, _, _ = O.sparse_attention(f64(lay["q"][b, 0]), rows, np.arange(rows.shape[0]), f64(lay["swa_kv"][b]),
                                           pos0, p, db.W)
            err = row_rel_err(f64(db.o[li][b, 0]), ref)
            assert err <= TOL, f"decode FP4 KV b{b} layer{li}: {err:.3e}"
            worst = max(worst, err)
            n_att += 1
    say(f"  worst attention row rel err {worst:.2e} over {n_att} outputs")
    assert n_att == 6


# ----------------------------------------------------- 1M decode with HSI C5

def test_million_context_hsi_decode_full_size(K):
    B, N, m, H_I, k, W, H, s_blk, nb = 4, 524288, 2, 32, 512, 128, 64, 64, 256
    say(f"case: 1M-context decode with HSI, {B} x {N} entries, s={s_blk}, n_b={nb}")
    bf = torch.bfloat16
    seed = 77
    kv = torch.empty(B, N, 512, dtype=bf, device=DEV)
    codes = torch.empty(B, N, 64, dtype=torch.uint8, device=DEV)
    scales = torch.empty(B, N, 4, dtype=torch.uint8, device=DEV)
    for b in range(B):
        kv[b] = synth.cache_rows(N, 512, seed, "kv_cache", b, DEV).to(bf)
        u = synth.cache_rows(N, 128, seed, "u", b, DEV)
        K.csa2_fp4_pack(u, codes[b], scales[b])
        del u
    p = N * m - 1
    q_pos = torch.full((B, 1), p, dtype=torch.int32, device=DEV)
    pos0 = torch.full((B,), p - W + 1, dtype=torch.int32, device=DEV)
    lay = [synth.decode_query_inputs(B, H, H_I, W, seed=3, layer=l, dtype=bf, device=DEV) for l in range(2)]
    tk_full = torch.empty(B, 1, k, dtype=torch.int32, device=DEV)
    cand = torch.empty(B, 1, nb, dtype=torch.int32, device=DEV)
    tk_re = torch.empty(B, 1, k, dtype=torch.int32, device=DEV)
    K.csa2_score_topk(None, lay[0]["q_idx"], lay[0]["w"], codes, scales, q_pos, tk_full, n_entries=N, m=m, k=k,
                      hsi=K.HSI_BUILD, hsi_s=s_blk, hsi_nb=nb, candidates=cand)
    K.csa2_score_topk(None, lay[1]["q_idx"], lay[1]["w"], codes, scales, q_pos, tk_re, n_entries=N, m=m, k=k,
                      hsi=K.HSI_USE, hsi_s=s_blk, hsi_nb=nb, candidates=cand)
    o = [torch.empty_like(lay[l]["q"]) for l in range(2)]
    K.csa2_sparse_attn(None, lay[0]["q"], kv, tk_full, lay[0]["swa_kv"], pos0, q_pos, o[0], W=W)
    K.csa2_sparse_attn(None, lay[1]["q"], kv, tk_re, lay[1]["swa_kv"], pos0, q_pos, o[1], W=W)
    torch.cuda.synchronize()
    tf, tr, cg = tk_full.cpu().numpy(), tk_re.cpu().numpy(), cand.cpu().numpy()
    worst, n_att = 0.0, 0
    for b in [0, 3]:
        # the sequence's index-K inputs drawn again and packed by the oracle
        codes_o, scales_o = O.fp4_pack(synth.cache_rows(N, 128, seed, "u", b, DEV).cpu().numpy())
        assert np.array_equal(codes[b].cpu().numpy(), codes_o) and np.array_equal(scales[b].cpu().numpy(), scales_o)
        kd = O.fp4_unpack(codes_o, scales_o)
        del codes_o, scales_o
        sc = O.index_scores(f64(lay[0]["q_idx"][b, 0]), f64(lay[0]["w"][b, 0]), kd, N)
        ex_full = check_topk_row(sc, np.arange(N), tf[b, 0], k, f"hsi full b{b}")
        nblk = N // s_blk
        beta = sc.reshape(nblk, s_blk).max(1)
        beta[-1] = np.inf
        beta_f = np.where(np.isinf(beta), np.max(np.abs(beta[:-1])) * 10 + 1, beta)
        ex_pool = check_topk_row(beta_f, np.arange(nblk), cg[b, 0], nb, f"hsi pool b{b}")
        assert (nblk - 1) in cg[b, 0]
        pool_o = O.hsi_pool(sc, N, s_blk, nb)
        sels = {0: O.topk_select(sc, k) if ex_full else None}
        if ex_pool:
            # Reindex: its own scores, restricted to the (oracle's = GPU's) pool
            assert np.array_equal(np.sort(pool_o[pool_o >= 0]), np.sort(cg[b, 0][cg[b, 0] >= 0]))
            sc2 = O.index_scores(f64(lay[1]["q_idx"][b, 0]), f64(lay[1]["w"][b, 0]), kd, N)
            ent = O.pool_entries(pool_o, N, s_blk)
            if check_topk_row(sc2[ent], ent, tr[b, 0], k, f"hsi reindex b{b}"):
                sels[1] = O.topk_select(sc2, k, ent)
        del kd
        say(f"  b{b}: exact full set {ex_full}, exact pool {ex_pool}, exact reindex set {1 in sels}")
        # floor: on these seeded inputs every sampled set is exact (deterministic
        # kernels on fixed data), so any difference is a regression
        assert ex_full and ex_pool and (1 in sels), f"hsi b{b}: a set is not exact"
        for li in (0, 1):
            sel = sels[li]
            n_att += 1
            rows = f64(kv[b][torch.from_numpy(sel[sel >= 0].astype(np.int64)).to(DEV)])
            ref, _, _ = O.sparse_attention(f64(lay[li]["q"][b, 0]), rows, np.arange(rows.shape[0]),
                                           f64(lay[li]["swa_kv"][b]), p - W + 1, p, W)
            err = row_rel_err(f64(o[li][b, 0]), ref)
            assert err <= TOL, f"hsi b{b} layer{li}: {err:.3e}"
            worst = max(worst, err)
    say(f"  worst attention row rel err {worst:.2e} over {n_att} outputs")
    assert n_att >= 4
