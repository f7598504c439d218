"""GPU parity of the decoder prefill with bounded replay: the decoder's Full layer
(m = 1) compresses the encoder output H20 of all L prompt tokens into the global
KV and index K (csa2_layer_io.T_x = L), and the Full, Reindex and Reuse layers
run through csa2_layer_forward for the last R positions only, each with the window
KV of the replayed positions (swa_pos0 = L - R); against the oracle's
decoder_replay."""
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
TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-3}


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def npy(t):
    if t is None:
        return None
    return t.detach().float().cpu().numpy().astype(np.float64) if t.is_floating_point() else t.cpu().numpy()


@pytest.mark.parametrize("dtype,L,R", [(torch.float32, 256, 48), (torch.bfloat16, 512, 96), (torch.bfloat16, 300, 300)])
def test_bounded_replay_through_layer_forward(dtype, L, R):
    B, D, H_I, k, W = 2, (256 if dtype == torch.float32 else 512), 4, 32, 16
    H = 8 if dtype == torch.float32 else 64
    say(f"case: bounded replay dtype={dtype} L={L} R={R} H={H}")
    cd = K.CSA2_BF16 if dtype == torch.bfloat16 else K.CSA2_F32
    h20 = synth.gaussian((B, L, D), 1.0, 93, "x", 0, dtype, DEV)
    w_kv = synth.linear_weight(512, D, 93, "w_kv", 0, dtype, DEV)
    w_ik = synth.linear_weight(128, 512, 93, "w_ik", 0, dtype, DEV)
    gamma = torch.ones(512, dtype=torch.float32, device=DEV)
    modes = [K.FULL, K.REINDEX, K.REUSE]
    lays = []
    for l, mode in enumerate(modes):
        lay = {"q": synth.gaussian((B, R, H, 512), 1.0, 93, "q", l, dtype, DEV),
               "swa_kv": synth.gaussian((B, R, 512), 1.0, 93, "swa_kv", l, dtype, DEV)}
        if mode != K.REUSE:
            lay["q_idx"] = synth.gaussian((B, R, H_I, 128), 1.0, 93, "q_idx", l, dtype, DEV)
            lay["w"] = synth.gaussian((B, R, H_I), 1.0, 93, "w", l, torch.float32, DEV)
        lays.append(lay)
    q_pos = torch.arange(L - R, L, dtype=torch.int32, device=DEV).repeat(B, 1).contiguous()
    pos0 = torch.full((B,), L - R, dtype=torch.int32, device=DEV)
    lat = torch.empty(B, L, 512, dtype=torch.float32, device=DEV)
    kv = torch.empty(B, L, 512, dtype=dtype, device=DEV)
    codes = torch.empty(B, L, 64, dtype=torch.uint8, device=DEV)
    scales = torch.empty(B, L, 4, dtype=torch.uint8, device=DEV)
    rt = K.Runtime()
    outs, tks = [], []
    for l, mode in enumerate(modes):
        lay = lays[l]
        cfg = K.layer_cfg(mode, cd, m=1, k=k, W=W, H_I=H_I, H=H)
        o = torch.empty_like(lay["q"])
        topk = torch.full((B, R, k), -9, dtype=torch.int32, device=DEV) if mode != K.REUSE else None
        kw = dict(B=B, T=R, q_pos=q_pos, q=lay["q"], swa_kv=lay["swa_kv"], swa_pos0=pos0, o=o, N_cap=L)
        if mode == K.FULL:
            kw.update(D=D, x=h20, w_kv=w_kv, w_gate=None, gamma=gamma, w_ik=w_ik, latent_pre=lat, kv_cache=kv,
                      ik_codes=codes, ik_scales=scales, T_x=L)
        if mode != K.REUSE:
            kw.update(q_idx=lay["q_idx"], w=lay["w"], topk=topk)
        ws = torch.empty(max(K.layer_workspace_bytes(cfg, K.layer_io(**kw)), 16), dtype=torch.uint8, device=DEV)
        K.csa2_layer_forward(rt, cfg, K.layer_io(workspace=ws, **kw))
        outs.append(o)
        tks.append(topk if topk is not None else tks[-1])
    torch.cuda.synchronize()
    assert rt.slot(K.SLOT_COMPRESS_KV).cols == L and rt.slot(K.SLOT_TOPK_IDXS).rows == R

    ocfgs = [O.LayerConfig(O.FULL, m=1, k=k, W=W, w_kv=npy(w_kv), w_gate=None, gamma=npy(gamma), w_ik=npy(w_ik)),
             O.LayerConfig(O.REINDEX, m=1, k=k, W=W), O.LayerConfig(O.REUSE, m=1, k=k, W=W)]
    oin = [O.LayerInputs(q=npy(ly["q"]), swa_kv=npy(ly["swa_kv"]), q_pos=None, swa_pos0=None,
                         q_idx=npy(ly.get("q_idx")), w=npy(ly.get("w"))) for ly in lays]
    ort = O.Runtime()
    refs = O.decoder_replay(ort, ocfgs, oin, npy(h20), R)
    # the global KV over all L tokens, and the selections of the replayed queries
    assert row_rel_err(npy(kv).reshape(-1, 512), ort.compress_kv.reshape(-1, 512)) <= TOL[dtype]
    worst, n_exact, n_sets = 0.0, 0, 0
    for b in range(B):
        lat_o, _, ids = O.compress(npy(h20[b]), npy(w_kv), None, npy(gamma), 1)
        u, _, _ = O.index_k(lat_o, npy(w_ik), ids)
        cg, sg = codes[b].cpu().numpy(), scales[b].cpu().numpy()
        check_fp4(u, cg, sg, f"b{b} index K")
        # entries whose GPU bytes differ at a rounding midpoint leave the band rule
        flips = np.where((cg != ort.index_k[0][b]).any(1) | (sg != ort.index_k[1][b]).any(1))[0]
        kd = O.fp4_unpack(ort.index_k[0][b], ort.index_k[1][b])
        for j in range(R):
            p = L - R + j
            for l in (0, 1):
                sc = O.index_scores(oin[l].q_idx[b, j], oin[l].w[b, j], kd, p + 1)
                row = tks[l][b, j].cpu().numpy()
                ex = check_topk_row(sc, np.arange(p + 1), row, k, f"b{b} l{l} p{p}", flips)
                n_exact += ex
                n_sets += 1
                # attention over the oracle's selection where the sets agree, else over
                # the GPU's (band-valid) set; the Reuse layer takes the Reindex set
                sel = O.topk_select(sc, k) if ex else row
                for lj in ((0,) if l == 0 else (1, 2)):
                    ref = O.sparse_attention(oin[lj].q[b, j], ort.compress_kv[b], sel, oin[lj].swa_kv[b], L - R,
                                             p, W)[0]
                    if ex:
                        assert np.allclose(ref, refs[lj][b, j], rtol=1e-9, atol=1e-9)
                    err = row_rel_err(npy(outs[lj][b, j]), ref)
                    worst = max(worst, err)
                    assert err <= TOL[dtype], f"b{b} layer {lj} p{p}: {err:.3e}"
    say(f"  exact sets {n_exact}/{n_sets}")
    say(f"  worst output row rel err {worst:.2e}")
