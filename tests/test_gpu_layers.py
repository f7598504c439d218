"""GPU parity of whole CSA2 layers (Full -> Reindex -> Reuse) through
csa2_layer_forward and the shared runtime slots, against the oracle's modes."""
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


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def npy(t):
    return t.detach().float().cpu().numpy().astype(np.float64) if t.is_floating_point() else t.cpu().numpy()


class GpuLayerStack:
    """Device buffers of one Full layer's caches plus per-layer call helpers."""

    def __init__(self, shape: synth.LayerShape, dtype, hsi=K.HSI_NONE if torch.cuda.is_available() else 0,
                 hsi_s=0, hsi_nb=0, kv_fp4=False, scale_fmt=0):
        s = shape
        self.scale_fmt = scale_fmt   # csa2_scale_fmt of the index K a Full layer writes
        self.s, self.dtype = s, dtype
        self.N = s.L // s.m
        self.rt = K.Runtime()
        self.lat = torch.empty(s.B, self.N, 512, dtype=torch.float32, device=DEV)
        self.kv_fp4 = kv_fp4
        if kv_fp4:   # FP4 main KV: codes in kv, E4M3 scales beside them
            self.kv = torch.zeros(s.B, self.N, 256, dtype=torch.uint8, device=DEV)
            self.kv_scales = torch.zeros(s.B, self.N, 32, dtype=torch.uint8, device=DEV)
        else:
            self.kv = torch.zeros(s.B, self.N, 512, dtype=dtype, device=DEV)
            self.kv_scales = None
        self.codes = torch.zeros(s.B, self.N, 64, dtype=torch.uint8, device=DEV)
        self.scales = torch.zeros(s.B, self.N, 4, dtype=torch.uint8, device=DEV)
        self.hsi, self.hsi_s, self.hsi_nb = hsi, hsi_s, hsi_nb
        self.cands = torch.full((s.B, s.L, max(hsi_nb, 1)), -3, dtype=torch.int32, device=DEV)

    def run(self, mode, inp, hsi=None, sink=None):
        s = self.s
        hsi = self.hsi if hsi is None else hsi
        cfg = K.layer_cfg(mode, K.CSA2_BF16 if self.dtype == torch.bfloat16 else K.CSA2_F32, m=s.m, k=s.k, W=s.W,
                          H_I=s.H_I, H=s.H, hsi=hsi, hsi_s=self.hsi_s, hsi_nb=self.hsi_nb,
                          kv_fmt=K.KV_FP4 if self.kv_fp4 else K.KV_DENSE, scale_fmt=self.scale_fmt)
        topk = torch.full((s.B, s.L, s.k), -9, dtype=torch.int32, device=DEV)
        o = torch.empty_like(inp["q"])
        kw = dict(B=s.B, T=s.L, q_pos=inp["q_pos"], q=inp["q"], swa_kv=inp["swa_kv"], swa_pos0=inp["swa_pos0"], o=o,
                  N_cap=self.N, sink=sink)
        if mode == K.FULL:
            kw.update(D=s.D, x=inp["x"], w_kv=inp["w_kv"], w_gate=inp["w_gate"], gamma=inp["gamma"],
                      w_ik=inp["w_ik"], latent_pre=self.lat, kv_cache=self.kv, ik_codes=self.codes,
                      ik_scales=self.scales, kv_scales=self.kv_scales)
        if mode != K.REUSE:
            kw.update(q_idx=inp["q_idx"], w=inp["w"], topk=topk,
                      candidates=self.cands if hsi == K.HSI_BUILD else None)
        io = K.layer_io(**kw)
        ws = torch.empty(max(K.layer_workspace_bytes(cfg, io), 16), dtype=torch.uint8, device=DEV)
        kw["workspace"] = ws
        io = K.layer_io(**kw)
        K.csa2_layer_forward(self.rt, cfg, io)
        torch.cuda.synchronize()
        return o, topk


def _np_inputs(inp, with_x):
    d = {k: (None if v is None else npy(v)) for k, v in inp.items()}
    return O.LayerInputs(q=d["q"], swa_kv=d["swa_kv"], q_pos=d["q_pos"], swa_pos0=d["swa_pos0"], q_idx=d["q_idx"],
                         w=d["w"], x=d["x"] if with_x else None)


def _compare_layer(tag, o_gpu, topk_gpu, rt_o: O.Runtime, o_ref, scores_fn, tol, check_sets=True):
    B, T = topk_gpu.shape[:2]
    tg = topk_gpu.cpu().numpy()
    og = npy(o_gpu)
    exact = np.zeros((B, T), bool)
    worst = 0.0
    for b in range(B):
        for t in range(T):
            if check_sets:
                sc, cands, exempt = scores_fn(b, t)
                exact[b, t] = check_topk_row(sc, cands, tg[b, t], tg.shape[-1], f"{tag} b{b} t{t}", exempt)
            else:
                exact[b, t] = np.array_equal(np.sort(tg[b, t]), np.sort(rt_o.topk_idxs[b, t]))
            if exact[b, t]:
                worst = max(worst, row_rel_err(og[b, t], o_ref[b, t]))
    say(f"  {tag}: exact sets {exact.sum()}/{B * T}, worst output row rel err {worst:.2e}")
    assert exact.mean() >= 0.97
    assert worst <= tol
    return exact


@pytest.mark.parametrize("dtype,sfmt", [(torch.float32, "e4m3"), (torch.bfloat16, "e4m3"),
                                       (torch.bfloat16, "ue8m0"), (torch.float32, "ue8m0")])
def test_full_reindex_reuse_tiny(dtype, sfmt):
    """sfmt: scale format of the Full layer's index K; the Reindex layer reads it
    from the index_k slot with the codes."""
    shape = synth.TINY if dtype == torch.float32 else synth.LayerShape(B=2, L=640, D=512, m=2, H_I=32, k=64, W=32, H=16)
    tol = 1e-3 if dtype == torch.float32 else 2e-2
    say(f"case: layers Full/Reindex/Reuse dtype={dtype} shape={shape} index-K scales {sfmt}")
    gfmt = K.SCALE_UE8M0 if sfmt == O.SCALE_UE8M0 else K.SCALE_E4M3
    g = GpuLayerStack(shape, dtype, scale_fmt=gfmt)
    full_in = synth.full_layer_inputs(shape, 0, dtype, DEV, layer=0)
    re_in = synth.full_layer_inputs(shape, 0, dtype, DEV, layer=1, with_x=False)
    ru_in = synth.full_layer_inputs(shape, 0, dtype, DEV, layer=2, with_x=False)

    rt_o = O.Runtime()
    cfg_full = O.LayerConfig(O.FULL, m=shape.m, k=shape.k, W=shape.W, w_kv=npy(full_in["w_kv"]),
                             w_gate=None if full_in["w_gate"] is None else npy(full_in["w_gate"]),
                             gamma=npy(full_in["gamma"]), w_ik=npy(full_in["w_ik"]), scale_fmt=sfmt)
    # ---- Full
    o_full, t_full = g.run(K.FULL, full_in)
    o_ref = O.layer_forward(rt_o, cfg_full, _np_inputs(full_in, True))
    codes_o, scales_o = rt_o.index_k
    for b in range(shape.B):
        lat_o, kv_o, ids = O.compress(npy(full_in["x"][b]), cfg_full.w_kv, cfg_full.w_gate, cfg_full.gamma, shape.m)
        assert row_rel_err(npy(g.kv[b]), kv_o) <= tol
        u, _, _ = O.index_k(lat_o, cfg_full.w_ik, ids * shape.m)
        nc, ns = check_fp4(u, g.codes[b].cpu().numpy(), g.scales[b].cpu().numpy(), f"full codes b{b}",
                           scale_fmt=sfmt)
        say(f"  full b={b}: FP4 code mismatches in band {nc}, scale {ns}")
    assert g.rt.slot(K.SLOT_INDEX_K).kv_fmt == gfmt   # the slot records the scale format
    kd = [O.fp4_unpack(codes_o[b], scales_o[b], scale_fmt=sfmt) for b in range(shape.B)]
    # entries whose GPU codes differ from the oracle's (each inside a rounding band, checked above)
    cg, sg = g.codes.cpu().numpy(), g.scales.cpu().numpy()
    flips = [np.where((cg[b] != codes_o[b]).any(1) | (sg[b] != scales_o[b]).any(1))[0] for b in range(shape.B)]

    def scores(inp):
        qi, ww = npy(inp["q_idx"]), npy(inp["w"])

        def fn(b, t):
            nv = O.visible_entries(t, shape.m)
            return O.index_scores(qi[b, t], ww[b, t], kd[b], nv), np.arange(nv), flips[b]
        return fn

    _compare_layer("full", o_full, t_full, rt_o, o_ref, scores(full_in), tol)
    info = g.rt.slot(K.SLOT_COMPRESS_KV)
    assert info.filled and info.ptr == g.kv.data_ptr() and info.cols == g.N
    # ---- Reindex (own indexer queries; KV and index K from the slots)
    o_re, t_re = g.run(K.REINDEX, re_in)
    o_ref = O.layer_forward(rt_o, O.LayerConfig(O.REINDEX, m=shape.m, k=shape.k, W=shape.W), _np_inputs(re_in, False))
    ex_re = _compare_layer("reindex", o_re, t_re, rt_o, o_ref, scores(re_in), tol)
    assert g.rt.slot(K.SLOT_TOPK_IDXS).ptr == t_re.data_ptr()
    # ---- Reuse (own queries; KV and top-k from the slots)
    o_ru, t_ru = g.run(K.REUSE, ru_in)
    o_ref = O.layer_forward(rt_o, O.LayerConfig(O.REUSE, m=shape.m, k=shape.k, W=shape.W), _np_inputs(ru_in, False))
    og, worst = npy(o_ru), 0.0
    for b in range(shape.B):
        for t in range(shape.L):
            if ex_re[b, t]:
                worst = max(worst, row_rel_err(og[b, t], o_ref[b, t]))
    say(f"  reuse: worst output row rel err {worst:.2e}")
    assert worst <= tol
    assert g.rt.slot(K.SLOT_TOPK_IDXS).ptr == t_re.data_ptr()   # Reuse wrote no slot


def test_reindex_with_full_queries_reproduces_full_selection():
    shape = synth.LayerShape(B=1, L=512, D=256, m=1, H_I=32, k=48, W=16, H=16)
    say("case: Reindex with the Full layer's indexer queries")
    g = GpuLayerStack(shape, torch.bfloat16)
    full_in = synth.full_layer_inputs(shape, 1, torch.bfloat16, DEV, layer=0)
    _, t_full = g.run(K.FULL, full_in)
    re_in = synth.full_layer_inputs(shape, 1, torch.bfloat16, DEV, layer=1, with_x=False)
    re_in["q_idx"], re_in["w"] = full_in["q_idx"], full_in["w"]
    gen_kv = g.rt.slot(K.SLOT_COMPRESS_KV).generation
    _, t_re = g.run(K.REINDEX, re_in)
    assert torch.equal(t_full, t_re)
    assert g.rt.slot(K.SLOT_COMPRESS_KV).generation == gen_kv   # Reindex does not write main KV


def test_hsi_layers():
    shape = synth.LayerShape(B=1, L=1024, D=256, m=1, H_I=32, k=32, W=16, H=16)
    s, nb = 16, 8
    say("case: Full (HSI build) then Reindex (HSI use)")
    g = GpuLayerStack(shape, torch.bfloat16, hsi=K.HSI_BUILD, hsi_s=s, hsi_nb=nb)
    full_in = synth.full_layer_inputs(shape, 2, torch.bfloat16, DEV, layer=0)
    _, t_full = g.run(K.FULL, full_in)
    re_in = synth.full_layer_inputs(shape, 2, torch.bfloat16, DEV, layer=1, with_x=False)
    _, t_re = g.run(K.REINDEX, re_in, hsi=K.HSI_USE)
    cg = g.cands.cpu().numpy()
    tr = t_re.cpu().numpy()
    # every Reindex selection lies inside the GPU pool of the same query, with the right size
    for t in range(shape.L):
        pool = set(O.pool_entries(cg[0, t], t + 1, s).tolist())
        sel = tr[0, t][tr[0, t] >= 0]
        assert set(sel.tolist()) <= pool
        assert len(sel) == min(shape.k, len(pool))
        assert (t // s) in cg[0, t]
