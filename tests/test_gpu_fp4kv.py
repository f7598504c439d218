"""GPU parity of the FP4 main KV ([P3] section six: 288 B per entry; section
seven: E2M1 data with an E4M3 scale per group of channels, dequantised before
attention).  The packer is bit-exact against the oracle codec; the compressor's
and the decode append's FP4 rows match the oracle's quantised latents up to
rounding-midpoint ties; attention over an FP4 cache equals the oracle's attention
over the dequantised rows in the few-query form (dequantised inside the gather)
and the many-query forms (dequantised once); a Full -> Reindex -> Reuse chain with
an FP4 cache matches the oracle's chain."""
import math

import numpy as np
import pytest
import torch

from oracle import csa2_oracle as O
from parity_utils import check_fp4, row_rel_err, say
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
    return t.detach().float().cpu().numpy().astype(np.float64) if t.is_floating_point() else t.cpu().numpy()


def test_kv_fp4_pack_bitexact():
    n = 3000
    say(f"case: kv_fp4_pack {n} rows")
    gen = np.random.default_rng(71)
    rows = synth.gaussian((n, 512), 1.0, 71, "u", 0, torch.float32, "cpu").numpy()
    rows *= np.exp(gen.uniform(-12, 8, (n, 1))).astype(np.float32)
    rows[0] = 0.0                                   # zero scale
    rows[1, :16] = -1e-9                            # rounds to -0 codes under a zero scale
    rows[2] *= 1e6                                  # saturating scale
    rows[3, 5] = 6.0 * 448.0 * 1.01                 # one saturating block
    codes = torch.zeros(n, 256, dtype=torch.uint8, device=DEV)
    scales = torch.zeros(n, 32, dtype=torch.uint8, device=DEV)
    K.csa2_kv_fp4_pack(torch.from_numpy(rows).to(DEV), codes, scales)
    torch.cuda.synchronize()
    c_o, s_o = O.kv_fp4_pack(rows)
    assert np.array_equal(scales.cpu().numpy(), s_o)
    assert np.array_equal(codes.cpu().numpy(), c_o)


@pytest.mark.parametrize("dtype,m", [(torch.bfloat16, 2), (torch.float32, 1), (torch.bfloat16, 4), (torch.bfloat16, 1)])
def test_compress_writes_fp4_kv(dtype, m):
    B, T, D = 2, 96 * m, 256
    N_cap = T // m + 5
    say(f"case: compress FP4 main KV dtype={dtype} m={m} B={B} T={T}")
    x = synth.gaussian((B, T, D), 1.0, 72, "x", 0, dtype, DEV)
    w_kv = synth.linear_weight(512, D, 72, "w_kv", 0, dtype, DEV)
    w_gate = synth.linear_weight(512, D, 72, "w_gate", 0, dtype, DEV) if m > 1 else None
    gamma = torch.ones(512, dtype=torch.float32, device=DEV)
    lat = torch.empty(B, T // m, 512, dtype=torch.float32, device=DEV)
    codes = torch.zeros(B, N_cap, 256, dtype=torch.uint8, device=DEV)
    scales = torch.zeros(B, N_cap, 32, dtype=torch.uint8, device=DEV)
    start = 2 * m
    K.csa2_compress(None, x, w_kv, w_gate, gamma, lat, codes, m=m, start_pos=start, kv_scales=scales)
    torch.cuda.synchronize()
    cg, sg = codes.cpu().numpy(), scales.cpu().numpy()
    g0, n = start // m, T // m
    for b in range(B):
        _, kv_o, _ = O.compress(npy(x[b]), npy(w_kv), None if w_gate is None else npy(w_gate), npy(gamma), m, start)
        nc, ns = check_fp4(kv_o, cg[b, g0:g0 + n], sg[b, g0:g0 + n], f"b{b}", block=16)
        say(f"  b{b}: code/scale differences at rounding midpoints {nc}/{ns}")
        assert nc + ns <= 0.002 * n * 512
        assert np.all(cg[b, :g0] == 0) and np.all(cg[b, g0 + n:] == 0) and np.all(sg[b, g0 + n:] == 0)


def _attn_case(dtype, B, T, H, k, W, N_cap, L_w, seed):
    gen = np.random.default_rng(seed)
    q = synth.gaussian((B, T, H, 512), 1.0, seed, "q", 0, dtype, DEV)
    rows = synth.gaussian((B * N_cap, 512), 1.0, seed, "kv_cache", 0, torch.float32, "cpu").numpy()
    rows *= np.exp(gen.uniform(-1.5, 1.5, (B * N_cap, 1))).astype(np.float32)
    c_o, s_o = O.kv_fp4_pack(rows)
    kv_deq = O.kv_fp4_unpack(c_o, s_o).reshape(B, N_cap, 512)
    codes = torch.from_numpy(c_o.reshape(B, N_cap, 256)).to(DEV)
    scales = torch.from_numpy(s_o.reshape(B, N_cap, 32)).to(DEV)
    swa = synth.gaussian((B, L_w, 512), 1.0, seed, "swa_kv", 0, dtype, DEV)
    pos0 = (gen.integers(0, 50, B)).astype(np.int32)
    pos = (pos0[:, None] + gen.integers(0, L_w, (B, T))).astype(np.int32)
    pos[0, 0] = pos0[0]                               # window of one row
    tk = np.full((B, T, k), -1, np.int32)
    for b in range(B):
        for t in range(T):
            nsel = [k, k // 2, 0, min(k, 7)][(b * T + t) % 4]
            ids = np.sort(gen.choice(N_cap, size=nsel, replace=False)).astype(np.int32)
            tk[b, t, :nsel] = ids
    if k > 1:
        tk[0, 0, -1] = N_cap + 5                      # out of range: skipped
    return q, codes, scales, kv_deq, swa, pos0, pos, tk


def _check_attn(q, kv_deq, swa, pos0, pos, tk, o, lse, W, N_cap, dtype, sample):
    og, lg, qn, swn = npy(o), lse.cpu().numpy(), npy(q), npy(swa)
    worst = 0.0
    for (b, t) in sample:
        sel = tk[b, t]
        sel = sel[(sel >= 0) & (sel < N_cap)]
        ref, _, rows = O.sparse_attention(qn[b, t], kv_deq[b], sel, swn[b], int(pos0[b]), int(pos[b, t]), W)
        worst = max(worst, row_rel_err(og[b, t], ref))
        lse_ref = O.attention_lse(qn[b, t], rows)
        assert np.allclose(lg[b, t], lse_ref, rtol=1e-4, atol=1e-3)
    say(f"  worst row rel err {worst:.2e} over {len(sample)} queries")
    assert worst <= TOL[dtype]


@pytest.mark.parametrize("H,k,W", [(64, 512, 128), (20, 77, 5), (16, 96, 40), (64, 40, 128)])
def test_decode_attention_fp4_kv(H, k, W):
    B, T, N_cap, L_w = 3, 2, 1500, 300
    say(f"case: decode attention FP4 KV H={H} k={k} W={W} B={B} T={T}")
    q, codes, scales, kv_deq, swa, pos0, pos, tk = _attn_case(torch.bfloat16, B, T, H, k, W, N_cap, L_w, 73)
    o = torch.empty_like(q)
    lse = torch.empty(B, T, H, dtype=torch.float32, device=DEV)
    K.csa2_sparse_attn(None, q, codes, torch.from_numpy(tk).to(DEV), swa, torch.from_numpy(pos0).to(DEV),
                       torch.from_numpy(pos).to(DEV), o, W=W, lse=lse, kv_scales=scales)
    torch.cuda.synchronize()
    _check_attn(q, kv_deq, swa, pos0, pos, tk, o, lse, W, N_cap, torch.bfloat16,
                [(b, t) for b in range(B) for t in range(T)])


@pytest.mark.parametrize("dtype,T", [(torch.bfloat16, 600), (torch.float32, 8)])
def test_many_query_attention_fp4_kv(dtype, T):
    B, H, k, W, N_cap, L_w = 2, 16 if dtype == torch.float32 else 64, 64, 32, 700, 700
    say(f"case: attention FP4 KV, dequantised once: dtype={dtype} B={B} T={T}")
    q, codes, scales, kv_deq, swa, pos0, pos, tk = _attn_case(dtype, B, T, H, k, W, N_cap, L_w, 74)
    o = torch.empty_like(q)
    lse = torch.empty(B, T, H, dtype=torch.float32, device=DEV)
    K.csa2_sparse_attn(None, q, codes, torch.from_numpy(tk).to(DEV), swa, torch.from_numpy(pos0).to(DEV),
                       torch.from_numpy(pos).to(DEV), o, W=W, lse=lse, kv_scales=scales)
    torch.cuda.synchronize()
    sample = [(b, t) for b in range(B) for t in range(0, T, max(1, T // 40))] + [(B - 1, T - 1)]
    _check_attn(q, kv_deq, swa, pos0, pos, tk, o, lse, W, N_cap, dtype, sample)


def test_decode_append_writes_fp4_kv():
    B, D, m = 3, 256, 2
    P, S = 8, 9
    L = P + S
    say(f"case: compress_step FP4 main KV B={B} D={D} m={m} prefill {P} + {S} steps")
    dtype = torch.bfloat16
    x = synth.gaussian((B, L, D), 1.0, 75, "x", 0, dtype, DEV)
    w_kv = synth.linear_weight(512, D, 75, "w_kv", 0, dtype, DEV)
    w_gate = synth.linear_weight(512, D, 75, "w_gate", 0, dtype, DEV)
    w_ik = synth.linear_weight(128, 512, 75, "w_ik", 0, dtype, DEV)
    gamma = torch.ones(512, dtype=torch.float32, device=DEV)
    N_cap = L // m + 2
    codes = torch.zeros(B, N_cap, 256, dtype=torch.uint8, device=DEV)
    scales = torch.zeros(B, N_cap, 32, dtype=torch.uint8, device=DEV)
    ikc = torch.zeros(B, N_cap, 64, dtype=torch.uint8, device=DEV)
    iks = torch.zeros(B, N_cap, 4, dtype=torch.uint8, device=DEV)
    lat = torch.empty(B, P // m, 512, dtype=torch.float32, device=DEV)
    K.csa2_compress(None, x[:, :P].contiguous(), w_kv, w_gate, gamma, lat, codes, m=m, start_pos=0,
                    kv_scales=scales)
    K.csa2_index_k(None, lat, w_ik, ikc, iks, m=m)
    state = torch.zeros(B, 3, 512, dtype=torch.float32, device=DEV)
    ws = None
    for s in range(S):
        t = P + s
        xs = x[:, t].contiguous()
        pos = torch.full((B,), t, dtype=torch.int32, device=DEV)
        ws = K.csa2_compress_step(None, xs, pos, w_kv, w_gate, gamma, w_ik, state, codes, ikc, iks, m=m,
                                  workspace=ws, kv_scales=scales)
    torch.cuda.synchronize()
    n_done = L // m
    cg, sg = codes.cpu().numpy(), scales.cpu().numpy()
    for b in range(B):
        _, kv_o, _ = O.compress(npy(x[b, :n_done * m]), npy(w_kv), npy(w_gate), npy(gamma), m, 0)
        nc, ns = check_fp4(kv_o, cg[b, :n_done], sg[b, :n_done], f"b{b}", block=16)
        say(f"  b{b}: {n_done - P // m} appended rows; differences at rounding midpoints {nc}/{ns}")
        assert np.all(cg[b, n_done:] == 0)


def test_layers_with_fp4_kv():
    from test_gpu_layers import GpuLayerStack, _compare_layer, _np_inputs
    shape = synth.LayerShape(B=2, L=640, D=512, m=2, H_I=32, k=64, W=32, H=16)
    dtype, tol = torch.bfloat16, 2e-2
    say(f"case: layers Full/Reindex/Reuse with FP4 main KV, shape={shape}")
    g = GpuLayerStack(shape, dtype, kv_fp4=True)
    full_in = synth.full_layer_inputs(shape, 0, dtype, DEV, layer=0)
    re_in = synth.full_layer_inputs(shape, 0, dtype, DEV, layer=1, with_x=False)
    ru_in = synth.full_layer_inputs(shape, 0, dtype, DEV, layer=2, with_x=False)
    rt_o = O.Runtime()
    cfg_full = O.LayerConfig(O.FULL, m=shape.m, k=shape.k, W=shape.W, w_kv=npy(full_in["w_kv"]),
                             w_gate=npy(full_in["w_gate"]), gamma=npy(full_in["gamma"]), w_ik=npy(full_in["w_ik"]),
                             kv_fp4=True)
    o_full, t_full = g.run(K.FULL, full_in)
    o_ref = O.layer_forward(rt_o, cfg_full, _np_inputs(full_in, True))
    codes_o, scales_o = rt_o.index_k
    for b in range(shape.B):
        _, kv_o, _ = O.compress(npy(full_in["x"][b]), cfg_full.w_kv, cfg_full.w_gate, cfg_full.gamma, shape.m)
        nc, ns = check_fp4(kv_o, g.kv[b].cpu().numpy(), g.kv_scales[b].cpu().numpy(), f"kv b{b}", block=16)
        say(f"  full b={b}: FP4 main-KV differences at rounding midpoints {nc}/{ns}")
    info = g.rt.slot(K.SLOT_COMPRESS_KV)
    assert info.kv_fmt == K.KV_FP4 and info.ptr == g.kv.data_ptr() and info.ptr2 == g.kv_scales.data_ptr()
    kd = [O.fp4_unpack(codes_o[b], scales_o[b]) for b in range(shape.B)]
    cg, sg = g.codes.cpu().numpy(), g.scales.cpu().numpy()
    flips = [np.where((cg[b] != codes_o[b]).any(1) | (sg[b] != scales_o[b]).any(1))[0] for b in range(shape.B)]

    def scores(inp):
        qi, ww = npy(inp["q_idx"]), npy(inp["w"])

        def fn(b, t):
            nv = O.visible_entries(t, shape.m)
            return O.index_scores(qi[b, t], ww[b, t], kd[b], nv), np.arange(nv), flips[b]
        return fn

    _compare_layer("full", o_full, t_full, rt_o, o_ref, scores(full_in), tol)
    o_re, t_re = g.run(K.REINDEX, re_in)
    o_ref = O.layer_forward(rt_o, O.LayerConfig(O.REINDEX, m=shape.m, k=shape.k, W=shape.W), _np_inputs(re_in, False))
    ex_re = _compare_layer("reindex", o_re, t_re, rt_o, o_ref, scores(re_in), tol)
    o_ru, _ = g.run(K.REUSE, ru_in)
    o_ref = O.layer_forward(rt_o, O.LayerConfig(O.REUSE, m=shape.m, k=shape.k, W=shape.W), _np_inputs(ru_in, False))
    og, worst = npy(o_ru), 0.0
    for b in range(shape.B):
        for t in range(shape.L):
            if ex_re[b, t]:
                worst = max(worst, row_rel_err(og[b, t], o_ref[b, t]))
    say(f"  reuse: worst output row rel err {worst:.2e}")
    assert worst <= tol
