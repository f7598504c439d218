"""GPU parity of the per-head attention sink (a logit that enters the softmax
denominator only; the pages name one sink per head in every layer but give no
formula, see the oracle's sparse_attention) on every attention path: the prefill
kernel (4- and 2-wave forms), few-query attention with one row split and with
several splits merged by the combine step, the fp32 path, and a Reuse layer
through csa2_layer_forward.  Rows with nothing to attend to must give a zero
output and the sink as log-sum-exp."""
import math

import numpy as np
import pytest
import torch

from oracle import csa2_oracle as O
from parity_utils import row_rel_err, say
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


def _case(dtype, B, T, H, k, W, N_cap, L_w, seed, empty_every=7):
    gen = np.random.default_rng(seed)
    q = synth.gaussian((B, T, H, 512), 1.0, seed, "q", 0, dtype, DEV)
    kv = synth.gaussian((B, N_cap, 512), 1.0, seed, "kv_cache", 0, dtype, DEV)
    swa = synth.gaussian((B, L_w, 512), 1.0, seed, "swa_kv", 0, dtype, DEV)
    # sink logits around the typical row logits (|q . r| / sqrt(512) ~ 1), some dominant
    sink = torch.from_numpy(gen.normal(1.0, 2.0, size=H).astype(np.float32)).to(DEV)
    pos0 = np.zeros(B, np.int32)
    pos0[-1] = 5
    pos = np.stack([gen.integers(0, L_w, size=T) for _ in range(B)]).astype(np.int32)
    tk = np.full((B, T, k), -1, np.int32)
    for b in range(B):
        for t in range(T):
            n = int(gen.integers(0, k + 1)) if t % empty_every else 0
            tk[b, t, :n] = np.sort(gen.choice(N_cap, size=n, replace=False))
            if n > 3 and t % 3 == 0:
                tk[b, t, 1] = -1
    # a query of the last sequence before its window buffer starts and with nothing selected
    pos[-1, 0] = 2
    tk[-1, 0, :] = -1
    return q, kv, swa, sink, pos0, pos, tk


def _check(tag, dtype, q, kv, swa, sink, pos0, pos, tk, W, o, lse, rows_of, every=1):
    og, lg = npy(o), lse.cpu().numpy()
    kvn, swn, qn, sk = npy(kv), npy(swa), npy(q), npy(sink)
    B, T = tk.shape[:2]
    N_cap = kv.shape[1]
    worst, n_empty, n_checked = 0.0, 0, 0
    for b in range(B):
        for t in sorted(set(list(range(0, T, every)) + [T - 1])):
            sel = tk[b, t]
            sel = sel[(sel >= 0) & (sel < N_cap)]
            ref, p, rows = O.sparse_attention(qn[b, t], kvn[b], sel, swn[b], int(pos0[b]), int(pos[b, t]), W, sink=sk)
            lse_ref = O.attention_lse(qn[b, t], rows, sink=sk)
            if rows.shape[0] == 0:
                assert np.all(og[b, t] == 0), f"{tag} b{b} t{t}: empty row must give 0"
                assert np.allclose(lg[b, t], sk, rtol=1e-6, atol=1e-6), f"{tag} b{b} t{t}: lse of an empty row"
                n_empty += 1
                continue
            worst = max(worst, row_rel_err(og[b, t], ref))
            assert np.allclose(lg[b, t], lse_ref, rtol=1e-4, atol=1e-3), f"{tag} b{b} t{t}: lse"
            n_checked += 1
    say(f"  {tag}: {n_checked} tokens, {n_empty} empty, worst row rel err {worst:.2e}")
    assert n_empty >= 1 and worst <= TOL[dtype]


@pytest.mark.parametrize("H", [64, 20])
def test_sink_prefill_path(H):
    q, kv, swa, sink, pos0, pos, tk = _case(torch.bfloat16, 2, 600, H, 96, 40, 700, 620, 41)
    say(f"case: attention sink, prefill path H={H}")
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    K.csa2_sparse_attn(None, q, kv, torch.from_numpy(tk).to(DEV), swa, torch.from_numpy(pos0).to(DEV),
                       torch.from_numpy(pos).to(DEV), o, W=40, lse=lse, sink=sink)
    torch.cuda.synchronize()
    _check(f"prefill H={H}", torch.bfloat16, q, kv, swa, sink, pos0, pos, tk, 40, o, lse, None, every=11)


@pytest.mark.parametrize("B,T", [(3, 100), (2, 4)])
def test_sink_decode_paths(B, T):
    """B*T = 300 queries: one row split each (direct output); 8 queries: many
    splits merged by the combine step, which adds the sink once."""
    q, kv, swa, sink, pos0, pos, tk = _case(torch.bfloat16, B, T, 64, 512, 128, 1200, 400, 43, empty_every=5)
    say(f"case: attention sink, decode path B={B} T={T}")
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    K.csa2_sparse_attn(None, q, kv, torch.from_numpy(tk).to(DEV), swa, torch.from_numpy(pos0).to(DEV),
                       torch.from_numpy(pos).to(DEV), o, W=128, lse=lse, sink=sink)
    torch.cuda.synchronize()
    _check(f"decode B={B} T={T}", torch.bfloat16, q, kv, swa, sink, pos0, pos, tk, 128, o, lse, None,
           every=7 if T > 10 else 1)


def test_sink_fp32_path():
    q, kv, swa, sink, pos0, pos, tk = _case(torch.float32, 2, 6, 8, 32, 16, 300, 120, 47, empty_every=3)
    say("case: attention sink, fp32 path")
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    K.csa2_sparse_attn(None, q, kv, torch.from_numpy(tk).to(DEV), swa, torch.from_numpy(pos0).to(DEV),
                       torch.from_numpy(pos).to(DEV), o, W=16, lse=lse, sink=sink)
    torch.cuda.synchronize()
    _check("fp32", torch.float32, q, kv, swa, sink, pos0, pos, tk, 16, o, lse, None)


@pytest.mark.parametrize("B,T", [(2, 600), (2, 4)])
def test_sink_minus_infinity_is_no_sink(B, T):
    """A sink of -inf leaves the result bit for bit as without a sink."""
    q, kv, swa, sink, pos0, pos, tk = _case(torch.bfloat16, B, T, 64, 96, 40, 700, 620, 53)
    args = (torch.from_numpy(tk).to(DEV), swa, torch.from_numpy(pos0).to(DEV), torch.from_numpy(pos).to(DEV))
    o1, o2 = torch.empty_like(q), torch.empty_like(q)
    K.csa2_sparse_attn(None, q, kv, args[0], args[1], args[2], args[3], o1, W=40)
    K.csa2_sparse_attn(None, q, kv, args[0], args[1], args[2], args[3], o2, W=40,
                       sink=torch.full((64,), -math.inf, dtype=torch.float32, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_sink_through_layer_forward():
    """A Reuse layer with a sink through csa2_layer_forward equals the direct call."""
    from test_gpu_layers import GpuLayerStack
    shape = synth.LayerShape(B=1, L=256, D=256, m=2, H_I=4, k=32, W=16, H=8)
    inp = synth.full_layer_inputs(shape, 9, torch.bfloat16, DEV, layer=0)
    reuse = synth.full_layer_inputs(shape, 9, torch.bfloat16, DEV, layer=2, with_x=False)
    st = GpuLayerStack(shape, torch.bfloat16)
    _, topk = st.run(K.FULL, inp)
    sink = torch.linspace(-2.0, 3.0, shape.H, device=DEV, dtype=torch.float32)
    o_layer, _ = st.run(K.REUSE, reuse, sink=sink)
    o_direct = torch.empty_like(reuse["q"])
    K.csa2_sparse_attn(None, reuse["q"], st.kv, topk, reuse["swa_kv"], reuse["swa_pos0"], reuse["q_pos"], o_direct,
                       W=shape.W, sink=sink)
    o_plain, _ = st.run(K.REUSE, reuse)
    torch.cuda.synchronize()
    assert torch.equal(o_layer, o_direct)
    assert not torch.equal(o_layer, o_plain)
