"""GPU parity of the FP8 window KV ring ([P3] section seven: the window KV is kept
in FP8): csa2_swa_append against the oracle's E4M3 encoding byte for byte (a
prefill block, decode appends that wrap the ring, saturation, ties, subnormals,
signed zero, skipped rows); attention that reads the ring on the few-query path
(dense and FP4 main KV), on the many-query path and through a Reuse layer,
against the oracle over the ring's dequantised rows and, bit for bit, against the
same kernels given those rows as a dense window."""
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

# values that reach each branch of the encoding: zeros of both signs, the
# largest finite value and beyond (saturation), ties between neighbours (to the
# even code), the subnormal range, a tie at half the smallest subnormal (to a
# signed zero), the smallest normal
SPECIALS = [0.0, -0.0, 448.0, -448.0, 460.0, 500.0, -1e6, 1.0625, -1.1875, 2.0 ** -10, -(2.0 ** -10),
            3 * 2.0 ** -10, 2.0 ** -9, -1e-5, 2.0 ** -6, 0.0137, 240.0, 232.0, -13.0]


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def npy(t):
    return t.detach().float().cpu().numpy().astype(np.float64) if t.is_floating_point() else t.cpu().numpy()


def window_rows(B, n, seed, dtype, with_specials=True):
    rows = synth.gaussian((B, n, 512), 1.0, seed, "swa_kv", 0, torch.float32, "cpu")
    if with_specials:
        # every row holds each special value once, at dims drawn per row
        gen = torch.Generator().manual_seed(seed)
        dims = torch.argsort(torch.rand(B, n, 512, generator=gen), dim=2)[:, :, :len(SPECIALS)]
        rows.scatter_(2, dims, torch.tensor(SPECIALS).expand(B, n, len(SPECIALS)).contiguous())
    return rows.to(dtype).to(DEV)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_swa_append_matches_oracle(dtype):
    B, L_w, n_pre, steps = 3, 96, [200, 96, 40], 130
    say(f"case: swa_append dtype={dtype} B={B} L_w={L_w} prefill {n_pre} + {steps} appends")
    total = max(n_pre) + steps
    rows = window_rows(B, total, 5, dtype)
    ring = torch.full((B, L_w, 512), 0x5A, dtype=torch.uint8, device=DEV)
    oring = np.full((B, L_w, 512), 0x5A, dtype=np.uint8)
    rn = npy(rows)
    # prefill: the last L_w rows of each sequence at once (absent rows: pos -1)
    pre_pos = np.full((B, L_w), -1, np.int32)
    pre_rows = torch.zeros(B, L_w, 512, dtype=dtype, device=DEV)
    for b in range(B):
        first = max(0, n_pre[b] - L_w)
        cnt = n_pre[b] - first
        pre_pos[b, :cnt] = np.arange(first, n_pre[b])
        pre_rows[b, :cnt] = rows[b, first:n_pre[b]]
        O.swa_ring_append(oring[b], rn[b, first:n_pre[b]], pre_pos[b, :cnt])
    K.csa2_swa_append(pre_rows, torch.from_numpy(pre_pos).to(DEV), ring)
    torch.cuda.synchronize()
    assert np.array_equal(ring.cpu().numpy(), oring), "after the prefill block"
    # decode: one row per sequence and step; sequence 2 skips every third step
    nxt = list(n_pre)
    for s in range(steps):
        pos = np.array([nxt[b] if (b != 2 or s % 3) else -1 for b in range(B)], np.int32)
        step_rows = torch.stack([rows[b, max(int(pos[b]), 0)] for b in range(B)])[:, None].contiguous()
        K.csa2_swa_append(step_rows, torch.from_numpy(pos[:, None]).to(DEV), ring)
        for b in range(B):
            if pos[b] >= 0:
                O.swa_ring_append(oring[b], rn[b, pos[b]][None], pos[b:b + 1])
                nxt[b] += 1
    torch.cuda.synchronize()
    got = ring.cpu().numpy()
    assert np.array_equal(got, oring), f"{np.count_nonzero(got != oring)} bytes differ after the appends"
    # every special value reached the ring with its expected byte somewhere
    vals = O.e4m3_decode(got)
    assert np.any(got == 0x80) and np.any(got == 0x7E) and np.any(got == 0xFE), "sign-zero / saturation"
    assert np.isfinite(vals).all()


def _ring_for(rows, n_pre, last, L_w, dtype):
    """Append window rows of positions 0..last[b] to a fresh ring the way a
    serving loop does (prefill block, then one row per step) on the GPU, and the
    same on the oracle's ring; returns (gpu ring, oracle ring)."""
    B = rows.shape[0]
    ring = torch.zeros(B, L_w, 512, dtype=torch.uint8, device=DEV)
    oring = np.zeros((B, L_w, 512), np.uint8)
    rn = npy(rows)
    pre_pos = np.full((B, L_w), -1, np.int32)
    pre_rows = torch.zeros(B, L_w, 512, dtype=dtype, device=DEV)
    for b in range(B):
        first = max(0, n_pre[b] - L_w)
        cnt = n_pre[b] - first
        pre_pos[b, :cnt] = np.arange(first, n_pre[b])
        pre_rows[b, :cnt] = rows[b, first:n_pre[b]]
        O.swa_ring_append(oring[b], rn[b, first:n_pre[b]], pre_pos[b, :cnt])
    K.csa2_swa_append(pre_rows, torch.from_numpy(pre_pos).to(DEV), ring)
    nxt = list(n_pre)
    while any(nxt[b] <= last[b] for b in range(B)):
        pos = np.array([nxt[b] if nxt[b] <= last[b] else -1 for b in range(B)], np.int32)
        step_rows = torch.stack([rows[b, max(int(pos[b]), 0)] for b in range(B)])[:, None].contiguous()
        K.csa2_swa_append(step_rows, torch.from_numpy(pos[:, None]).to(DEV), ring)
        for b in range(B):
            if pos[b] >= 0:
                O.swa_ring_append(oring[b], rn[b, pos[b]][None], pos[b:b + 1])
                nxt[b] += 1
    torch.cuda.synchronize()
    assert np.array_equal(ring.cpu().numpy(), oring), "ring bytes"
    return ring, oring


def _dense_from_ring(oring, pos0, L_w, dtype):
    """The oracle ring's rows of positions pos0[b] .. pos0[b] + L_w - 1 as a dense
    window (rows past what the ring holds stay zero; no query reaches them)."""
    B = oring.shape[0]
    dense = np.zeros((B, L_w, 512))
    for b in range(B):
        hi = pos0[b] + L_w - 1
        dense[b] = O.swa_ring_rows(oring[b], pos0[b], hi)
    return torch.from_numpy(dense).to(dtype).to(DEV)


def _ring_vs_dense(o_ring, o_dense, lse_ring=None, lse_dense=None, exact=True):
    """The ring call against the same call over the ring's rows as a dense window.
    Where both run the same kernel over the same splits the results are equal bit
    for bit.  The bf16 decode kernel gives a ring's window rows splits of their own
    (read and widened from the ring), while a dense window shares splits with bf16
    selected rows: the same rows, but partials merged in another grouping, so the
    two agree to the bf16 partials' rounding."""
    if exact:
        assert torch.equal(o_ring, o_dense), "ring vs dense window of its rows"
        if lse_ring is not None:
            assert torch.equal(lse_ring, lse_dense), "ring vs dense window: lse"
        return
    err = row_rel_err(npy(o_ring), npy(o_dense))
    assert err <= 1e-2, f"ring vs dense window of its rows: {err:.2e}"
    if lse_ring is not None:
        assert torch.allclose(lse_ring, lse_dense, rtol=1e-5, atol=1e-5), "ring vs dense window: lse"


@pytest.mark.parametrize("dtype,kv_fp4,L_w,W,H", [
    (torch.bfloat16, False, 128, 128, 64), (torch.bfloat16, True, 160, 128, 64), (torch.float32, False, 128, 64, 8),
    (torch.bfloat16, False, 96, 64, 16), (torch.bfloat16, True, 96, 64, 32), (torch.bfloat16, True, 128, 100, 16),
])
def test_ring_attention_decode(dtype, kv_fp4, L_w, W, H):
    B, k, N_cap = 3, 32, 80
    last = [300, 77, 20]              # newest position of each sequence
    n_pre = [200, 50, 10]
    say(f"case: ring attention decode dtype={dtype} fp4kv={kv_fp4} L_w={L_w} W={W} H={H}")
    rows = window_rows(B, max(last) + 1, 17, dtype, with_specials=False)
    ring, oring = _ring_for(rows, n_pre, last, L_w, dtype)
    q = synth.gaussian((B, 1, H, 512), 1.0, 17, "q", 0, dtype, DEV)
    kvf = synth.gaussian((B, N_cap, 512), 1.0, 17, "kv_cache", 0, torch.float32, DEV)
    gen = np.random.default_rng(17)
    tk_np = np.stack([gen.choice(N_cap, size=k, replace=False) for _ in range(B)]).astype(np.int32)[:, None]
    tk = torch.from_numpy(tk_np).to(DEV)
    if kv_fp4:
        codes = torch.empty(B, N_cap, 256, dtype=torch.uint8, device=DEV)
        scs = torch.empty(B, N_cap, 32, dtype=torch.uint8, device=DEV)
        K.csa2_kv_fp4_pack(kvf.contiguous(), codes, scs)
        kv, kv_scales = codes, scs
        kv_rows = [O.kv_fp4_unpack(*O.kv_fp4_pack(npy(kvf[b]).astype(np.float32))) for b in range(B)]
    else:
        kv, kv_scales = kvf.to(dtype), None
        kv_rows = [npy(kv[b]) for b in range(B)]
    swa_pos0 = torch.zeros(B, dtype=torch.int32, device=DEV)
    q_pos = torch.tensor(last, dtype=torch.int32, device=DEV)[:, None].contiguous()
    o_ring = torch.empty_like(q)
    lse_ring = torch.empty(B, 1, H, dtype=torch.float32, device=DEV)
    K.csa2_sparse_attn(None, q, kv, tk, ring, swa_pos0, q_pos, o_ring, W=W, lse=lse_ring, kv_scales=kv_scales)
    # the same kernels over the ring's rows given as a dense window
    pos0 = [max(0, last[b] - L_w + 1) for b in range(B)]
    dense = _dense_from_ring(oring, pos0, L_w, dtype)
    o_dense = torch.empty_like(q)
    lse_dense = torch.empty_like(lse_ring)
    K.csa2_sparse_attn(None, q, kv, tk, dense, torch.tensor(pos0, dtype=torch.int32, device=DEV), q_pos, o_dense,
                       W=W, lse=lse_dense, kv_scales=kv_scales)
    torch.cuda.synchronize()
    _ring_vs_dense(o_ring, o_dense, lse_ring, lse_dense, exact=kv_fp4 or dtype == torch.float32)
    og, qn = npy(o_ring), npy(q)
    worst = 0.0
    for b in range(B):
        win = O.swa_ring_rows(oring[b], pos0[b], last[b])
        ref, _, rows_used = O.sparse_attention(qn[b, 0], kv_rows[b], tk_np[b, 0].astype(np.int64), win, pos0[b],
                                               last[b], W)
        worst = max(worst, row_rel_err(og[b, 0], ref))
        assert np.allclose(lse_ring[b, 0].cpu().numpy(), O.attention_lse(qn[b, 0], rows_used), rtol=1e-4,
                           atol=1e-3), b
    say(f"  worst row rel err {worst:.2e}")
    assert worst <= TOL[dtype]


@pytest.mark.parametrize("T,L_w", [(300, 448), (8, 160)])
def test_ring_attention_many_queries(T, L_w):
    """Several queries per sequence, all within L_w - W of the newest position so
    that every window lies inside the ring: 600 queries take the many-query
    kernel, 16 the decode kernel, which finds the ring's first position from each
    sequence's newest query itself."""
    dtype, B, H, k, W, N_cap = torch.bfloat16, 2, 16, 16, 128, 64
    last = [700, 400]
    n_pre = [600, 300]
    say(f"case: ring attention many queries B={B} T={T} H={H} L_w={L_w} W={W}")
    rows = window_rows(B, max(last) + 1, 23, dtype, with_specials=False)
    ring, oring = _ring_for(rows, n_pre, last, L_w, dtype)
    q = synth.gaussian((B, T, H, 512), 1.0, 23, "q", 0, dtype, DEV)
    kv = synth.gaussian((B, N_cap, 512), 1.0, 23, "kv_cache", 0, dtype, DEV)
    gen = np.random.default_rng(23)
    tk_np = np.stack([np.stack([gen.choice(N_cap, size=k, replace=False) for _ in range(T)])
                      for _ in range(B)]).astype(np.int32)
    qp = np.stack([np.arange(last[b] - T + 1, last[b] + 1) for b in range(B)]).astype(np.int32)
    gen.shuffle(qp, axis=1)
    tk, q_pos = torch.from_numpy(tk_np).to(DEV), torch.from_numpy(qp).to(DEV)
    swa_pos0 = torch.zeros(B, dtype=torch.int32, device=DEV)
    o_ring = torch.empty_like(q)
    K.csa2_sparse_attn(None, q, kv, tk, ring, swa_pos0, q_pos, o_ring, W=W)
    pos0 = [max(0, last[b] - L_w + 1) for b in range(B)]
    dense = _dense_from_ring(oring, pos0, L_w, dtype)
    o_dense = torch.empty_like(q)
    K.csa2_sparse_attn(None, q, kv, tk, dense, torch.tensor(pos0, dtype=torch.int32, device=DEV), q_pos, o_dense,
                       W=W)
    torch.cuda.synchronize()
    _ring_vs_dense(o_ring, o_dense, exact=B * T >= 512)
    og, qn, kvn = npy(o_ring), npy(q), npy(kv)
    worst = 0.0
    for b in range(B):
        for t in sorted(set([0, 1, T - 1] + list(range(0, T, 29)))):
            p = int(qp[b, t])
            win = O.swa_ring_rows(oring[b], pos0[b], last[b])
            ref, _, _ = O.sparse_attention(qn[b, t], kvn[b], tk_np[b, t].astype(np.int64), win, pos0[b], p, W)
            worst = max(worst, row_rel_err(og[b, t], ref))
    say(f"  worst row rel err {worst:.2e}")
    assert worst <= TOL[dtype]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_ring_through_reuse_layer(dtype):
    """A Full layer's prefill (dense window) fills the slots; a Reuse layer then
    attends with its window KV in an FP8 ring (cfg.swa_fmt) holding all prefill
    positions; equal to the same layer given the ring's rows as a dense window,
    and to the oracle's layer_forward over those rows."""
    B, m, P = 2, 2, 16
    D = 512 if dtype == torch.bfloat16 else 256
    H_I, H, k, W, L_w = 4, 8, 4, 8, 32
    say(f"case: ring through a Reuse layer dtype={dtype} B={B} P={P} L_w={L_w}")
    shape = synth.LayerShape(B=B, L=P, D=D, m=m, H_I=H_I, k=k, W=W, H=H)
    f = synth.full_layer_inputs(shape, 61, dtype, DEV, layer=0, with_x=True)
    g = synth.full_layer_inputs(shape, 61, dtype, DEV, layer=1, with_x=False)
    cd = K.CSA2_BF16 if dtype == torch.bfloat16 else K.CSA2_F32
    rt = K.Runtime()
    N_cap = P // m
    lat = torch.empty(B, N_cap, 512, dtype=torch.float32, device=DEV)
    kv = torch.zeros(B, N_cap, 512, dtype=dtype, device=DEV)
    codes = torch.zeros(B, N_cap, 64, dtype=torch.uint8, device=DEV)
    scales = torch.zeros(B, N_cap, 4, dtype=torch.uint8, device=DEV)
    cfg_full = K.layer_cfg(K.FULL, cd, m=m, k=k, W=W, H_I=H_I, H=H)
    o_full = torch.empty_like(f["q"])
    tk = torch.empty(B, P, k, dtype=torch.int32, device=DEV)
    kw = dict(B=B, T=P, q_pos=f["q_pos"], q=f["q"], swa_kv=f["swa_kv"], swa_pos0=f["swa_pos0"], o=o_full,
              N_cap=N_cap, D=D, x=f["x"], w_kv=f["w_kv"], w_gate=f["w_gate"], gamma=f["gamma"], w_ik=f["w_ik"],
              latent_pre=lat, kv_cache=kv, ik_codes=codes, ik_scales=scales, q_idx=f["q_idx"], w=f["w"], topk=tk)
    ws = torch.empty(max(K.layer_workspace_bytes(cfg_full, K.layer_io(**kw)), 16), dtype=torch.uint8, device=DEV)
    K.csa2_layer_forward(rt, cfg_full, K.layer_io(workspace=ws, **kw))

    # the Reuse layer's window rows (positions 0..P-1) in a ring of L_w >= P rows
    pos0 = npy(g["swa_pos0"]).astype(np.int32)
    assert np.all(pos0 == 0)
    rows = g["swa_kv"][:, :P].contiguous()
    ring = torch.zeros(B, L_w, 512, dtype=torch.uint8, device=DEV)
    K.csa2_swa_append(rows, torch.arange(P, dtype=torch.int32, device=DEV).repeat(B, 1).contiguous(), ring)
    oring = np.zeros((B, L_w, 512), np.uint8)
    for b in range(B):
        O.swa_ring_append(oring[b], npy(rows[b]), np.arange(P))
    outs = {}
    for fmt in (K.SWA_FP8_RING, K.SWA_DENSE):
        cfg = K.layer_cfg(K.REUSE, cd, m=m, k=k, W=W, H_I=H_I, H=H, swa_fmt=fmt)
        swa = ring if fmt == K.SWA_FP8_RING else _dense_from_ring(oring, [0] * B, L_w, dtype)
        o = torch.empty_like(g["q"])
        kw = dict(B=B, T=P, q_pos=g["q_pos"], q=g["q"], swa_kv=swa, swa_pos0=g["swa_pos0"], o=o, N_cap=N_cap)
        need = K.layer_workspace_bytes(cfg, K.layer_io(**kw))
        if fmt == K.SWA_FP8_RING and dtype == torch.float32:   # widened into a dense window first
            assert need >= B * L_w * 512 * 4
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)
        K.csa2_layer_forward(rt, cfg, K.layer_io(workspace=ws, **kw))
        outs[fmt] = o
    torch.cuda.synchronize()
    assert np.array_equal(ring.cpu().numpy(), oring)
    _ring_vs_dense(outs[K.SWA_FP8_RING], outs[K.SWA_DENSE], exact=dtype == torch.float32)

    def cpu(t):
        return npy(t)
    ort = O.Runtime()
    ocfg = O.LayerConfig(O.FULL, m=m, k=k, W=W, w_kv=cpu(f["w_kv"]), w_gate=cpu(f["w_gate"]), gamma=cpu(f["gamma"]),
                         w_ik=cpu(f["w_ik"]))
    O.layer_forward(ort, ocfg, O.LayerInputs(q=cpu(f["q"]), swa_kv=cpu(f["swa_kv"]), q_pos=cpu(f["q_pos"]),
                                             swa_pos0=cpu(f["swa_pos0"]), q_idx=cpu(f["q_idx"]), w=cpu(f["w"]),
                                             x=cpu(f["x"])))
    # the GPU's selection may differ from the oracle's only where scores tie
    # within the band; the Reuse layer attends the GPU's own selection
    ort.topk_idxs = tk.cpu().numpy().astype(np.int64)
    win = np.stack([O.swa_ring_rows(oring[b], 0, L_w - 1) for b in range(B)])
    ref = O.layer_forward(ort, O.LayerConfig(O.REUSE, m=m, k=k, W=W),
                          O.LayerInputs(q=cpu(g["q"]), swa_kv=win, q_pos=cpu(g["q_pos"]), swa_pos0=pos0))
    err = row_rel_err(npy(outs[K.SWA_FP8_RING]), ref)
    say(f"  row rel err {err:.2e}")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("kv_fp4,H", [(False, 64), (True, 16)])
def test_ring_attention_window_only(kv_fp4, H):
    """k = 0 with the window in a ring, on the decode kernel that reads the ring
    itself: the selected-row split has no rows (an empty partial the merge must
    ignore) and the window rows come from the FP8 splits; compared with the
    oracle's window-only attention and with the same call over a dense copy."""
    dtype, B, W, L_w, N_cap = torch.bfloat16, 3, 128, 160, 40
    last = [300, 140, 60]
    n_pre = [250, 100, 30]
    say(f"case: ring attention window only k=0 fp4kv={kv_fp4} H={H}")
    rows = window_rows(B, max(last) + 1, 29, dtype, with_specials=False)
    ring, oring = _ring_for(rows, n_pre, last, L_w, dtype)
    q = synth.gaussian((B, 1, H, 512), 1.0, 29, "q", 0, dtype, DEV)
    kvf = synth.gaussian((B, N_cap, 512), 1.0, 29, "kv_cache", 0, torch.float32, DEV)
    if kv_fp4:
        kv = torch.empty(B, N_cap, 256, dtype=torch.uint8, device=DEV)
        kv_scales = torch.empty(B, N_cap, 32, dtype=torch.uint8, device=DEV)
        K.csa2_kv_fp4_pack(kvf.contiguous(), kv, kv_scales)
    else:
        kv, kv_scales = kvf.to(dtype), None
    tk = torch.full((B, 1, 1), 3, dtype=torch.int32, device=DEV)   # never read with k = 0
    q_pos = torch.tensor(last, dtype=torch.int32, device=DEV)[:, None].contiguous()
    swa_pos0 = torch.zeros(B, dtype=torch.int32, device=DEV)
    o_ring = torch.empty_like(q)
    lse_ring = torch.empty(B, 1, H, dtype=torch.float32, device=DEV)
    K.csa2_sparse_attn(None, q, kv, tk, ring, swa_pos0, q_pos, o_ring, W=W, k=0, lse=lse_ring, kv_scales=kv_scales)
    pos0 = [max(0, last[b] - L_w + 1) for b in range(B)]
    dense = _dense_from_ring(oring, pos0, L_w, dtype)
    o_dense = torch.empty_like(q)
    lse_dense = torch.empty_like(lse_ring)
    K.csa2_sparse_attn(None, q, kv, tk, dense, torch.tensor(pos0, dtype=torch.int32, device=DEV), q_pos, o_dense,
                       W=W, k=0, lse=lse_dense, kv_scales=kv_scales)
    torch.cuda.synchronize()
    _ring_vs_dense(o_ring, o_dense, lse_ring, lse_dense, exact=kv_fp4)
    og, lg, qn = npy(o_ring), lse_ring.cpu().numpy(), npy(q)
    worst = 0.0
    for b in range(B):
        win = O.swa_ring_rows(oring[b], pos0[b], last[b])
        ref, _, used = O.sparse_attention(qn[b, 0], np.zeros((0, 512)), np.zeros(0, np.int64), win, pos0[b],
                                          last[b], W)
        worst = max(worst, row_rel_err(og[b, 0], ref))
        assert np.allclose(lg[b, 0], O.attention_lse(qn[b, 0], used), rtol=1e-4, atol=1e-3), b
    say(f"  worst row rel err {worst:.2e}")
    assert worst <= TOL[dtype]
