"""GPU parity of the decode append path (csa2_compress_step): a prefill with
csa2_compress + csa2_index_k, then one token per sequence and step, must leave
the cache rows and index-K rows the whole-sequence oracle computes (the step's
partial-group state carries a group's earlier tokens).  One sequence lags one
step behind (its first step has no token, pos = -1), so sequences sit at
different positions inside their groups."""
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


@pytest.mark.parametrize("dtype,m,sfmt", [(torch.bfloat16, 2, "e4m3"), (torch.bfloat16, 1, "e4m3"),
                                          (torch.bfloat16, 4, "e4m3"), (torch.float32, 2, "e4m3"),
                                          (torch.bfloat16, 2, "ue8m0"), (torch.float32, 1, "ue8m0")])
def test_compress_step_continues_the_prefill(dtype, m, sfmt):
    """sfmt: scale format of the index-K rows (the prefill's and the steps')."""
    B, D = 3, (512 if dtype == torch.bfloat16 else 256)
    P, S = 8 * m, 6 * m + 1                 # prefill tokens, then S append steps
    L = P + S
    gfmt = K.SCALE_UE8M0 if sfmt == O.SCALE_UE8M0 else K.SCALE_E4M3
    say(f"case: compress_step dtype={dtype} m={m} B={B} D={D} prefill {P} + {S} steps, index-K scales {sfmt}")
    x = synth.gaussian((B, L, D), 1.0, 61, "x", 0, dtype, DEV)
    w_kv = synth.linear_weight(512, D, 61, "w_kv", 0, dtype, DEV)
    w_gate = synth.linear_weight(512, D, 61, "w_gate", 0, dtype, DEV) if m > 1 else None
    w_ik = synth.linear_weight(128, 512, 61, "w_ik", 0, dtype, DEV)
    gamma = (1.0 + 0.1 * synth.gaussian((512,), 1.0, 61, "w", 0, torch.float32, DEV)).contiguous()
    N_cap = L // m + 2
    kv = torch.zeros(B, N_cap, 512, dtype=dtype, device=DEV)
    codes = torch.zeros(B, N_cap, 64, dtype=torch.uint8, device=DEV)
    scales = torch.zeros(B, N_cap, 4, dtype=torch.uint8, device=DEV)
    lat = torch.empty(B, P // m, 512, dtype=torch.float32, device=DEV)
    K.csa2_compress(None, x[:, :P].contiguous(), w_kv, w_gate, gamma, lat, kv, m=m, start_pos=0)
    K.csa2_index_k(None, lat, w_ik, codes, scales, m=m, scale_fmt=gfmt)
    state = torch.full((B, 3, 512), float("nan"), dtype=torch.float32, device=DEV) if m > 1 else None
    lat_step = torch.zeros(B, 512, dtype=torch.float32, device=DEV)
    ws = None
    done = [P - 1] * B                        # last position folded in, per sequence
    for s in range(S):
        t = P + s
        pos = [t, t, t - 1 if s > 0 else -1]   # sequence 2 lags one step
        xs = torch.stack([x[b, max(pos[b], 0)] for b in range(B)]).contiguous()
        ws = K.csa2_compress_step(None, xs, torch.tensor(pos, dtype=torch.int32, device=DEV), w_kv, w_gate, gamma,
                                  w_ik, state, kv, codes, scales, m=m, latent_pre=lat_step, workspace=ws,
                                  scale_fmt=gfmt)
        for b in range(B):
            if pos[b] >= 0:
                done[b] = pos[b]
    torch.cuda.synchronize()
    kvg, cg, sg = npy(kv), codes.cpu().numpy(), scales.cpu().numpy()
    worst = 0.0
    for b in range(B):
        n_done = (done[b] + 1) // m           # complete groups
        lp, kvo, ids = O.compress(npy(x[b, :n_done * m]), npy(w_kv), None if w_gate is None else npy(w_gate),
                                  npy(gamma), m, 0)
        u, _, _ = O.index_k(lp, npy(w_ik), ids * m)
        g0 = P // m                            # rows written by the steps
        worst = max(worst, row_rel_err(kvg[b, g0:n_done], kvo[g0:]))
        check_fp4(u[:g0], cg[b, :g0], sg[b, :g0], f"prefill b{b}", scale_fmt=sfmt)
        nc, ns = check_fp4(u[g0:], cg[b, g0:n_done], sg[b, g0:n_done], f"step b{b}", scale_fmt=sfmt)
        assert np.all(kvg[b, n_done:] == 0) and np.all(cg[b, n_done:] == 0), f"b{b}: rows past the last group"
        say(f"  b{b}: {n_done - g0} appended rows, fp4 code/scale differences at rounding midpoints {nc}/{ns}")
    assert worst <= TOL[dtype], worst
    # the last completed group's latent (before RoPE) of a sequence whose last step closed a group
    for b in range(B):
        if (done[b] + 1) % m == 0 and done[b] >= P:
            lp, _, _ = O.compress(npy(x[b, :done[b] + 1]), npy(w_kv), None if w_gate is None else npy(w_gate),
                                  npy(gamma), m, 0)
            assert row_rel_err(npy(lat_step[b])[None], lp[-1:]) <= 1e-4
