"""The no-alloc score/top-k entry point (csa2_score_topk_noalloc, fixed device
scratch inside the library) against csa2_score_topk with a caller workspace, on
calls in a row through the C ABI, each with a smaller input than the one before:
a flat scan, then an HSI pool build with the merge pre-filter (which use more of
the scratch's regions), then a flat scan over UE8M0-scaled index K: top-k ids
and pool blocks must be bit-identical.  Also: a call too large for the scratch is
refused before anything is enqueued."""
import ctypes as C

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from compressed_sparse_attention_compress_amd import csa2 as K

DEV = "cuda"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _inputs(B, N, seed, H_I=32, ue8m0=False):
    codes = torch.empty(B, N, 64, dtype=torch.uint8, device=DEV)
    scales = torch.empty(B, N, 4, dtype=torch.uint8, device=DEV)
    for b in range(B):
        u = synth.cache_rows(N, 128, seed, "u", b, DEV)
        if ue8m0:   # UE8M0 block scales, packed by the oracle's encoder
            from oracle import csa2_oracle as O
            c, sc = O.fp4_pack(u.cpu().numpy(), 32, O.SCALE_UE8M0)
            codes[b], scales[b] = torch.from_numpy(c).to(DEV), torch.from_numpy(sc).to(DEV)
        else:
            K.csa2_fp4_pack(u, codes[b], scales[b])
    q = synth.decode_query_inputs(B, 8, H_I, 8, seed=seed, dtype=torch.bfloat16, device=DEV)
    return codes, scales, q["q_idx"], q["w"]


def test_noalloc_matches_workspace_entry_on_two_calls():
    m, k = 2, 512
    sf_ue = K.SCALE_UE8M0
    calls = [dict(B=16, N=65536, hsi=K.HSI_NONE, s=0, nb=0, seed=81, sf=K.SCALE_E4M3),
             dict(B=4, N=100000, hsi=K.HSI_BUILD, s=64, nb=32, seed=82, sf=K.SCALE_E4M3),
             dict(B=2, N=30000, hsi=K.HSI_NONE, s=0, nb=0, seed=83, sf=sf_ue)]
    refs, outs = [], []
    data = []
    for c in calls:
        codes, scales, q_idx, w = _inputs(c["B"], c["N"], c["seed"], ue8m0=c["sf"] == sf_ue)
        q_pos = torch.full((c["B"], 1), c["N"] * m - 1 - 3, dtype=torch.int32, device=DEV)
        data.append((codes, scales, q_idx, w, q_pos))
    # reference: the workspace entry point
    for c, (codes, scales, q_idx, w, q_pos) in zip(calls, data):
        tk = torch.full((c["B"], 1, k), -7, dtype=torch.int32, device=DEV)
        cand = torch.full((c["B"], 1, max(c["nb"], 1)), -7, dtype=torch.int32, device=DEV)
        K.csa2_score_topk(None, q_idx, w, codes, scales, q_pos, tk, n_entries=c["N"], m=m, k=k, hsi=c["hsi"],
                          hsi_s=c["s"], hsi_nb=c["nb"], candidates=cand if c["hsi"] else None, scale_fmt=c["sf"])
        refs.append((tk, cand))
    # the no-alloc entry point: two calls in a row, the second smaller
    for c, (codes, scales, q_idx, w, q_pos) in zip(calls, data):
        tk = torch.full((c["B"], 1, k), -5, dtype=torch.int32, device=DEV)
        cand = torch.full((c["B"], 1, max(c["nb"], 1)), -5, dtype=torch.int32, device=DEV)
        K.csa2_score_topk_noalloc(None, q_idx, w, codes, scales, q_pos, tk, n_entries=c["N"], m=m, k=k,
                                  hsi=c["hsi"], hsi_s=c["s"], hsi_nb=c["nb"], candidates=cand if c["hsi"] else None,
                                  scale_fmt=c["sf"])
        outs.append((tk, cand))
    torch.cuda.synchronize()
    for i, c in enumerate(calls):
        print(f"call {i}: B={c['B']} N={c['N']} hsi={c['hsi']}", flush=True)
        assert torch.equal(outs[i][0], refs[i][0]), f"call {i}: top-k ids differ"
        assert bool((refs[i][0] >= 0).all()), f"call {i}: the reference selected fewer than k"
        if c["hsi"]:
            assert torch.equal(outs[i][1], refs[i][1]), f"call {i}: pool blocks differ"


def test_noalloc_refuses_oversized_calls_and_workspaces():
    # 512 queries over 8192 entries need a 16 MiB key matrix + 256 B: one byte too many
    a = K.ScoreTopkArgs(dtype=1, B=1, T=512, H_I=32, N_cap=8192, n_entries=8192, m=1, k=512, q_idx=0x1000,
                        w=0x1000, codes=0x1000, scales=0x1000, q_pos=0x1000, topk=0x1000)
    assert K.STATUS[K.lib().csa2_score_topk_noalloc(None, C.byref(a), None)] == "CSA2_ERR_WORKSPACE"
    assert b"scratch" in K.lib().csa2_last_error()
    a.T, a.workspace, a.workspace_bytes = 1, 0x1000, 1 << 20
    assert K.STATUS[K.lib().csa2_score_topk_noalloc(None, C.byref(a), None)] == "CSA2_ERR_INVALID_ARG"
