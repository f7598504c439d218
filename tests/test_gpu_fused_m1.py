"""A Full layer with m = 1, bf16 operands and a bf16 cache makes its cache rows,
pre-RoPE latent and index K in one kernel when it runs through
csa2_layer_forward.  Those outputs must equal, bit for bit, what csa2_compress
followed by csa2_index_k write (the two-call path, pinned to the oracle by the
kernel and full-size tests), for both index-K scale formats, token counts that
are not a multiple of the 128-token workgroup tile, several sequences and a
nonzero start position; the slots must advertise the same entry counts."""
import pytest
import torch

from parity_utils import say
import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from compressed_sparse_attention_compress_amd import csa2 as K

DEV = "cuda"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("B,T_x,D,start,extra,sfmt", [
    (2, 300, 256, 0, 0, 0),
    (1, 1000, 512, 40, 60, 1),
    (1, 128, 4096, 0, 0, 0),
    (3, 77, 256, 5, 3, 1),
    (1, 1, 64, 0, 0, 0),       # one token, one 64-wide k-step
    (2, 129, 64, 7, 0, 1),     # a second tile holding a single token
])
def test_fused_full_layer_equals_two_calls(B, T_x, D, start, extra, sfmt):
    say(f"case: fused m=1 Full layer B={B} T_x={T_x} D={D} start={start} scale_fmt={sfmt}")
    bf = torch.bfloat16
    H, H_I, k, W = 16, 4, 16, 8
    R = min(8, T_x)
    N_cap = start + T_x + extra
    x = synth.gaussian((B, T_x, D), 1.0, 61, "x", 0, bf, DEV)
    w_kv = synth.linear_weight(512, D, 61, "w_kv", 0, bf, DEV)
    w_ik = synth.linear_weight(128, 512, 61, "w_ik", 0, bf, DEV)
    gamma = (0.5 + torch.rand(512, generator=torch.Generator().manual_seed(61))).float().to(DEV)

    def bufs():
        return (torch.full((B, T_x, 512), float("nan"), dtype=torch.float32, device=DEV),
                torch.zeros(B, N_cap, 512, dtype=bf, device=DEV),
                torch.zeros(B, N_cap, 64, dtype=torch.uint8, device=DEV),
                torch.zeros(B, N_cap, 4, dtype=torch.uint8, device=DEV))

    # two calls
    lat2, kv2, c2, s2 = bufs()
    K.csa2_compress(None, x, w_kv, None, gamma, lat2, kv2, m=1, start_pos=start)
    K.csa2_index_k(None, lat2, w_ik, c2, s2, m=1, entry0=start, scale_fmt=sfmt)

    # one layer call (its queries: the last R positions)
    lat1, kv1, c1, s1 = bufs()
    q = synth.gaussian((B, R, H, 512), 1.0, 61, "q", 0, bf, DEV)
    swa = synth.gaussian((B, R, 512), 1.0, 61, "swa_kv", 0, bf, DEV)
    q_idx = synth.gaussian((B, R, H_I, 128), 1.0, 61, "q_idx", 0, bf, DEV)
    w = synth.gaussian((B, R, H_I), 1.0, 61, "w", 0, torch.float32, DEV)
    p_last = start + T_x - 1
    q_pos = torch.arange(p_last - R + 1, p_last + 1, dtype=torch.int32, device=DEV).repeat(B, 1).contiguous()
    pos0 = torch.full((B,), p_last - R + 1, dtype=torch.int32, device=DEV)
    o = torch.empty_like(q)
    topk = torch.empty(B, R, k, dtype=torch.int32, device=DEV)
    cfg = K.layer_cfg(K.FULL, K.CSA2_BF16, m=1, k=k, W=W, H_I=H_I, H=H, scale_fmt=sfmt)
    kw = dict(B=B, T=R, q_pos=q_pos, q=q, swa_kv=swa, swa_pos0=pos0, o=o, N_cap=N_cap, D=D, start_pos=start, x=x,
              w_kv=w_kv, w_gate=None, gamma=gamma, w_ik=w_ik, latent_pre=lat1, kv_cache=kv1, ik_codes=c1,
              ik_scales=s1, q_idx=q_idx, w=w, topk=topk, T_x=T_x)
    ws = torch.empty(max(K.layer_workspace_bytes(cfg, K.layer_io(**kw)), 16), dtype=torch.uint8, device=DEV)
    rt = K.Runtime()
    K.csa2_layer_forward(rt, cfg, K.layer_io(workspace=ws, **kw))
    torch.cuda.synchronize()

    assert not torch.isnan(lat1).any()
    assert torch.equal(lat1, lat2), "pre-RoPE latent differs"
    assert torch.equal(kv1, kv2), "cache rows differ"
    assert torch.equal(c1, c2), "index-K codes differ"
    assert torch.equal(s1, s2), "index-K scales differ"
    # untouched rows outside [start, start + T_x) stay zero in both
    assert not kv1[:, :start].any() and not kv1[:, start + T_x:].any()
    assert not c1[:, start + T_x:].any() and not s1[:, start + T_x:].any()
    assert rt.slot(K.SLOT_COMPRESS_KV).cols == start + T_x
    assert rt.slot(K.SLOT_INDEX_K).cols == start + T_x
