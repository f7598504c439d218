"""The benchmark's steps captured as a HIP graph (stream capture of the C-ABI
calls) and replayed: every replay must reproduce the eager result bit for bit.
Between replays the outputs are overwritten by eager kernels and the device is
synchronised, so a replay that skipped or reused work would show."""
from __future__ import annotations

import pytest
import torch

import synth
from parity_utils import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    from compressed_sparse_attention_compress_amd import csa2 as lib
    lib.lib()
    return lib


def _replays_match(step, outputs, n_replays=3):
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(n_replays):
        for t in outputs:
            if t.dtype.is_floating_point:
                t.fill_(float("nan"))
            else:
                t.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for j, (a, b) in enumerate(zip(outputs, ref)):
            assert torch.equal(a, b), f"replay {rep}: output {j} differs from the eager step"
    del g


def test_decode_step_graph_replay(K):
    import bench
    say("case: decode step (score/top-k + two attention calls) as a HIP graph, 8 x 16384 entries")
    db = bench.DecodeBench(torch, K, synth, B=8, n_entries=16384)
    _replays_match(db.step, [db.topk, db.o[0], db.o[1]])


def test_prefill_step_graph_replay(K):
    import bench
    say("case: prefill step (compress, index K, score/top-k, attention) as a HIP graph, L=1024, hidden 512")
    pb = bench.PrefillBench(torch, K, synth, L=1024, D=512)
    _replays_match(pb.step, [pb.lat, pb.kv, pb.codes, pb.scales, pb.topk, pb.o])


def test_hsi_decode_step_graph_replay(K):
    import bench
    say("case: HSI decode step (Full scan + pool build with the merge pre-filter, pool scan, two attention calls) "
        "as a HIP graph, 4 x 131072 entries")
    hb = bench.HsiDecodeBench(torch, K, synth, B=4, n_entries=131072, copies=1)
    _replays_match(hb.step, [hb.tk[0], hb.tk[1], hb.cand, hb.o[0], hb.o[1]])
