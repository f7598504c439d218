#!/usr/bin/env python3
"""Benchmark of the CSA2 layer hot path on one MI355X.

Headline (the `value` of the JSON line): encoder Full-layer prefill throughput in
tokens/s -- one step = compressor + index K + score/top-k + sparse attention over
one batch (B=1, L=8192, hidden 4096, m=2, 32x128 FP4 indexer heads, top-512, window
128, 64 heads, bf16 in / fp32 accumulate).  A second record ("decode") times the
batched decode step (Reindex + Reuse over 64 sequences x 131072 m=2 entries), and
a third ("decode_hsi_1m") the 1M-context decode step with the HSI candidate pool
(4 sequences x 524288 entries), a fourth ("decode_append") the Full layer's
decode append of one token per sequence, a fifth ("decode_fp4kv") the batched
decode step with the main KV stored as FP4, and two more the decoder macro-block
prefill at L=32768, m=1 (Full, Reindex, Reuse, Reuse through csa2_layer_forward):
"decoder_block" over all positions and "decoder_replay" with only the last R
positions replayed through the decoder layers.

Every input is seeded synthetic data already resident in HBM when timing starts.
Per-kernel times come from HIP events recorded on the stream the library launches
on (torch's current stream).  The CPU oracle is timed on this host beside each
record (`cpu_baseline`): the whole prefill step unsampled for the headline; a
stated sample, extrapolated and labelled so, for the decode and decoder records;
all sequences for the decode append.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3        # fp32 (vector and MFMA)

METRIC = "CSA2 layer prefill tokens/s + decode µs/step; % HBM/MFMA roofline"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# --------------------------------------------------------------------------- C2

class PrefillBench:
    """Encoder Full-layer prefill (B=1, L=8192, D=4096, m=2)."""

    def __init__(self, torch, K, synth, L=8192, D=4096, m=2, H_I=32, k=512, W=128, H=64, B=1):
        self.t, self.K = torch, K
        self.shape = synth.LayerShape(B=B, L=L, D=D, m=m, H_I=H_I, k=k, W=W, H=H)
        s = self.shape
        dev = "cuda"
        self.inp = synth.full_layer_inputs(s, seed=0, dtype=torch.bfloat16, device=dev, layer=0,
                                           w_from_linear=True)
        self.N = L // m
        self.lat = torch.empty(B, self.N, 512, dtype=torch.float32, device=dev)
        self.kv = torch.empty(B, self.N, 512, dtype=torch.bfloat16, device=dev)
        self.codes = torch.empty(B, self.N, 64, dtype=torch.uint8, device=dev)
        self.scales = torch.empty(B, self.N, 4, dtype=torch.uint8, device=dev)
        self.topk = torch.empty(B, L, k, dtype=torch.int32, device=dev)
        self.o = torch.empty_like(self.inp["q"])
        nb = K.score_topk_workspace_bytes(q_idx=self.inp["q_idx"], w=self.inp["w"], codes=self.codes,
                                          scales=self.scales, q_pos=self.inp["q_pos"], topk=self.topk,
                                          n_entries=self.N, m=m, k=k, N_cap=self.N)
        self.ws = torch.empty(nb, dtype=torch.uint8, device=dev)
        self.ev = None

    def step(self, events=None):
        K, i, s = self.K, self.inp, self.shape
        if events is not None:
            events[0].record()
        K.csa2_compress(None, i["x"], i["w_kv"], i["w_gate"], i["gamma"], self.lat, self.kv, m=s.m)
        if events is not None:
            events[1].record()
        K.csa2_index_k(None, self.lat, i["w_ik"], self.codes, self.scales, m=s.m)
        if events is not None:
            events[2].record()
        K.csa2_score_topk(None, i["q_idx"], i["w"], self.codes, self.scales, i["q_pos"], self.topk,
                          n_entries=self.N, m=s.m, k=s.k, workspace=self.ws)
        if events is not None:
            events[3].record()
        K.csa2_sparse_attn(None, i["q"], self.kv, self.topk, i["swa_kv"], i["swa_pos0"], i["q_pos"], self.o, W=s.W)
        if events is not None:
            events[4].record()

    # algorithmic work of each stage for this workload
    def work(self):
        s = self.shape
        L, m, k, W, H = s.L, s.m, s.k, s.W, s.H
        n_t = [(t + 1) // m for t in range(L)]
        pairs = sum(n_t)
        rows = sum(min(k, n) + min(W, t + 1) for t, n in enumerate(n_t))
        g = 1 if m == 1 else 2
        return {
            "compress": {"flop": 2.0 * s.B * L * s.D * 512 * g},
            "index_k": {"flop": 2.0 * s.B * self.N * 512 * 128},
            "score_topk": {"flop": 2.0 * s.B * pairs * s.H_I * 128, "pairs": s.B * pairs},
            "sparse_attn": {"flop": 4.0 * s.B * rows * H * 512, "rows": s.B * rows},
        }


# --------------------------------------------------------------------------- C1

class TinyLayerBench:
    """Tiny Full layer, fp32 (B=1, L=512, hidden 256, m=2, 4 indexer heads, top-32,
    SWA 16, 8 heads): one csa2_layer_forward call (compressor, index K, score +
    top-k, attention); a latency figure, the oracle timed beside it."""

    def __init__(self, torch, K, synth):
        self.t, self.K = torch, K
        self.shape = s = synth.TINY
        dev = "cuda"
        self.inp = synth.full_layer_inputs(s, 0, torch.float32, dev, layer=0)
        self.N = s.L // s.m
        self.lat = torch.empty(s.B, self.N, 512, dtype=torch.float32, device=dev)
        self.kv = torch.empty(s.B, self.N, 512, dtype=torch.float32, device=dev)
        self.codes = torch.empty(s.B, self.N, 64, dtype=torch.uint8, device=dev)
        self.scales = torch.empty(s.B, self.N, 4, dtype=torch.uint8, device=dev)
        self.topk = torch.empty(s.B, s.L, s.k, dtype=torch.int32, device=dev)
        self.o = torch.empty_like(self.inp["q"])
        self.rt = K.Runtime()
        self.cfg = K.layer_cfg(K.FULL, K.CSA2_F32, m=s.m, k=s.k, W=s.W, H_I=s.H_I, H=s.H)
        i = self.inp
        self.kw = dict(B=s.B, T=s.L, q_pos=i["q_pos"], q=i["q"], swa_kv=i["swa_kv"], swa_pos0=i["swa_pos0"], o=self.o,
                       N_cap=self.N, D=s.D, x=i["x"], w_kv=i["w_kv"], w_gate=i["w_gate"], gamma=i["gamma"],
                       w_ik=i["w_ik"], latent_pre=self.lat, kv_cache=self.kv, ik_codes=self.codes,
                       ik_scales=self.scales, q_idx=i["q_idx"], w=i["w"], topk=self.topk)
        nb = K.layer_workspace_bytes(self.cfg, K.layer_io(**self.kw))
        self.ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=dev)
        self.io = K.layer_io(workspace=self.ws, **self.kw)
        torch.cuda.synchronize()

    def step(self, events=None):
        if events is not None:
            events[0].record()
        self.K.csa2_layer_forward(self.rt, self.cfg, self.io)
        if events is not None:
            events[1].record()

    def work(self):
        s = self.shape
        n_t = [(t + 1) // s.m for t in range(s.L)]
        rows = sum(min(s.k, n) + min(s.W, t + 1) for t, n in enumerate(n_t))
        return (2.0 * s.B * s.L * s.D * 512 * (1 if s.m == 1 else 2) + 2.0 * s.B * self.N * 512 * 128
                + 2.0 * s.B * sum(n_t) * s.H_I * 128 + 4.0 * s.B * rows * s.H * 512)


# --------------------------------------------------------------------------- C4

class DecodeBench:
    """Batched decode step, Reindex + Reuse: 64 sequences x 131072 m=2 entries."""

    def __init__(self, torch, K, synth, B=64, n_entries=131072, m=2, H_I=32, k=512, W=128, H=64, kv_fp4=False,
                 swa_fp8=False):
        self.t, self.K = torch, K
        dev = "cuda"
        self.B, self.N, self.m, self.H_I, self.k, self.W, self.H = B, n_entries, m, H_I, k, W, H
        self.kv_fp4, self.swa_fp8 = kv_fp4, swa_fp8
        self.seed = seed = 11   # per-sequence cache rows: synth.cache_rows(n, d, seed, name, b)
        if kv_fp4:   # FP4 main KV: N(0,1) latent rows packed by the (bit-exact) FP4 packer
            self.kv = torch.empty(B, n_entries, 256, dtype=torch.uint8, device=dev)
            self.kv_scales = torch.empty(B, n_entries, 32, dtype=torch.uint8, device=dev)
            for b in range(B):
                r = synth.cache_rows(n_entries, 512, seed, "kv_cache", b, dev)
                K.csa2_kv_fp4_pack(r, self.kv[b], self.kv_scales[b])
            del r
        else:
            self.kv = torch.empty(B, n_entries, 512, dtype=torch.bfloat16, device=dev)
            for b in range(B):
                self.kv[b] = synth.cache_rows(n_entries, 512, seed, "kv_cache", b, dev).to(torch.bfloat16)
            self.kv_scales = None
        self.codes = torch.empty(B, n_entries, 64, dtype=torch.uint8, device=dev)
        self.scales = torch.empty(B, n_entries, 4, dtype=torch.uint8, device=dev)
        for b in range(B):  # index K: N(0,1) rows packed by the (bit-exact) FP4 packer
            u = synth.cache_rows(n_entries, 128, seed, "u", b, dev)
            K.csa2_fp4_pack(u, self.codes[b], self.scales[b])
        del u
        p = n_entries * m - 1  # newest token; all entries visible
        self.q_pos = torch.full((B, 1), p, dtype=torch.int32, device=dev)
        self.swa_pos0 = torch.full((B,), p - W + 1, dtype=torch.int32, device=dev)
        self.layers = [synth.decode_query_inputs(B, H, H_I, W, seed=0, layer=l, dtype=torch.bfloat16, device=dev)
                       for l in range(2)]
        self.topk = torch.empty(B, 1, k, dtype=torch.int32, device=dev)
        self.o = [torch.empty_like(self.layers[l]["q"]) for l in range(2)]
        self.win = [self.layers[l]["swa_kv"] for l in range(2)]
        if swa_fp8:
            # each layer's window KV in an FP8 ring of W rows holding positions p-W+1..p;
            # every step re-appends the newest token's row (what a decode step writes)
            wpos = torch.arange(p - W + 1, p + 1, dtype=torch.int32, device=dev).repeat(B, 1).contiguous()
            self.win = []
            self.new_rows = []
            for l in range(2):
                ring = torch.zeros(B, W, 512, dtype=torch.uint8, device=dev)
                K.csa2_swa_append(self.layers[l]["swa_kv"], wpos, ring)
                self.win.append(ring)
                self.new_rows.append(self.layers[l]["swa_kv"][:, W - 1:].contiguous())
        nb = K.score_topk_workspace_bytes(q_idx=self.layers[0]["q_idx"], w=self.layers[0]["w"], codes=self.codes,
                                          scales=self.scales, q_pos=self.q_pos, topk=self.topk, n_entries=n_entries,
                                          m=m, k=k, N_cap=n_entries)
        self.ws = torch.empty(nb, dtype=torch.uint8, device=dev)
        na = K.sparse_attn_workspace_bytes(self.layers[0]["q"], k, W, kv_fp4, n_entries, swa_fp8, W)
        self.ws_attn = torch.empty(max(na, 16), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()

    def step(self, events=None):
        K = self.K
        r, u = self.layers
        if events is not None:
            events[0].record()
        K.csa2_score_topk(None, r["q_idx"], r["w"], self.codes, self.scales, self.q_pos, self.topk,
                          n_entries=self.N, m=self.m, k=self.k, workspace=self.ws)
        if events is not None:
            events[1].record()
        if self.swa_fp8:
            K.csa2_swa_append(self.new_rows[0], self.q_pos, self.win[0])
        K.csa2_sparse_attn(None, r["q"], self.kv, self.topk, self.win[0], self.swa_pos0, self.q_pos, self.o[0],
                           W=self.W, workspace=self.ws_attn, kv_scales=self.kv_scales)
        if events is not None:
            events[2].record()
        if self.swa_fp8:
            K.csa2_swa_append(self.new_rows[1], self.q_pos, self.win[1])
        K.csa2_sparse_attn(None, u["q"], self.kv, self.topk, self.win[1], self.swa_pos0, self.q_pos, self.o[1],
                           W=self.W, workspace=self.ws_attn, kv_scales=self.kv_scales)
        if events is not None:
            events[3].record()

    def work(self):
        B, N = self.B, self.N
        rows = B * (min(self.k, N) + self.W)
        sel_row_bytes = 288.0 if self.kv_fp4 else 1024.0     # FP4 main KV row, or bf16 row
        win_row_bytes = 512.0 if self.swa_fp8 else 1024.0     # FP8 ring row, or bf16 row
        append_bytes = B * (1024.0 + 512.0) if self.swa_fp8 else 0.0   # newest row read, ring slot written
        return {
            "score_topk": {"bytes": 68.0 * B * N + B * self.H_I * (128 * 2 + 4) + B * self.k * 4,
                           "flop": 2.0 * B * N * self.H_I * 128},
            "sparse_attn": {"bytes": B * min(self.k, N) * sel_row_bytes + B * self.W * win_row_bytes
                            + 2.0 * B * self.H * 512 * 2 + append_bytes,
                            "flop": 4.0 * rows * self.H * 512},
        }


# --------------------------------------------------------------------------- C5

class HsiDecodeBench:
    """1M-context decode with the HSI candidate pool: 4 sequences x 524288 m=2
    entries.  The Full layer scores every entry, keeps its top-512 and the block
    maxima (s=64) and picks the 256 best blocks (newest forced); the Reindex layer
    scores the 16384-entry pool only; both attend.  The 142.6 MB of index K would
    sit in the 256 MB MALL if one copy were re-read every step, so the steps rotate
    over three copies (428 MB) and every scan comes from HBM."""

    def __init__(self, torch, K, synth, B=4, n_entries=524288, m=2, H_I=32, k=512, W=128, H=64, s_blk=64, n_b=256,
                 copies=3):
        self.t, self.K = torch, K
        dev = "cuda"
        self.B, self.N, self.m, self.H_I, self.k, self.W, self.H = B, n_entries, m, H_I, k, W, H
        self.s_blk, self.n_b, self.copies = s_blk, n_b, copies
        self.seed = seed = 12
        self.kv = torch.empty(B, n_entries, 512, dtype=torch.bfloat16, device=dev)
        codes = torch.empty(B, n_entries, 64, dtype=torch.uint8, device=dev)
        scales = torch.empty(B, n_entries, 4, dtype=torch.uint8, device=dev)
        for b in range(B):
            self.kv[b] = synth.cache_rows(n_entries, 512, seed, "kv_cache", b, dev).to(torch.bfloat16)
            u = synth.cache_rows(n_entries, 128, seed, "u", b, dev)
            K.csa2_fp4_pack(u, codes[b], scales[b])
        del u
        self.ik = [(codes, scales)] + [(codes.clone(), scales.clone()) for _ in range(copies - 1)]
        p = n_entries * m - 1
        self.q_pos = torch.full((B, 1), p, dtype=torch.int32, device=dev)
        self.swa_pos0 = torch.full((B,), p - W + 1, dtype=torch.int32, device=dev)
        self.layers = [synth.decode_query_inputs(B, H, H_I, W, seed=5, layer=l, dtype=torch.bfloat16, device=dev)
                       for l in range(2)]
        self.tk = [torch.empty(B, 1, k, dtype=torch.int32, device=dev) for _ in range(2)]
        self.cand = torch.empty(B, 1, n_b, dtype=torch.int32, device=dev)
        self.o = [torch.empty_like(self.layers[l]["q"]) for l in range(2)]
        common = dict(codes=codes, scales=scales, q_pos=self.q_pos, n_entries=n_entries, m=m, k=k, N_cap=n_entries,
                      hsi_s=s_blk, hsi_nb=n_b, candidates=self.cand)
        nb = max(K.score_topk_workspace_bytes(q_idx=self.layers[l]["q_idx"], w=self.layers[l]["w"], topk=self.tk[l],
                                              hsi=(K.HSI_BUILD, K.HSI_USE)[l], **common) for l in range(2))
        self.ws = torch.empty(nb, dtype=torch.uint8, device=dev)
        na = K.sparse_attn_workspace_bytes(self.layers[0]["q"], k, W)
        self.ws_attn = torch.empty(max(na, 16), dtype=torch.uint8, device=dev)
        self.rep = 0
        torch.cuda.synchronize()

    def step(self, events=None):
        K = self.K
        f, r = self.layers
        codes, scales = self.ik[self.rep]
        self.rep = (self.rep + 1) % self.copies
        kw = dict(q_pos=self.q_pos, n_entries=self.N, m=self.m, k=self.k, hsi_s=self.s_blk, hsi_nb=self.n_b,
                  candidates=self.cand, workspace=self.ws)
        if events is not None:
            events[0].record()
        K.csa2_score_topk(None, f["q_idx"], f["w"], codes, scales, topk=self.tk[0], hsi=K.HSI_BUILD, **kw)
        if events is not None:
            events[1].record()
        K.csa2_score_topk(None, r["q_idx"], r["w"], codes, scales, topk=self.tk[1], hsi=K.HSI_USE, **kw)
        if events is not None:
            events[2].record()
        for l, lay in enumerate((f, r)):
            K.csa2_sparse_attn(None, lay["q"], self.kv, self.tk[l], lay["swa_kv"], self.swa_pos0, self.q_pos,
                               self.o[l], W=self.W, workspace=self.ws_attn)
        if events is not None:
            events[3].record()

    def work(self):
        B, N = self.B, self.N
        pool = self.n_b * self.s_blk
        rows = B * (self.k + self.W)
        q_bytes = B * self.H_I * (128 * 2 + 4)
        return {
            "score_full": {"bytes": 68.0 * B * N + q_bytes + B * (self.k + self.n_b) * 4},
            "score_pool": {"bytes": 68.0 * B * pool + q_bytes + B * (self.n_b + self.k) * 4},
            "attn_2_layers": {"bytes": 2 * (rows * 1024.0 + 2.0 * B * self.H * 512 * 2)},
        }


# --------------------------------------------------------------------------- C3

class DecoderBench:
    """Decoder macro-block prefill: one Full layer at m=1 compresses the encoder
    output H20 of all L prompt tokens into the shared global KV and index K, then
    the block's four layers (Full, Reindex, Reuse, Reuse) run through
    csa2_layer_forward for the last R prompt positions, each layer with its own
    queries and its window KV of the replayed positions.  R = L is the full
    decoder prefill; R < L is the bounded replay (only the prompt's tail passes
    through the decoder layers, their windows limited to that tail)."""

    def __init__(self, torch, K, synth, L=32768, R=None, D=4096, H_I=32, k=512, W=128, H=64, seed=31):
        self.t, self.K = torch, K
        dev = "cuda"
        R = L if R is None else R
        self.L, self.R, self.D, self.H_I, self.k, self.W, self.H = L, R, D, H_I, k, W, H
        self.modes = [K.FULL, K.REINDEX, K.REUSE, K.REUSE]
        bf = torch.bfloat16
        self.seed = seed
        self.x = synth.gaussian((1, L, D), 1.0, seed, "x", 0, bf, dev)
        self.w_kv = synth.linear_weight(512, D, seed, "w_kv", 0, bf, dev)
        self.w_ik = synth.linear_weight(128, 512, seed, "w_ik", 0, bf, dev)
        self.gamma = torch.ones(512, dtype=torch.float32, device=dev)
        self.q_pos = torch.arange(L - R, L, dtype=torch.int32, device=dev)[None].contiguous()
        self.swa_pos0 = torch.full((1,), L - R, dtype=torch.int32, device=dev)
        self.layers = []
        for l in range(4):
            lay = {"q": synth.gaussian((1, R, H, 512), 1.0, seed, "q", l, bf, dev),
                   "swa_kv": synth.gaussian((1, R, 512), 1.0, seed, "swa_kv", l, bf, dev),
                   "o": torch.empty(1, R, H, 512, dtype=bf, device=dev)}
            if self.modes[l] != K.REUSE:
                lay["q_idx"] = synth.gaussian((1, R, H_I, 128), 1.0, seed, "q_idx", l, bf, dev)
                lay["w"] = synth.gaussian((1, R, H_I), 1.0, seed, "w", l, torch.float32, dev)
                lay["topk"] = torch.empty(1, R, k, dtype=torch.int32, device=dev)
            self.layers.append(lay)
        self.lat = torch.empty(1, L, 512, dtype=torch.float32, device=dev)
        self.kv = torch.empty(1, L, 512, dtype=bf, device=dev)
        self.codes = torch.empty(1, L, 64, dtype=torch.uint8, device=dev)
        self.scales = torch.empty(1, L, 4, dtype=torch.uint8, device=dev)
        self.rt = K.Runtime()
        self.cfgs = [K.layer_cfg(mde, K.CSA2_BF16, m=1, k=k, W=W, H_I=H_I, H=H) for mde in self.modes]
        need = max(K.layer_workspace_bytes(c, self._io(l)) for l, c in enumerate(self.cfgs))
        self.ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()

    def _io(self, l, ws=None):
        K, lay = self.K, self.layers[l]
        kw = dict(B=1, T=self.R, q_pos=self.q_pos, q=lay["q"], swa_kv=lay["swa_kv"], swa_pos0=self.swa_pos0,
                  o=lay["o"], N_cap=self.L, workspace=ws)
        if self.modes[l] == K.FULL:
            kw.update(D=self.D, x=self.x, w_kv=self.w_kv, w_gate=None, gamma=self.gamma, w_ik=self.w_ik,
                      latent_pre=self.lat, kv_cache=self.kv, ik_codes=self.codes, ik_scales=self.scales,
                      T_x=self.L)
        if self.modes[l] != K.REUSE:
            kw.update(q_idx=lay["q_idx"], w=lay["w"], topk=lay["topk"])
        return K.layer_io(**kw)

    def step(self, events=None):
        for l, cfg in enumerate(self.cfgs):
            if events is not None:
                events[l].record()
            self.K.csa2_layer_forward(self.rt, cfg, self._io(l, self.ws))
        if events is not None:
            events[4].record()

    def compress_only(self):
        self.K.csa2_compress(None, self.x, self.w_kv, None, self.gamma, self.lat, self.kv, m=1)

    def work(self):
        L, R, k, W, H = self.L, self.R, self.k, self.W, self.H
        pos = range(L - R, L)
        pairs = sum(p + 1 for p in pos)                       # m = 1: entry g visible at p >= g
        rows = sum(min(k, p + 1) + min(W, p - (L - R) + 1) for p in pos)
        return {"compress_flop": 2.0 * L * self.D * 512, "index_k_flop": 2.0 * L * 512 * 128,
                "score_flop_per_layer": 2.0 * pairs * self.H_I * 128, "attn_flop_per_layer": 4.0 * rows * H * 512,
                "flop": 2.0 * L * self.D * 512 + 2.0 * L * 512 * 128 + 2 * 2.0 * pairs * self.H_I * 128
                        + 4 * 4.0 * rows * H * 512}


# ------------------------------------------------------------ decode append

class AppendBench:
    """Full-layer decode append: one new token per sequence per step for 64
    sequences (hidden 4096, m=2).  A step pair covers both kinds of step: the
    group's first token (C and Z, then the running pool), and its last (C and Z,
    pool, norm, RoPE, cache row, index-K row)."""

    def __init__(self, torch, K, synth, B=64, D=4096, m=2, N_cap=131072):
        self.t, self.K = torch, K
        dev = "cuda"
        self.B, self.D, self.m = B, D, m
        bf = torch.bfloat16
        self.x = [synth.gaussian((B, D), 1.0, 71, "x", l, bf, dev) for l in range(m)]
        self.w_kv = synth.linear_weight(512, D, 71, "w_kv", 0, bf, dev)
        self.w_gate = synth.linear_weight(512, D, 71, "w_gate", 0, bf, dev)
        self.w_ik = synth.linear_weight(128, 512, 71, "w_ik", 0, bf, dev)
        self.gamma = torch.ones(512, dtype=torch.float32, device=dev)
        self.state = torch.zeros(B, 3, 512, dtype=torch.float32, device=dev)
        self.kv = torch.zeros(B, N_cap, 512, dtype=bf, device=dev)
        self.codes = torch.zeros(B, N_cap, 64, dtype=torch.uint8, device=dev)
        self.scales = torch.zeros(B, N_cap, 4, dtype=torch.uint8, device=dev)
        p0 = 2 * (N_cap // 2) - 2 * m
        self.pos = [torch.full((B,), p0 + i, dtype=torch.int32, device=dev) for i in range(m)]
        self.ws = torch.empty(B * 1024 * 4 * 4, dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()

    def step(self, events=None):
        K = self.K
        for i in range(self.m):
            if events is not None:
                events[i].record()
            K.csa2_compress_step(None, self.x[i], self.pos[i], self.w_kv, self.w_gate, self.gamma, self.w_ik,
                                 self.state, self.kv, self.codes, self.scales, m=self.m, workspace=self.ws)
        if events is not None:
            events[self.m].record()

    def bytes_per_step(self):
        B, D = self.B, self.D
        w = 2 * 512 * D * 2 + 128 * 512 * 2                    # W_kv, W_gate, W_ik (bf16)
        return w + B * D * 2 + B * 3 * 512 * 4 * 2 + B * 1024 * 4 * 4 * 2   # x, state in/out, C/Z partials


def time_steps(torch, bench, n_stages, steps, warmup):
    for _ in range(warmup):
        bench.step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_stages + 1)] for _ in range(steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        bench.step(evs[i])
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    per_stage = [sum(evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(steps)) / steps for j in range(n_stages)]
    return total_ms / steps, per_stage


def time_graph(torch, bench, steps, warmup, per_graph=1):
    """The step captured once as a HIP graph (stream capture of the C-ABI calls,
    which launch on torch's current stream and neither allocate nor synchronise),
    then replayed: the launch gaps and the Python/ctypes overhead between kernels
    go away, the kernels are the same.  With per_graph > 1 the graph holds that
    many consecutive steps (a bench that rotates input copies captures one step
    per copy).  Returns ms per step."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            bench.step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(per_graph):
            bench.step()
    reps = max(1, steps // per_graph)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        g.replay()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / (reps * per_graph)
    del g
    return ms


def kernel_src_hash(names):
    h = hashlib.sha256()
    for n in names:
        p = os.path.join(ROOT, "compressed_sparse_attention_compress_amd", "csrc", n)
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel, src_files):
    """HBM bytes per launch from committed rocprofv3 PMC summaries, or None when
    the kernel source changed since they were taken."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
        e = d.get(kernel)
        if not e or e.get("src_hash") != kernel_src_hash(src_files):
            return None
        return e.get("bytes_per_launch")
    except Exception:
        return None


# -------------------------------------------------------------- CPU baseline

def cpu_baseline_prefill(bench, min_seconds=10.0):
    """Oracle on this host over the whole workload: compressor + index K over all
    tokens, then score/top-k and attention for every query; the whole step is
    repeated until at least `min_seconds` have passed and the mean is reported."""
    import numpy as np
    from oracle import csa2_oracle as O
    s, i = bench.shape, bench.inp
    try:
        cores = len(os.sched_getaffinity(0))
    except Exception:
        cores = os.cpu_count() or 1

    def f64(x):
        return x.detach().float().cpu().numpy().astype(np.float64)
    x = f64(i["x"][0])
    w_kv, w_gate, gamma, w_ik = f64(i["w_kv"]), f64(i["w_gate"]), f64(i["gamma"]), f64(i["w_ik"])
    qi, ww, qq, sw = f64(i["q_idx"][0]), f64(i["w"][0]), f64(i["q"][0]), f64(i["swa_kv"][0])
    runs, t_build, t_q = 0, 0.0, 0.0
    while runs == 0 or t_build + t_q < min_seconds:
        t0 = time.perf_counter()
        lat, kv, ids = O.compress(x, w_kv, w_gate, gamma, s.m, 0)
        _, codes, scales = O.index_k(lat, w_ik, ids * s.m)
        kd = O.fp4_unpack(codes, scales)
        t1 = time.perf_counter()
        for tok in range(s.L):
            nv = O.visible_entries(tok, s.m)
            sc = O.index_scores(qi[tok], ww[tok], kd, nv)
            sel = O.topk_select(sc, s.k)
            O.sparse_attention(qq[tok], kv, sel, sw, 0, tok, s.W)
        t2 = time.perf_counter()
        t_build += t1 - t0
        t_q += t2 - t1
        runs += 1
    per_step = (t_build + t_q) / runs
    return {"value": s.B * s.L / per_step, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": (f"the whole workload, unsampled: compressor + index K on all {s.L} tokens, then score + "
                       f"top-k + attention for all {s.L} queries; {runs} run(s), mean {per_step:.2f} s per step "
                       f"({t_build / runs:.2f} s build, {t_q / runs:.2f} s queries); numpy float64, "
                       f"BLAS threads = {cores}"),
            "measured_s": round(t_build + t_q, 2)}


def cpu_baseline_tiny(tb, min_seconds=2.0):
    """The oracle's whole Full layer (compressor, index K, score + top-k and
    attention for all 512 queries) on the same inputs, repeated for at least
    `min_seconds`."""
    import numpy as np
    from oracle import csa2_oracle as O
    s, i = tb.shape, tb.inp

    def f64(x):
        return None if x is None else x.detach().float().cpu().numpy().astype(np.float64)
    cfg = O.LayerConfig(O.FULL, m=s.m, k=s.k, W=s.W, w_kv=f64(i["w_kv"]), w_gate=f64(i["w_gate"]),
                        gamma=f64(i["gamma"]), w_ik=f64(i["w_ik"]))
    li = O.LayerInputs(q=f64(i["q"]), swa_kv=f64(i["swa_kv"]), q_pos=i["q_pos"].cpu().numpy(),
                       swa_pos0=i["swa_pos0"].cpu().numpy(), q_idx=f64(i["q_idx"]), w=f64(i["w"]), x=f64(i["x"]))
    runs, t = 0, 0.0
    while runs == 0 or t < min_seconds:
        t0 = time.perf_counter()
        O.layer_forward(O.Runtime(), cfg, li)
        t += time.perf_counter() - t0
        runs += 1
    per = t / runs
    return {"value": round(per * 1e6, 1), "unit": "us per layer call", "cores": _cores(), "kind": "oracle",
            "sample": f"the whole tiny Full layer, unsampled; {runs} runs, mean {per:.3f} s; numpy float64",
            "measured_s": round(t, 2)}


def _cores():
    try:
        return len(os.sched_getaffinity(0))
    except Exception:
        return os.cpu_count() or 1


def cpu_baseline_decoder(db, every=256):
    """Oracle on this host for the decoder block: the compressor and index K over
    all L prompt tokens in full, then score + top-k + attention of every
    `every`-th replayed query through the four layers; the query part is
    extrapolated to all R replayed queries (work per query is the same up to its
    visible-entry count, which the sample spans evenly)."""
    import numpy as np
    from oracle import csa2_oracle as O
    K = db.K

    def f64(x):
        return x.detach().float().cpu().numpy().astype(np.float64)
    x, w_kv, gamma, w_ik = f64(db.x[0]), f64(db.w_kv), f64(db.gamma), f64(db.w_ik)
    lays = [{n: f64(v[0]) for n, v in lay.items() if n in ("q", "q_idx", "w", "swa_kv")} for lay in db.layers]
    t0 = time.perf_counter()
    lat, kv, ids = O.compress(x, w_kv, None, gamma, 1, 0)
    _, codes, scales = O.index_k(lat, w_ik, ids)
    kd = O.fp4_unpack(codes, scales)
    t1 = time.perf_counter()
    sample = list(range(0, db.R, every))
    for j in sample:
        p = db.L - db.R + j
        sel = None
        for l, lay in enumerate(lays):
            if db.modes[l] != K.REUSE:
                sel = O.topk_select(O.index_scores(lay["q_idx"][j], lay["w"][j], kd, O.visible_entries(p, 1)),
                                    db.k)
            O.sparse_attention(lay["q"][j], kv, sel, lay["swa_kv"], db.L - db.R, p, db.W)
    t2 = time.perf_counter()
    total = (t1 - t0) + (t2 - t1) / len(sample) * db.R
    return {"value": db.L / total, "unit": "tokens/s", "cores": _cores(), "kind": "oracle",
            "sample": (f"compressor + index K on all {db.L} tokens in full ({t1 - t0:.2f} s), then score + top-k + "
                       f"attention through the 4 layers for every {every}th of the {db.R} replayed queries "
                       f"({len(sample)} queries, {t2 - t1:.2f} s), extrapolated by the query count to "
                       f"{total:.1f} s per step; numpy float64, BLAS threads = {_cores()}"),
            "measured_s": round(t2 - t0, 2)}


def cpu_baseline_decode(db, seqs=(0, 21, 42, 63)):
    """Oracle on this host for the batched decode step on `seqs` of the B
    sequences: index-K dequantisation, scores over all entries, top-k, then the
    Reindex and the Reuse layer's attention; extrapolated by the sequence count.
    The sequence's caches are drawn again from their seeds before the clock.
    With FP4 main KV the selected rows are dequantised inside the clock; with the
    FP8 window ring each layer appends the newest row and reads its window from
    the ring inside the clock (the ring holding the earlier rows is built
    before it)."""
    import numpy as np
    import torch
    import synth
    from oracle import csa2_oracle as O

    def f64(x):
        return x.detach().float().cpu().numpy().astype(np.float64)
    p = int(db.q_pos[0, 0].item())
    pos0 = int(db.swa_pos0[0].item())
    W = db.W
    spent = 0.0
    for b in seqs:
        codes, scales = O.fp4_pack(synth.cache_rows(db.N, 128, db.seed, "u", b, "cuda").cpu().numpy())
        lay = [{n: f64(v[b]) for n, v in db.layers[l].items()} for l in range(2)]
        if db.kv_fp4:
            # FP4 rows of the entries the step selects (packing all N rows here would
            # take ~10 s a sequence; the step reads only these)
            sel0 = O.topk_select(O.index_scores(lay[0]["q_idx"][0], lay[0]["w"][0], O.fp4_unpack(codes, scales),
                                                db.N), db.k)
            ids0 = np.sort(sel0[sel0 >= 0])
            rows = synth.cache_rows(db.N, 512, db.seed, "kv_cache", b, "cuda")[torch.from_numpy(ids0).cuda()]
            kvc, kvs = O.kv_fp4_pack(rows.cpu().numpy())
        else:
            kv = f64(synth.cache_rows(db.N, 512, db.seed, "kv_cache", b, "cuda").to(torch.bfloat16))
        rings = []
        if db.swa_fp8:
            for l in range(2):
                ring = np.zeros((W, 512), dtype=np.uint8)
                O.swa_ring_append(ring, lay[l]["swa_kv"], np.arange(p - W + 1, p + 1))
                rings.append(ring)
        t0 = time.perf_counter()
        kd = O.fp4_unpack(codes, scales)
        sel = O.topk_select(O.index_scores(lay[0]["q_idx"][0], lay[0]["w"][0], kd, db.N), db.k)
        if db.kv_fp4:
            j = np.searchsorted(ids0, sel[sel >= 0])
            kv_a, sel_a = O.kv_fp4_unpack(kvc[j], kvs[j]), np.arange(j.size)
        else:
            kv_a, sel_a = kv, sel
        for l in range(2):
            if db.swa_fp8:
                O.swa_ring_append(rings[l], lay[l]["swa_kv"][W - 1:], [p])
                win, w0 = O.swa_ring_rows(rings[l], p - W + 1, p), p - W + 1
            else:
                win, w0 = lay[l]["swa_kv"], pos0
            O.sparse_attention(lay[l]["q"][0], kv_a, sel_a, win, w0, p, W)
        spent += time.perf_counter() - t0
        del kv_a, kd
    per_step = spent / len(seqs) * db.B
    extra = (" (FP4 main KV: the selected rows dequantised" + ("; FP8 window ring: append + window read per layer)"
                                                                if db.swa_fp8 else ")")) if db.kv_fp4 else ""
    return {"value": per_step * 1e6, "unit": "us/step", "cores": _cores(), "kind": "oracle",
            "sample": (f"{len(seqs)} of the {db.B} sequences (index-K dequantisation, scores over all {db.N} entries, "
                       f"top-{db.k}, attention of the Reindex and the Reuse layer{extra}), {spent:.2f} s, "
                       f"extrapolated by the sequence count; numpy float64, BLAS threads = {_cores()}"),
            "measured_s": round(spent, 2)}


def cpu_baseline_append(ab):
    """Oracle on this host for the decode append record: `compress_step` and, at
    a group's last token, `index_k`, for every sequence over the m steps of one
    group (the record's step); all B sequences, no sampling."""
    import numpy as np
    from oracle import csa2_oracle as O

    def f64(x):
        return x.detach().float().cpu().numpy().astype(np.float64)
    xs = [f64(x) for x in ab.x]
    w_kv, w_gate, w_ik, gamma = f64(ab.w_kv), f64(ab.w_gate), f64(ab.w_ik), f64(ab.gamma)
    pos = [int(p[0].item()) for p in ab.pos]
    reps, spent = 0, 0.0
    while reps == 0 or spent < 2.0:
        t0 = time.perf_counter()
        for b in range(ab.B):
            pending = []
            for i in range(ab.m):
                pending, ent = O.compress_step(pending, xs[i][b], w_kv, w_gate, gamma, pos[i], ab.m)
                if ent is not None:
                    g, lat, _ = ent
                    O.index_k(lat[None], w_ik, np.array([g * ab.m]))
        spent += time.perf_counter() - t0
        reps += 1
    per_step = spent / reps / ab.m
    return {"value": per_step * 1e6, "unit": "us/token step", "cores": _cores(), "kind": "oracle",
            "sample": (f"all {ab.B} sequences, the {ab.m} steps of one group (C and Z projections, pool; at the "
                       f"group's last token RMSNorm, RoPE and the index-K row), {reps} run(s), {spent:.2f} s; "
                       f"numpy float64, BLAS threads = {_cores()}"),
            "measured_s": round(spent, 2)}


def cpu_baseline_hsi(hb, seqs=(0,)):
    """Oracle on this host for the 1M-context HSI decode step on `seqs` of the 4
    sequences: the Full layer (scores over all entries, top-k, block maxima and
    the pool), the Reindex layer inside the pool, and both layers' attention;
    extrapolated by the sequence count."""
    import numpy as np
    import torch
    import synth
    from oracle import csa2_oracle as O

    def f64(x):
        return x.detach().float().cpu().numpy().astype(np.float64)
    p = int(hb.q_pos[0, 0].item())
    pos0 = int(hb.swa_pos0[0].item())
    spent = 0.0
    for b in seqs:
        codes, scales = O.fp4_pack(synth.cache_rows(hb.N, 128, hb.seed, "u", b, "cuda").cpu().numpy())
        kv = f64(synth.cache_rows(hb.N, 512, hb.seed, "kv_cache", b, "cuda").to(torch.bfloat16))
        lay = [{n: f64(v[b]) for n, v in hb.layers[l].items()} for l in range(2)]
        t0 = time.perf_counter()
        kd = O.fp4_unpack(codes, scales)
        sc = O.index_scores(lay[0]["q_idx"][0], lay[0]["w"][0], kd, hb.N)
        sels = [O.topk_select(sc, hb.k)]
        pool = O.pool_entries(O.hsi_pool(sc, hb.N, hb.s_blk, hb.n_b), hb.N, hb.s_blk)
        sc2 = O.index_scores(lay[1]["q_idx"][0], lay[1]["w"][0], kd, hb.N)
        sels.append(O.topk_select(sc2, hb.k, pool))
        for l in range(2):
            O.sparse_attention(lay[l]["q"][0], kv, sels[l], lay[l]["swa_kv"], pos0, p, hb.W)
        spent += time.perf_counter() - t0
        del kv, kd
    per_step = spent / len(seqs) * hb.B
    return {"value": per_step * 1e6, "unit": "us/step", "cores": _cores(), "kind": "oracle",
            "sample": (f"{len(seqs)} of the {hb.B} sequences (Full layer: scores over all {hb.N} entries, top-{hb.k}, "
                       f"block maxima and pool; Reindex layer inside the pool; both attentions), {spent:.2f} s, "
                       f"extrapolated by the sequence count; numpy float64, BLAS threads = {_cores()}"),
            "measured_s": round(spent, 2)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode record")
    ap.add_argument("--decode-seqs", type=int, default=64)
    ap.add_argument("--no-hsi", action="store_true", help="skip the 1M-context HSI decode record")
    ap.add_argument("--no-append", action="store_true", help="skip the decode-append record")
    ap.add_argument("--no-tiny", action="store_true", help="skip the tiny fp32 layer latency record")
    ap.add_argument("--no-fp4kv", action="store_true", help="skip the decode record with FP4 main KV")
    ap.add_argument("--no-fp8swa", action="store_true",
                    help="skip the decode record with FP4 main KV and the FP8 window ring")
    ap.add_argument("--no-decoder", action="store_true",
                    help="skip the decoder macro-block records (full prefill and bounded replay)")
    ap.add_argument("--replay", type=int, default=2048,
                    help="replayed tail length R of the bounded-replay decoder record")
    ap.add_argument("--no-graph", dest="graph", action="store_false",
                    help="time eager launches instead of a HIP graph replay of the step")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="before timing, copy a buffer of this many MiB device-to-device once (a plain copy "
                         "kernel of known size, used to calibrate rocprofv3 FETCH_SIZE / WRITE_SIZE readings)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the path shards by sequence across GPUs, with no cross-GPU traffic on the hot path); got --gpus "
              f"{args.gpus}", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    from compressed_sparse_attention_compress_amd import csa2 as K
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(3)
    K.lib()
    if args.copy_calib_mib > 0:
        n = args.copy_calib_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {args.copy_calib_mib} MiB read + {args.copy_calib_mib} MiB written")
        del src, dst

    log("prefill: building inputs")
    pb = PrefillBench(torch, K, synth)
    log("prefill: timing")
    ms_eager, stages = time_steps(torch, pb, 4, args.steps, args.warmup)
    ms = time_graph(torch, pb, args.steps, args.warmup) if args.graph else ms_eager
    work = pb.work()
    names = ["compress", "index_k", "score_topk", "sparse_attn"]
    stage_rec = {}
    for n, t_ms in zip(names, stages):
        w = work[n]
        rec = {"ms": round(t_ms, 4), "tflops": round(w["flop"] / (t_ms * 1e-3) / 1e12, 2),
               "mfma_frac": round(w["flop"] / (t_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
        stage_rec[n] = rec
    dom = max(names, key=lambda n: stage_rec[n]["ms"])
    dom_files = {"compress": ["k_compress.hip"], "index_k": ["k_index_k.hip"], "score_topk": ["k_score.hip"],
                 "sparse_attn": ["k_attn.hip"]}[dom]
    achieved = work[dom]["flop"] / (stage_rec[dom]["ms"] * 1e-3) / 1e12
    tokens = pb.shape.B * pb.shape.L
    value = tokens / (ms * 1e-3)
    total_flop = sum(w["flop"] for w in work.values())
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "ms_per_step_eager": round(ms_eager, 4),
        "timing": "HIP graph replay of the step" if args.graph else "eager launches",
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "encoder Full-layer prefill: B=1, L=8192, hidden 4096, m=2 (4096 entries), latent 512, "
                               "indexer 32x128 FP4 (E4M3 scale / 32 dims), top-512, SWA 128, 64 heads x 512",
                   "global_batch": tokens, "seq_len": pb.shape.L, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": traffic_for(dom, dom_files)},
        "stages": stage_rec,
        "step_tflops": round(total_flop / (ms * 1e-3) / 1e12, 2),
    }
    if not args.no_decode:
        del pb
        torch.cuda.empty_cache()
        log("decode: building caches")
        db = DecodeBench(torch, K, synth, B=args.decode_seqs)
        log("decode: timing")
        dms_eager, dst = time_steps(torch, db, 3, max(args.steps, 20), args.warmup)
        dms = time_graph(torch, db, max(args.steps, 20), args.warmup) if args.graph else dms_eager
        dw = db.work()
        sc_gbs = dw["score_topk"]["bytes"] / (dst[0] * 1e-3) / 1e9
        attn_gbs = (dw["sparse_attn"]["bytes"] * 2) / ((dst[1] + dst[2]) * 1e-3) / 1e9
        step_bytes = dw["score_topk"]["bytes"] + 2 * dw["sparse_attn"]["bytes"]
        out["decode"] = {
            "workload": f"batched decode, Reindex + Reuse: {db.B} sequences x {db.N} m=2 entries (262144-token "
                        f"context), bf16 latent, FP4 index K, 32x128 indexer heads, top-512, SWA 128, 64 heads",
            "us_per_step": round(dms * 1e3, 2), "us_per_step_eager": round(dms_eager * 1e3, 2),
            "stages_us": {"score_topk": round(dst[0] * 1e3, 2), "attn_reindex": round(dst[1] * 1e3, 2),
                          "attn_reuse": round(dst[2] * 1e3, 2)},
            "roofline": {"bound": "hbm", "kernel": "score_topk", "achieved": round(sc_gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(sc_gbs / HBM_PEAK_GBS, 4),
                         "traffic": traffic_for("score_topk_decode", ["k_score.hip"])},
            "attn_GBps": round(attn_gbs, 1),
            "step_frac_of_hbm_roofline": round(step_bytes / HBM_PEAK_GBS / 1e9 / (dms * 1e-3), 4),
        }
        if not args.no_cpu:
            log("decode: cpu baseline (oracle, 4 of the sequences)")
            out["decode"]["cpu_baseline"] = cpu_baseline_decode(db)
        del db
        torch.cuda.empty_cache()
    if not args.no_decode and not args.no_fp4kv:
        log("decode (FP4 main KV): building caches")
        fb = DecodeBench(torch, K, synth, B=args.decode_seqs, kv_fp4=True)
        log("decode (FP4 main KV): timing")
        fms_eager, fst = time_steps(torch, fb, 3, max(args.steps, 20), args.warmup)
        fms = time_graph(torch, fb, max(args.steps, 20), args.warmup) if args.graph else fms_eager
        fw = fb.work()
        attn_gbs = fw["sparse_attn"]["bytes"] / (fst[1] * 1e-3) / 1e9
        step_bytes = fw["score_topk"]["bytes"] + 2 * fw["sparse_attn"]["bytes"]
        out["decode_fp4kv"] = {
            "workload": f"batched decode, Reindex + Reuse, FP4 main KV (288 B per entry, E2M1 + E4M3 per 16 dims): "
                        f"{fb.B} sequences x {fb.N} m=2 entries, FP4 index K, 32x128 indexer heads, top-512, "
                        f"SWA 128 (bf16), 64 heads",
            "us_per_step": round(fms * 1e3, 2), "us_per_step_eager": round(fms_eager * 1e3, 2),
            "stages_us": {"score_topk": round(fst[0] * 1e3, 2), "attn_reindex": round(fst[1] * 1e3, 2),
                          "attn_reuse": round(fst[2] * 1e3, 2)},
            "roofline": {"bound": "hbm", "kernel": "sparse_attn_fp4kv", "achieved": round(attn_gbs, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(attn_gbs / HBM_PEAK_GBS, 4),
                         "traffic": traffic_for("sparse_attn_fp4kv", ["k_attn.hip"])},
            "attn_bytes_per_layer": fw["sparse_attn"]["bytes"],
            "step_frac_of_hbm_roofline": round(step_bytes / HBM_PEAK_GBS / 1e9 / (fms * 1e-3), 4),
        }
        if not args.no_cpu:
            log("decode (FP4 main KV): cpu baseline (oracle, 4 of the sequences)")
            out["decode_fp4kv"]["cpu_baseline"] = cpu_baseline_decode(fb)
        del fb
        torch.cuda.empty_cache()
    if not args.no_decode and not args.no_fp8swa:
        log("decode (FP4 main KV, FP8 window ring): building caches")
        wb = DecodeBench(torch, K, synth, B=args.decode_seqs, kv_fp4=True, swa_fp8=True)
        log("decode (FP4 main KV, FP8 window ring): timing")
        wms_eager, wst = time_steps(torch, wb, 3, max(args.steps, 20), args.warmup)
        wms = time_graph(torch, wb, max(args.steps, 20), args.warmup) if args.graph else wms_eager
        ww = wb.work()
        attn_gbs = ww["sparse_attn"]["bytes"] / (wst[1] * 1e-3) / 1e9
        step_bytes = ww["score_topk"]["bytes"] + 2 * ww["sparse_attn"]["bytes"]
        out["decode_fp4kv_fp8swa"] = {
            "workload": f"batched decode, Reindex + Reuse, FP4 main KV (288 B per entry) and each layer's SWA 128 "
                        f"window KV in an FP8 ring (E4M3, 512 B per row; the step appends the newest row): "
                        f"{wb.B} sequences x {wb.N} m=2 entries, FP4 index K, 32x128 indexer heads, top-512, "
                        f"64 heads",
            "us_per_step": round(wms * 1e3, 2), "us_per_step_eager": round(wms_eager * 1e3, 2),
            "stages_us": {"score_topk": round(wst[0] * 1e3, 2), "append_attn_reindex": round(wst[1] * 1e3, 2),
                          "append_attn_reuse": round(wst[2] * 1e3, 2)},
            "roofline": {"bound": "hbm", "kernel": "swa_append + sparse_attn (FP4 KV, FP8 ring)",
                         "achieved": round(attn_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(attn_gbs / HBM_PEAK_GBS, 4),
                         "traffic": traffic_for("sparse_attn_fp4kv_fp8swa", ["k_attn.hip", "k_swa.hip"])},
            "attn_bytes_per_layer": ww["sparse_attn"]["bytes"],
            "step_frac_of_hbm_roofline": round(step_bytes / HBM_PEAK_GBS / 1e9 / (wms * 1e-3), 4),
        }
        if not args.no_cpu:
            log("decode (FP4 main KV, FP8 window ring): cpu baseline (oracle, 4 of the sequences)")
            out["decode_fp4kv_fp8swa"]["cpu_baseline"] = cpu_baseline_decode(wb)
        del wb
        torch.cuda.empty_cache()
    if not args.no_hsi:
        log("hsi decode: building caches")
        hb = HsiDecodeBench(torch, K, synth)
        log("hsi decode: timing")
        n_hsi = 3 * max(args.steps, 20)
        hms_eager, hst = time_steps(torch, hb, 3, n_hsi, args.warmup)
        hms = time_graph(torch, hb, n_hsi, args.warmup, per_graph=hb.copies) if args.graph else hms_eager
        hw = hb.work()
        full_gbs = hw["score_full"]["bytes"] / (hst[0] * 1e-3) / 1e9
        step_bytes = sum(v["bytes"] for v in hw.values())
        out["decode_hsi_1m"] = {
            "workload": f"1M-context decode with the HSI candidate pool: {hb.B} sequences x {hb.N} m=2 entries "
                        f"(1048576-token context), blocks of {hb.s_blk}, top-{hb.n_b} blocks (16384-entry pool), "
                        f"Full layer (scan + pool build) + Reindex layer (pool only), top-512, SWA 128, 64 heads; "
                        f"index K rotated over {hb.copies} copies so scans come from HBM",
            "us_per_step": round(hms * 1e3, 2), "us_per_step_eager": round(hms_eager * 1e3, 2),
            "stages_us": {"score_full_build": round(hst[0] * 1e3, 2), "score_reindex_pool": round(hst[1] * 1e3, 2),
                          "attn_2_layers": round(hst[2] * 1e3, 2)},
            "roofline": {"bound": "hbm", "kernel": "score_full_build", "achieved": round(full_gbs, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(full_gbs / HBM_PEAK_GBS, 4),
                         "traffic": traffic_for("score_hsi_full", ["k_score.hip"])},
            "step_bytes": step_bytes,
            "step_frac_of_hbm_roofline": round(step_bytes / HBM_PEAK_GBS / 1e9 / (hms * 1e-3), 4),
        }
        if not args.no_cpu:
            log("hsi decode: cpu baseline (oracle, 1 of the sequences)")
            out["decode_hsi_1m"]["cpu_baseline"] = cpu_baseline_hsi(hb)
        del hb
        torch.cuda.empty_cache()
    if not args.no_decoder:
        for rec, R in (("decoder_block", None), ("decoder_replay", args.replay)):
            log(f"{rec}: building inputs")
            dcb = DecoderBench(torch, K, synth, R=R)
            n_dec = max(3, args.steps // 2)
            dec_eager, dec_st = time_steps(torch, dcb, 4, n_dec, 1)
            dec_ms = time_graph(torch, dcb, n_dec, 1) if args.graph else dec_eager
            dw = dcb.work()
            # the projections' MFMA fraction, from the compressor call timed alone
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            dcb.compress_only()
            ev[0].record()
            for _ in range(5):
                dcb.compress_only()
            ev[1].record()
            torch.cuda.synchronize()
            c_ms = ev[0].elapsed_time(ev[1]) / 5
            c_tf = dw["compress_flop"] / (c_ms * 1e-3) / 1e12
            step_tf = dw["flop"] / (dec_ms * 1e-3) / 1e12
            out[rec] = {
                "workload": (f"decoder macro-block prefill: the Full layer (m=1) compresses H20 of all {dcb.L} "
                             f"prompt tokens (hidden 4096) into the global KV and FP4 index K; Full, Reindex, Reuse, "
                             f"Reuse through csa2_layer_forward for the last {dcb.R} positions (window KV of those "
                             f"positions only), 32x128 indexer heads, top-512, SWA 128, 64 heads"
                             + ("" if dcb.R == dcb.L else f"; bounded replay R={dcb.R}")),
                "tokens_per_s": round(dcb.L / (dec_ms * 1e-3), 1), "ms_per_step": round(dec_ms, 4),
                "ms_per_step_eager": round(dec_eager, 4),
                "stages_ms": {n: round(t, 4) for n, t in zip(("full", "reindex", "reuse", "reuse2"), dec_st)},
                "roofline": {"bound": "mfma", "kernel": "compress (projections)", "achieved": round(c_tf, 2),
                             "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": round(c_tf / MFMA_BF16_PEAK_TFLOPS, 4),
                             "traffic": traffic_for("compress_decoder", ["k_compress.hip"])},
                "step_tflops": round(step_tf, 2),
                "step_frac_of_mfma_peak": round(step_tf / MFMA_BF16_PEAK_TFLOPS, 4),
            }
            if not args.no_cpu:
                log(f"{rec}: cpu baseline (oracle)")
                out[rec]["cpu_baseline"] = cpu_baseline_decoder(dcb)
            del dcb
            torch.cuda.empty_cache()
    if not args.no_append:
        log("decode append: building inputs")
        ab = AppendBench(torch, K, synth)
        n_app = max(args.steps, 20)
        ams_eager, ast = time_steps(torch, ab, ab.m, n_app, args.warmup)
        ams = time_graph(torch, ab, n_app, args.warmup) if args.graph else ams_eager
        per_tok = ams / ab.m                      # one append call = one new token per sequence
        gbs = ab.bytes_per_step() / (per_tok * 1e-3) / 1e9
        out["decode_append"] = {
            "workload": f"Full-layer decode append: {ab.B} sequences, hidden {ab.D}, m={ab.m}; one new token per "
                        f"sequence per call (C/Z projection, running group pool, and at a group's last token the "
                        f"cache row and its FP4 index-K row)",
            "us_per_token_step": round(per_tok * 1e3, 2), "us_per_token_step_eager": round(ams_eager / ab.m * 1e3, 2),
            "stages_us": {"group_first_token": round(ast[0] * 1e3, 2), "group_last_token": round(ast[1] * 1e3, 2)},
            "roofline": {"bound": "hbm", "kernel": "compress_step", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": traffic_for("compress_step", ["k_compress.hip"])},
        }
        if not args.no_cpu:
            log("decode append: cpu baseline (oracle, all sequences)")
            out["decode_append"]["cpu_baseline"] = cpu_baseline_append(ab)
        del ab
        torch.cuda.empty_cache()
    if not args.no_tiny:
        log("tiny layer: timing")
        tb = TinyLayerBench(torch, K, synth)
        n_tiny = max(args.steps, 50)
        tms_eager, _ = time_steps(torch, tb, 1, n_tiny, args.warmup)
        tms = time_graph(torch, tb, n_tiny, args.warmup) if args.graph else tms_eager
        tflops = tb.work() / (tms * 1e-3) / 1e12
        out["tiny_layer"] = {
            "workload": "tiny Full layer, fp32: B=1, L=512, hidden 256, m=2 (256 entries), latent 512, indexer 4x128 "
                        "FP4, top-32, SWA 16, 8 heads x 512; one csa2_layer_forward call (compressor, index K, "
                        "score + top-k, attention)",
            "us_per_call": round(tms * 1e3, 2), "us_per_call_eager": round(tms_eager * 1e3, 2),
            "roofline": {"bound": "latency", "kernel": "layer (fp32)", "achieved": round(tflops, 3),
                         "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tflops / FP32_PEAK_TFLOPS, 5),
                         "traffic": None},
        }
        if not args.no_cpu:
            log("tiny layer: cpu baseline (oracle, whole layer)")
            out["tiny_layer"]["cpu_baseline"] = cpu_baseline_tiny(tb)
        del tb
    if not args.no_cpu:
        log("cpu baseline: the oracle on the whole prefill step")
        pb2 = PrefillBench(torch, K, synth)
        out["cpu_baseline"] = cpu_baseline_prefill(pb2)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
