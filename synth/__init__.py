"""Seeded synthetic inputs for the CSA2 hot path.

This module only draws random tensors of the right shapes, dtypes and scales; it
holds none of the method's arithmetic (no pooling, norm, RoPE, quantisation,
scoring, selection or attention).  Both the HIP library's tests/benchmark and the
CPU oracle consume what it produces.

Distributions (one generator per tensor, derived from one seed):
  * hidden states, queries, indexer queries, head weights, window KV and cache
    latents: N(0, 1);
  * projection weights W [out, in]: N(0, 1/sqrt(in)) (standard deviation);
  * RMSNorm gain: ones.
The pages evaluate on agentic long-context benchmarks; no data or trained weights
exist here, so these Gaussian tensors stand in for them at the same shapes.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional

import torch

_SALT = {
    "x": 1, "w_kv": 2, "w_gate": 3, "w_ik": 4, "q": 5, "q_idx": 6, "w": 7, "swa_kv": 8,
    "w_w": 9, "kv_cache": 10, "u": 11, "plant": 12,
}


def _gen(seed: int, name: str, layer: int = 0, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + _SALT[name] * 7919 + layer * 104_729) & 0x7FFFFFFFFFFF)
    return g


def gaussian(shape, std: float, seed: int, name: str, layer: int = 0, dtype=torch.float32,
             device="cpu") -> torch.Tensor:
    """N(0, std) in float32 on ``device``, then cast to ``dtype`` (round to nearest)."""
    g = _gen(seed, name, layer, device)
    t = torch.randn(*shape, generator=g, dtype=torch.float32, device=device)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def linear_weight(out_f: int, in_f: int, seed: int, name: str, layer: int = 0,
                  dtype=torch.float32, device="cpu") -> torch.Tensor:
    """Weight [out, in] with entries N(0, 1/sqrt(in))."""
    return gaussian((out_f, in_f), 1.0 / math.sqrt(in_f), seed, name, layer, dtype, device)


@dataclass
class LayerShape:
    B: int
    L: int            # tokens of hidden state (Full layer input)
    D: int            # hidden size
    m: int            # compress ratio
    H_I: int          # indexer heads
    k: int            # top-k
    W: int            # sliding window
    H: int            # attention heads
    d: int = 512      # latent width
    d_I: int = 128    # indexer head dim


def full_layer_inputs(shape: LayerShape, seed: int = 0, dtype=torch.float32, device="cpu",
                      layer: int = 0, w_from_linear: bool = False, with_x: bool = True):
    """Inputs of one prefill layer over tokens 0..L-1 of each sequence.

    Returns a dict of tensors: x [B,L,D], w_kv/w_gate [512,D] (w_gate None when
    m == 1), gamma [512] (float32), w_ik [128,512], q [B,L,H,512],
    q_idx [B,L,H_I,128], w [B,L,H_I] (float32), swa_kv [B,L,512],
    q_pos [B,L] int32, swa_pos0 [B] int32.
    """
    s = shape
    out = {}
    if with_x:
        out["x"] = gaussian((s.B, s.L, s.D), 1.0, seed, "x", 0, dtype, device)
        out["w_kv"] = linear_weight(s.d, s.D, seed, "w_kv", layer, dtype, device)
        out["w_gate"] = linear_weight(s.d, s.D, seed, "w_gate", layer, dtype, device) if s.m > 1 else None
        out["gamma"] = torch.ones(s.d, dtype=torch.float32, device=device)
        out["w_ik"] = linear_weight(s.d_I, s.d, seed, "w_ik", layer, dtype, device)
    out["q"] = gaussian((s.B, s.L, s.H, s.d), 1.0, seed, "q", layer, dtype, device)
    out["q_idx"] = gaussian((s.B, s.L, s.H_I, s.d_I), 1.0, seed, "q_idx", layer, dtype, device)
    if w_from_linear and with_x:
        ww = linear_weight(s.H_I, s.D, seed, "w_w", layer, torch.float32, device)
        out["w"] = (out["x"].float() @ ww.T).contiguous()
    else:
        out["w"] = gaussian((s.B, s.L, s.H_I), 1.0, seed, "w", layer, torch.float32, device)
    out["swa_kv"] = gaussian((s.B, s.L, s.d), 1.0, seed, "swa_kv", layer, dtype, device)
    out["q_pos"] = torch.arange(s.L, dtype=torch.int32, device=device).repeat(s.B, 1).contiguous()
    out["swa_pos0"] = torch.zeros(s.B, dtype=torch.int32, device=device)
    return out


def decode_cache_inputs(B: int, n_entries: int, seed: int = 0, dtype=torch.bfloat16,
                        device="cpu", d: int = 512, d_I: int = 128,
                        seq_slice: Optional[range] = None):
    """Pre-filled caches for decode: latent kv [B,N,512] and the float32 index-K
    rows u [B,N,128] that are to be quantised to FP4.  Each sequence has its own
    generator, so one sequence can be regenerated alone (``seq_slice``)."""
    seqs = range(B) if seq_slice is None else seq_slice
    kv = torch.empty((len(seqs), n_entries, d), dtype=dtype, device=device)
    u = torch.empty((len(seqs), n_entries, d_I), dtype=torch.float32, device=device)
    for i, b in enumerate(seqs):
        kv[i] = gaussian((n_entries, d), 1.0, seed, "kv_cache", b, dtype, device)
        u[i] = gaussian((n_entries, d_I), 1.0, seed, "u", b, torch.float32, device)
    return kv, u


def cache_rows(n: int, d: int, seed: int, name: str, seq: int, device="cpu") -> torch.Tensor:
    """N(0, 1) float32 rows [n, d] of one sequence's pre-filled cache (latent rows,
    or index-K values before quantisation), from a generator of its own per
    (seed, name, sequence), so that any one sequence can be drawn again alone."""
    return gaussian((n, d), 1.0, seed, name, seq, torch.float32, device)


def decode_query_inputs(B: int, H: int, H_I: int, W: int, seed: int = 0, layer: int = 0,
                        dtype=torch.bfloat16, device="cpu", d: int = 512, d_I: int = 128):
    """One new query token per sequence for one layer: q [B,1,H,512],
    q_idx [B,1,H_I,128], w [B,1,H_I] float32, swa_kv [B,W,512]."""
    return {
        "q": gaussian((B, 1, H, d), 1.0, seed, "q", layer, dtype, device),
        "q_idx": gaussian((B, 1, H_I, d_I), 1.0, seed, "q_idx", layer, dtype, device),
        "w": gaussian((B, 1, H_I), 1.0, seed, "w", layer, torch.float32, device),
        "swa_kv": gaussian((B, W, d), 1.0, seed, "swa_kv", layer, dtype, device),
    }


# The five workloads (hidden 4096, latent 512, 32x128 indexer heads, top-512,
# window 128, 64 query heads; a tiny fp32 case for the oracle).
TINY = LayerShape(B=1, L=512, D=256, m=2, H_I=4, k=32, W=16, H=8)
ENCODER_PREFILL = LayerShape(B=1, L=8192, D=4096, m=2, H_I=32, k=512, W=128, H=64)
DECODER_PREFILL = LayerShape(B=1, L=32768, D=4096, m=1, H_I=32, k=512, W=128, H=64)
