"""Seeded synthetic inputs for the CSA / HCA workloads.

This module only draws random tensors; it holds none of the attention
method's arithmetic.  Both the HIP path and the CPU oracle receive the values
it produces (the oracle as float64 copies of the very same rounded values).

Every tensor is drawn from its own generator, keyed by (seed, workload name,
tensor name, chunk), so any chunk can be regenerated on its own.  Large
tensors are drawn on the GPU (torch's Philox generator); small ones may be
drawn on the CPU.  Values from the two devices differ for the same key, so a
parity test always draws once and copies to the other side.
"""
from __future__ import annotations

import hashlib

import torch

TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def key_seed(*parts) -> int:
    """A 63-bit seed from an arbitrary key tuple (stable across runs)."""
    h = hashlib.sha256("/".join(str(p) for p in parts).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, *key):
    g = torch.Generator(device=device)
    g.manual_seed(key_seed(*key))
    return g


def normal(shape, key, std=1.0, dtype="f32", device="cpu", chunk_rows=None):
    """N(0, std^2) values rounded to `dtype`.  With chunk_rows, rows are drawn
    in chunks of that many leading-axis rows, each from its own generator."""
    out = torch.empty(shape, dtype=TORCH_DTYPES[dtype], device=device)
    if chunk_rows is None:
        x = torch.randn(shape, generator=_gen(device, *key), device=device, dtype=torch.float32)
        out.copy_(x.mul_(std))
        return out
    for c0 in range(0, shape[0], chunk_rows):
        out[c0:c0 + chunk_rows].copy_(normal_chunk(shape, key, c0 // chunk_rows, chunk_rows, std, device))
    return out


def normal_chunk(shape, key, chunk, chunk_rows, std=1.0, device="cpu"):
    """Chunk `chunk` (leading-axis rows [chunk*chunk_rows, ...)) of a chunked
    `normal` tensor, in float32 before rounding."""
    rows = min(chunk_rows, shape[0] - chunk * chunk_rows)
    x = torch.randn((rows,) + tuple(shape[1:]), generator=_gen(device, *key, "chunk", chunk),
                    device=device, dtype=torch.float32)
    return x.mul_(std)


def uniform(shape, key, lo=0.0, hi=1.0, dtype="f32", device="cpu"):
    """U(lo, hi) values rounded to `dtype`."""
    x = torch.rand(shape, generator=_gen(device, *key), device=device, dtype=torch.float32)
    return x.mul_(hi - lo).add_(lo).to(TORCH_DTYPES[dtype])


def csa_prefill_inputs(cfg, seed=0, device="cpu", with_indexer=True, with_window=True):
    """Every input of one CSA (or HCA) prefill layer for workload `cfg`.

    Weights are given output-major ([out_channels, d], a linear layer's weight
    layout); mathematically the projection is H . W^T.  Distributions follow
    the workload statement: H ~ N(0,1), projections ~ N(0, 1/d), position
    biases ~ N(0,1), queries ~ N(0,1), indexer weights ~ U(0,1), sink ~ N(0,1).
    """
    name, dt = cfg["name"], cfg["dtype"]
    n, d, c, m = cfg["n"], cfg["d"], cfg["c"], cfg["m"]
    w = (1 + cfg["overlap"]) * c
    sd = d ** -0.5
    big = dict(device=device, dtype=dt)
    t = {}
    t["H"] = normal((n, d), (seed, name, "H"), chunk_rows=8192, **big)
    t["W_kv"] = normal((w, d), (seed, name, "W_kv"), std=sd, **big)
    t["W_z"] = normal((w, d), (seed, name, "W_z"), std=sd, **big)
    t["ape"] = normal((m, w), (seed, name, "ape"), device=device)
    if with_window:
        t["W_win"] = normal((c, d), (seed, name, "W_win"), std=sd, **big)
    nh = cfg["nh"]
    t["q"] = normal((n, nh, c), (seed, name, "q"), chunk_rows=4096, **big)
    t["sink"] = normal((nh,), (seed, name, "sink"), device=device)
    if with_indexer and cfg.get("hI"):
        hI, cI = cfg["hI"], cfg["cI"]
        wI_ = (1 + cfg["overlap"]) * cI
        t["WI_kv"] = normal((wI_, d), (seed, name, "WI_kv"), std=sd, **big)
        t["WI_z"] = normal((wI_, d), (seed, name, "WI_z"), std=sd, **big)
        t["apeI"] = normal((m, wI_), (seed, name, "apeI"), device=device)
        t["qI"] = normal((n, hI, cI), (seed, name, "qI"), chunk_rows=8192, **big)
        t["wI"] = uniform((n, hI), (seed, name, "wI"), **big)
    return t
