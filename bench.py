"""Benchmark: CSA/HCA hybrid compressed attention on one MI355X.

Headline (`value`): prefill tokens/s of one CSA layer at 64K tokens (bf16,
d=4096, m=4 overlapped compression, 16x64 indexer, top-512, 64 query heads of
width 512, partial RoPE on 64 dims, window 128, sinks).  One step = the whole
prefill hot path on one synthetic sequence: compressor projections + pooling
(main entries, window rows, indexer keys), indexer scoring + top-k, sparse
shared-KV MQA.  Inputs are resident in HBM before timing starts.

Also reported (`decode`): one CSA+HCA decode step (both layers, one new token
per sequence) at batch 32 x 128K context and batch 4 x 1M context, in us per
step and us per token, with the caches built beforehand by the library's own
prefill from seeded N(0,1) hidden states.

`roofline` is measured live for the dominant kernel (sparse MQA prefill) with
HIP events on the stream it runs on; its `traffic` (HBM bytes per launch) is
read from the committed rocprofv3 counter summary of that kernel, and is null
when the kernel source no longer matches the one the counters were taken on.
`cpu_baseline` times the CPU fp64 oracle on a bounded sample of the same
workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-decode]
                       [--no-cpu-baseline] [--pmc-probe [mqa|hca|decode]]
                       [--oracle-times]
  --pmc-probe: run only a 1 GiB device copy (the counter scale reference) and
               one workload's kernels (the 64K sparse MQA prefill by default,
               the 16K HCA prefill step, or decode step replays), for
               rocprofv3 --pmc passes.
  --oracle-times: time the CPU oracle on whole workloads (no GPU).
"""
import hashlib
import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import long_context_attention_10_amd as L  # noqa: E402
from long_context_attention_10_amd import configs, inputs as I  # noqa: E402

PEAK_BF16 = 2.5e15      # dense bf16 matrix FLOP/s, MI355X
PEAK_HBM = 8.0e12       # HBM3E bytes/s, MI355X
PEAK_FP32 = 157.3e12    # fp32 vector FLOP/s, MI355X
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "mqa_prefill_bf16_64k_traffic.txt")
MQA_SOURCE = os.path.join(ROOT, "long_context_attention_10_amd", "csrc", "attention_bf16.hip")


# --------------------------------------------------------------------------
# prefill (headline)
# --------------------------------------------------------------------------
class CsaPrefill:
    def __init__(self, cfg, device="cuda"):
        self.cfg = cfg
        self.t = I.csa_prefill_inputs(cfg, device=device)
        n, c, m, k, nh = cfg["n"], cfg["c"], cfg["m"], cfg["k"], cfg["nh"]
        dt = I.TORCH_DTYPES[cfg["dtype"]]
        self.comp = torch.empty((n // m, c), dtype=dt, device=device)
        self.win = torch.empty((n, c), dtype=dt, device=device)
        self.kI = torch.empty((n // m, cfg["cI"]), dtype=dt, device=device)
        self.idx = torch.empty((n, k), dtype=torch.int32, device=device)
        self.out = torch.empty((n, nh, c), dtype=dt, device=device)

    def compress(self):
        self.compress_main()
        self.compress_indexer()

    def compress_main(self):
        c, t = self.cfg, self.t
        L.csa_compress_prefill(t["H"], t["W_kv"], t["W_z"], t["ape"], c["m"], c["overlap"],
                               W_win=t["W_win"], rope_dims=c["rope_dims"], out_comp=self.comp,
                               out_win=self.win)

    def compress_indexer(self):
        c, t = self.cfg, self.t
        L.csa_compress_prefill(t["H"], t["WI_kv"], t["WI_z"], t["apeI"], c["m"], c["overlap"],
                               out_comp=self.kI, ws_slot="prefill_indexer")

    def index(self):
        c, t = self.cfg, self.t
        L.csa_index_topk_prefill(t["qI"], t["wI"], self.kI, c["m"], c["k"], out=self.idx)

    def attend(self):
        c, t = self.cfg, self.t
        L.csa_sparse_mqa_prefill(t["q"], self.win, self.comp, self.idx, t["sink"],
                                 n_win=c["n_win"], rope_dims=c["rope_dims"], out=self.out)

    def step(self, streams=False):
        """One prefill pass.  The indexer chain (its compressor, then the
        top-k) and the main compressor are independent until the attention:
        with `streams` the indexer chain runs on a forked side stream
        (default priority) while the main compressor runs on the current
        stream, which joins it before the attention.  Off by default: at 64K
        both chains fill the chip, and the overlap measured no faster."""
        if not streams:
            self.compress()
            self.index()
            self.attend()
            return
        main = torch.cuda.current_stream()
        if getattr(self, "side", None) is None:
            self.side = torch.cuda.Stream()
        self.side.wait_stream(main)
        with torch.cuda.stream(self.side):
            self.compress_indexer()
            self.index()
        self.compress_main()
        main.wait_stream(self.side)
        self.attend()

    def step_chunked(self, chunk=8192):
        """The same prefill in block-aligned chunks of `chunk` tokens: each
        chunk compresses its tokens (with the block before it under overlap)
        into the shared entry buffers, then selects and attends for its own
        rows over the entries so far and the window rows before it."""
        c, t = self.cfg, self.t
        n, m, ov, nw, r = c["n"], c["m"], c["overlap"], c["n_win"], c["rope_dims"]
        for p0 in range(0, n, chunk):
            p1 = min(n, p0 + chunk)
            h0 = p0 - m if ov and p0 > 0 else p0
            e0, e1 = p0 // m, p1 // m
            L.csa_compress_prefill(t["H"][h0:p1], t["W_kv"], t["W_z"], t["ape"], m, ov,
                                   W_win=t["W_win"], rope_dims=r, out_comp=self.comp[e0:e1],
                                   out_win=self.win[p0:p1], pos0=p0)
            L.csa_compress_prefill(t["H"][h0:p1], t["WI_kv"], t["WI_z"], t["apeI"], m, ov,
                                   out_comp=self.kI[e0:e1], pos0=p0)
            L.csa_index_topk_prefill(t["qI"][p0:p1], t["wI"][p0:p1], self.kI[:e1], m, c["k"],
                                     out=self.idx[p0:p1], t0=p0)
            w0 = max(0, p0 - nw + 1)
            L.csa_sparse_mqa_prefill(t["q"][p0:p1], self.win[w0:p1], self.comp[:e1],
                                     self.idx[p0:p1], t["sink"], n_win=nw, rope_dims=r,
                                     out=self.out[p0:p1], t0=p0)

    def attn_flops(self):
        """Algorithmic FLOPs of the sparse MQA: 2 matmuls x 2 FLOP per
        multiply-add x heads x width, per (token, candidate) pair."""
        c = self.cfg
        t = np.arange(c["n"], dtype=np.int64)
        pairs = np.minimum(c["n_win"], t + 1) + np.minimum(c["k"], (t + 1) // c["m"])
        return 4.0 * c["nh"] * c["c"] * float(pairs.sum()), int(pairs.sum())


class HcaPrefill:
    """One HCA layer prefill (compressor with window rows, then dense MQA over
    every visible entry) on the workload's synthetic inputs."""

    def __init__(self, cfg, device="cuda"):
        self.cfg = cfg
        self.t = I.csa_prefill_inputs(cfg, device=device, with_indexer=False)
        n, c, m, nh = cfg["n"], cfg["c"], cfg["m"], cfg["nh"]
        dt = I.TORCH_DTYPES[cfg["dtype"]]
        self.comp = torch.empty((n // m, c), dtype=dt, device=device)
        self.win = torch.empty((n, c), dtype=dt, device=device)
        self.out = torch.empty((n, nh, c), dtype=dt, device=device)

    def compress(self):
        c, t = self.cfg, self.t
        L.csa_compress_prefill(t["H"], t["W_kv"], t["W_z"], t["ape"], c["m"], 0,
                               W_win=t["W_win"], rope_dims=c.get("rope_dims", 0),
                               out_comp=self.comp, out_win=self.win)

    def attend(self):
        c, t = self.cfg, self.t
        L.hca_dense_mqa_prefill(t["q"], self.win, self.comp, t["sink"], c["m"], n_win=c["n_win"],
                                rope_dims=c.get("rope_dims", 0), out=self.out)

    def step(self):
        self.compress()
        self.attend()

    def attn_flops(self):
        c = self.cfg
        t = np.arange(c["n"], dtype=np.int64)
        pairs = np.minimum(c["n_win"], t + 1) + (t + 1) // c["m"]
        return 4.0 * c["nh"] * c["c"] * float(pairs.sum())


def chunk_at_context(pf, ctx, chunk, steps, device="cuda"):
    """One prefill chunk of `chunk` tokens ending a `ctx`-token context, with
    the earlier entries, indexer keys and window rows synthetic N(0, 1)
    stand-ins (the 64K workload's weights and per-token inputs): compress
    (main + indexer, with the halo block), select over up to ctx/m entries,
    attend.  Returns the stage times in ms."""
    c, t = pf.cfg, pf.t
    m, ov, nw, r, k = c["m"], c["overlap"], c["n_win"], c["rope_dims"], c["k"]
    p0 = ctx - chunk
    name = ("chunk_at", ctx)
    kw = dict(dtype=c["dtype"], device=device)
    H = I.normal((chunk + m, c["d"]), name + ("H",), **kw)
    comp = I.normal((ctx // m, c["c"]), name + ("comp",), **kw)
    kI = I.normal((ctx // m, c["cI"]), name + ("kI",), **kw)
    w0 = p0 - nw + 1
    win = I.normal((ctx - w0, c["c"]), name + ("win",), **kw)
    q, qI, wI = t["q"][:chunk], t["qI"][:chunk], t["wI"][:chunk]
    idx = torch.empty((chunk, k), dtype=torch.int32, device=device)
    out = torch.empty_like(q)
    e0, e1 = p0 // m, ctx // m

    def compress():
        L.csa_compress_prefill(H, t["W_kv"], t["W_z"], t["ape"], m, ov, W_win=t["W_win"],
                               rope_dims=r, out_comp=comp[e0:e1], out_win=win[p0 - w0:], pos0=p0)
        L.csa_compress_prefill(H, t["WI_kv"], t["WI_z"], t["apeI"], m, ov, out_comp=kI[e0:e1],
                               pos0=p0)

    def index():
        L.csa_index_topk_prefill(qI, wI, kI, m, k, out=idx, t0=p0)

    def attend():
        L.csa_sparse_mqa_prefill(q, win, comp, idx, t["sink"], n_win=nw, rope_dims=r, out=out,
                                 t0=p0)
    res = {}
    for nm, fn in (("compress", compress), ("index_topk", index), ("sparse_mqa", attend)):
        res[nm] = float(np.mean(time_region(fn, steps, 1)))
    del H, comp, kI, win, idx, out
    torch.cuda.empty_cache()
    return res


def time_region(fn, steps, warmup, flush=None):
    """Per-step event times (ms) on the current stream."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    times = []
    if flush is None:
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(steps):
            fn()
        e.record()
        torch.cuda.synchronize()
        return [s.elapsed_time(e) / steps] * steps
    for _ in range(steps):
        flush()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        torch.cuda.synchronize()
        times.append(s.elapsed_time(e))
    return times


def time_ahead(fn, steps, warmup, pre):
    """Per-step GPU times (ms) of fn, each step enqueued after pre() on the
    current stream.  The host enqueues every iteration before it reads any
    event, so no step waits for the host to launch its kernels; pre() (a
    cache flush, or a GPU sleep for warm steps) gives the host the time to
    run ahead."""
    for _ in range(warmup):
        pre()
        fn()
    torch.cuda.synchronize()
    ev = []
    for _ in range(steps):
        pre()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        ev.append((s, e))
    torch.cuda.synchronize()
    return [s.elapsed_time(e) for s, e in ev]


class CacheFlush:
    """Evicts the step's data from the caches before a cold step.

    clean(): write 1 GiB, then read 512 MiB of another buffer, so that the
    256 MiB last-level cache holds clean lines of neither buffer and the
    write-back of the flush's own dirty lines happens before the step, not
    inside it.  dirty(): the write alone (the step then also pays that
    write-back).  warm(): evicts nothing.  Each ends with a GPU sleep of
    about 0.5 ms, which touches no memory and gives the host the time to
    enqueue the next step before the GPU reaches it."""

    def __init__(self, dev):
        self.w = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        self.r = torch.ones(1 << 27, dtype=torch.float32, device=dev)

    def clean(self):
        self.w.random_(0, 255)
        self.r.sum()
        torch.cuda._sleep(1000000)

    def dirty(self):
        self.w.random_(0, 255)
        torch.cuda._sleep(1000000)

    def warm(self):
        torch.cuda._sleep(1000000)


def graph_of(fn):
    """Capture fn (after a warm call that sizes every workspace) in a HIP graph."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def measured_traffic():
    """HBM bytes per sparse-MQA-prefill launch from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE, each scaled by the factor a plain 1 GiB
    copy gives), or None if that summary is absent or was taken on another
    version of the kernel source."""
    try:
        kv = {}
        with open(TRAFFIC_FILE) as fh:
            for line in fh:
                if ":" in line and not line.startswith("#"):
                    a, b = line.split(":", 1)
                    kv[a.strip()] = b.strip()
        with open(MQA_SOURCE, "rb") as fh:
            sha = hashlib.sha256(fh.read()).hexdigest()
        if kv.get("source_sha256") != sha:
            return None
        return float(kv["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def pmc_probe(target="mqa"):
    """One 1 GiB device-to-device copy (counter scale reference), then the
    kernels of `target` for counter passes: "mqa" the sparse MQA prefill of
    the 64K workload twice; "hca" the 16K HCA prefill step (compressor and
    dense MQA) twice; "decode" four graph replays of each decode workload's
    step (both after a clean cache flush)."""
    dev = "cuda"
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    if target == "mqa":
        pf = CsaPrefill(configs.get("csa_prefill_64k_bf16"), dev)
        pf.compress()
        pf.index()
        torch.cuda.synchronize()
        for _ in range(2):
            pf.attend()
    elif target == "hca":
        hp = HcaPrefill(configs.get("hca_prefill_16k_bf16"), dev)
        for _ in range(2):
            hp.step()
    elif target == "decode":
        cf = CacheFlush(dev)
        for wname in ("decode_b32_128k_bf16", "decode_b4_1m_bf16"):
            hd = HybridDecode(configs.get(wname), dev)
            g = graph_of(hd.step)
            for _ in range(4):
                cf.clean()
                g.replay()
            torch.cuda.synchronize()
            del g, hd
            torch.cuda.empty_cache()
    else:
        raise SystemExit(f"unknown probe target {target}")
    torch.cuda.synchronize()
    print(f"[bench] pmc probe done: 1 GiB copy, then {target}", flush=True)


# --------------------------------------------------------------------------
# decode (CSA layer + HCA layer, one token per sequence)
# --------------------------------------------------------------------------
class CsaLayer:
    """The whole CSA layer forward of one prefill workload: the query path
    (latent RMSNorm, q, q^I, w^I), the four calls, and the grouped output
    projection.  Shares the prefill's compressed-entry buffers; its own q, q^I
    and w^I come from H."""

    def __init__(self, pf, device="cuda", seed=0):
        self.pf = pf
        c = pf.cfg
        n, d, nh, cc, hI, cI = c["n"], c["d"], c["nh"], c["c"], c["hI"], c["cI"]
        dc, g, dg = c["d_c"], c["groups"], c["d_g"]
        name, kw = c["name"], dict(dtype=c["dtype"], device=device)
        dt = I.TORCH_DTYPES[c["dtype"]]
        kg = nh * cc // g
        self.w = dict(
            W_DQ=I.normal((dc, d), (seed, name, "W_DQ"), std=d ** -0.5, **kw),
            g_q=1.0 + 0.1 * I.normal((dc,), (seed, name, "g_q"), device=device),
            W_UQ=I.normal((nh * cc, dc), (seed, name, "W_UQ"), std=dc ** -0.5, **kw),
            W_IUQ=I.normal((hI * cI, dc), (seed, name, "W_IUQ"), std=dc ** -0.5, **kw),
            W_w=I.normal((hI, d), (seed, name, "W_w"), std=d ** -0.5, **kw),
            wo_a=I.normal((g, dg, kg), (seed, name, "wo_a"), std=kg ** -0.5, **kw),
            wo_b=I.normal((d, g * dg), (seed, name, "wo_b"), std=(g * dg) ** -0.5, **kw))
        self.q = torch.empty((n, nh, cc), dtype=dt, device=device)
        self.qI = torch.empty((n, hI, cI), dtype=dt, device=device)
        self.wI = torch.empty((n, hI), dtype=dt, device=device)
        self.y = torch.empty((n, d), dtype=dt, device=device)

    def qproj(self):
        c, w = self.pf.cfg, self.w
        L.csa_query_proj(self.pf.t["H"], w["W_DQ"], w["W_UQ"], c["nh"], W_IUQ=w["W_IUQ"],
                         W_w=w["W_w"], n_heads_i=c["hI"], g_q=w["g_q"], eps=c["eps"],
                         out=(self.q, self.qI, self.wI))

    def oproj(self):
        L.csa_output_proj(self.pf.out, self.w["wo_a"], self.w["wo_b"], out=self.y)

    def step(self):
        pf, c = self.pf, self.pf.cfg
        self.qproj()
        pf.compress()
        L.csa_index_topk_prefill(self.qI, self.wI, pf.kI, c["m"], c["k"], out=pf.idx)
        L.csa_sparse_mqa_prefill(self.q, pf.win, pf.comp, pf.idx, pf.t["sink"], n_win=c["n_win"],
                                 rope_dims=c["rope_dims"], out=pf.out)
        self.oproj()

    def proj_flops(self):
        """(query path, output projection) matrix FLOPs: 2 per multiply-add."""
        c = self.pf.cfg
        n, d, dc, hI, cI = c["n"], c["d"], c["d_c"], c["hI"], c["cI"]
        width = c["nh"] * c["c"]
        qf = 2.0 * n * d * (dc + hI) + 2.0 * n * dc * (width + hI * cI)
        of = 2.0 * n * width * c["d_g"] + 2.0 * n * c["groups"] * c["d_g"] * d
        return qf, of


class HybridDecode:
    """State for B sequences at position t = ctx-1 (caches hold [0, t))."""

    def __init__(self, cfg, device="cuda", seed=0):
        self.cfg = cfg
        B, ctx, d, c, m, ov = cfg["batch"], cfg["ctx"], cfg["d"], cfg["c"], cfg["m"], cfg["overlap"]
        mh, hI, cI, nh, nw = cfg["m_hca"], cfg["hI"], cfg["cI"], cfg["nh"], cfg["n_win"]
        r = cfg["rope_dims"]
        name = cfg["name"]
        dt = I.TORCH_DTYPES[cfg["dtype"]]
        sd = d ** -0.5
        kw = dict(dtype=cfg["dtype"], device=device)
        w, wI = (1 + ov) * c, (1 + ov) * cI
        g = {}
        for lay in ("csa", "hca"):
            wl = w if lay == "csa" else c
            g[lay + "_Wkv"] = I.normal((wl, d), (seed, name, lay, "Wkv"), std=sd, **kw)
            g[lay + "_Wz"] = I.normal((wl, d), (seed, name, lay, "Wz"), std=sd, **kw)
            g[lay + "_ape"] = I.normal((m if lay == "csa" else mh, wl), (seed, name, lay, "ape"), device=device)
            g[lay + "_Wwin"] = I.normal((c, d), (seed, name, lay, "Wwin"), std=sd, **kw)
            g[lay + "_q"] = I.normal((B, nh, c), (seed, name, lay, "q"), **kw)
            g[lay + "_sink"] = I.normal((nh,), (seed, name, lay, "sink"), device=device)
        g["WI_kv"] = I.normal((wI, d), (seed, name, "WI_kv"), std=sd, **kw)
        g["WI_z"] = I.normal((wI, d), (seed, name, "WI_z"), std=sd, **kw)
        g["apeI"] = I.normal((m, wI), (seed, name, "apeI"), device=device)
        g["qI"] = I.normal((B, hI, cI), (seed, name, "qI"), **kw)
        g["wI"] = I.uniform((B, hI), (seed, name, "wI"), **kw)
        self.g = g
        t = ctx - 1
        self.pos = torch.full((B,), t, dtype=torch.int64, device=device)
        self.h = torch.empty((B, d), dtype=dt, device=device)
        self.cache = torch.empty((B, ctx // m, c), dtype=dt, device=device)
        self.kcache = torch.empty((B, ctx // m, cI), dtype=dt, device=device)
        self.hcache = torch.empty((B, ctx // mh, c), dtype=dt, device=device)
        self.ring = torch.empty((B, nw, c), dtype=dt, device=device)
        self.hring = torch.empty((B, nw, c), dtype=dt, device=device)
        dsc = L.compress_desc(batch=B, d=d, c=c, m=m, overlap=ov)
        dsi = L.compress_desc(batch=B, d=d, c=cI, m=m, overlap=ov)
        dsh = L.compress_desc(batch=B, d=d, c=c, m=mh, overlap=0)
        self.st = torch.empty(L.csa_state_bytes(dsc) // 4, dtype=torch.float32, device=device)
        self.sti = torch.empty(L.csa_state_bytes(dsi) // 4, dtype=torch.float32, device=device)
        self.sth = torch.empty(L.csa_state_bytes(dsh) // 4, dtype=torch.float32, device=device)
        self.idx = torch.empty((B, cfg["k"]), dtype=torch.int32, device=device)
        self.side = None  # side streams of the decode step, made on first use
        self.out_c = torch.empty((B, nh, c), dtype=dt, device=device)
        self.out_h = torch.empty((B, nh, c), dtype=dt, device=device)
        # build the caches: prefill of tokens [0, t) for every sequence
        ps, psi, psh = self.st.numel() // B, self.sti.numel() // B, self.sth.numel() // B
        for b in range(B):
            Hb = I.normal((t + 1, d), (seed, name, "H", b), chunk_rows=65536, **kw)
            self.h[b] = Hb[t]
            Hp = Hb[:t]
            a = L.csa_compress_prefill(Hp, g["csa_Wkv"], g["csa_Wz"], g["csa_ape"], m, ov,
                                       W_win=g["csa_Wwin"], rope_dims=r, n_win=nw, want_win=False,
                                       want_ring=True, want_state=True, out_comp=self.cache[b, : t // m])
            self.ring[b].copy_(a["ring"])
            self.st[b * ps:(b + 1) * ps].copy_(a["state"])
            a = L.csa_compress_prefill(Hp, g["WI_kv"], g["WI_z"], g["apeI"], m, ov, want_state=True,
                                       out_comp=self.kcache[b, : t // m])
            self.sti[b * psi:(b + 1) * psi].copy_(a["state"])
            a = L.csa_compress_prefill(Hp, g["hca_Wkv"], g["hca_Wz"], g["hca_ape"], mh, 0,
                                       W_win=g["hca_Wwin"], rope_dims=r, n_win=nw, want_win=False,
                                       want_ring=True, want_state=True, out_comp=self.hcache[b, : t // mh])
            self.hring[b].copy_(a["ring"])
            self.sth[b * psh:(b + 1) * psh].copy_(a["state"])
            del Hb, Hp, a
        torch.cuda.synchronize()
        for key in [k for k in L._WS if k[1] == "default"]:  # free the build scratch
            L._WS.pop(key)
        torch.cuda.empty_cache()

    def make_kv8(self):
        """FP8 copies of the two window rings and entry caches (the format of
        csa_kv_fp8_quant), for step(kv8=True)."""
        r = self.cfg["rope_dims"]
        self.kv8 = {n: L.csa_kv_fp8_quant(getattr(self, n), r)
                    for n in ("ring", "cache", "hring", "hcache")}
        torch.cuda.synchronize()

    def step(self, streams=True, kv8=False):
        """One decode step.  Its chains are independent until the sparse
        attention: (indexer compressor -> selection), (scoring of the cached
        indexer keys -> selection), (CSA compressor) and (HCA compressor ->
        dense attention).  The scoring reads only keys that precede this
        step, so it starts with the step, beside the compressors.  With
        `streams` each compressor has a forked stream (the HCA chain runs on
        the current one); the scoring's stream then waits for the indexer
        compressor's, selects, waits for the CSA compressor's and runs the
        sparse attention; the current stream joins the others at the end.
        The scoring is enqueued first (the compressors finish long before
        their results are needed; in a graph the branch enqueued first starts
        with the step, the others some microseconds later).  Each chain has
        its own workspaces.  With `kv8` the
        attention reads FP8 rings and caches (make_kv8): each compressor's new
        bf16 row (window slot, and the entry when one is emitted) is converted
        into them by csa_kv_fp8_quant_decode on the compressor's stream."""
        c, g = self.cfg, self.g
        m, ov, r = c["m"], c["overlap"], c["rope_dims"]
        main = torch.cuda.current_stream()
        if streams:
            if self.side is None or len(self.side) < 3:
                self.side = (torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream())
            sb, sc, sd = self.side
            sb.wait_stream(main)
            sc.wait_stream(main)
            sd.wait_stream(main)
        else:
            sb = sc = sd = main
        # the scoring first: it is the one chain without slack, and in a graph
        # the branch enqueued first starts with the step
        with torch.cuda.stream(sd):
            L.csa_index_topk_decode_score(g["qI"], g["wI"], self.kcache, self.pos, m, c["k"])
        with torch.cuda.stream(sb):
            L.csa_compress_decode(self.h, self.pos, g["WI_kv"], g["WI_z"], g["apeI"], m, ov, self.sti,
                                  self.kcache, ws_slot="decode_proj_idx")
        with torch.cuda.stream(sc):
            L.csa_compress_decode(self.h, self.pos, g["csa_Wkv"], g["csa_Wz"], g["csa_ape"], m, ov,
                                  self.st, self.cache, W_win=g["csa_Wwin"], win_ring=self.ring,
                                  rope_dims=r, ws_slot="decode_proj_csa")
            if kv8:
                L.csa_kv_fp8_quant_decode(self.cache, self.pos, self.kv8["cache"], r, m=m)
                L.csa_kv_fp8_quant_decode(self.ring, self.pos, self.kv8["ring"], r, ring=True)
        L.csa_compress_decode(self.h, self.pos, g["hca_Wkv"], g["hca_Wz"], g["hca_ape"],
                              c["m_hca"], 0, self.sth, self.hcache, W_win=g["hca_Wwin"],
                              win_ring=self.hring, rope_dims=r, ws_slot="decode_proj_hca")
        if kv8:
            L.csa_kv_fp8_quant_decode(self.hcache, self.pos, self.kv8["hcache"], r, m=c["m_hca"])
            L.csa_kv_fp8_quant_decode(self.hring, self.pos, self.kv8["hring"], r, ring=True)
        with torch.cuda.stream(sd):
            if streams:
                sd.wait_stream(sb)
            L.csa_index_topk_decode_select(g["qI"], g["wI"], self.kcache, self.pos, m, c["k"],
                                           out=self.idx)
            if streams:
                sd.wait_stream(sc)
            if kv8:
                L.csa_sparse_mqa_decode_fp8(g["csa_q"], self.kv8["ring"], self.kv8["cache"],
                                            self.idx, self.pos, g["csa_sink"], r, out=self.out_c)
            else:
                L.csa_sparse_mqa_decode(g["csa_q"], self.ring, self.cache, self.idx, self.pos,
                                        g["csa_sink"], rope_dims=r, out=self.out_c)
        if kv8:
            L.hca_dense_mqa_decode_fp8(g["hca_q"], self.kv8["hring"], self.kv8["hcache"], self.pos,
                                       g["hca_sink"], c["m_hca"], r, out=self.out_h)
        else:
            L.hca_dense_mqa_decode(g["hca_q"], self.hring, self.hcache, self.pos, g["hca_sink"],
                                   c["m_hca"], rope_dims=r, out=self.out_h)
        if streams:
            main.wait_stream(sb)
            main.wait_stream(sc)
            main.wait_stream(sd)

    def step_fp4(self, streams=True):
        """The same step with the FP4 indexer path: q^I is rotated and
        quantised, the indexer compressor's new entry is quantised into the
        FP4 key cache, and the top-k reads FP4 keys (the attention and the
        other chains are unchanged)."""
        c, g = self.cfg, self.g
        m, ov, r = c["m"], c["overlap"], c["rope_dims"]
        if getattr(self, "kc", None) is None:  # the FP4 key cache, made once
            self.kc, self.ke = L.csa_indexer_fp4_quant(self.kcache)
            self.qc, self.qe = L.csa_indexer_fp4_quant(g["qI"])
        main = torch.cuda.current_stream()
        if streams:
            if self.side is None:
                self.side = (torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream())
            sb, sc = self.side[:2]
            sb.wait_stream(main)
            sc.wait_stream(main)
        else:
            sb = sc = main
        with torch.cuda.stream(sb):
            L.csa_indexer_fp4_quant(g["qI"], out=(self.qc, self.qe))
            L.csa_compress_decode(self.h, self.pos, g["WI_kv"], g["WI_z"], g["apeI"], m, ov, self.sti,
                                  self.kcache, ws_slot="decode_proj_idx")
            L.csa_indexer_fp4_quant_decode(self.kcache, self.pos, m, self.kc, self.ke)
            L.csa_index_topk_decode_fp4(self.qc, self.qe, g["wI"], self.kc, self.ke, self.pos, m,
                                        c["k"], out=self.idx)
        with torch.cuda.stream(sc):
            L.csa_compress_decode(self.h, self.pos, g["csa_Wkv"], g["csa_Wz"], g["csa_ape"], m, ov,
                                  self.st, self.cache, W_win=g["csa_Wwin"], win_ring=self.ring,
                                  rope_dims=r, ws_slot="decode_proj_csa")
        L.csa_compress_decode(self.h, self.pos, g["hca_Wkv"], g["hca_Wz"], g["hca_ape"],
                              c["m_hca"], 0, self.sth, self.hcache, W_win=g["hca_Wwin"],
                              win_ring=self.hring, rope_dims=r, ws_slot="decode_proj_hca")
        L.hca_dense_mqa_decode(g["hca_q"], self.hring, self.hcache, self.pos, g["hca_sink"],
                               c["m_hca"], rope_dims=r, out=self.out_h)
        if streams:
            main.wait_stream(sb)
            main.wait_stream(sc)
        L.csa_sparse_mqa_decode(g["csa_q"], self.ring, self.cache, self.idx, self.pos, g["csa_sink"],
                                rope_dims=r, out=self.out_c)

    def paginate(self, page_tokens=128, seed=0):
        """Copies of the three entry caches as shuffled pools of pages of
        `page_tokens` raw tokens (page_tokens / m entries each) with their
        page tables, for step_paged."""
        dev = self.cache.device
        gen = torch.Generator(device="cpu").manual_seed(seed)
        self.pg = {}
        for name, cache, m in (("cache", self.cache, self.cfg["m"]),
                               ("kcache", self.kcache, self.cfg["m"]),
                               ("hcache", self.hcache, self.cfg["m_hca"])):
            B, ne, w = cache.shape
            pe = max(1, page_tokens // m)
            npg = -(-ne // pe)
            table = torch.randperm(B * npg, generator=gen).to(torch.int32).reshape(B, npg)
            e = torch.arange(ne)
            rows = (table[:, e // pe].long() * pe + (e % pe)[None]).reshape(-1).to(dev)
            pool = torch.empty((B * npg * pe, w), dtype=cache.dtype, device=dev)
            pool[rows] = cache.reshape(B * ne, w)
            self.pg[name] = (pool, table.to(dev), pe)
        torch.cuda.synchronize()

    def step_paged(self, streams=True):
        """The decode step over the paged caches of paginate(): the same calls
        as step() through their _paged entry points."""
        c, g = self.cfg, self.g
        m, ov, r = c["m"], c["overlap"], c["rope_dims"]
        (cp, ct, ce), (kp, kt, ke), (hp, ht, he) = (self.pg["cache"], self.pg["kcache"],
                                                    self.pg["hcache"])
        main = torch.cuda.current_stream()
        if streams:
            if self.side is None:
                self.side = (torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream())
            sb, sc = self.side[:2]
            sb.wait_stream(main)
            sc.wait_stream(main)
        else:
            sb = sc = main
        with torch.cuda.stream(sb):
            L.csa_compress_decode_paged(self.h, self.pos, g["WI_kv"], g["WI_z"], g["apeI"], m, ov,
                                        self.sti, kp, kt, ke, n_entries=self.kcache.shape[1],
                                        ws_slot="decode_proj_idx")
            L.csa_index_topk_decode_paged(g["qI"], g["wI"], kp, kt, ke, self.pos, m, c["k"],
                                          n_entries=self.kcache.shape[1], out=self.idx)
        with torch.cuda.stream(sc):
            L.csa_compress_decode_paged(self.h, self.pos, g["csa_Wkv"], g["csa_Wz"], g["csa_ape"],
                                        m, ov, self.st, cp, ct, ce, W_win=g["csa_Wwin"],
                                        win_ring=self.ring, n_entries=self.cache.shape[1],
                                        rope_dims=r, ws_slot="decode_proj_csa")
        L.csa_compress_decode_paged(self.h, self.pos, g["hca_Wkv"], g["hca_Wz"], g["hca_ape"],
                                    c["m_hca"], 0, self.sth, hp, ht, he, W_win=g["hca_Wwin"],
                                    win_ring=self.hring, n_entries=self.hcache.shape[1],
                                    rope_dims=r, ws_slot="decode_proj_hca")
        L.hca_dense_mqa_decode_paged(g["hca_q"], self.hring, hp, ht, he, self.pos, g["hca_sink"],
                                     c["m_hca"], n_entries=self.hcache.shape[1], rope_dims=r,
                                     out=self.out_h)
        if streams:
            main.wait_stream(sb)
            main.wait_stream(sc)
        L.csa_sparse_mqa_decode_paged(g["csa_q"], self.ring, cp, ct, ce, self.idx, self.pos,
                                      g["csa_sink"], n_entries=self.cache.shape[1], rope_dims=r,
                                      out=self.out_c)

    def algorithmic_bytes(self, kv8=False):
        """Bytes a decode step must move at least once (bf16 = 2 B; with
        `kv8` the attention's window rows and entries are FP8 rows)."""
        c = self.cfg
        B, ctx, d, cc, m, ov = c["batch"], c["ctx"], c["d"], c["c"], c["m"], c["overlap"]
        t = ctx - 1
        vis, vis_h = (t + 1) // m, (t + 1) // c["m_hca"]
        nw = min(c["n_win"], t + 1)
        e = 2
        w, wI = (1 + ov) * cc, (1 + ov) * c["cI"]
        weights = d * (2 * w + cc + 2 * wI + 2 * cc + cc) * e
        keys = B * vis * c["cI"] * e
        row = L.kv_fp8_row_bytes(cc, c["rope_dims"]) if kv8 else cc * e
        csa = B * (nw + min(c["k"], vis)) * row
        hca = B * (nw + vis_h) * row
        qo = 4 * B * c["nh"] * cc * e + B * (c["hI"] * c["cI"] + c["hI"]) * e + B * d * e
        return weights + keys + csa + hca + qo


def prefill_flops(cfg):
    """Algorithmic FLOPs of one CSA prefill step, by stage: the projections
    (2 d per output column per token: C, Z and window rows of the main
    compressor, C and Z of the indexer's), the index scores (2 hI cI per
    visible (token, entry) pair) and the attention (4 nh c per (token,
    candidate) pair)."""
    n, d, c, m, ov = cfg["n"], cfg["d"], cfg["c"], cfg["m"], cfg["overlap"]
    w, wI = (1 + ov) * c, (1 + ov) * cfg["cI"]
    t = np.arange(n, dtype=np.int64)
    vis = (t + 1) // m
    pairs = np.minimum(cfg["n_win"], t + 1) + np.minimum(cfg["k"], vis)
    return {"projection": 2.0 * n * d * (2 * w + c + 2 * wI),
            "index": 2.0 * cfg["hI"] * cfg["cI"] * float(vis.sum()),
            "attention": 4.0 * cfg["nh"] * c * float(pairs.sum())}


def c1_record(steps, warmup, dev):
    """The 2K-token fp32 CSA workload end to end (compressors, index + top-k,
    sparse attention): step time and its fraction of the fp32 peak."""
    cfg = configs.get("csa_prefill_2k_f32")
    pf = CsaPrefill(cfg, dev)
    ms = float(np.mean(time_region(pf.step, steps, warmup)))
    st = {nm: float(np.mean(time_region(fn, max(3, steps), 1)))
          for nm, fn in (("compress", pf.compress), ("index_topk", pf.index),
                         ("sparse_mqa", pf.attend))}
    fl = prefill_flops(cfg)
    tot = sum(fl.values())
    return {"workload": cfg["name"], "ms_per_step": ms, "tokens_per_s": cfg["n"] / (ms * 1e-3),
            "stages_ms": st, "gflop": {k_: v / 1e9 for k_, v in fl.items()},
            "tflops": tot / (ms * 1e-3) / 1e12, "frac_fp32_peak": tot / (ms * 1e-3) / PEAK_FP32}


def oracle_times():
    """The CPU fp64 oracle timed on whole workloads (no GPU): the 2K fp32 CSA
    prefill and the 16K bf16 HCA prefill in full, and one decode step of one
    sequence at 128K and at 1M context (the new token's projections by the
    three compressors with the pooling and epilogue of the block it closes,
    the index scores over every visible key and the top-k, the sparse and the
    dense attention rows), scaled by the batch for a whole step."""
    from oracle import csa_oracle as O
    cores = len(os.sched_getaffinity(0))
    f = lambda x: x.detach().to("cpu", torch.float64).numpy()  # noqa: E731
    out = {"cores": cores}
    # 2K fp32 CSA prefill, every stage for every token
    cfg = configs.get("csa_prefill_2k_f32")
    t = I.csa_prefill_inputs(cfg)
    n, m, ov, k, c = cfg["n"], cfg["m"], cfg["overlap"], cfg["k"], cfg["c"]
    H = f(t["H"])
    t0 = time.perf_counter()
    comp = O.compress_prefill(H, f(t["W_kv"]).T, f(t["W_z"]).T, f(t["ape"]), m, ov)
    win = O.window_rows(H, f(t["W_win"]).T)
    KI = O.compress_prefill(H, f(t["WI_kv"]).T, f(t["WI_z"]).T, f(t["apeI"]), m, ov)
    t1 = time.perf_counter()
    idx = O.topk(O.index_scores(f(t["qI"]), f(t["wI"]), KI, m), k, m)
    t2 = time.perf_counter()
    O.sparse_mqa_prefill(f(t["q"]), win, comp, idx, f(t["sink"]), cfg["n_win"], c ** -0.5)
    t3 = time.perf_counter()
    out[cfg["name"]] = {"s": t3 - t0, "stages_s": {"compress": t1 - t0, "index_topk": t2 - t1,
                                                    "sparse_mqa": t3 - t2}}
    # 16K bf16 HCA prefill
    cfg = configs.get("hca_prefill_16k_bf16")
    t = I.csa_prefill_inputs(cfg, with_indexer=False)
    n, m, c = cfg["n"], cfg["m"], cfg["c"]
    H = f(t["H"])
    t0 = time.perf_counter()
    comp = O.compress_prefill(H, f(t["W_kv"]).T, f(t["W_z"]).T, f(t["ape"]), m, 0, store="bf16")
    win = O.window_rows(H, f(t["W_win"]).T, store="bf16")
    t1 = time.perf_counter()
    O.dense_mqa_prefill(f(t["q"]), win, comp, f(t["sink"]), m, cfg["n_win"], c ** -0.5,
                        store="bf16")
    t2 = time.perf_counter()
    out[cfg["name"]] = {"s": t2 - t0, "stages_s": {"compress": t1 - t0, "dense_mqa": t2 - t1}}
    del H, comp, win
    # one decode step of one sequence
    rng = np.random.default_rng(0)
    for wname in ("decode_b32_128k_bf16", "decode_b4_1m_bf16"):
        dc = configs.get(wname)
        d, c, m, mh, ov, r = dc["d"], dc["c"], dc["m"], dc["m_hca"], dc["overlap"], dc["rope_dims"]
        tpos = dc["ctx"] - 1
        vis, vis_h, nw = (tpos + 1) // m, (tpos + 1) // mh, min(dc["n_win"], tpos + 1)
        w, wI = (1 + ov) * c, (1 + ov) * dc["cI"]
        h = rng.standard_normal((1, d))
        Wm = rng.standard_normal((d, 2 * w + c)) * d ** -0.5
        Wi = rng.standard_normal((d, 2 * wI)) * d ** -0.5
        Wh = rng.standard_normal((d, 3 * c)) * d ** -0.5
        blk = lambda rows, cols: rng.standard_normal((rows, cols))  # noqa: E731
        Cm, Zm, Ci, Zi, Ch, Zh = (blk((1 + ov) * m, w), blk((1 + ov) * m, w),
                                  blk((1 + ov) * m, wI), blk((1 + ov) * m, wI),
                                  blk(mh, c), blk(mh, c))
        qI, wIv = blk(dc["hI"], dc["cI"])[None], rng.uniform(size=(1, dc["hI"]))
        KI = blk(vis, dc["cI"])
        q = blk(dc["nh"], c)
        sink = blk(1, dc["nh"])[0]
        ent = O.rms_norm(blk(dc["k"], c), 1e-6)
        ent_h = O.rms_norm(blk(vis_h, c), 1e-6)
        wrows = O.rms_norm(blk(nw, c), 1e-6)
        t0 = time.perf_counter()
        O.project(h, Wm), O.project(h, Wi), O.project(h, Wh)
        for C_, Z_, ape_, mm, ovv in ((Cm, Zm, blk(m, w), m, ov), (Ci, Zi, blk(m, wI), m, ov),
                                      (Ch, Zh, blk(mh, c), mh, 0)):
            e_ = O.pool(C_, Z_, ape_, mm, ovv)[-1:]
            O.entry_epilogue(e_[:, :c] if e_.shape[1] > c else e_, [tpos], True, 1e-6, r,
                             10000.0, "bf16")
        t1 = time.perf_counter()
        sc = O.index_scores(qI, wIv, KI, m, t0=tpos)
        O.topk(sc, dc["k"], m, t0=tpos)
        t2 = time.perf_counter()
        O.attend_decode_row(q, tpos, wrows, ent, sink, c ** -0.5, rope_dims=r, store="bf16")
        O.attend_decode_row(q, tpos, wrows, ent_h, sink, c ** -0.5, rope_dims=r, store="bf16")
        t3 = time.perf_counter()
        out[wname] = {"s_per_sequence": t3 - t0, "s_per_step": (t3 - t0) * dc["batch"],
                      "batch": dc["batch"],
                      "stages_s_per_sequence": {"compressors": t1 - t0, "index_topk": t2 - t1,
                                                "attention": t3 - t2}}
        del KI
    return out


def cpu_baseline(pf, sample_tokens=2048, sample_rows=48):
    """Time the CPU fp64 oracle on a bounded sample of the prefill workload and
    scale to tokens/s: compressor on the first `sample_tokens` tokens, indexer
    + top-k and core attention on `sample_rows` query rows spread over the
    sequence (reusing the GPU's entries as the stage inputs)."""
    from oracle import csa_oracle as O
    cfg, t = pf.cfg, pf.t
    n, m, ov, r, k = cfg["n"], cfg["m"], cfg["overlap"], cfg["rope_dims"], cfg["k"]
    cores = len(os.sched_getaffinity(0))
    f = lambda x: x.detach().to("cpu", torch.float64).numpy()  # noqa: E731
    H = f(t["H"][:sample_tokens])
    Wkv, Wz, Ww, WIk, WIz = (f(t[x]).T for x in ("W_kv", "W_z", "W_win", "WI_kv", "WI_z"))
    ape, apeI = f(t["ape"]), f(t["apeI"])
    t0 = time.perf_counter()
    O.compress_prefill(H, Wkv, Wz, ape, m, ov, rope_dims=r, store="bf16")
    O.window_rows(H, Ww, rope_dims=r, store="bf16")
    O.compress_prefill(H, WIk, WIz, apeI, m, ov, store="bf16")
    t_comp = (time.perf_counter() - t0) / sample_tokens
    rows = np.linspace(n // 8, n - 1, sample_rows).astype(np.int64)
    KI = f(pf.kI)
    comp, win = f(pf.comp), f(pf.win)
    qI, wI = f(t["qI"][rows]), f(t["wI"][rows])
    q, sink = f(t["q"][rows]), f(t["sink"])
    t0 = time.perf_counter()
    idx = np.full((len(rows), k), -1, dtype=np.int64)
    for i, tok in enumerate(rows):
        sc = O.index_scores(qI[i][None], wI[i][None], KI[: (tok + 1) // m], m, t0=int(tok))
        idx[i] = O.topk(sc, k, m, t0=int(tok))[0]
    t_idx = (time.perf_counter() - t0) / len(rows)
    t0 = time.perf_counter()
    for i, tok in enumerate(rows):
        sel = idx[i][idx[i] >= 0]
        lo = max(0, tok - cfg["n_win"] + 1)
        O.attend_decode_row(q[i], int(tok), win[lo:tok + 1], comp[sel], sink, cfg["c"] ** -0.5,
                            rope_dims=r, store="bf16")
    t_att = (time.perf_counter() - t0) / len(rows)
    per_tok = t_comp + t_idx + t_att
    return {"value": 1.0 / per_tok, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"CPU fp64 oracle, {cores} host threads: compressor (main, window, indexer) on "
                      f"the first {sample_tokens} tokens; indexer+top-k and sparse MQA on "
                      f"{sample_rows} query rows spread over the 64K sequence; per-token stage "
                      f"times summed (compress {t_comp * 1e3:.3f} ms, index {t_idx * 1e3:.3f} ms, "
                      f"attention {t_att * 1e3:.3f} ms per token)"}


def backward_record(steps, dev="cuda"):
    """csa_sparse_mqa_backward and hca_dense_mqa_backward on the 2K-token fp32
    CSA workload's shapes (8 heads x 128, k = 64, window 128, m = 4; the
    dense call over the same entries), timed with events; algorithmic work
    10 nh c FLOP per (query, candidate) pair (logits, dp, dq and both parts
    of the row gradient), against the fp32 vector peak."""
    cfg = configs.get("csa_prefill_2k_f32")
    t = I.csa_prefill_inputs(cfg, device=dev)
    m, ov, k, nw, c, nh = cfg["m"], cfg["overlap"], cfg["k"], cfg["n_win"], cfg["c"], cfg["nh"]
    main_ = L.csa_compress_prefill(t["H"], t["W_kv"], t["W_z"], t["ape"], m, ov, W_win=t["W_win"])
    kI = L.csa_compress_prefill(t["H"], t["WI_kv"], t["WI_z"], t["apeI"], m, ov)
    idx = L.csa_index_topk_prefill(t["qI"], t["wI"], kI["comp"], m, k)
    dout = I.normal(tuple(t["q"].shape), (0, cfg["name"], "dout"), device=dev)
    n = cfg["n"]
    tt = torch.arange(n, device=dev)
    win_pairs = int(torch.clamp(tt + 1, max=nw).sum().item())
    pairs_s = win_pairs + int((idx >= 0).sum().item())
    pairs_d = win_pairs + int(torch.clamp((tt + 1) // m, max=main_["comp"].shape[0]).sum().item())
    res = {"workload": cfg["name"] + " attention backward", "n": n, "nh": nh, "c": c, "k": k}
    for nm, fn, pairs in (
            ("sparse", lambda: L.csa_sparse_mqa_backward(t["q"], main_["win"], main_["comp"], idx,
                                                         t["sink"], dout, n_win=nw), pairs_s),
            ("dense", lambda: L.hca_dense_mqa_backward(t["q"], main_["win"], main_["comp"],
                                                       t["sink"], dout, m, n_win=nw), pairs_d)):
        ms = float(np.median(time_region(fn, max(5, steps), 2)))
        fl = 10.0 * nh * c * pairs
        res[nm] = {"ms": ms, "pairs": pairs, "tokens_per_s": n / (ms * 1e-3),
                   "tflops": fl / (ms * 1e-3) / 1e12, "frac_fp32": fl / (ms * 1e-3) / PEAK_FP32}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pmc-probe", nargs="?", const="mqa", default=None,
                    choices=("mqa", "hca", "decode"),
                    help="only the copy reference and the kernels of one workload, for "
                         "counter passes")
    ap.add_argument("--oracle-times", action="store_true",
                    help="only time the CPU oracle on whole workloads (no GPU) and print that")
    a = ap.parse_args()
    if a.oracle_times:
        print(json.dumps({"oracle_times": oracle_times()}), flush=True)
        return
    if a.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {a.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    L.load()
    if a.pmc_probe:
        pmc_probe(a.pmc_probe)
        return
    dev = "cuda"
    cfg = configs.get("csa_prefill_64k_bf16")
    print(f"[bench] building inputs for {cfg['name']}", file=sys.stderr, flush=True)
    pf = CsaPrefill(cfg, dev)
    torch.cuda.synchronize()
    print("[bench] timing prefill steps", file=sys.stderr, flush=True)
    times = time_region(pf.step, a.steps, a.warmup)
    ms = float(np.mean(times))
    n = cfg["n"]
    # dominant kernel, timed live with events on the stream it runs on
    att_t = time_region(pf.attend, max(3, a.steps), 1)
    att_ms = float(np.mean(att_t))
    flops, pairs = pf.attn_flops()
    comp_ms = float(np.mean(time_region(pf.compress, max(3, a.steps), 1)))
    idx_ms = float(np.mean(time_region(pf.index, max(3, a.steps), 1)))
    achieved = flops / (att_ms * 1e-3)
    rec = {
        "metric": "CSA prefill tokens/s at 64K (1 GPU); decode us/token at 128K and 1M context",
        "value": n / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1) / U(0,1) inputs)",
        "config": {"workload": cfg["name"], "layer": "CSA", "n": n, "d": cfg["d"], "c": cfg["c"],
                   "m": cfg["m"], "overlap": cfg["overlap"], "indexer": f"{cfg['hI']}x{cfg['cI']}",
                   "k": cfg["k"], "nh": cfg["nh"], "n_win": cfg["n_win"],
                   "rope_dims": cfg["rope_dims"], "parallelism": "none (1 GPU)"},
        "stages_ms": {"compress": comp_ms, "index_topk": idx_ms, "sparse_mqa": att_ms},
        "roofline": {"kernel": "mqa_prefill_bf16_kernel (csa_sparse_mqa_prefill)", "bound": "mfma",
                     "achieved": achieved / 1e12, "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16, "traffic": measured_traffic(),
                     "algorithmic": f"{flops:.4g} FLOP per launch = 4 x 64 heads x 512 x "
                                    f"{pairs} (token, candidate) pairs"},
    }
    del att_t
    # the same prefill in 8 chunks of 8192 tokens (chunked prefill): its time,
    # and whether its outputs equal the one-shot prefill's bit for bit
    pf.step()
    one_shot = [x.clone() for x in (pf.comp, pf.kI, pf.idx, pf.out)]
    pf.step_chunked(8192)
    same = all(torch.equal(a_.view(torch.int16) if a_.dtype == torch.bfloat16 else a_,
                           b_.view(torch.int16) if b_.dtype == torch.bfloat16 else b_)
               for a_, b_ in zip(one_shot, (pf.comp, pf.kI, pf.idx, pf.out)))
    ch_ms = float(np.mean(time_region(lambda: pf.step_chunked(8192), a.steps, 1)))
    rec["chunked_prefill"] = {"chunk_tokens": 8192, "chunks": -(-n // 8192), "ms_per_step": ch_ms,
                              "tokens_per_s": n / (ch_ms * 1e-3),
                              "outputs_equal_one_shot": bool(same)}
    del one_shot
    # one 8192-token chunk ending a 1M-token context: its rows see up to
    # 262144 entries, so the selection runs the decode top-k over row batches
    st1m = chunk_at_context(pf, 1 << 20, 8192, max(3, a.steps), dev)
    rec["chunked_prefill"]["chunk_ending_1m_context"] = {
        "stages_ms": st1m, "ms": sum(st1m.values()),
        "tokens_per_s": 8192 / (sum(st1m.values()) * 1e-3)}
    # the HCA layer's prefill at its own workload (16K) and at 64K tokens
    rec["hca_prefill"] = {}
    for n_h in (16384, 65536):
        hcfg = dict(configs.get("hca_prefill_16k_bf16", n=n_h))
        hp = HcaPrefill(hcfg, dev)
        h_ms = float(np.mean(time_region(hp.step, a.steps, a.warmup)))
        ha_ms = float(np.mean(time_region(hp.attend, max(3, a.steps), 1)))
        hf = hp.attn_flops()
        rec["hca_prefill"][f"n{n_h}"] = {
            "ms_per_step": h_ms, "tokens_per_s": n_h / (h_ms * 1e-3),
            "stages_ms": {"compress": h_ms - ha_ms, "dense_mqa": ha_ms},
            "dense_mqa_tflops": hf / (ha_ms * 1e-3) / 1e12,
            "dense_mqa_frac": hf / (ha_ms * 1e-3) / PEAK_BF16,
            # q and out, window rows and entries, each once (bf16)
            "dense_mqa_hbm_frac": 2.0 * hcfg["c"] * (2 * n_h * hcfg["nh"] + n_h + n_h // hcfg["m"])
                                  / (ha_ms * 1e-3) / PEAK_HBM}
        del hp
        torch.cuda.empty_cache()
    # the 2K-token fp32 workload end to end, against the fp32 peak
    rec["c1_prefill_2k_f32"] = c1_record(a.steps, a.warmup, dev)
    # the 64K workload without overlapping compression (ov = 0)
    pf0 = CsaPrefill(dict(cfg, overlap=0), dev)
    ms0 = float(np.mean(time_region(pf0.step, a.steps, a.warmup)))
    rec["ov0_prefill"] = {
        "overlap": 0, "ms_per_step": ms0, "tokens_per_s": n / (ms0 * 1e-3),
        "stages_ms": {nm: float(np.mean(time_region(fn, max(3, a.steps), 1)))
                      for nm, fn in (("compress", pf0.compress), ("index_topk", pf0.index),
                                     ("sparse_mqa", pf0.attend))}}
    del pf0
    torch.cuda.empty_cache()
    # the deterministic attention backward at the 2K fp32 workload: entries,
    # window rows and the selection from the forward path, dout ~ N(0, 1)
    rec["backward"] = backward_record(a.steps)
    # selection on bf16-rounded index scores ([R] section 4.4): its time and
    # its recall of the fp32-score selection, row by row (-1 slots excluded)
    idx32 = pf.idx.clone()
    idx16 = torch.empty_like(idx32)

    def index_bf16():
        L.csa_index_topk_prefill(pf.t["qI"], pf.t["wI"], pf.kI, cfg["m"], cfg["k"], out=idx16,
                                 scores="bf16")
    ib_ms = float(np.mean(time_region(index_bf16, max(3, a.steps), 1)))
    pos = torch.searchsorted(idx16, idx32).clamp_(max=idx16.shape[1] - 1)
    hit = (idx16.gather(1, pos) == idx32) & (idx32 >= 0)
    rec["index_bf16_scores"] = {
        "index_topk_ms": ib_ms, "index_topk_fp32_ms": idx_ms, "speedup": idx_ms / ib_ms,
        "recall_of_fp32_selection": float(hit.sum().item()) / float((idx32 >= 0).sum().item())}
    # the FP4 indexer path at prefill ([R] section 4.4): q^I and the keys
    # rotated and quantised to E2M1, scores from the scaled FP4 matrix
    # instruction; its time, the quantisation it adds, and its recall of the
    # fp32-score selection on the same inputs
    qc, qe = L.csa_indexer_fp4_quant(pf.t["qI"])
    kc, ke = L.csa_indexer_fp4_quant(pf.kI)

    def quant_fp4():
        L.csa_indexer_fp4_quant(pf.t["qI"], out=(qc, qe))
        L.csa_indexer_fp4_quant(pf.kI, out=(kc, ke))

    def index_fp4():
        L.csa_index_topk_prefill_fp4(qc, qe, pf.t["wI"], kc, ke, cfg["m"], cfg["k"], out=idx16)
    i4_ms = float(np.mean(time_region(index_fp4, max(3, a.steps), 1)))
    q4_ms = float(np.mean(time_region(quant_fp4, max(3, a.steps), 1)))
    index_fp4()
    pos = torch.searchsorted(idx16, idx32).clamp_(max=idx16.shape[1] - 1)
    hit = (idx16.gather(1, pos) == idx32) & (idx32 >= 0)
    rec["index_fp4"] = {
        "index_topk_ms": i4_ms, "quant_ms": q4_ms, "index_topk_fp32_ms": idx_ms,
        "speedup_with_quant": idx_ms / (i4_ms + q4_ms),
        "key_bytes_per_entry": [kc.shape[-1] + ke.shape[-1], 2 * pf.kI.shape[-1]],
        "recall_of_fp32_selection": float(hit.sum().item()) / float((idx32 >= 0).sum().item())}
    del idx32, idx16, pos, hit, qc, qe, kc, ke
    # the whole layer around the four calls (query path and output projection
    # added), on the same workload
    print("[bench] timing the full CSA layer", file=sys.stderr, flush=True)
    lay = CsaLayer(pf, dev)
    lay_ms = float(np.mean(time_region(lay.step, a.steps, a.warmup)))
    qp_ms = float(np.mean(time_region(lay.qproj, max(3, a.steps), 1)))
    op_ms = float(np.mean(time_region(lay.oproj, max(3, a.steps), 1)))
    qf, of = lay.proj_flops()
    rec["layer"] = {
        "workload": cfg["name"] + " + query path + grouped output projection",
        "widths": {"d_c": cfg["d_c"], "groups": cfg["groups"], "d_g": cfg["d_g"]},
        "ms_per_step": lay_ms, "tokens_per_s": n / (lay_ms * 1e-3),
        "stages_ms": {"query_proj": qp_ms, "output_proj": op_ms},
        "query_proj_tflops": qf / (qp_ms * 1e-3) / 1e12,
        "output_proj_tflops": of / (op_ms * 1e-3) / 1e12,
        "output_proj_frac": of / (op_ms * 1e-3) / PEAK_BF16,
        "algorithmic": f"query path {qf:.4g} FLOP, output projection {of:.4g} FLOP per step"}
    del lay
    torch.cuda.empty_cache()
    if not a.no_decode:
        dec = {}
        cf = CacheFlush(dev)
        flush = cf.clean

        def med_us(ts):
            return float(np.median(ts)) * 1e3

        for wname in ("decode_b32_128k_bf16", "decode_b4_1m_bf16"):
            dc = configs.get(wname)
            print(f"[bench] building decode state for {wname}", file=sys.stderr, flush=True)
            hd = HybridDecode(dc, dev)
            print(f"[bench] timing {wname}", file=sys.stderr, flush=True)
            nd = max(20, a.steps)  # decode steps are short: at least 20 timed
            tt = time_ahead(hd.step, nd, 3, cf.clean)
            tw = time_ahead(hd.step, nd, 3, cf.warm)
            td = time_ahead(hd.step, nd, 3, cf.dirty)
            g = graph_of(hd.step)  # the same step, launched as one HIP graph
            tg = time_ahead(g.replay, nd, 3, cf.clean)
            tgw = time_ahead(g.replay, nd, 3, cf.warm)
            us, ug = med_us(tt), med_us(tg)
            byts = hd.algorithmic_bytes()
            dec[wname] = {"us_per_step": us, "us_per_token": us / dc["batch"],
                          "us_per_step_p10_p90": [float(np.percentile(tt, 10)) * 1e3,
                                                  float(np.percentile(tt, 90)) * 1e3],
                          "graph_us_per_step_p10_p90": [float(np.percentile(tg, 10)) * 1e3,
                                                        float(np.percentile(tg, 90)) * 1e3],
                          "us_per_step_warm_cache": med_us(tw),
                          "us_per_step_dirty_flush": med_us(td),
                          "graph_us_per_step": ug, "graph_us_per_token": ug / dc["batch"],
                          "graph_us_per_step_warm_cache": med_us(tgw),
                          "batch": dc["batch"], "ctx": dc["ctx"], "k": dc["k"],
                          "hbm_bytes_algorithmic": byts,
                          "hbm_frac": byts / (us * 1e-6) / PEAK_HBM,
                          "graph_hbm_frac": byts / (ug * 1e-6) / PEAK_HBM}
            # the step at t = ctx, which emits no entry (the graph reads the
            # position from device memory)
            hd.pos.fill_(dc["ctx"])
            tne = time_ahead(hd.step, nd, 3, flush)
            tneg = time_ahead(g.replay, nd, 3, flush)
            hd.pos.fill_(dc["ctx"] - 1)
            dec[wname]["no_emission_t_ctx"] = {"us_per_step": med_us(tne),
                                               "graph_us_per_step": med_us(tneg)}
            del g
            # the FP4 indexer path (rotation + E2M1 keys and q^I): the top-k
            # over FP4 keys against the same call over bf16 keys, and how much
            # of the bf16-key selection it recalls
            c_, g_ = hd.cfg, hd.g
            kc, ke = L.csa_indexer_fp4_quant(hd.kcache)
            qc, qe = L.csa_indexer_fp4_quant(g_["qI"])
            idx4 = torch.empty_like(hd.idx)

            def topk_bf16():
                L.csa_index_topk_decode(g_["qI"], g_["wI"], hd.kcache, hd.pos, c_["m"], c_["k"],
                                        out=hd.idx)

            def topk_fp4():
                L.csa_index_topk_decode_fp4(qc, qe, g_["wI"], kc, ke, hd.pos, c_["m"], c_["k"],
                                            out=idx4)
            t16 = med_us(time_ahead(graph_of(topk_bf16).replay, nd, 3, flush))
            t4 = med_us(time_ahead(graph_of(topk_fp4).replay, nd, 3, flush))
            topk_bf16()
            topk_fp4()
            pos_ = torch.searchsorted(idx4, hd.idx).clamp_(max=idx4.shape[1] - 1)
            hit = (idx4.gather(1, pos_) == hd.idx) & (hd.idx >= 0)
            tstep = time_ahead(hd.step_fp4, nd, 3, flush)
            gf = graph_of(hd.step_fp4)
            tgs = time_ahead(gf.replay, nd, 3, flush)
            del gf
            dec[wname]["fp4_indexer"] = {
                "us_per_step": float(np.median(tstep)) * 1e3,
                "graph_us_per_step": float(np.median(tgs)) * 1e3,
                "topk_us_fp4_keys": t4, "topk_us_bf16_keys": t16,
                "key_bytes_per_entry": [kc.shape[-1] + ke.shape[-1], 2 * hd.kcache.shape[-1]],
                "recall_of_bf16_selection": float(hit.sum().item()) / float((hd.idx >= 0).sum().item())}
            del kc, ke, qc, qe, idx4, pos_, hit
            # FP8 KV rows (E4M3 codes with block-64 scales, RoPE channels in
            # bf16): the same step with the attention reading FP8 rings and
            # caches, and each attention call alone beside its bf16 twin
            hd.make_kv8()
            k8 = hd.kv8

            def att(fp8, sparse):
                if sparse and fp8:
                    return lambda: L.csa_sparse_mqa_decode_fp8(
                        g_["csa_q"], k8["ring"], k8["cache"], hd.idx, hd.pos, g_["csa_sink"],
                        c_["rope_dims"], out=hd.out_c)
                if sparse:
                    return lambda: L.csa_sparse_mqa_decode(
                        g_["csa_q"], hd.ring, hd.cache, hd.idx, hd.pos, g_["csa_sink"],
                        rope_dims=c_["rope_dims"], out=hd.out_c)
                if fp8:
                    return lambda: L.hca_dense_mqa_decode_fp8(
                        g_["hca_q"], k8["hring"], k8["hcache"], hd.pos, g_["hca_sink"],
                        c_["m_hca"], c_["rope_dims"], out=hd.out_h)
                return lambda: L.hca_dense_mqa_decode(
                    g_["hca_q"], hd.hring, hd.hcache, hd.pos, g_["hca_sink"], c_["m_hca"],
                    rope_dims=c_["rope_dims"], out=hd.out_h)
            att_us = {}
            for nm, fp8, sp in (("sparse_bf16", False, True), ("sparse_fp8", True, True),
                                ("dense_bf16", False, False), ("dense_fp8", True, False)):
                att_us[nm] = med_us(time_ahead(graph_of(att(fp8, sp)).replay, nd, 3, flush))
            s8 = lambda: hd.step(kv8=True)  # noqa: E731
            t8 = time_ahead(s8, nd, 3, flush)
            g8 = graph_of(s8)
            tg8 = time_ahead(g8.replay, nd, 3, flush)
            del g8
            b8 = hd.algorithmic_bytes(kv8=True)
            dec[wname]["fp8_kv"] = {
                "us_per_step": med_us(t8), "graph_us_per_step": med_us(tg8),
                "row_bytes": [L.kv_fp8_row_bytes(c_["c"], c_["rope_dims"]), 2 * c_["c"]],
                "hbm_bytes_algorithmic": b8, "hbm_frac": b8 / (med_us(t8) * 1e-6) / PEAK_HBM,
                "attention_graph_us_cold": att_us}
            del hd.kv8, k8
            # the same step over caches in shuffled pages of 128 raw tokens
            hd.paginate(128)
            gp = graph_of(hd.step_paged)
            tgp = time_ahead(gp.replay, nd, 3, flush)
            tgpw = time_ahead(gp.replay, nd, 3, cf.warm)
            del gp
            dec[wname]["paged"] = {
                "page_tokens": 128,
                "page_entries": {"csa": hd.pg["cache"][2], "indexer": hd.pg["kcache"][2],
                                 "hca": hd.pg["hcache"][2]},
                "graph_us_per_step": float(np.median(tgp)) * 1e3,
                "graph_us_per_step_warm_cache": med_us(tgpw)}
            del hd
            torch.cuda.empty_cache()
            # the same step without overlapping compression (ov = 0)
            hd0 = HybridDecode(dict(dc, overlap=0), dev)
            g0 = graph_of(hd0.step)
            t0e = time_ahead(hd0.step, nd, 3, flush)
            t0g = time_ahead(g0.replay, nd, 3, flush)
            b0 = hd0.algorithmic_bytes()
            dec[wname]["ov0"] = {"overlap": 0, "us_per_step": med_us(t0e),
                                 "graph_us_per_step": med_us(t0g), "hbm_bytes_algorithmic": b0,
                                 "hbm_frac": b0 / (med_us(t0e) * 1e-6) / PEAK_HBM}
            del g0, hd0
            torch.cuda.empty_cache()
        rec["decode"] = dec
    if not a.no_cpu_baseline:
        print("[bench] timing the CPU oracle sample", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(pf)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
