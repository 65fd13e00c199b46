"""The benchmark's decode step with its three independent chains on forked
streams gives bitwise the results of the same step on one stream, eagerly
and as a captured graph replayed several times."""
import pytest
import torch

import bench

pytestmark = pytest.mark.gpu


def _cfg():
    return dict(name="streams-check", kind="decode", dtype="bf16", batch=3, ctx=4100, d=512, c=512,
                m=4, overlap=1, m_hca=128, hI=16, cI=64, k=256, nh=64, n_win=128, rope_dims=64,
                qk_norm=1, eps=1e-6, theta=10000.0)


def test_decode_step_streams_match_one_stream(lib):
    print("[streams] decode step B=3 ctx=4100 d=512", flush=True)
    hd = bench.HybridDecode(_cfg(), "cuda")
    mutable = [hd.cache, hd.kcache, hd.hcache, hd.ring, hd.hring, hd.st, hd.sti, hd.sth]
    outs = [hd.idx, hd.out_c, hd.out_h] + mutable
    names = ["idx", "out_c", "out_h", "cache", "kcache", "hcache", "ring", "hring", "st", "sti", "sth"]
    snap = [x.clone() for x in mutable]

    def restore():
        for x, s in zip(mutable, snap):
            x.copy_(s)

    hd.step(streams=False)
    torch.cuda.synchronize()
    ref = [x.clone() for x in outs]

    restore()
    hd.step(streams=True)
    torch.cuda.synchronize()
    for n, a, b in zip(names, outs, ref):
        assert torch.equal(a, b), f"streams: {n} differs from the one-stream step"

    restore()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        hd.step(streams=True)
    for rep in range(3):
        restore()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"[streams] graph replay {rep}", flush=True)
        for n, a, b in zip(names, outs, ref):
            assert torch.equal(a, b), f"graph replay {rep}: {n} differs from the one-stream step"


def test_prefill_step_streams_match_one_stream(lib):
    """The benchmark's prefill step with the indexer chain on a forked stream
    gives bitwise the one-stream results."""
    from long_context_attention_10_amd import configs
    print("[streams] prefill step n=4096", flush=True)
    cfg = dict(configs.get("csa_prefill_64k_bf16", n=4096))
    cfg["name"] = "streams-check-prefill"
    pf = bench.CsaPrefill(cfg, "cuda")
    outs = [pf.comp, pf.win, pf.kI, pf.idx, pf.out]
    names = ["comp", "win", "kI", "idx", "out"]
    pf.step(streams=False)
    torch.cuda.synchronize()
    ref = [x.clone() for x in outs]
    for x in outs:
        x.zero_()
    for _ in range(2):
        pf.step(streams=True)
        torch.cuda.synchronize()
        for n, a, b in zip(names, outs, ref):
            assert torch.equal(a, b), f"streams: {n} differs from the one-stream step"
