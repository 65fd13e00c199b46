"""Comparison helpers for the GPU-vs-oracle parity tests."""
import numpy as np
import torch

from oracle import csa_oracle as O


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def bf16_ulp(x):
    """Spacing of bfloat16 values at |x| (8 significant bits)."""
    x = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -126)))
    return 2.0 ** (e - 7)


BF16_ABS_SLACK = 1e-5


def bf16_midpoint_dist(x):
    """Distance from x to the nearest point halfway between two adjacent
    bfloat16 values (where round-to-nearest changes its decision)."""
    x = np.abs(np.asarray(x, np.float64))
    u = bf16_ulp(x)
    frac = np.mod(x / u, 1.0)
    return np.abs(frac - 0.5) * u


def _pair_max(a, rope_dims):
    """For the last rope_dims channels (adjacent pairs rotated together),
    the larger of each pair's two values; other channels unchanged."""
    a = np.array(a, np.float64, copy=True)
    if rope_dims:
        c = a.shape[-1]
        t = a[..., c - rope_dims:].reshape(a.shape[:-1] + (rope_dims // 2, 2))
        t[:] = t.max(axis=-1, keepdims=True)
        a[..., c - rope_dims:] = t.reshape(a.shape[:-1] + (rope_dims,))
    return a


def assert_stored_close(gpu, ref, dtype, what, atol_f32=3e-5, unrounded=None, prenorm=None,
                        rope_dims=0):
    """Stored entries / window rows (unit-RMS after QK-RMSNorm).

    fp32: within atol_f32 (fp32 accumulation of the projection and pooling).

    bf16: within one bf16 ulp of the oracle value (itself rounded to bf16)
    plus BF16_ABS_SLACK.  The slack covers fp32 accumulation error before the
    rounding: a value that nearly cancels (|x| ~ 1e-5) carries the same
    ~2e-6 absolute fp32 error as any other, which is many bf16 ulps of x.

    The row is rounded twice, before its RMSNorm and at store.  Where the
    GPU's fp32 pre-norm value and the oracle's fp64 one straddle a bf16
    rounding midpoint, the first rounding differs by one pre-norm ulp, i.e.
    by at most 2^-7 |y| after the norm (y the stored value), and the store
    rounding adds at most one ulp of y: such elements may differ by up to
    ulp(y) + 2^-7 |y|.  In the last rope_dims channels RoPE mixes each
    adjacent pair, so a flip in either member moves both by up to 2^-7 times
    the pair's norm.  These elements are allowed only as the rare event this
    is (at most 1 % of the elements, plus 8), and, when the oracle's pre-norm
    values are given, only where that value (or, in a rotated pair, either
    member's) lies within 1e-4 * max(1, |x|) of a midpoint (the fp32
    accumulation error of the pre-norm value)."""
    g, r = f64(gpu) if isinstance(gpu, torch.Tensor) else gpu, ref
    assert g.shape == r.shape, (what, g.shape, r.shape)
    err = np.abs(g - r)
    if dtype == "f32":
        bad = err > atol_f32
    else:
        tight = bf16_ulp(r) * 1.0001 + BF16_ABS_SLACK
        mag = np.abs(r)
        if rope_dims:
            c = r.shape[-1]
            pr = r[..., c - rope_dims:].reshape(r.shape[:-1] + (rope_dims // 2, 2))
            pn_ = np.repeat(np.sqrt((pr * pr).sum(-1)), 2, axis=-1)
            mag = mag.copy()
            mag[..., c - rope_dims:] = pn_
        wide = bf16_ulp(r) * 1.0001 + 2.0 ** -7 * mag * 1.01 + BF16_ABS_SLACK
        flip = (err > tight) & (err <= wide)
        if prenorm is not None:
            pn = np.asarray(prenorm, np.float64).reshape(r.shape)
            near = (bf16_midpoint_dist(pn) <= 1e-4 * np.maximum(1.0, np.abs(pn))).astype(np.float64)
            flip &= _pair_max(near, rope_dims) > 0
        nflip = int(flip.sum())
        assert nflip <= 0.01 * r.size + 8, (
            f"{what}: {nflip} of {r.size} elements need the pre-norm rounding allowance")
        bad = (err > tight) & ~flip
    if bad.any():
        where = np.argwhere(bad)[:5]
        detail = []
        for w in where:
            w = tuple(w)
            u = "" if unrounded is None else f" unrounded {unrounded[w]!r}"
            pn = "" if prenorm is None else f" pre-norm {np.asarray(prenorm).reshape(r.shape)[w]!r}"
            detail.append(f"at {w}: gpu {g[w]!r} oracle {r[w]!r}{u}{pn}")
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} elements off, max err "
                             f"{err.max():.3g}; " + "; ".join(detail))
    return float(err.max())


def assert_out_close(gpu, ref, dtype, what):
    """Attention outputs: max abs error <= 1e-4 (fp32) / 2e-2 (bf16)."""
    tol = 1e-4 if dtype == "f32" else 2e-2
    g = f64(gpu) if isinstance(gpu, torch.Tensor) else gpu
    err = np.abs(g - ref)
    assert err.max() <= tol, f"{what}: max abs err {err.max():.3g} > {tol}"
    return float(err.max())


def check_topk_sets(gpu_idx, scores, k, m, t0=0, rel_tau=1e-5):
    """Compare the GPU index rows with the oracle's top-k of `scores`
    (oracle fp64 scores from the same inputs the GPU used).  Sets must be
    equal except for members whose score lies within tau of the k-th score
    (tau = rel_tau * max(1, |k-th|)); padding must be exact.  Returns the
    number of rows whose sets differ inside the tie band."""
    g = np.asarray(gpu_idx)
    ref = O.topk(scores, k, m, t0=t0)
    n_tie_rows = 0
    for r in range(g.shape[0]):
        vis = int(min(scores.shape[1], (t0 + r + 1) // m))
        kt = min(k, vis)
        gr = g[r]
        assert np.all(gr[kt:] == -1), f"row {r}: padding wrong"
        gs = gr[:kt]
        assert np.all((gs >= 0) & (gs < vis)), f"row {r}: index out of visible range"
        assert len(set(gs.tolist())) == kt, f"row {r}: duplicate indices"
        assert np.all(np.diff(gs) > 0), f"row {r}: not ascending"
        os_ = set(ref[r, :kt].tolist())
        diff = set(gs.tolist()) ^ os_
        if diff:
            kth = np.sort(scores[r, :vis])[::-1][kt - 1]
            tau = rel_tau * max(1.0, abs(kth))
            for s in diff:
                assert abs(scores[r, s] - kth) <= tau, (
                    f"row {r}: entry {s} score {scores[r, s]!r} vs k-th {kth!r} outside tie band")
            n_tie_rows += 1
    return n_tie_rows


def check_bf16_selection(got, sc, k, m, t0=0):
    """GPU rows selected on bf16 scores against the oracle's selection on the
    fp64 scores rounded to bf16.  The GPU rounds fp32 scores, so an entry
    whose score sits within one bf16 step of the k-th rounded score may round
    the other way; only such entries may differ.  Returns the rows that
    differ."""
    ref = O.topk_bf16_scores(sc, k, m, t0=t0)
    rb = O.round_bf16(sc)
    nd = 0
    for r in range(got.shape[0]):
        vis = int(min(sc.shape[1], (t0 + r + 1) // m))
        kt = min(k, vis)
        g = got[r]
        assert np.all(g[kt:] == -1) and np.all(np.diff(g[:kt]) > 0), f"row {r}: layout"
        diff = set(g[:kt].tolist()) ^ set(ref[r, :kt].tolist())
        if diff:
            kth = np.sort(rb[r, :vis])[::-1][kt - 1]
            band = 1.01 * float(bf16_ulp(kth)) + 1e-6
            for s_ in diff:
                assert abs(sc[r, s_] - kth) <= band, f"row {r}: entry {s_} off the bf16 tie band"
            nd += 1
    return nd
