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


def assert_stored_close(gpu, ref, dtype, what, atol_f32=3e-5, unrounded=None):
    """Stored entries/rows (unit-RMS after QK-RMSNorm): fp32 within atol_f32;
    bf16 within one bf16 ulp of the oracle value (itself rounded to bf16) plus
    BF16_ABS_SLACK.  The slack covers fp32 accumulation error before the
    rounding: a value that nearly cancels (|x| ~ 1e-5) carries the same
    ~2e-6 absolute fp32 error as any other, which is many bf16 ulps of x."""
    g, r = f64(gpu) if isinstance(gpu, torch.Tensor) else gpu, ref
    assert g.shape == r.shape, (what, g.shape, r.shape)
    err = np.abs(g - r)
    if dtype == "f32":
        bad = err > atol_f32
    else:
        bad = err > bf16_ulp(r) * 1.0001 + BF16_ABS_SLACK
    if bad.any():
        where = np.argwhere(bad)[:5]
        detail = []
        for w in where:
            w = tuple(w)
            u = "" if unrounded is None else f" unrounded {unrounded[w]!r}"
            detail.append(f"at {w}: gpu {g[w]!r} oracle {r[w]!r}{u}")
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
