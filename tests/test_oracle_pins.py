"""Pins for the CPU fp64 oracle: each test ties an oracle function to something
other than itself -- a hand-derived worked example, a closed form, an
invariant, a textbook/library routine, or brute force on tiny inputs.

Citation keys: [R] = page "DeepSeek-V4 技术解读报告" (juejin.cn), section 2.3;
[A] = page "DeepSeek-V4：算法架构" (1zeryu.github.io), code excerpts."""
import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import csa_oracle as O

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")))
RNG = np.random.default_rng(1234)


# --------------------------------------------------------------- pooling (O2)
def test_pool_hand_no_overlap():
    g = GOLD["pool_no_overlap"]
    out = O.pool(np.array(g["C"]), np.array(g["Z"]), np.array(g["ape"]), g["m"], g["overlap"])
    np.testing.assert_allclose(out, g["expected"], rtol=0, atol=1e-12)


def test_pool_hand_overlap():
    g = GOLD["pool_overlap"]
    out = O.pool(np.array(g["C"]), np.array(g["Z"]), np.array(g["ape"]), g["m"], g["overlap"])
    np.testing.assert_allclose(out, g["expected"], rtol=0, atol=1e-12)


@pytest.mark.parametrize("m,overlap", [(1, False), (3, False), (4, False), (2, True), (3, True), (4, True)])
def test_pool_weights_sum_to_one(m, overlap):
    n, c = 5 * m + 2, 6
    w = 2 if overlap else 1
    C = RNG.normal(size=(n, w * c))
    Z = RNG.normal(size=(n, w * c)) * 3
    ape = RNG.normal(size=(m, w * c))
    S = O.pool_weights(C, Z, ape, m, overlap)
    assert S.shape == (n // m, (2 if overlap else 1) * m, c)
    np.testing.assert_allclose(S.sum(axis=1), 1.0, atol=1e-12)
    assert np.all(S >= 0)
    if overlap:  # block 0 takes nothing from the (absent) previous block
        assert np.all(S[0, m:] == 0)


def test_pool_m1_is_identity():
    C = RNG.normal(size=(7, 4))
    Z = RNG.normal(size=(7, 4))
    out = O.pool(C, Z, RNG.normal(size=(1, 4)), 1, False)
    np.testing.assert_allclose(out, C, atol=1e-15)


def test_pool_constant_logits_give_mean():
    m, c = 4, 3
    C = RNG.normal(size=(8, c))
    Z = np.full((8, c), 0.7)
    out = O.pool(C, Z, np.zeros((m, c)), m, False)
    np.testing.assert_allclose(out, C.reshape(2, m, c).mean(axis=1), atol=1e-14)


def test_overlap_with_empty_b_series_equals_plain_pooling():
    m, c, n = 4, 5, 16
    Ca, Za = RNG.normal(size=(n, c)), RNG.normal(size=(n, c))
    Cb = RNG.normal(size=(n, c))
    Zb = np.full((n, c), -np.inf)
    ape_a = RNG.normal(size=(m, c))
    out_ov = O.pool(np.hstack([Cb, Ca]), np.hstack([Zb, Za]), np.hstack([np.zeros((m, c)), ape_a]), m, True)
    out_plain = O.pool(Ca, Za, ape_a, m, False)
    np.testing.assert_allclose(out_ov, out_plain, atol=1e-13)


def test_overlap_block_uses_previous_block_b_series():
    """Entry i of the overlapped compressor equals the plain softmax pool of
    the 2m rows (block i's a-series, block i-1's b-series) built by hand."""
    m, c, n = 3, 2, 9
    C = RNG.normal(size=(n, 2 * c))
    Z = RNG.normal(size=(n, 2 * c))
    ape = RNG.normal(size=(m, 2 * c))
    out = O.pool(C, Z, ape, m, True)
    i = 2
    logits = np.concatenate([Z[m * i:m * i + m, c:] + ape[:, c:], Z[m * (i - 1):m * i, :c] + ape[:, :c]])
    vals = np.concatenate([C[m * i:m * i + m, c:], C[m * (i - 1):m * i, :c]])
    wts = np.exp(logits) / np.exp(logits).sum(axis=0)
    np.testing.assert_allclose(out[i], (wts * vals).sum(axis=0), atol=1e-13)


# ------------------------------------------------------ norm / RoPE (O3, O7)
def test_rms_norm_hand():
    g = GOLD["rms_norm"]
    np.testing.assert_allclose(O.rms_norm(np.array(g["x"], float), g["eps"]), g["expected"], atol=1e-12)


def test_rms_norm_unit_rms_and_scale_invariance():
    x = RNG.normal(size=(10, 64)) * 5
    y = O.rms_norm(x, 0.0)
    np.testing.assert_allclose(np.sqrt((y * y).mean(-1)), 1.0, atol=1e-12)
    np.testing.assert_allclose(O.rms_norm(3.7 * x, 0.0), y, atol=1e-12)


@pytest.mark.parametrize("case", range(2))
def test_rope_hand(case):
    g = GOLD["rope"]["cases"][case]
    out = O.rope(np.array([g["x"]], float), [g["pos"]], g["rope_dims"], g["theta"])[0]
    np.testing.assert_allclose(out, g["expected"], atol=1e-12)


def test_rope_inverse_norm_and_relative_position():
    r, c, theta = 8, 12, 10000.0
    x = RNG.normal(size=(3, c))
    pos = np.array([0.0, 5.0, 1234.0])
    y = O.rope(x, pos, r, theta)
    np.testing.assert_allclose(O.rope(y, pos, r, theta, inverse=True), x, atol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), atol=1e-12)
    np.testing.assert_array_equal(y[:, : c - r], x[:, : c - r])
    # score between rotated q (pos a) and k (pos b) depends only on a - b
    q, k = RNG.normal(size=(1, c)), RNG.normal(size=(1, c))
    s1 = O.rope(q, [100.0], r, theta) @ O.rope(k, [40.0], r, theta).T
    s2 = O.rope(q, [1060.0], r, theta) @ O.rope(k, [1000.0], r, theta).T
    np.testing.assert_allclose(s1, s2, atol=1e-10)


def test_rope_three_axis_broadcast():
    x = RNG.normal(size=(4, 3, 16))
    pos = np.arange(4.0) * 7
    y = O.rope(x, pos, 8, 10000.0)
    for t in range(4):
        for h in range(3):
            np.testing.assert_allclose(y[t, h], O.rope(x[t, h][None], [pos[t]], 8, 10000.0)[0], atol=1e-14)


# ------------------------------------------------------------- number format
def test_bf16_rounding_hand():
    g = GOLD["bf16"]
    np.testing.assert_array_equal(O.round_bf16(np.array(g["inputs"])), g["expected"])


def test_bf16_rounding_matches_torch_for_fp32_inputs():
    torch = pytest.importorskip("torch")
    x = (RNG.normal(size=20000) * np.exp(RNG.normal(size=20000) * 4)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.round_bf16(x.astype(np.float64)), ref)


# ------------------------------------------------------- indexer (O5, O6)
def test_index_scores_and_topk_hand():
    g = GOLD["index_scores"]
    n = g["n_tokens"]
    qI = np.array([g["q_per_token"]] * n, float)
    wI = np.array([g["w_per_token"]] * n, float)
    KI = np.array(g["K"], float)
    sc = O.index_scores(qI, wI, KI, g["m"])
    exp = np.array([[np.nan if v is None else v for v in row] for row in g["expected_scores"]])
    np.testing.assert_allclose(np.where(np.isinf(sc), np.nan, sc), exp, atol=1e-12)
    assert np.all(np.isneginf(sc[np.isnan(exp)]))
    np.testing.assert_array_equal(O.topk(sc, g["k"], g["m"]), g["expected_idx"])


def test_index_scores_nonneg_and_head_permutation():
    n, h, d, m = 9, 4, 8, 2
    qI = RNG.normal(size=(n, h, d))
    wI = RNG.uniform(size=(n, h))
    KI = RNG.normal(size=(n // m, d))
    sc = O.index_scores(qI, wI, KI, m)
    fin = np.isfinite(sc)
    assert np.all(sc[fin] >= 0)
    perm = RNG.permutation(h)
    np.testing.assert_allclose(O.index_scores(qI[:, perm], wI[:, perm], KI, m), sc, atol=1e-12)


def test_index_mask_is_causal_block_end():
    """Entry s is visible to t exactly when its last token m(s+1)-1 <= t."""
    n, m = 23, 4
    sc = O.index_scores(RNG.normal(size=(n, 1, 3)), np.ones((n, 1)), RNG.normal(size=(n // m, 3)), m)
    for t in range(n):
        for s in range(n // m):
            assert np.isfinite(sc[t, s]) == (m * (s + 1) - 1 <= t)


@pytest.mark.parametrize("trial", range(20))
def test_topk_brute_force_subsets(trial):
    """Exhaustive check on tiny rows: the chosen set is the unique k_t-subset
    that beats every other subset in (score, then smaller index) order."""
    rng = np.random.default_rng(trial)
    m, ne, k = 1, 7, 3
    n = ne
    sc = rng.integers(0, 4, size=(n, ne)).astype(float)  # many ties on purpose
    t = np.arange(n)
    s = np.arange(ne)
    sc = np.where(s[None] < (t[:, None] + 1) // m, sc, -np.inf)
    idx = O.topk(sc, k, m)
    for r in range(n):
        v = (r + 1) // m
        kt = min(k, v)
        assert np.all(idx[r, kt:] == -1)
        got = set(idx[r, :kt].tolist())

        def key(j):
            return (sc[r, j], -j)

        # every subset whose members all beat every non-member; must be unique
        valid = [set(S) for S in itertools.combinations(range(v), kt)
                 if all(key(a) > key(b) for a in S for b in range(v) if b not in S)]
        assert valid == [got]


def test_topk_padding_count_and_causality():
    n, m, k = 40, 4, 6
    sc = O.index_scores(RNG.normal(size=(n, 2, 4)), RNG.uniform(size=(n, 2)), RNG.normal(size=(n // m, 4)), m)
    idx = O.topk(sc, k, m)
    for t in range(n):
        v = (t + 1) // m
        assert np.sum(idx[t] == -1) == k - min(k, v)
        sel = idx[t][idx[t] >= 0]
        assert np.all(m * (sel + 1) - 1 <= t)


# ------------------------------------------------------ attention (O7-O10)
def test_attention_sink_hand():
    g = GOLD["attention_sink"]
    p, ps = O.attention_probs(np.array(g["q"]), np.array(g["kv"]), np.array(g["sink"]), g["scale"])
    np.testing.assert_allclose(p, g["expected_p"], atol=1e-15)
    np.testing.assert_allclose(ps, g["expected_p_sink"], atol=1e-15)
    np.testing.assert_allclose(O.attend(np.array(g["q"]), np.array(g["kv"]), np.array(g["sink"]), g["scale"]),
                               g["expected_o"], atol=1e-15)


def test_attention_probabilities_sum_to_one():
    qh, kv = RNG.normal(size=(5, 16)), RNG.normal(size=(30, 16))
    sink = RNG.normal(size=5)
    p, ps = O.attention_probs(qh, kv, sink, 0.25)
    np.testing.assert_allclose(p.sum(1) + ps, 1.0, atol=1e-14)


def test_attention_equal_logits_closed_form_and_huge_sink():
    N, c = 11, 8
    kv = RNG.normal(size=(N, c))
    sink = np.array([0.3, -1.2])
    o = O.attend(np.zeros((2, c)), kv, sink, 1.0)  # all logits 0
    expect = (N / (N + np.exp(sink)))[:, None] * kv.mean(0)[None]
    np.testing.assert_allclose(o, expect, atol=1e-14)
    o_big = O.attend(RNG.normal(size=(1, c)), kv, np.array([80.0]), 0.1)
    assert np.max(np.abs(o_big)) < 1e-30


def _sdpa_causal(q, k, v):
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    Q = torch.from_numpy(q).permute(1, 0, 2)[None]  # [1, nh, n, c]
    K = torch.from_numpy(k)[None, None].expand(1, q.shape[1], -1, -1)
    V = torch.from_numpy(v)[None, None].expand(1, q.shape[1], -1, -1)
    out = F.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=1.0)
    lse = torch.logsumexp((Q @ K.transpose(-1, -2)).masked_fill(
        torch.ones(q.shape[0], q.shape[0], dtype=torch.bool).triu(1), float("-inf")), dim=-1)
    return out[0].permute(1, 0, 2).numpy(), lse[0].permute(1, 0).numpy()


@pytest.mark.parametrize("overlap", [False])
def test_csa_m1_all_entries_no_window_is_dense_causal_mqa(overlap):
    """m = 1, k >= n, n_win = 0, no RoPE: CSA is dense causal shared-KV MQA
    over the normalised per-token rows, including the token itself.  Checked
    against torch's scaled_dot_product_attention (fp64, CPU) with the sink
    folded in through the closed form o_sink = o * S / (S + e^z')."""
    n, d, c, nh = 12, 10, 8, 3
    H = RNG.normal(size=(n, d))
    Wkv, Wz = RNG.normal(size=(d, c)), RNG.normal(size=(d, c))
    comp = O.compress_prefill(H, Wkv, Wz, np.zeros((1, c)), 1, overlap, qk_norm=True, eps=1e-6, store="f64")
    q = RNG.normal(size=(n, nh, c))
    sc = O.index_scores(RNG.normal(size=(n, 2, c)), RNG.uniform(size=(n, 2)), comp, 1)
    idx = O.topk(sc, n, 1)
    sink = RNG.normal(size=nh)
    scale = c ** -0.5
    out = O.sparse_mqa_prefill(q, np.zeros((n, c)), comp, idx, sink, 0, scale, qk_norm=True, store="f64")
    qn = O.rms_norm(q, 1e-6) * scale
    ref, lse = _sdpa_causal(qn, comp, comp)
    S = np.exp(lse)
    ref = ref * (S / (S + np.exp(sink)[None]))[..., None]
    np.testing.assert_allclose(out, ref, atol=1e-12)
    # with the sink pushed to -inf the result is exactly softmax attention
    out_ns = O.sparse_mqa_prefill(q, np.zeros((n, c)), comp, idx, np.full(nh, -np.inf), 0, scale, store="f64")
    np.testing.assert_allclose(out_ns, _sdpa_causal(qn, comp, comp)[0], atol=1e-12)


def test_sparse_with_all_entries_equals_dense_hca():
    n, c, nh, m, n_win = 37, 8, 2, 4, 5
    q = RNG.normal(size=(n, nh, c))
    win = RNG.normal(size=(n, c))
    comp = RNG.normal(size=(n // m, c))
    sink = RNG.normal(size=nh)
    idx = np.full((n, n), -1)
    for t in range(n):
        v = (t + 1) // m
        idx[t, :v] = RNG.permutation(v)  # order of the selected set is irrelevant
    a = O.sparse_mqa_prefill(q, win, comp, idx, sink, n_win, 0.3, rope_dims=4, store="f64")
    b = O.dense_mqa_prefill(q, win, comp, sink, m, n_win, 0.3, rope_dims=4, store="f64")
    np.testing.assert_allclose(a, b, atol=1e-13)


def test_window_extent_and_dense_hand_count():
    """With identical candidates the output is N/(N+e^z') times the row, where
    N = window rows + visible entries; this pins the candidate counting."""
    n, c, m, n_win = 20, 4, 4, 3
    row = RNG.normal(size=c)
    win = np.tile(row, (n, 1))
    comp = np.tile(row, (n // m, 1))
    sink = np.array([0.5])
    q = RNG.normal(size=(n, 1, c))
    out = O.dense_mqa_prefill(q, win, comp, sink, m, n_win, 0.7, qk_norm=False, store="f64")
    for t in range(n):
        N = min(n_win, t + 1) + (t + 1) // m
        z = 0.7 * q[t, 0] @ row  # every candidate has this same logit
        np.testing.assert_allclose(out[t, 0], N / (N + np.exp(0.5 - z)) * row, atol=1e-13)


def test_output_inverse_rope_makes_output_relative():
    """Shifting every position by the same offset leaves the output unchanged
    when entries, window rows and queries are all rotated consistently
    ([R] 2.3.3: inverse RoPE at the query position)."""
    n, c, nh, r = 6, 16, 2, 8
    q0 = RNG.normal(size=(n, nh, c))
    raw = RNG.normal(size=(n, c))
    sink = RNG.normal(size=nh)

    def run(shift):
        win = O.rope(raw, shift + np.arange(n, dtype=float), r, 100.0)
        outs = []
        for t in range(n):
            qh = O.rope(q0[t][None], [shift + t], r, 100.0)[0]
            o = O.attend(qh, win[: t + 1], sink, 0.5)
            outs.append(O.rope(o[None], [shift + t], r, 100.0, inverse=True)[0])
        return np.array(outs)

    np.testing.assert_allclose(run(0.0), run(37.0), atol=1e-10)


def _positions_case():
    """The worked example's inputs, built through the oracle's own entry and
    window-row functions (identity projections, no QK-RMSNorm), so that each
    position the oracle assigns is exercised."""
    g = GOLD["attention_positions"]
    c, r, th, m, t = g["c"], g["rope_dims"], g["theta"], g["m"], g["t"]
    n = t + 1
    H = np.zeros((n, c))
    H[t] = g["raw_window_row_at_t"]
    win = O.window_rows(H, np.eye(c), qk_norm=False, rope_dims=r, theta=th, store="f64")
    # entries: m = 2 identical token rows per block, so pooling returns the row
    Hc = np.zeros((n, c))
    Hc[0:2] = g["raw_entry_0"]
    Hc[2:4] = g["raw_entry_1"]
    comp = O.compress_prefill(Hc, np.eye(c), np.zeros((c, c)), np.zeros((m, c)), m, False,
                              qk_norm=False, rope_dims=r, theta=th, store="f64")
    q = np.zeros((n, 1, c))
    q[t, 0] = g["raw_q_at_t"]
    return g, q, win, comp


def test_attention_positions_worked_example_sparse():
    """Query rotated by +t, window row j at j, entry i at m*i, output rotated
    back by -t: the contribution of each candidate depends only on its
    distance to the query, and the values match the hand derivation."""
    g, q, win, comp = _positions_case()
    t = g["t"]
    idx = np.full((t + 1, 1), -1)
    idx[t, 0] = 1
    out = O.sparse_mqa_prefill(q, win, comp, idx, np.array(g["sink"]), g["n_win"], g["scale"],
                               qk_norm=False, rope_dims=g["rope_dims"], theta=g["theta"],
                               store="f64", rows=[t])
    np.testing.assert_allclose(out[0, 0], g["expected_sparse"], rtol=0, atol=1e-15)


def test_attention_positions_worked_example_dense():
    g, q, win, comp = _positions_case()
    t = g["t"]
    out = O.dense_mqa_prefill(q, win, comp, np.array(g["sink"]), g["m"], g["n_win"], g["scale"],
                              qk_norm=False, rope_dims=g["rope_dims"], theta=g["theta"],
                              store="f64", rows=[t])
    np.testing.assert_allclose(out[0, 0], g["expected_dense"], rtol=0, atol=1e-15)


def test_attention_positions_single_window_row_is_relative():
    """One token, n_win = 1, no entries, r = c: the query and its own window
    row carry the same rotation, so the logit is the unrotated q.v and the
    output rotated back is p_self * v with p_self = e^z / (e^z + e^z')."""
    c, r, t = 4, 4, 9
    rng = np.random.default_rng(5)
    raw_v = rng.normal(size=c)
    qraw = rng.normal(size=c)
    sink = np.array([0.25])
    H = np.zeros((t + 1, c))
    H[t] = raw_v
    win = O.window_rows(H, np.eye(c), qk_norm=False, rope_dims=r, theta=100.0, store="f64")
    q = np.zeros((t + 1, 1, c))
    q[t, 0] = qraw
    idx = np.full((t + 1, 1), -1)
    out = O.sparse_mqa_prefill(q, win, np.zeros((0, c)), idx, sink, 1, 0.5, qk_norm=False,
                               rope_dims=r, theta=100.0, store="f64", rows=[t])
    z = 0.5 * float(qraw @ raw_v)
    p_self = math.exp(z) / (math.exp(z) + math.exp(0.25))
    np.testing.assert_allclose(out[0, 0], p_self * raw_v, rtol=0, atol=1e-14)


@pytest.mark.parametrize("r", [0, 8])
def test_attend_decode_row_equals_prefill_rows(r):
    """One decode query at t over its window rows and the entries a prefill
    row would attend to gives that prefill row, for the sparse (selected
    entries) and the dense (all visible entries) modes."""
    rng = np.random.default_rng(11 + r)
    n, c, nh, m, n_win, k = 29, 16, 3, 4, 5, 3
    q = rng.normal(size=(n, nh, c))
    win = O.rope(rng.normal(size=(n, c)), np.arange(n, dtype=float), r, 1000.0)
    comp = O.rope(rng.normal(size=(n // m, c)), m * np.arange(n // m, dtype=float), r, 1000.0)
    sink = rng.normal(size=nh)
    idx = np.full((n, k), -1)
    for t in range(n):
        v = (t + 1) // m
        sel = rng.permutation(v)[:k]
        idx[t, :len(sel)] = sel
    kw = dict(qk_norm=True, eps=1e-6, rope_dims=r, theta=1000.0, store="f64")
    sp = O.sparse_mqa_prefill(q, win, comp, idx, sink, n_win, 0.3, **kw)
    de = O.dense_mqa_prefill(q, win, comp, sink, m, n_win, 0.3, **kw)
    for t in (0, 3, 4, 17, n - 1):
        wr = win[O.window_range(t, n_win)]
        sel = [s for s in idx[t] if s >= 0]
        a = O.attend_decode_row(q[t], t, wr, comp[sel], sink, 0.3, **kw)
        np.testing.assert_allclose(a, sp[t], rtol=0, atol=1e-13)
        b = O.attend_decode_row(q[t], t, wr, comp[: (t + 1) // m], sink, 0.3, **kw)
        np.testing.assert_allclose(b, de[t], rtol=0, atol=1e-13)


def test_prenorm_rounding_worked_example():
    """A17: the pooled value is rounded to the storage type before its
    RMSNorm; in this example the cast changes the stored bf16 value."""
    g = GOLD["prenorm_rounding"]
    x = np.array([g["x"]])
    got = O.entry_epilogue(x, [0.0], True, g["eps"], 0, 10000.0, g["store"])
    np.testing.assert_array_equal(got[0], g["expected"])
    no_cast = O.round_bf16(O.rms_norm(x, g["eps"]))
    np.testing.assert_array_equal(no_cast[0], g["expected_without_prenorm_rounding"])


def test_prenorm_rounding_reaches_entries_and_window_rows():
    """Entries and window rows both pass through the pre-norm rounding: with
    identity projections they equal the epilogue of the bf16-rounded input,
    which differs from the single-rounding result on these inputs."""
    x = np.array([[1.00390625, 0.0], [1.01171875, 0.2], [0.75, -1.0]])
    win = O.window_rows(x, np.eye(2), eps=1.0, store="bf16")
    ref = O.round_bf16(O.rms_norm(O.round_bf16(x), 1.0))
    np.testing.assert_array_equal(win, ref)
    assert np.any(win != O.round_bf16(O.rms_norm(x, 1.0)))
    comp = O.compress_prefill(x, np.eye(2), np.zeros((2, 2)), np.zeros((1, 2)), 1, False,
                              eps=1.0, store="bf16")
    np.testing.assert_array_equal(comp, ref)


# --------------------------------------------------------- decode (OD)
@pytest.mark.parametrize("overlap,m", [(False, 4), (True, 4), (False, 8), (True, 3)])
def test_stateful_decode_equals_prefill(overlap, m):
    """The pages' token-at-a-time compressor emits, block by block, exactly
    the prefill entries (prefill(n) followed by decode steps == prefill(n+s))."""
    n, d, c = 6 * m + 1, 12, 8
    w = 2 if overlap else 1
    H = RNG.normal(size=(n, d))
    Wkv, Wz = RNG.normal(size=(d, w * c)), RNG.normal(size=(d, w * c))
    ape = RNG.normal(size=(m, w * c))
    ref = O.compress_prefill(H, Wkv, Wz, ape, m, overlap, rope_dims=4, store="f64")
    dec = O.CompressorDecodeOracle(c, m, overlap, ape, rope_dims=4, store="f64")
    C, Z = O.project(H, Wkv), O.project(H, Wz)
    got = []
    for t in range(n):
        e = dec.append(t, C[t], Z[t])
        assert (e is not None) == ((t + 1) % m == 0)
        if e is not None:
            got.append(e)
    np.testing.assert_allclose(np.array(got), ref, atol=1e-12)


def test_causality_perturbation():
    """Changing token j's hidden state leaves every output row t < j unchanged."""
    n, d, c, nh, m, k, n_win = 24, 10, 8, 2, 4, 3, 4
    H = RNG.normal(size=(n, d))
    W = [RNG.normal(size=(d, 2 * c)) for _ in range(2)] + [RNG.normal(size=(d, c))]
    WI = [RNG.normal(size=(d, 2 * 4)) for _ in range(2)]
    ape, apeI = RNG.normal(size=(m, 2 * c)), RNG.normal(size=(m, 2 * 4))
    q, qI, wI = RNG.normal(size=(n, nh, c)), RNG.normal(size=(n, 2, 4)), RNG.uniform(size=(n, 2))
    sink = RNG.normal(size=nh)

    def layer(Hx):
        comp = O.compress_prefill(Hx, W[0], W[1], ape, m, True, rope_dims=4, store="f64")
        KI = O.compress_prefill(Hx, WI[0], WI[1], apeI, m, True, store="f64")
        win = O.window_rows(Hx, W[2], rope_dims=4, store="f64")
        idx = O.topk(O.index_scores(qI, wI, KI, m), k, m)
        return O.sparse_mqa_prefill(q, win, comp, idx, sink, n_win, 0.35, rope_dims=4, store="f64")

    base = layer(H)
    j = 13
    H2 = H.copy()
    H2[j] += 5.0
    pert = layer(H2)
    np.testing.assert_array_equal(pert[:j], base[:j])
    assert np.max(np.abs(pert[j:] - base[j:])) > 1e-6


# ------------------------------------------------- query path / output (O8)
def test_query_proj_worked_example():
    """h = (3, 4), W_DQ = I: the latent (3, 4) has mean square 12.5, so with
    eps = 0 its RMSNorm is (3, 4)/sqrt(12.5); a weight scales it per channel."""
    H = np.array([[3.0, 4.0]])
    I2 = np.eye(2)
    cq, q, qI, wI = O.query_proj(H, I2, np.array([2.0, 0.5]), np.array([[1.0], [-1.0]]), I2,
                                 np.array([[1.0], [1.0]]), 0.0, lambda x: x)
    s = 1 / math.sqrt(12.5)
    np.testing.assert_allclose(cq, [[6 * s, 2 * s]], rtol=1e-15)
    np.testing.assert_allclose(q, cq, rtol=1e-15)               # W_UQ = I
    np.testing.assert_allclose(qI, [[8 * s]], rtol=1e-15)      # (6s + 2s)
    np.testing.assert_allclose(wI, [[-1.0]], rtol=1e-15)       # 3 - 4


def test_query_proj_latent_norm_and_scale_invariance():
    """Without a weight, every latent row has mean square ms/(ms+eps); the
    latent, q and q^I do not change when h is scaled (eps = 0)."""
    n, d, dc = 7, 12, 8
    H = RNG.normal(size=(n, d))
    W = RNG.normal(size=(d, dc))
    Wu, Wi, Ww = RNG.normal(size=(dc, 6)), RNG.normal(size=(dc, 4)), RNG.normal(size=(d, 3))
    eps = 1e-3
    cq = O.query_proj(H, W, None, Ww, Wu, Wi, eps, lambda x: x)[0]
    lat = H @ W
    ms = np.mean(lat * lat, axis=1)
    np.testing.assert_allclose(np.mean(cq * cq, axis=1), ms / (ms + eps), rtol=1e-12)
    a = O.query_proj(H, W, None, Ww, Wu, Wi, 0.0, lambda x: x)
    b = O.query_proj(5.0 * H, W, None, Ww, Wu, Wi, 0.0, lambda x: x)
    for x, y in zip(a[:3], b[:3]):
        np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(b[3], 5.0 * a[3], rtol=1e-12)   # w^I is linear in h


def test_output_proj_equals_block_diagonal_product():
    """The grouped projection is the dense product with the block-diagonal
    matrix of the group weights, followed by wo_b."""
    import scipy.linalg
    n, g, kg, dg, d = 5, 3, 4, 2, 7
    o = RNG.normal(size=(n, g * kg))
    wo_a = RNG.normal(size=(g, dg, kg))
    wo_b = RNG.normal(size=(d, g * dg))
    bd = scipy.linalg.block_diag(*[wo_a[j] for j in range(g)])  # [g*dg, g*kg]
    ref = o @ bd.T @ wo_b.T
    np.testing.assert_allclose(O.output_proj(o, wo_a, wo_b, lambda x: x), ref, rtol=1e-12)


def test_output_proj_single_group_identity():
    """g = 1 with wo_a = I leaves o . wo_b^T; storing rounds once per stage."""
    n, k, d = 4, 6, 3
    o = RNG.normal(size=(n, k))
    wo_b = RNG.normal(size=(d, k))
    out = O.output_proj(o, np.eye(k)[None], wo_b, lambda x: x)
    np.testing.assert_allclose(out, o @ wo_b.T, rtol=1e-13)
    outb = O.output_proj(o, np.eye(k)[None], wo_b, O.round_bf16)
    np.testing.assert_array_equal(outb, O.round_bf16(O.round_bf16(o) @ wo_b.T))


def test_topk_on_bf16_scores_worked_example():
    """Scores 1.0, 1.001, 0.5, 1.003: in bf16 (8 significant bits, step 2^-7
    at 1) the first, second and fourth all become exactly 1.0, so with k = 2
    the two smallest indices of that tie win (0 and 1), while on the exact
    scores the two largest (3 and 1) would."""
    sc = np.array([[1.0, 1.001, 0.5, 1.003]])
    np.testing.assert_array_equal(O.round_bf16(sc), [[1.0, 1.0, 0.5, 1.0]])
    got = O.topk_bf16_scores(sc, 2, 1, t0=3)
    assert sorted(got[0].tolist()) == [0, 1]
    assert sorted(O.topk(sc, 2, 1, t0=3)[0].tolist()) == [1, 3]


# ------------------------------------------- quantised indexer path (O9)
def test_hadamard_worked_example_and_orthogonality():
    """H_2 / sqrt(2) maps (1, 0) to (1, 1)/sqrt(2); the normalised transform is
    its own inverse and keeps dot products, so the scores of rotated q and k
    equal the unrotated ones."""
    np.testing.assert_allclose(O.hadamard(np.array([1.0, 0.0])), [2 ** -0.5, 2 ** -0.5], rtol=1e-15)
    np.testing.assert_allclose(O.hadamard(np.array([1.0, 2.0, 3.0, 4.0])), [5.0, -1.0, -2.0, 0.0],
                               rtol=1e-15, atol=1e-15)  # (10, -2, -4, 0) / 2
    x = RNG.normal(size=(5, 64))
    np.testing.assert_allclose(O.hadamard(O.hadamard(x)), x, rtol=1e-12, atol=1e-12)
    q, K = RNG.normal(size=(3, 4, 64)), RNG.normal(size=(9, 64))
    w = RNG.uniform(size=(3, 4))
    np.testing.assert_allclose(O.index_scores(O.hadamard(q), w, O.hadamard(K), 1, t0=8),
                               O.index_scores(q, w, K, 1, t0=8), rtol=1e-12, atol=1e-12)


def test_fp4_quant_worked_examples():
    """A block with amax 12 takes 2^e = 2 (12/6 = 2 exactly); 3.0 -> 1.5 is on
    the grid; 2.5 -> 1.25 is a tie between 1 and 1.5 and goes to the even 1;
    -7.0 -> -3.5, a tie between 3 and 4, goes to 4; 0.4 -> 0.2 rounds to 0 and
    keeps no sign; 12 -> 6 is the largest code."""
    x = np.zeros(32)
    x[:6] = [12.0, 3.0, 2.5, -7.0, -0.4, 0.9]
    codes, exps = O.fp4_quant(x)
    assert exps.tolist() == [1]
    assert codes[:6].tolist() == [7, 3, 2, 8 + 6, 0, 1]  # 0.9/2 = 0.45 -> 0.5 (index 1)
    np.testing.assert_array_equal(O.fp4_dequant(codes, exps)[:6], [12.0, 3.0, 2.0, -8.0, 0.0, 1.0])
    z, ez = O.fp4_quant(np.zeros((2, 64)))
    assert (z == 0).all() and (ez == 0).all()


def test_fp4_quant_round_trip_and_error_bound():
    """Grid values times the block scale come back exactly; any value is off
    by at most half of the widest grid gap (1 at the top, times 2^e), and
    each block's largest magnitude stays within 6 * 2^e."""
    e = -3
    vals = np.zeros(32)
    vals[:8], vals[8:15], vals[15:23] = O.FP4_GRID, -O.FP4_GRID[1:], O.FP4_GRID
    vals *= 2.0 ** e
    vals[0] = 6 * 2.0 ** e  # pin the block amax so that e is -3
    c, ex = O.fp4_quant(vals)
    assert ex.tolist() == [e]
    np.testing.assert_array_equal(O.fp4_dequant(c, ex), vals)
    x = RNG.normal(size=(50, 128)) * np.exp(RNG.normal(size=(50, 1)))
    c, ex = O.fp4_quant(x)
    dq = O.fp4_dequant(c, ex)
    scale = np.repeat(np.ldexp(1.0, ex), 32, axis=-1)
    assert np.all(np.abs(dq - x) <= scale * 1.0 + 1e-15)
    assert np.all(np.abs(x) <= 6 * scale * (1 + 1e-12))
    assert np.all(np.abs(x).reshape(50, 4, 32).max(-1) > 3 * np.ldexp(1.0, ex) * (1 - 1e-12))


# ------------------------------------------------- attention backward (O11)
def _bwd_case(seed, rope_dims, qk_norm):
    rng = np.random.default_rng(seed)
    n, nh, c, m, n_win, k = 9, 2, 6, 2, 3, 2
    q = rng.normal(size=(n, nh, c))
    win = rng.normal(size=(n, c))
    comp = rng.normal(size=(n // m, c))
    sink = rng.normal(size=nh)
    dout = rng.normal(size=(n, nh, c))
    idx = np.full((n, k), -1)
    for t in range(n):
        v = (t + 1) // m
        sel = rng.permutation(v)[:k]
        idx[t, :len(sel)] = sel
    kw = dict(qk_norm=qk_norm, eps=1e-3, rope_dims=rope_dims, theta=100.0)
    return q, win, comp, idx, sink, dout, m, n_win, kw


@pytest.mark.parametrize("rope_dims,qk_norm", [(0, False), (2, True), (4, True)])
def test_attention_backward_matches_finite_differences(rope_dims, qk_norm):
    """Central differences of L = sum(dout * out) in fp64 (step 1e-6) agree
    with every gradient of the hand-derived backward, sparse and dense."""
    q, win, comp, idx, sink, dout, m, n_win, kw = _bwd_case(3 + rope_dims, rope_dims, qk_norm)
    scale = 0.4

    def loss_sparse(q_, win_, comp_, sink_):
        return float(np.sum(dout * O.sparse_mqa_prefill(q_, win_, comp_, idx, sink_, n_win, scale,
                                                        store="f64", **kw)))

    def loss_dense(q_, win_, comp_, sink_):
        return float(np.sum(dout * O.dense_mqa_prefill(q_, win_, comp_, sink_, m, n_win, scale,
                                                       store="f64", **kw)))

    for loss, grads in (
            (loss_sparse, O.sparse_mqa_backward(q, win, comp, idx, sink, dout, n_win, scale, **kw)),
            (loss_dense, O.dense_mqa_backward(q, win, comp, sink, dout, m, n_win, scale, **kw))):
        args = [q, win, comp, sink]
        for a, (x, g) in enumerate(zip(args, grads)):
            num = np.zeros_like(x)
            h = 1e-6
            for pos in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[pos] += h
                xm[pos] -= h
                ap, am = list(args), list(args)
                ap[a], am[a] = xp, xm
                num[pos] = (loss(*ap) - loss(*am)) / (2 * h)
            np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-7)


def test_attention_backward_matches_torch_autograd():
    """The same gradients from torch's automatic differentiation (fp64, CPU)
    of the forward written with torch operations."""
    torch = pytest.importorskip("torch")
    q, win, comp, idx, sink, dout, m, n_win, kw = _bwd_case(11, 4, True)
    scale, eps, r, theta = 0.4, kw["eps"], kw["rope_dims"], kw["theta"]
    T = lambda x: torch.tensor(x, dtype=torch.float64, requires_grad=True)  # noqa: E731
    tq, tw, tc, ts = T(q), T(win), T(comp), T(sink)
    n, nh, c = q.shape

    def rot(x, pos, sign):
        x0, x1 = x[..., c - r::2], x[..., c - r + 1::2]
        ang = sign * pos * theta ** (-2.0 * torch.arange(r // 2, dtype=torch.float64) / r)
        y0 = x0 * torch.cos(ang) - x1 * torch.sin(ang)
        y1 = x0 * torch.sin(ang) + x1 * torch.cos(ang)
        out = x.clone()
        out[..., c - r::2] = y0
        out[..., c - r + 1::2] = y1
        return out

    outs = []
    for t in range(n):
        qn = tq[t] / torch.sqrt((tq[t] ** 2).mean(-1, keepdim=True) + eps)
        qh = rot(qn, float(t), 1.0)
        wr = O.window_range(t, n_win).tolist()
        sel = [s for s in idx[t].tolist() if s >= 0]
        kv = torch.cat([tw[wr], tc[sel]], 0)
        z = scale * qh @ kv.T
        allz = torch.cat([z, ts[:, None]], 1)
        pz = torch.softmax(allz, 1)[:, :-1]
        outs.append(rot(pz @ kv, float(t), -1.0))
    (torch.stack(outs) * torch.tensor(dout)).sum().backward()
    got = O.sparse_mqa_backward(q, win, comp, idx, sink, dout, n_win, scale, **kw)
    for g, x in zip(got, (tq, tw, tc, ts)):
        np.testing.assert_allclose(g, x.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_attention_backward_logit_gradients_sum_to_zero():
    """Adding one constant to every logit and the sink leaves the output
    unchanged, so the logit gradients of a row (candidates and sink) sum to
    zero: checked through a query of all zeros (qk_norm off), where the
    gradient of the sink equals minus the summed candidate-logit gradients."""
    rng = np.random.default_rng(7)
    nh, c, N = 2, 4, 5
    kv = rng.normal(size=(N, c))
    sink = rng.normal(size=nh)
    dout = rng.normal(size=(nh, c))
    q = rng.normal(size=(nh, c))
    dq, dkv, dsink = O.attention_backward_row(q, 0, kv, sink, dout, 1.0, qk_norm=False)
    # d(loss)/d(shift all candidate logits) = sum_j dz_j = -dsink by the identity;
    # shifting every candidate logit by s is adding s / scale to q . kv_j for all j,
    # which the direction q -> q + s * v with kv v = 1 would do: use finite differences
    s = 1e-6
    def out(sh):
        z = q @ kv.T + sh
        M = np.maximum(z.max(1), sink)
        e, es = np.exp(z - M[:, None]), np.exp(sink - M)
        return ((e / (e.sum(1) + es)[:, None]) @ kv * dout).sum()
    dz_sum = (out(s) - out(-s)) / (2 * s)
    np.testing.assert_allclose(dz_sum, -dsink.sum(), rtol=1e-6)


# ------------------------------------------------------- FP8 KV rows (O12)
def test_fp8_quant_worked_examples():
    g = GOLD["fp8_kv"]
    for blk in ("a", "b"):
        x = np.zeros(64)
        vals = g["block_" + blk]
        x[:len(vals)] = vals
        codes, e = O.fp8_quant(x)
        assert e.tolist() == [g["exp_" + blk]]
        assert codes[:len(vals)].tolist() == g["codes_" + blk]
        np.testing.assert_array_equal(O.fp8_dequant(codes, e)[:len(vals)], g["values_" + blk])
    # a negative value that rounds to zero keeps no sign: -2^-10 is half the
    # subnormal step below zero (block scale 1, set by a 448 in the block)
    x = np.zeros(64)
    x[0], x[1] = 448.0, -2.0 ** -10
    assert O.fp8_quant(x)[0][1] == 0


def test_fp8_scale_floor():
    """The scale exponent stops at -117 (smallest grid step 2^-126, the
    smallest normal fp32 number).  A block with largest magnitude 2^-110 would
    take e = -118 (2^-110 = 0.5 * 2^-109); floored, 2^-110 / 2^-117 = 128 =
    field 14, mantissa 0 (code 112); 3 * 2^-127 / 2^-117 = 1.5 steps of 2^-9,
    a tie between 1 and 2, even 2 (code 2, value 2^-125); 2^-130 is 1/16 of a
    step and rounds to 0."""
    x = np.zeros(64)
    x[0], x[1], x[2], x[3] = 2.0 ** -110, 3 * 2.0 ** -127, 2.0 ** -130, -(2.0 ** -110)
    c, e = O.fp8_quant(x)
    assert e.tolist() == [-117]
    assert c[:4].tolist() == [112, 2, 0, 128 + 112]
    np.testing.assert_array_equal(O.fp8_dequant(c, e)[:4],
                                  [2.0 ** -110, 2.0 ** -125, 0.0, -(2.0 ** -110)])


def test_fp8_grid_round_trip_and_error_bound():
    """Grid values times the scale come back exactly; otherwise the error is
    at most half a grid step (2^-4 of the value for normals, 2^-10 of the
    scale below 2^-6), and the scale is the smallest power of two that holds
    the block's largest magnitude."""
    grid = O.fp8_e4m3_values()[:127]
    x = np.concatenate([grid, -grid[1:65]]) * 2.0 ** 3  # 191 values: three blocks less one
    x = x[:128].reshape(2, 64)
    x[:, 0] = 448 * 8.0  # pin e = 3 in both blocks
    c, e = O.fp8_quant(x)
    assert e.tolist() == [[3], [3]]
    np.testing.assert_array_equal(O.fp8_dequant(c, e), x)
    rng = np.random.default_rng(21)
    y = rng.normal(size=(40, 256)) * np.exp(rng.normal(size=(40, 1)) * 3)
    c, e = O.fp8_quant(y)
    d = O.fp8_dequant(c, e)
    scale = np.repeat(np.ldexp(1.0, e), 64, axis=-1)
    normal = np.abs(y) >= 2.0 ** -6 * scale
    assert np.all(np.abs(d - y)[normal] <= 2.0 ** -4 * np.abs(y)[normal] * (1 + 1e-12))
    assert np.all(np.abs(d - y)[~normal] <= 2.0 ** -10 * scale[~normal] * (1 + 1e-12))
    amax = np.abs(y).reshape(40, 4, 64).max(-1)
    assert np.all(amax <= 448 * np.ldexp(1.0, e)) and np.all(amax > 224 * np.ldexp(1.0, e))
    z, ez = O.fp8_quant(np.zeros((2, 64)))
    assert (z == 0).all() and (ez == 0).all()


def test_kv_fp8_keeps_rope_channels():
    rng = np.random.default_rng(4)
    x = rng.normal(size=(5, 512))
    y = O.kv_fp8(x, 64)
    np.testing.assert_array_equal(y[:, 448:], x[:, 448:])
    c, e = O.fp8_quant(x[:, :448])
    np.testing.assert_array_equal(y[:, :448], O.fp8_dequant(c, e))
    np.testing.assert_array_equal(O.kv_fp8(x, 512), x)
