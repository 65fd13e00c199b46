"""Plain CPU fp64 oracle for CSA / HCA hybrid compressed attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test-suite, the package smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP library.

Every function is a direct, unblocked statement of a definition from the
pages, in float64 numpy.  A library primitive (matmul, argsort, exp) may serve
as a step; there is no fusion or reordering beyond what the definition states.

Citation keys used below (page title, then where on the page):
  [R]  "DeepSeek-V4 技术解读报告" (juejin.cn/post/7631898635937497134),
       section 2.3 "混合注意力架构 (CSA + HCA)", equations 9-23 and 27.
  [A]  "DeepSeek-V4：算法架构" (1zeryu.github.io/p/deepseek-v4/), the
       "Q, K, V 映射与位置编码注入", "Sparse Attention", "CSA 选择器层代码
       实现" (classes Compressor and Indexer), "HCA 选择函数代码实现" and
       "输出投影" code excerpts.

Readings where the pages are silent or ambiguous (each is also listed in the
design notes of the repository):
  * visibility: compressed entry s is visible to 0-indexed query t iff
    s < floor((t+1)/m), i.e. its block ends at or before t ([A] Indexer causal
    mask; [R] eq 16 read with a 1-indexed t);
  * overlap column packing: the first c columns of an overlapped projection
    are the b-series (feed block i+1), the last c the a-series ([A] Compressor
    constructor comment and overlap transform);
  * window: the n_win most recent positions including t itself;
  * RoPE: adjacent pairs (2p, 2p+1) of the last r dims, angle pos*theta^(-2p/r);
    entry i sits at position m*i; the output is rotated back by -t;
  * QK-RMSNorm has unit weight; core-attention scale is passed in (c^-1/2);
  * rounding (bf16 configs): a pooled entry, and a window row's projection,
    is rounded to the storage type before its RMSNorm ([A] Compressor casts
    the pooled value to the model dtype before its norm; the attention's wkv
    is a model-dtype linear layer); norm and RoPE then run in high precision
    with one more round-to-nearest-even at store; attention output rounded
    once.

Parity pins for every function live in tests/test_oracle_pins.py.
"""
from __future__ import annotations

import math

import numpy as np

F64 = np.float64


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------
def round_bf16(x):
    """Round float64 values to the nearest bfloat16 (ties to even), returned
    as float64.  bfloat16 keeps 8 significant bits and fp32's exponent range;
    frexp gives x = f * 2**e with 0.5 <= |f| < 1, so rounding f*2**8 to an
    integer (numpy rounds half to even) keeps exactly 8 significant bits.
    Values in fp32's subnormal range are not produced by any workload here."""
    x = np.asarray(x, dtype=F64)
    f, e = np.frexp(x)
    r = np.ldexp(np.round(f * 256.0), e - 8)
    big = np.abs(r) > 3.3895313892515355e38  # beyond bf16's largest finite
    return np.where(big, np.copysign(np.inf, x), r)


def round_to(x, dtype: str):
    """One rounding to the storage type ('f32' or 'bf16'), back in float64."""
    if dtype == "f32":
        return np.asarray(x, dtype=F64).astype(np.float32).astype(F64)
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f64":
        return np.asarray(x, dtype=F64)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# O1: projections  ([R] eq 9-10 for CSA, eq 20-21 for HCA)
# ---------------------------------------------------------------------------
def project(H, W):
    """C = H . W (and Z = H . W_Z): rows are tokens, columns channels."""
    return np.asarray(H, F64) @ np.asarray(W, F64)


# ---------------------------------------------------------------------------
# O2: block softmax pooling  ([R] eq 11-12, eq 22-23; [A] Compressor)
# ---------------------------------------------------------------------------
def pool_terms(C, Z, ape, m: int, overlap: bool):
    """The logits and values that enter each compressed entry.

    Returns (logits, values), both [n_c, L, c] with L = m (no overlap) or
    2m (overlap).  For overlap, rows 0..m-1 of L are block i's a-series
    (Z_a + B_a, C_a) and rows m..2m-1 are block i-1's b-series
    (Z_b + B_b, C_b); for i = 0 the b-terms are -inf logits with zero values
    ([R] text under eq 12).  Only complete blocks are pooled."""
    C = np.asarray(C, F64)
    Z = np.asarray(Z, F64)
    ape = np.asarray(ape, F64)
    n = C.shape[0]
    nc = n // m
    if not overlap:
        c = C.shape[1]
        vals = C[: nc * m].reshape(nc, m, c)
        logits = Z[: nc * m].reshape(nc, m, c) + ape[None, :, :]
        return logits, vals
    c = C.shape[1] // 2
    Cb, Ca = C[:, :c], C[:, c:]
    Zb, Za = Z[:, :c], Z[:, c:]
    Bb, Ba = ape[:, :c], ape[:, c:]
    la = Za[: nc * m].reshape(nc, m, c) + Ba[None]
    va = Ca[: nc * m].reshape(nc, m, c)
    lb = np.full((nc, m, c), -np.inf)
    vb = np.zeros((nc, m, c))
    if nc > 1:
        lb[1:] = Zb[: (nc - 1) * m].reshape(nc - 1, m, c) + Bb[None]
        vb[1:] = Cb[: (nc - 1) * m].reshape(nc - 1, m, c)
    return np.concatenate([la, lb], axis=1), np.concatenate([va, vb], axis=1)


def softmax(x, axis):
    """Softmax with the maximum subtracted (exact in exact arithmetic)."""
    x = np.asarray(x, F64)
    mx = np.max(x, axis=axis, keepdims=True)
    e = np.exp(x - mx)
    return e / np.sum(e, axis=axis, keepdims=True)


def pool_weights(C, Z, ape, m, overlap):
    """S of eq 11 / eq 22: per (block, channel) softmax over its L rows."""
    logits, _ = pool_terms(C, Z, ape, m, overlap)
    return softmax(logits, axis=1)


def pool(C, Z, ape, m, overlap):
    """C^Comp_i = sum_j S_j (.) C_j  (eq 12 / eq 23) for every complete block."""
    logits, vals = pool_terms(C, Z, ape, m, overlap)
    return np.sum(softmax(logits, axis=1) * vals, axis=1)


# ---------------------------------------------------------------------------
# O3: entry epilogue - QK RMSNorm and partial RoPE ([R] 2.3.3; [A] Compressor)
# ---------------------------------------------------------------------------
def rms_norm(x, eps):
    """x / sqrt(mean(x^2) + eps) over the last axis, unit weight."""
    x = np.asarray(x, F64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def rope(x, pos, rope_dims: int, theta: float, inverse: bool = False):
    """Rotate the last `rope_dims` channels of x by position `pos`.

    Pairs are adjacent channels (2p, 2p+1) of that tail, rotated by the angle
    pos * theta^(-2p/r) (negated when inverse).  `pos` broadcasts against the
    leading axes of x (one position per row)."""
    x = np.array(x, F64, copy=True)
    r = rope_dims
    if r == 0:
        return x
    c = x.shape[-1]
    pos = np.asarray(pos, F64)
    p = np.arange(r // 2, dtype=F64)
    freq = theta ** (-2.0 * p / r)
    ang = pos[..., None] * freq  # [..., r/2]
    if inverse:
        ang = -ang
    cos, sin = np.cos(ang), np.sin(ang)
    while cos.ndim < x.ndim:  # broadcast over any axes between rows and channels
        cos = cos[..., None, :]
        sin = sin[..., None, :]
    x0 = x[..., c - r :: 2].copy()
    x1 = x[..., c - r + 1 :: 2].copy()
    x[..., c - r :: 2] = x0 * cos - x1 * sin
    x[..., c - r + 1 :: 2] = x0 * sin + x1 * cos
    return x


def entry_epilogue(x, positions, qk_norm, eps, rope_dims, theta, store):
    """Round the pooled (or projected) row to the storage type, as [A]
    Compressor's cast to the model dtype before its RMSNorm does; normalise;
    rotate at the entry's position; round to storage again."""
    y = round_to(x, store)
    y = rms_norm(y, eps) if qk_norm else y
    y = rope(y, positions, rope_dims, theta)
    return round_to(y, store)


def compress_prefill(H, W_kv, W_z, ape, m, overlap, qk_norm=True, eps=1e-6,
                     rope_dims=0, theta=10000.0, store="f32"):
    """Compressed entries of one sequence: O1 -> O2 -> O3.  Entry i sits at
    position m*i for RoPE ([A] Compressor: positions 0, m, 2m, ...)."""
    C = project(H, W_kv)
    Z = project(H, W_z)
    ent = pool(C, Z, ape, m, overlap)
    pos = m * np.arange(ent.shape[0], dtype=F64)
    return entry_epilogue(ent, pos, qk_norm, eps, rope_dims, theta, store)


def window_rows(H, W_win, qk_norm=True, eps=1e-6, rope_dims=0, theta=10000.0,
                store="f32", pos0=0):
    """Uncompressed per-token KV for the sliding window ([A] attention wkv ->
    kv_norm -> RoPE at the token's own position)."""
    V = project(H, W_win)
    pos = pos0 + np.arange(V.shape[0], dtype=F64)
    return entry_epilogue(V, pos, qk_norm, eps, rope_dims, theta, store)


# ---------------------------------------------------------------------------
# O5 / O6: lightning indexer and top-k  ([R] eq 16-17; [A] Indexer)
# ---------------------------------------------------------------------------
def visible_entries(t, m):
    """Number of compressed entries visible to 0-indexed token t."""
    return (np.asarray(t) + 1) // m


def index_scores(qI, wI, KI, m, t0=0):
    """I[t, s] = sum_h w[t,h] * ReLU(q[t,h] . K[s]) for visible s, -inf
    otherwise.  qI [n, hI, cI], wI [n, hI], KI [n_e, cI]; rows are tokens
    t0 .. t0+n-1."""
    qI = np.asarray(qI, F64)
    wI = np.asarray(wI, F64)
    KI = np.asarray(KI, F64)
    dots = np.einsum("thd,sd->ths", qI, KI)
    I = np.einsum("th,ths->ts", wI, np.maximum(dots, 0.0))
    t = t0 + np.arange(qI.shape[0])
    vis = visible_entries(t, m)
    s = np.arange(KI.shape[0])
    return np.where(s[None, :] < vis[:, None], I, -np.inf)


def topk(scores, k, m, t0=0):
    """Per row, the k_t = min(k, visible) entries of largest score, ties to
    the smaller index; slots k_t..k-1 hold -1.  Row order: descending score."""
    scores = np.asarray(scores, F64)
    n, ne = scores.shape
    out = np.full((n, k), -1, dtype=np.int64)
    for r in range(n):
        v = int(min(ne, visible_entries(t0 + r, m)))
        kt = min(k, v)
        if kt == 0:
            continue
        order = np.argsort(-scores[r, :v], kind="stable")
        out[r, :kt] = order[:kt]
    return out


# ---------------------------------------------------------------------------
# O7 - O10: shared-KV MQA with window and sink  ([R] eq 18-19, 27; 2.3.3)
# ---------------------------------------------------------------------------
def topk_bf16_scores(scores, k, m, t0=0):
    """The selector on index scores quantised from fp32 to bf16 ([R] section
    4.4, the indexer QK path under quantisation-aware training: bf16 scores
    for a faster top-k): the top-k of the scores rounded to bf16, ties still
    broken toward the smaller entry index."""
    return topk(round_bf16(scores), k, m, t0=t0)


def query_prologue(q, pos, qk_norm, eps, rope_dims, theta):
    """Per-head RMSNorm, then RoPE of the last r dims at the query position.
    q [rows, nh, c]; pos [rows]."""
    y = rms_norm(q, eps) if qk_norm else np.asarray(q, F64)
    return rope(y, np.asarray(pos, F64), rope_dims, theta)


def attention_probs(qh, kv, sink, scale):
    """Eq 27: p_j = exp(z_j) / (sum_k exp(z_k) + exp(z')), z = scale q.kv.
    qh [nh, c], kv [N, c], sink [nh].  Returns (p [nh, N], p_sink [nh])."""
    z = scale * (np.asarray(qh, F64) @ np.asarray(kv, F64).T)
    zs = np.asarray(sink, F64)
    M = np.maximum(np.max(z, axis=1, initial=-np.inf), zs)
    e = np.exp(z - M[:, None])
    es = np.exp(zs - M)
    den = np.sum(e, axis=1) + es
    return e / den[:, None], es / den


def attend(qh, kv, sink, scale):
    """o_h = sum_j p_j kv_j: each candidate is both key and value (eq 19)."""
    kv = np.asarray(kv, F64)
    if kv.shape[0] == 0:
        return np.zeros(np.shape(qh))
    p, _ = attention_probs(qh, kv, sink, scale)
    return p @ kv


def window_range(t, n_win):
    """Positions of the uncompressed window of token t: [t-n_win+1, t]."""
    return np.arange(max(0, t - n_win + 1), t + 1)


def output_epilogue(o, pos, rope_dims, theta, store):
    """Inverse RoPE on the last r dims at the query position, then round."""
    return round_to(rope(o, np.asarray(pos, F64), rope_dims, theta, inverse=True), store)


def sparse_mqa_prefill(q, win_kv, comp, idx, sink, n_win, scale, qk_norm=True,
                       eps=1e-6, rope_dims=0, theta=10000.0, store="f32", rows=None):
    """CSA core attention: window rows of t plus the selected entries idx[t]
    (-1 = empty slot); no de-duplication between the two ([A] topk_idxs
    concatenation).  q [n, nh, c]; win_kv [n, c]; comp [n_e, c]; idx [n, k]."""
    q = np.asarray(q, F64)
    n, nh, c = q.shape
    rows = range(n) if rows is None else rows
    out = np.zeros((len(rows), nh, c))
    for i, t in enumerate(rows):
        qh = query_prologue(q[t][None], [t], qk_norm, eps, rope_dims, theta)[0]
        sel = [s for s in np.asarray(idx[t]).tolist() if s >= 0]
        kv = np.concatenate([np.asarray(win_kv, F64)[window_range(t, n_win)],
                             np.asarray(comp, F64)[sel]], axis=0)
        out[i] = attend(qh, kv, sink, scale)
        out[i] = output_epilogue(out[i][None], [t], rope_dims, theta, "f64")[0]
    return round_to(out, store)


def dense_mqa_prefill(q, win_kv, comp, sink, m, n_win, scale, qk_norm=True,
                      eps=1e-6, rope_dims=0, theta=10000.0, store="f32", rows=None):
    """HCA core attention: window rows plus every visible entry
    s < floor((t+1)/m) ([A] HCA selection rule)."""
    q = np.asarray(q, F64)
    n, nh, c = q.shape
    rows = range(n) if rows is None else rows
    comp = np.asarray(comp, F64)
    out = np.zeros((len(rows), nh, c))
    for i, t in enumerate(rows):
        qh = query_prologue(q[t][None], [t], qk_norm, eps, rope_dims, theta)[0]
        v = int(min(comp.shape[0], visible_entries(t, m)))
        kv = np.concatenate([np.asarray(win_kv, F64)[window_range(t, n_win)], comp[:v]], axis=0)
        o = attend(qh, kv, sink, scale)
        out[i] = output_epilogue(o[None], [t], rope_dims, theta, "f64")[0]
    return round_to(out, store)


# ---------------------------------------------------------------------------
# OD: decode - the pages' stateful compressor  ([A] Compressor decode branch)
# ---------------------------------------------------------------------------
class CompressorDecodeOracle:
    """Token-at-a-time compressor.  Keeps the raw projected rows (C, Z + B)
    of the current block and, under overlap, of the previous block; when the
    token at `pos` closes a block ((pos+1) mod m == 0) it pools that block
    (plus the previous block's b-series) and returns the finished entry.

    Written independently of `pool`: the prefill/decode agreement is a pin."""

    def __init__(self, c, m, overlap, ape, qk_norm=True, eps=1e-6,
                 rope_dims=0, theta=10000.0, store="f32"):
        self.c, self.m, self.overlap = c, m, bool(overlap)
        self.ape = np.asarray(ape, F64)
        self.cfg = (qk_norm, eps, rope_dims, theta, store)
        self.rows = {}  # block index -> list of (C row, Z+B row) per position

    def append(self, pos, c_row, z_row):
        m = self.m
        blk, r = divmod(int(pos), m)
        c_row = np.asarray(c_row, F64)
        lg = np.asarray(z_row, F64) + self.ape[r]
        self.rows.setdefault(blk, []).append((c_row, lg))
        assert len(self.rows[blk]) == r + 1, "tokens must arrive in order"
        for old in [b for b in self.rows if b < blk - 1]:
            del self.rows[old]
        if r != m - 1:
            return None
        c = self.c
        if self.overlap:
            vals = [cr[c:] for cr, _ in self.rows[blk]]
            logs = [lg[c:] for _, lg in self.rows[blk]]
            if blk >= 1:
                vals += [cr[:c] for cr, _ in self.rows[blk - 1]]
                logs += [lg[:c] for _, lg in self.rows[blk - 1]]
        else:
            vals = [cr for cr, _ in self.rows[blk]]
            logs = [lg for _, lg in self.rows[blk]]
        vals = np.stack(vals)
        logs = np.stack(logs)
        w = np.exp(logs - logs.max(axis=0))
        ent = (w * vals).sum(axis=0) / w.sum(axis=0)
        qk_norm, eps, rd, theta, store = self.cfg
        return entry_epilogue(ent[None], [m * blk], qk_norm, eps, rd, theta, store)[0]


def attend_decode_row(q_row, pos, win_rows, entries, sink, scale, qk_norm=True,
                      eps=1e-6, rope_dims=0, theta=10000.0, store="f32"):
    """One decode query at position `pos`: the window rows (positions
    pos-n_win+1..pos, oldest first) plus the given compressed entries."""
    qh = query_prologue(np.asarray(q_row, F64)[None], [pos], qk_norm, eps, rope_dims, theta)[0]
    kv = np.concatenate([np.asarray(win_rows, F64), np.asarray(entries, F64)], axis=0)
    o = attend(qh, kv, sink, scale)
    return round_to(output_epilogue(o[None], [pos], rope_dims, theta, "f64")[0], store)


# ---------------------------------------------------------------------------
# O8: the layer around the four calls -- query path and grouped output
# projection ([R] eq 13-15 and 18, section 2.3.1 (d); [A] "Q, K, V 映射与位置
# 编码注入" excerpt (wq_a -> q_norm -> wq_b) and "输出投影" excerpt)
# ---------------------------------------------------------------------------
def query_proj(H, W_DQ, g_q, W_w, W_UQ, W_IUQ, eps, store):
    """c^Q = q_norm(H . W_DQ) (RMSNorm over the latent, weight g_q; None =
    unit), stored; q = c^Q . W_UQ and q^I = c^Q . W_IUQ, stored; w^I = H . W_w,
    stored.  Weights in the pages' orientation [in, out].  The per-head query
    RMSNorm and RoPE belong to the attention call, not here.  Returns
    (c^Q, q, q^I, w^I) as [n, width] arrays."""
    lat = rms_norm(project(H, W_DQ), eps)
    if g_q is not None:
        lat = lat * np.asarray(g_q, F64)
    cq = store(lat)
    q = store(project(cq, W_UQ))
    qI = store(project(cq, W_IUQ))
    wI = store(project(H, W_w))
    return cq, q, qI, wI


def output_proj(o, wo_a, wo_b, store):
    """Grouped low-rank output projection.  o [n, n_h*c] (the attention
    output, already rotated back) is split into g consecutive groups of
    n_h*c/g channels; group j is projected by wo_a[j] [d_g, n_h*c/g] to d_g
    channels (stored); the g*d_g concatenation is projected by wo_b [d, g*d_g]
    to d (stored).  wo_a and wo_b are linear-layer weights [out, in]."""
    o = np.asarray(o, F64)
    n, g = o.shape[0], wo_a.shape[0]
    kg = o.shape[1] // g
    mid = np.empty((n, g, wo_a.shape[1]))
    for j in range(g):
        mid[:, j, :] = o[:, j * kg:(j + 1) * kg] @ np.asarray(wo_a[j], F64).T
    mid = store(mid.reshape(n, -1))
    return store(mid @ np.asarray(wo_b, F64).T)


# ---------------------------------------------------------------------------
# O9: the indexer's quantised QK path ([A] Compressor with rotate=True and the
# Indexer forward: rotate_activation, then fp4_act_quant of q^I and of the
# stored keys; [R] section 4.4: the indexer QK path cached, loaded and
# multiplied in FP4)
# ---------------------------------------------------------------------------
FP4_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])  # E2M1 magnitudes
FP4_BLOCK = 32


def hadamard(x):
    """rotate_activation: the normalised Walsh-Hadamard transform over the last
    axis (length a power of two), x . H_n / sqrt(n) with H_n the Sylvester
    matrix (H_1 = [1], H_2k = [[H_k, H_k], [H_k, -H_k]])."""
    x = np.asarray(x, F64)
    n = x.shape[-1]
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    assert h.shape[0] == n, "length must be a power of two"
    return x @ h / math.sqrt(n)


def fp4_quant(x):
    """fp4_act_quant, read as the MX-style format: every block of 32
    consecutive values along the last axis shares a power-of-two scale 2^e,
    e = ceil(log2(amax / 6)) (e = 0 for an all-zero block), so that every
    |x| / 2^e <= 6; each x / 2^e is then rounded to the nearest E2M1 value,
    ties to the even mantissa (0, 1, 2, 4).  Returns (codes, exps): codes in
    0..15, bit 3 the sign (set only for a nonzero magnitude), bits 0-2 the
    index into FP4_GRID; exps the block exponents e."""
    x = np.asarray(x, F64)
    nb = x.shape[-1] // FP4_BLOCK
    xb = x.reshape(x.shape[:-1] + (nb, FP4_BLOCK))
    amax = np.max(np.abs(xb), axis=-1)
    # the smallest e with amax <= 6 * 2^e, without a rounded division:
    # amax = f * 2^k (0.5 <= f < 1) gives e = k - 3 when f <= 0.75, else k - 2
    f, k = np.frexp(amax)
    e = np.where(amax > 0, np.where(f <= 0.75, k - 3, k - 2), 0).astype(np.int64)
    a = np.abs(xb) / np.ldexp(1.0, e)[..., None]
    idx = np.searchsorted(FP4_GRID, a, side="right") - 1   # largest grid value <= a
    idx = np.clip(idx, 0, 7)
    up = np.minimum(idx + 1, 7)
    dlo, dhi = a - FP4_GRID[idx], FP4_GRID[up] - a
    pick_up = (dhi < dlo) | ((dhi == dlo) & (idx % 2 == 1))
    mag = np.where(pick_up, up, idx)
    sign = (xb < 0) & (mag > 0)
    codes = (mag + 8 * sign).reshape(x.shape)
    return codes.astype(np.int64), e


def fp4_dequant(codes, exps):
    """Values of fp4_quant's output: sign * FP4_GRID[code & 7] * 2^e."""
    codes = np.asarray(codes)
    nb = codes.shape[-1] // FP4_BLOCK
    cb = codes.reshape(codes.shape[:-1] + (nb, FP4_BLOCK))
    v = np.where(cb >= 8, -1.0, 1.0) * FP4_GRID[cb & 7] * np.ldexp(1.0, np.asarray(exps))[..., None]
    return v.reshape(codes.shape)


def index_scores_fp4(qI, wI, KI, m, t0=0):
    """Index scores of the quantised path: q^I and the keys rotated and
    FP4-quantised, then eq 16 on the dequantised values."""
    qc, qe = fp4_quant(hadamard(qI))
    kc, ke = fp4_quant(hadamard(KI))
    return index_scores(fp4_dequant(qc, qe), wI, fp4_dequant(kc, ke), m, t0=t0)


# ---------------------------------------------------------------------------
# O11: backward of the core attention.  [R] section 4.3 asks for a
# deterministic attention backward (no atomic adds: per-unit accumulation
# buffers and a deterministic global sum); what it computes is the chain rule
# through the forward of eq 19 and 27 with the query RMSNorm / RoPE and the
# output's inverse RoPE of section 2.3.3.  Gradients are taken with respect
# to the raw queries, the stored window rows and entries (the compressor's
# own backward is not part of it) and the sink logits, for an upstream
# gradient dout of the output.
# ---------------------------------------------------------------------------
def attention_backward_row(q_row, t, kv, sink, dout_row, scale, qk_norm=True, eps=1e-6,
                           rope_dims=0, theta=10000.0):
    """One query token t: q_row [nh, c] (raw), kv [N, c] its candidates (keys
    and values), dout_row [nh, c] the gradient of its output.  Returns
    (dq_row [nh, c], dkv [N, c], dsink [nh])."""
    q = np.asarray(q_row, F64)
    kv = np.asarray(kv, F64)
    zs = np.asarray(sink, F64)
    # forward, keeping what the backward needs
    if qk_norm:
        rr = np.sqrt(np.mean(q * q, axis=-1, keepdims=True) + eps)
        nq = q / rr
    else:
        nq = q
    qh = rope(nq, [t], rope_dims, theta)                         # the rotated query
    z = scale * (qh @ kv.T)                                      # [nh, N]
    M = np.maximum(np.max(z, axis=1, initial=-np.inf), zs)
    e = np.exp(z - M[:, None])
    es = np.exp(zs - M)
    den = np.sum(e, axis=1) + es
    p = e / den[:, None]
    ps = es / den
    o_rot = p @ kv                                               # before the inverse RoPE
    # backward: o = R(-t) o_rot, so the gradient reaching o_rot is R(t) dout
    do = rope(np.asarray(dout_row, F64), [t], rope_dims, theta)
    dp = do @ kv.T                                               # [nh, N]
    dd = np.sum(do * o_rot, axis=-1)                             # sum_j p_j dp_j
    dz = p * (dp - dd[:, None])                                  # softmax with the sink term
    dsink = -ps * dd
    dqh = scale * (dz @ kv)
    dkv = p.T @ do + scale * (dz.T @ qh)                         # as value, then as key
    dn = rope(dqh, [t], rope_dims, theta, inverse=True)          # R(t)^T = R(-t)
    if qk_norm:
        dq = (dn - nq * np.mean(dn * nq, axis=-1, keepdims=True)) / rr
    else:
        dq = dn
    return dq, dkv, dsink


def sparse_mqa_backward(q, win_kv, comp, idx, sink, dout, n_win, scale, qk_norm=True,
                        eps=1e-6, rope_dims=0, theta=10000.0):
    """Gradients of sparse_mqa_prefill (unrounded) for upstream gradient dout
    [n, nh, c]: (dq [n, nh, c], dwin [n, c], dcomp [n_e, c], dsink [nh]).  A
    row that is a candidate of several queries sums their contributions."""
    q = np.asarray(q, F64)
    win_kv = np.asarray(win_kv, F64)
    comp = np.asarray(comp, F64)
    n, nh, c = q.shape
    dq = np.zeros_like(q)
    dwin = np.zeros_like(win_kv)
    dcomp = np.zeros_like(comp)
    dsink = np.zeros(nh)
    for t in range(n):
        wr = window_range(t, n_win)
        sel = [s for s in np.asarray(idx[t]).tolist() if s >= 0]
        kv = np.concatenate([win_kv[wr], comp[sel]], axis=0)
        g_q, g_kv, g_s = attention_backward_row(q[t], t, kv, sink, dout[t], scale, qk_norm, eps,
                                                rope_dims, theta)
        dq[t] = g_q
        dwin[wr] += g_kv[: len(wr)]
        for a, s in enumerate(sel):
            dcomp[s] += g_kv[len(wr) + a]
        dsink += g_s
    return dq, dwin, dcomp, dsink


def dense_mqa_backward(q, win_kv, comp, sink, dout, m, n_win, scale, qk_norm=True, eps=1e-6,
                       rope_dims=0, theta=10000.0):
    """Gradients of dense_mqa_prefill: every visible entry s < floor((t+1)/m)
    is a candidate of token t."""
    n = np.asarray(q).shape[0]
    ne = np.asarray(comp).shape[0]
    idx = np.full((n, max(1, ne)), -1)
    for t in range(n):
        v = int(min(ne, visible_entries(t, m)))
        idx[t, :v] = np.arange(v)
    return sparse_mqa_backward(q, win_kv, comp, idx, sink, dout, n_win, scale, qk_norm, eps,
                               rope_dims, theta)


# ---------------------------------------------------------------------------
# O12: FP8 storage of the KV rows ([A] "Q, K, V 映射与位置编码注入" and the
# Compressor: act_quant of kv[..., :-rd] with block size 64 -- the channels
# without RoPE are quantised to FP8, the RoPE channels keep their precision;
# [R] section 2.3.4: the KV cache stores the RoPE dims in BF16 and the rest
# in FP8).  Read as E4M3 (4 exponent bits, bias 7, 3 mantissa bits, largest
# finite 448, subnormal step 2^-9) with one power-of-two scale per block of
# 64 values, the smallest 2^e with max |x| <= 448 * 2^e; each x / 2^e rounds
# to the nearest E4M3 value, ties to the even mantissa.  The pages leave the
# scale's range open; it is stored as one byte e + 127, and here e is floored
# at -117 so that the smallest step of the grid, 2^(e-9), is 2^-126, the
# smallest normal fp32 number: a block whose largest magnitude is below
# 448 * 2^-117 is rounded on that fixed grid.
# ---------------------------------------------------------------------------
FP8_BLOCK = 64
FP8_MAX = 448.0
FP8_E_MIN = -117


def fp8_e4m3_values():
    """Every non-negative finite E4M3 value, indexed by its 7-bit code
    (exponent field << 3 | mantissa): subnormals m * 2^-9 for field 0, else
    (1 + m/8) * 2^(field - 7); field 15 with mantissa 7 is not a number."""
    v = []
    for ef in range(16):
        for mt in range(8):
            if ef == 15 and mt == 7:
                v.append(np.nan)
            elif ef == 0:
                v.append(mt * 2.0 ** -9)
            else:
                v.append((1 + mt / 8.0) * 2.0 ** (ef - 7))
    return np.array(v)


def fp8_quant(x):
    """Returns (codes, exps): codes 0..255 (bit 7 the sign, set only for a
    nonzero magnitude), exps the block exponents e."""
    x = np.asarray(x, F64)
    nb = x.shape[-1] // FP8_BLOCK
    xb = x.reshape(x.shape[:-1] + (nb, FP8_BLOCK))
    amax = np.max(np.abs(xb), axis=-1)
    # smallest e with amax <= 448 * 2^e: amax = f * 2^k, 448 = 0.875 * 2^9
    f, k = np.frexp(amax)
    e = np.where(amax > 0, np.where(f <= 0.875, k - 9, k - 8), 0).astype(np.int64)
    e = np.maximum(e, FP8_E_MIN)
    a = np.abs(xb) / np.ldexp(1.0, e)[..., None]
    grid = fp8_e4m3_values()[:127]                      # finite magnitudes, ascending
    lo = np.clip(np.searchsorted(grid, a, side="right") - 1, 0, 126)
    hi = np.minimum(lo + 1, 126)
    dlo, dhi = a - grid[lo], grid[hi] - a
    pick_up = (dhi < dlo) | ((dhi == dlo) & (lo % 2 == 1))
    mag = np.where(pick_up, hi, lo)
    sign = (xb < 0) & (mag > 0)
    codes = (mag + 128 * sign).reshape(x.shape)
    return codes.astype(np.int64), e


def fp8_dequant(codes, exps):
    """sign * E4M3 magnitude * 2^e of fp8_quant's output."""
    codes = np.asarray(codes)
    nb = codes.shape[-1] // FP8_BLOCK
    cb = codes.reshape(codes.shape[:-1] + (nb, FP8_BLOCK))
    v = np.where(cb >= 128, -1.0, 1.0) * fp8_e4m3_values()[cb & 127]
    v = v * np.ldexp(1.0, np.asarray(exps))[..., None]
    return v.reshape(codes.shape)


def kv_fp8(rows, rope_dims):
    """A stored KV row as its FP8 form holds it: the first c - r channels
    quantised and dequantised, the last r (the RoPE channels) unchanged."""
    rows = np.asarray(rows, F64)
    c = rows.shape[-1]
    out = rows.copy()
    if c - rope_dims:
        codes, e = fp8_quant(rows[..., : c - rope_dims])
        out[..., : c - rope_dims] = fp8_dequant(codes, e)
    return out
