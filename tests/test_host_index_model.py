"""Host model of the index arithmetic of the prefill index scorer
(index_scores_prefill_kernel) and the decode scorer's workspace offsets,
with bounds checks, at the sizes a long-row selection reaches (1024 rows of
a chunk that ends a 1M-token context, 262144 keys) and at the 64K workload.

The formulas below restate the kernel's own: grid, per-workgroup query block
q0 = blockIdx.x * TQ, key chunk [blockIdx.y * key_chunk, kend), the clamped
key row of each staged load, the query rows read, and the 32-bit score offset
tq * ld + si from the workgroup's row base.  Every extreme is evaluated; the
asserts are that each stays inside its buffer and below 2^31 where the
kernel holds it in 32 bits."""
import pytest

ROWS_PER_WG = 256  # 4 waves x 2 blocks x 32 (query, head) rows


def prefill_scorer_extremes(n, n_entries, m, hI, cI, t0, ld, key_chunk=2048):
    """Largest index each access of index_scores_prefill_kernel can form."""
    TQ = ROWS_PER_WG // hI
    nvis = min((t0 + n) // m, n_entries)
    gx, gy = -(-n // TQ), -(-nvis // key_chunk)
    worst = dict(score_off32=0, score_elem=0, key_row=0, q_elem=0, w_elem=0)
    for bx in (0, gx - 1):
        q0 = bx * TQ
        tlast = min(q0 + TQ, n) - 1
        for by in (0, gy - 1):
            kend = min(min((t0 + tlast + 1) // m, n_entries), (by + 1) * key_chunk)
            kbeg = by * key_chunk
            if kbeg >= kend:
                continue
            # staged key rows: min(k0 + key, kend - 1)
            worst["key_row"] = max(worst["key_row"], kend - 1)
            # query rows read: t < n only
            worst["q_elem"] = max(worst["q_elem"], ((min(q0 + TQ, n) - 1) * hI + hI - 1) * cI + cI - 1)
            worst["w_elem"] = max(worst["w_elem"], (min(q0 + TQ, n) - 1) * hI + hI - 1)
            # stores: query q0 + tq (tq < TQ, t < n), entry si < vis(t) <= kend
            for tq in (0, min(TQ, n - q0) - 1):
                t = q0 + tq
                vq = min((t0 + t + 1) // m, n_entries)
                si = min(kend, vq) - 1
                if si < kbeg:
                    continue
                off32 = tq * ld + si
                worst["score_off32"] = max(worst["score_off32"], off32)
                worst["score_elem"] = max(worst["score_elem"], q0 * ld + off32)
    return worst


@pytest.mark.parametrize("name,n,n_entries,m,hI,cI,t0", [
    ("64K workload", 65536, 16384, 4, 16, 64, 0),
    ("chunk of 8192 ending 1M", 8192, 262144, 4, 16, 64, (1 << 20) - 8192),
    ("1024 rows x 262144 keys", 1024, 262144, 4, 16, 64, (1 << 20) - 1024),
    ("4 heads, 1024 rows x 262144 keys", 1024, 262144, 4, 4, 128, (1 << 20) - 1024),
])
def test_prefill_scorer_indices_in_bounds(name, n, n_entries, m, hI, cI, t0):
    nvis_last = min((t0 + n) // m, n_entries)
    ld = (nvis_last + 3) // 4 * 4  # the score rows' stride
    TQ = ROWS_PER_WG // hI
    assert TQ * ld < 2 ** 31  # the launcher's check, which the 32-bit offsets rely on
    w = prefill_scorer_extremes(n, n_entries, m, hI, cI, t0, ld)
    assert w["score_off32"] < 2 ** 31, name
    assert w["score_elem"] < n * ld, name
    assert w["key_row"] < n_entries, name
    assert w["q_elem"] < n * hI * cI, name
    assert w["w_elem"] < n * hI, name


def test_decode_selector_offsets_at_long_rows():
    """The decode selector over batches of long prefill rows: every workspace
    offset is formed in 64 bits (scores b * n_entries + s, candidates
    (b * chunks + chunk) * L + i) and stays inside the carved regions."""
    import long_context_attention_10_amd as L
    B, ne, k = 1024, 262144, 512
    d = L.IndexDesc(0, B, 16, 64, 4, k, L.CSA_BF16, ne)
    total = L.workspace_bytes("index_topk_decode", d)
    chunks = -(-ne // 1024)
    per = min(1024, (2 * k // chunks + 16 + 7) // 8 * 8)
    scores = B * ne * 4
    cand = B * chunks * per * 8
    meta = B * chunks * 16
    assert scores + cand + meta <= total


def long_path_batches(n, n_entries, m, t0, rows_per_batch):
    """The long-row selection's sub-batches as its launcher forms them: rows
    r0 .. r0 + R - 1 at positions t0 + r0 .., scored by the prefill scorer
    into the decode workspace's score rows (stride = the entries the last row
    of the chunk sees)."""
    ne = min((t0 + n) // m, n_entries)
    for r0 in range(0, n, rows_per_batch):
        yield min(rows_per_batch, n - r0), t0 + r0, ne


@pytest.mark.parametrize("name,n,n_entries,m,hI,cI,t0,rows", [
    ("chunk of 8192 ending 1M, 16 heads", 8192, 262144, 4, 16, 64, (1 << 20) - 8192, 1024),
    ("chunk of 8192 ending 1M, 4 heads", 8192, 262144, 4, 4, 128, (1 << 20) - 8192, 1024),
    ("chunk crossing 16384 entries", 700, 20000, 4, 16, 64, 65000, 700),
    ("ragged last batch", 3000, 100000, 4, 8, 64, 390000, 1024),
])
def test_long_path_scorer_indices_in_bounds(name, n, n_entries, m, hI, cI, t0, rows):
    """Each sub-batch of the long-row selection runs the prefill scorer with
    the decode workspace's unpadded score stride: every index stays inside
    the batch's score rows, key table, query rows and weights, and every
    32-bit offset below 2^31."""
    TQ = ROWS_PER_WG // hI
    for R, t0b, ne in long_path_batches(n, n_entries, m, t0, rows):
        ld = ne
        assert TQ * ld < 2 ** 31
        w = prefill_scorer_extremes(R, ne, m, hI, cI, t0b, ld)
        assert w["score_off32"] < 2 ** 31, name
        assert w["score_elem"] < R * ld, name  # the carved score region: R rows of ne
        assert w["key_row"] < ne <= n_entries, name
        assert w["q_elem"] < R * hI * cI, name
        assert w["w_elem"] < R * hI, name
        # candidates from the stored scores: row b reads s < vis(b) <= ne
        for b in (0, R - 1):
            vis = min((t0b + b + 1) // m, ne)
            assert b * ne + vis - 1 < R * ld
