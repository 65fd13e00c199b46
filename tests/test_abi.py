"""C-ABI checks that need no GPU: the library loads, exports every function
that include/csa.h declares, and rejects bad arguments on the host before
anything is enqueued (the documented error codes)."""
import ctypes
import os
import re

import pytest

import long_context_attention_10_amd as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?(?:int|size_t|char\s*\*|const char\s*\*)\s*\**\s*(\w+)\s*\(",
                       src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.fail("libcsa.so is not built (run python -m long_context_attention_10_amd.build)")
    return L.load()


def test_header_declares_the_eight_entry_points():
    names = declared_functions()
    for f in ["csa_compress_prefill", "csa_compress_decode", "csa_index_topk_prefill",
              "csa_index_topk_decode", "csa_sparse_mqa_prefill", "csa_sparse_mqa_decode",
              "hca_dense_mqa_prefill", "hca_dense_mqa_decode"]:
        assert f in names


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 12
    for f in names:
        assert hasattr(lib, f), f"libcsa.so does not export {f}"
    assert set(names) == set(L.EXPORTED)


def test_abi_version_and_status_strings(lib):
    assert lib.csa_abi_version() == 10
    for code in (0, -1, -2, -3, -4):
        assert len(lib.csa_status_string(code)) > 0
    assert lib.csa_status_string(-99) == b"unknown status"


def test_struct_sizes_match_c_layout(tmp_path):
    """The binding's ctypes descriptors have the C compiler's size and field
    offsets for every descriptor in include/csa.h."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    pairs = [("csa_compress_desc", L.CompressDesc), ("csa_index_desc", L.IndexDesc),
             ("csa_attn_desc", L.AttnDesc), ("csa_query_desc", L.QueryDesc),
             ("csa_oproj_desc", L.OprojDesc), ("csa_fp4_desc", L.Fp4Desc),
             ("csa_kv8_desc", L.Kv8Desc)]
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "csa.h"', "int main(void) {"]
    for cname, py in pairs:
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'  printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines.append("  return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run([cc, "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = dict(l.rsplit(" ", 1) for l in subprocess.run([str(exe)], capture_output=True, text=True,
                                                        check=True).stdout.splitlines())
    for cname, py in pairs:
        assert int(got[f"{cname} size"]) == ctypes.sizeof(py), cname
        for f, _ in py._fields_:
            assert int(got[f"{cname} {f}"]) == getattr(py, f).offset, (cname, f)


def test_workspace_and_state_sizes(lib):
    d = L.compress_desc(n=2048, d=1024, c=128, m=4, overlap=0)
    assert L.workspace_bytes("compress_prefill", d) >= 2048 * (2 * 128 + 128) * 4
    d1 = L.compress_desc(batch=4, d=4096, c=512, m=4, overlap=1)
    assert L.csa_state_bytes(d1) == 4 * 3 * 3 * 512 * 4
    d0 = L.compress_desc(batch=4, d=4096, c=512, m=128, overlap=0)
    assert L.csa_state_bytes(d0) == 4 * 1 * 3 * 512 * 4
    idx = L.IndexDesc(65536, 1, 16, 64, 4, 512, L.CSA_BF16, 16384)
    assert L.workspace_bytes("index_topk_prefill", idx) >= 65536 * 16384 * 4
    ad = L.attn_desc(batch=4, nh=64, c=512, k=1024, n_entries=262144, dtype=L.CSA_BF16)
    assert L.workspace_bytes("sparse_mqa_decode", ad) > 0
    assert lib.csa_workspace_bytes(0, None) == 0
    # no entry carries state between calls in its workspace: nothing needs clearing
    dd = L.IndexDesc(0, 4, 16, 64, 4, 1024, L.CSA_BF16, 262144)
    assert L.workspace_zero_bytes("index_topk_decode", dd) == 0
    # scores (4 B per entry) plus each 1024-entry chunk's candidates (8 B each) and record
    chunks, per_chunk = 256, 2 * 1024 // 256 + 16
    assert L.workspace_bytes("index_topk_decode", dd) == (
        4 * 262144 * 4 + 4 * chunks * per_chunk * 8 + 4 * chunks * 16)
    assert L.workspace_zero_bytes("index_topk_prefill", idx) == 0
    assert L.workspace_zero_bytes("sparse_mqa_decode", ad) == 0
    assert lib.csa_workspace_zero_bytes(3, None) == 0


def _p(v=1):
    return ctypes.c_void_p(v)  # never dereferenced: validation fails first


@pytest.mark.parametrize("change,code", [
    (dict(c=96), -2),            # entry width outside the kernels' set
    (dict(d=100), -2),           # hidden size not a multiple of 64
    (dict(dtype=7), -2),         # unknown dtype
    (dict(m=0), -1),
    (dict(overlap=2), -1),
    (dict(rope_dims=3), -1),
    (dict(n=-1), -1),
])
def test_compress_prefill_rejects(lib, change, code):
    kw = dict(n=64, d=128, c=128, m=4, overlap=0)
    kw.update(change)
    d = L.compress_desc(**kw)
    st = lib.csa_compress_prefill(ctypes.byref(d), _p(), _p(), _p(), _p(), None, _p(), None, None,
                                  None, _p(), 1 << 40, None)
    assert st == code


def test_null_descriptor_and_pointers(lib):
    assert lib.csa_compress_prefill(None, *([None] * 10), 0, None) == -1
    d = L.compress_desc(n=64, d=128, c=128, m=4)
    # H missing
    assert lib.csa_compress_prefill(ctypes.byref(d), None, _p(), _p(), _p(), None, _p(), None, None,
                                    None, _p(), 1 << 40, None) == -1
    # window output requested without window weights
    assert lib.csa_compress_prefill(ctypes.byref(d), _p(), _p(), _p(), _p(), None, _p(), _p(), None,
                                    None, _p(), 1 << 40, None) == -1
    # workspace too small
    assert lib.csa_compress_prefill(ctypes.byref(d), _p(), _p(), _p(), _p(), None, _p(), None, None,
                                    None, _p(), 16, None) == -3


def test_index_and_attention_reject(lib):
    bad = L.IndexDesc(16, 1, 5, 64, 4, 8, L.CSA_BF16, 4)  # 5 indexer heads
    assert lib.csa_index_topk_prefill(ctypes.byref(bad), _p(), _p(), _p(), _p(), _p(), 1 << 30, None) == -2
    big_k = L.IndexDesc(16, 1, 16, 64, 4, 4096, L.CSA_BF16, 4)
    assert lib.csa_index_topk_prefill(ctypes.byref(big_k), _p(), _p(), _p(), _p(), _p(), 1 << 30, None) == -2
    # rows beyond the register selector take the decode top-k: fp32 scores only
    too_many = L.IndexDesc(1 << 20, 1, 16, 64, 4, 512, L.CSA_BF16, 1 << 18, L.CSA_BF16)
    assert lib.csa_index_topk_prefill(ctypes.byref(too_many), _p(), _p(), _p(), _p(), _p(), 1 << 40, None) == -2
    long_rows = L.IndexDesc(1 << 20, 1, 16, 64, 4, 512, L.CSA_BF16, 1 << 18)
    assert lib.csa_index_topk_prefill(ctypes.byref(long_rows), _p(), _p(), _p(), _p(), _p(), 8, None) == -3
    assert L.workspace_zero_bytes("index_topk_prefill", long_rows) == 0
    short_rows = L.IndexDesc(1 << 14, 1, 16, 64, 4, 512, L.CSA_BF16, 1 << 12)
    assert L.workspace_zero_bytes("index_topk_prefill", short_rows) == 0
    dd = L.IndexDesc(0, 2, 16, 64, 4, 8, L.CSA_BF16, 100)
    assert lib.csa_index_topk_decode(ctypes.byref(dd), _p(), _p(), _p(), _p(), _p(), _p(), 8, None) == -3
    a = L.attn_desc(n=8, nh=65, c=128, k=4)
    assert lib.csa_sparse_mqa_prefill(ctypes.byref(a), _p(), _p(), _p(), _p(), _p(), _p(), None, 0, None) == -2
    a = L.attn_desc(n=8, nh=8, c=96, k=4)
    assert lib.csa_sparse_mqa_prefill(ctypes.byref(a), _p(), _p(), _p(), _p(), _p(), _p(), None, 0, None) == -2
    a = L.attn_desc(n=8, nh=8, c=128, k=0)
    assert lib.csa_sparse_mqa_prefill(ctypes.byref(a), _p(), _p(), _p(), _p(), _p(), _p(), None, 0, None) == -1
    a = L.attn_desc(batch=2, nh=8, c=128, m=4, n_entries=64)
    assert lib.hca_dense_mqa_decode(ctypes.byref(a), _p(), _p(), _p(), _p(), _p(), _p(), _p(), 8, None) == -3


def test_binding_keeps_the_zero_region(lib):
    """The binding clears a workspace's leading zero bytes only when the buffer
    is new or the region grew past what the last call left zero (host-side
    logic, exercised on CPU tensors)."""
    import torch
    slot = "zero-region-test"
    key = ("cpu", slot)
    L._WS.pop(key, None)
    L._WS_ZERO.pop(key, None)
    t, n = L.workspace(4096, "cpu", slot, zero_bytes=1024)
    assert n == 4096 and int(torch.count_nonzero(t[:1024])) == 0
    t[1024:2048] = 7           # the call's other regions: scores, lists, ...
    t2, _ = L.workspace(4096, "cpu", slot, zero_bytes=1024)
    assert t2.data_ptr() == t.data_ptr() and int(t2[1500]) == 7  # nothing cleared
    t2[:16] = 3                # (a call never leaves this; shows no clearing happens)
    L.workspace(4096, "cpu", slot, zero_bytes=512)  # smaller region: no clearing
    assert int(t2[0]) == 3
    t2[:16] = 0
    t3, _ = L.workspace(4096, "cpu", slot, zero_bytes=2048)  # grew past 512: cleared
    assert int(torch.count_nonzero(t3[:2048])) == 0
    L.workspace(4096, "cpu", slot)  # an entry without zero bytes forgets the state
    assert key not in L._WS_ZERO
    t4, _ = L.workspace(8192, "cpu", slot, zero_bytes=1024)  # new buffer: cleared
    assert t4.numel() == 8192 and int(torch.count_nonzero(t4[:1024])) == 0
    L._WS.pop(key, None)
    L._WS_ZERO.pop(key, None)


def test_layer_projection_calls_reject(lib):
    q = L.QueryDesc(64, 256, 128, 8, 128, 4, 64, L.CSA_BF16, 1e-6)
    args = [_p()] * 10 + [1 << 40, None]
    bad = L.QueryDesc(64, 256, 128, 8, 128, 4, 64, L.CSA_F32, 1e-6)
    assert lib.csa_query_proj(ctypes.byref(bad), *args) == -2      # bf16 only
    bad = L.QueryDesc(64, 100, 128, 8, 128, 4, 64, L.CSA_BF16, 1e-6)
    assert lib.csa_query_proj(ctypes.byref(bad), *args) == -2      # d not a multiple of 64
    assert lib.csa_query_proj(None, *args) == -1
    assert lib.csa_query_proj(ctypes.byref(q), None, *([_p()] * 9), 1 << 40, None) == -1  # H
    assert lib.csa_query_proj(ctypes.byref(q), *([_p()] * 9), None, 0, None) == -3  # no ws
    o = L.OprojDesc(64, 8, 128, 2, 64, 256, L.CSA_BF16)
    oargs = [_p()] * 5 + [1 << 40, None]
    bad = L.OprojDesc(64, 8, 128, 3, 64, 256, L.CSA_BF16)
    assert lib.csa_output_proj(ctypes.byref(bad), *oargs) == -1   # groups must divide 8*128
    bad = L.OprojDesc(64, 8, 128, 32, 64, 256, L.CSA_BF16)
    assert lib.csa_output_proj(ctypes.byref(bad), *oargs) == -2   # 32-channel groups
    assert lib.csa_output_proj(ctypes.byref(o), None, _p(), _p(), _p(), _p(), 1 << 40, None) == -1
    assert lib.csa_output_proj(ctypes.byref(o), _p(), _p(), _p(), _p(), None, 0, None) == -3
    assert L.workspace_bytes("output_proj", o) == 64 * 2 * 64 * 2
    assert L.workspace_bytes("query_proj", q) >= 64 * (128 + 4) * 4 + 64 * 128 * 2


def test_index_score_dtype(lib):
    """Prefill selects on fp32 or bf16 scores (half the workspace); decode only
    on fp32; anything else is rejected before a launch."""
    d32 = L.IndexDesc(4096, 1, 16, 64, 4, 512, L.CSA_BF16, 1024, L.CSA_F32)
    d16 = L.IndexDesc(4096, 1, 16, 64, 4, 512, L.CSA_BF16, 1024, L.CSA_BF16)
    assert L.workspace_bytes("index_topk_prefill", d16) * 2 == L.workspace_bytes("index_topk_prefill", d32)
    bad = L.IndexDesc(4096, 1, 16, 64, 4, 512, L.CSA_BF16, 1024, 7)
    assert lib.csa_index_topk_prefill(ctypes.byref(bad), _p(), _p(), _p(), _p(), _p(), 1 << 40, None) == -2
    dec = L.IndexDesc(0, 2, 16, 64, 4, 512, L.CSA_BF16, 1024, L.CSA_BF16)
    assert lib.csa_index_topk_decode(ctypes.byref(dec), _p(), _p(), _p(), _p(), _p(), _p(), 1 << 40,
                                     None) == -2


def test_fp4_calls_reject(lib):
    d = L.Fp4Desc(16, 96, L.CSA_BF16)
    assert lib.csa_indexer_fp4_quant(ctypes.byref(d), _p(), _p(), _p(), None) == -2  # width
    d = L.Fp4Desc(16, 64, 9)
    assert lib.csa_indexer_fp4_quant(ctypes.byref(d), _p(), _p(), _p(), None) == -2  # dtype
    d = L.Fp4Desc(16, 64, L.CSA_BF16)
    assert lib.csa_indexer_fp4_quant(ctypes.byref(d), None, _p(), _p(), None) == -1
    assert lib.csa_indexer_fp4_quant(None, _p(), _p(), _p(), None) == -1
    dec = L.IndexDesc(0, 2, 16, 64, 4, 512, L.CSA_F32, 1024)
    assert lib.csa_index_topk_decode_fp4(ctypes.byref(dec), *([_p()] * 8), 1 << 40, None) == -2
    dec = L.IndexDesc(0, 2, 16, 64, 4, 512, L.CSA_BF16, 1024)
    assert lib.csa_index_topk_decode_fp4(ctypes.byref(dec), *([_p()] * 7), None, 0, None) == -3
    assert lib.csa_index_topk_decode_fp4(ctypes.byref(dec), None, *([_p()] * 7), 1 << 40, None) == -1
    # code arrays off a 16-byte boundary (the other pointers aligned, the
    # workspace large enough): rejected before anything is enqueued
    a = [_p(4096)] * 8
    for i in (0, 3):  # qI_codes, K_codes
        bad = list(a)
        bad[i] = _p(4096 + 8)
        assert lib.csa_index_topk_decode_fp4(ctypes.byref(dec), *bad, 1 << 40, None) == -1
    assert L.workspace_bytes("index_topk_decode_fp4", dec) == L.workspace_bytes("index_topk_decode", dec)
    assert L.workspace_zero_bytes("index_topk_decode_fp4", dec) == 0


def test_paged_calls_reject(lib):
    """The paged decode calls reject a missing page table, a page size below
    one, and fp32 attention, before anything is enqueued."""
    d = L.compress_desc(batch=2, d=128, c=128, m=4, max_entries=64)
    args = [_p()] * 7  # h, pos, W_kv, W_z, ape, W_win, state
    assert lib.csa_compress_decode_paged(ctypes.byref(d), *args, _p(), None, 32, _p(), _p(),
                                         1 << 40, None) == -1
    assert lib.csa_compress_decode_paged(ctypes.byref(d), *args, _p(), _p(), 0, _p(), _p(),
                                         1 << 40, None) == -1
    assert lib.csa_compress_decode_paged(None, *args, _p(), _p(), 32, _p(), _p(), 1 << 40,
                                         None) == -1
    dd = L.IndexDesc(0, 2, 16, 64, 4, 8, L.CSA_BF16, 100)
    assert lib.csa_index_topk_decode_paged(ctypes.byref(dd), _p(), _p(), _p(), None, 32, _p(),
                                           _p(), _p(), 1 << 40, None) == -1
    assert lib.csa_index_topk_decode_paged(ctypes.byref(dd), _p(), _p(), _p(), _p(), -4, _p(),
                                           _p(), _p(), 1 << 40, None) == -1
    assert lib.csa_index_topk_decode_paged(ctypes.byref(dd), _p(), _p(), _p(), _p(), 32, _p(),
                                           _p(), _p(), 8, None) == -3
    a = L.attn_desc(batch=2, nh=8, c=128, k=4, n_entries=64, dtype=L.CSA_F32)
    assert lib.csa_sparse_mqa_decode_paged(ctypes.byref(a), _p(), _p(), _p(), _p(), 32, _p(),
                                           _p(), _p(), _p(), _p(), 1 << 40, None) == -2
    a = L.attn_desc(batch=2, nh=8, c=128, m=4, n_entries=64, dtype=L.CSA_BF16)
    assert lib.hca_dense_mqa_decode_paged(ctypes.byref(a), _p(), _p(), _p(), None, 1, _p(), _p(),
                                          _p(), _p(), 1 << 40, None) == -1
    assert lib.hca_dense_mqa_decode_paged(ctypes.byref(a), _p(), _p(), _p(), _p(), 1, _p(), _p(),
                                          _p(), _p(), 8, None) == -3


def test_compress_prefill_paged_rejects(lib):
    """The paged prefill compressor rejects a missing page table, a page
    size below one, a chunk whose entries pass max_entries, a capacity past
    32-bit entry numbers and a missing descriptor, before anything is
    enqueued."""
    f = lib.csa_compress_prefill_paged
    args = [_p()] * 6  # H, W_kv, W_z, ape, W_win, comp_pool
    tail = [None, None, None, _p(), 1 << 40, None]  # out_win, ring, state, ws, ws_bytes, stream
    pd = L.compress_desc(n=64, d=128, c=128, m=4, max_entries=16)
    assert f(ctypes.byref(pd), *args, None, 32, *tail) == -1
    assert f(ctypes.byref(pd), *args, _p(), 0, *tail) == -1
    small = L.compress_desc(n=64, d=128, c=128, m=4, max_entries=15)  # 16 entries
    assert f(ctypes.byref(small), *args, _p(), 32, *tail) == -1
    chunk = L.compress_desc(n=64, d=128, c=128, m=4, max_entries=19, pos0=16)  # entries 4 .. 19
    assert f(ctypes.byref(chunk), *args, _p(), 32, *tail) == -1
    big = L.compress_desc(n=64, d=128, c=128, m=4, max_entries=1 << 31)
    assert f(ctypes.byref(big), *args, _p(), 32, *tail) == -2
    assert f(None, *args, _p(), 32, *tail) == -1


def test_fp4_paged_calls_reject(lib):
    """The two FP4 paged calls reject a missing page table, a page size below
    one, a capacity past 32-bit entry numbers and missing pools, before
    anything is enqueued."""
    f = L.Fp4Desc(2, 64, L.CSA_BF16)
    q = lib.csa_indexer_fp4_quant_decode_paged
    assert q(ctypes.byref(f), _p(), 64, _p(), 4, _p(), _p(), None, 32, None) == -1
    assert q(ctypes.byref(f), _p(), 64, _p(), 4, _p(), _p(), _p(), 0, None) == -1
    assert q(ctypes.byref(f), _p(), 64, _p(), 4, _p(), _p(), _p(), -2, None) == -1
    assert q(ctypes.byref(f), _p(), 1 << 31, _p(), 4, _p(), _p(), _p(), 32, None) == -2
    assert q(ctypes.byref(f), None, 64, _p(), 4, _p(), _p(), _p(), 32, None) == -1
    assert q(ctypes.byref(f), _p(), 64, _p(), 4, None, _p(), _p(), 32, None) == -1
    assert q(ctypes.byref(f), _p(), 64, _p(), 4, _p(), None, _p(), 32, None) == -1
    assert q(None, _p(), 64, _p(), 4, _p(), _p(), _p(), 32, None) == -1
    t = lib.csa_index_topk_decode_fp4_paged
    dd = L.IndexDesc(0, 2, 16, 64, 4, 8, L.CSA_BF16, 100)
    assert t(ctypes.byref(dd), _p(), _p(), _p(), _p(), _p(), None, 32, _p(), _p(), _p(),
             1 << 40, None) == -1
    assert t(ctypes.byref(dd), _p(), _p(), _p(), _p(), _p(), _p(), 0, _p(), _p(), _p(),
             1 << 40, None) == -1
    assert t(ctypes.byref(dd), _p(), _p(), _p(), None, _p(), _p(), 32, _p(), _p(), _p(),
             1 << 40, None) == -1
    assert t(ctypes.byref(dd), _p(), _p(), _p(), _p(), None, _p(), 32, _p(), _p(), _p(),
             1 << 40, None) == -1
    assert t(ctypes.byref(dd), _p(), _p(), _p(), _p(), _p(), _p(), 32, _p(), _p(), _p(),
             8, None) == -3
    for i in (0, 3):  # qI_codes, K_codes_pool off a 16-byte boundary
        a = [_p(4096)] * 5
        a[i] = _p(4096 + 4)
        assert t(ctypes.byref(dd), *a, _p(4096), 32, _p(4096), _p(4096), _p(4096),
                 1 << 40, None) == -1
    big = L.IndexDesc(0, 2, 16, 64, 4, 8, L.CSA_BF16, 1 << 31)
    assert t(ctypes.byref(big), _p(), _p(), _p(), _p(), _p(), _p(), 32, _p(), _p(), _p(),
             1 << 40, None) == -2
    f32 = L.IndexDesc(0, 2, 16, 64, 4, 8, L.CSA_F32, 100)
    assert t(ctypes.byref(f32), _p(), _p(), _p(), _p(), _p(), _p(), 32, _p(), _p(), _p(),
             1 << 40, None) == -2


def test_chunked_prefill_rejects(lib):
    """A chunk must start at a block boundary and at a position >= 0."""
    d = L.compress_desc(n=64, d=128, c=128, m=4, pos0=6)
    assert lib.csa_compress_prefill(ctypes.byref(d), *([_p()] * 10), 1 << 40, None) == -2
    d = L.compress_desc(n=64, d=128, c=128, m=4, pos0=-4)
    assert lib.csa_compress_prefill(ctypes.byref(d), *([_p()] * 10), 1 << 40, None) == -1
    # under overlap a chunk projects the halo block too
    d0 = L.compress_desc(n=64, d=128, c=128, m=4, overlap=1)
    d1 = L.compress_desc(n=64, d=128, c=128, m=4, overlap=1, pos0=8)
    assert L.workspace_bytes("compress_prefill", d1) > L.workspace_bytes("compress_prefill", d0)
    di = L.IndexDesc(16, 1, 16, 64, 4, 8, L.CSA_BF16, 4, 0, -1)
    assert lib.csa_index_topk_prefill(ctypes.byref(di), *([_p()] * 5), 1 << 30, None) == -1
    # the last row's visible count decides which selector runs
    di = L.IndexDesc(16, 1, 16, 64, 4, 512, L.CSA_BF16, 1 << 20, L.CSA_BF16, 4 * 16384)
    assert lib.csa_index_topk_prefill(ctypes.byref(di), *([_p()] * 5), 1 << 40, None) == -2
    di = L.IndexDesc(16, 1, 16, 64, 4, 512, L.CSA_BF16, 1 << 20, L.CSA_F32, 4 * 16384)
    long_ws = L.workspace_bytes("index_topk_prefill", di)  # the decode selector's workspace
    di.t0 = 0
    assert L.workspace_bytes("index_topk_prefill", di) != long_ws  # the register selector's
    assert L.workspace_zero_bytes("index_topk_prefill", di) == 0
    a = L.attn_desc(n=8, nh=8, c=128, k=4, t0=-1)
    assert lib.csa_sparse_mqa_prefill(ctypes.byref(a), *([_p()] * 6), None, 0, None) == -1


def test_noalloc_topk_rejects(lib):
    """The no-allocation top-k rejects descriptors whose scratch exceeds the
    library's static array, and null pointers, before touching the GPU."""
    assert lib.csa_noalloc_scratch_bytes() == 32 << 20
    ok = L.IndexDesc(0, 32, 16, 64, 4, 512, L.CSA_BF16, 32768)
    assert L.workspace_bytes("index_topk_decode", ok) <= lib.csa_noalloc_scratch_bytes()
    big = L.IndexDesc(0, 128, 16, 64, 4, 512, L.CSA_BF16, 65536)
    assert L.workspace_bytes("index_topk_decode", big) > lib.csa_noalloc_scratch_bytes()
    f = lib.csa_index_topk_decode_noalloc
    assert f(ctypes.byref(big), _p(), _p(), _p(), _p(), _p(), None) == -3
    assert f(ctypes.byref(ok), None, _p(), _p(), _p(), _p(), None) == -1
    assert f(ctypes.byref(ok), _p(), _p(), _p(), None, _p(), None) == -1
    assert f(None, _p(), _p(), _p(), _p(), _p(), None) == -1
    bad = L.IndexDesc(0, 2, 16, 64, 4, 0, L.CSA_BF16, 100)
    assert f(ctypes.byref(bad), _p(), _p(), _p(), _p(), _p(), None) in (-1, -2)


def test_split_topk_calls_reject(lib):
    """The two halves of the decode top-k validate like the single call."""
    d = L.IndexDesc(0, 2, 16, 64, 4, 8, L.CSA_BF16, 100)
    need = L.workspace_bytes("index_topk_decode", d)
    sc, se = lib.csa_index_topk_decode_score, lib.csa_index_topk_decode_select
    assert sc(ctypes.byref(d), None, _p(), _p(), _p(), _p(), need, None) == -1
    assert sc(ctypes.byref(d), _p(), _p(), _p(), _p(), _p(), need - 1, None) == -3
    assert sc(None, _p(), _p(), _p(), _p(), _p(), need, None) == -1
    assert se(ctypes.byref(d), _p(), _p(), _p(), _p(), None, _p(), need, None) == -1
    assert se(ctypes.byref(d), _p(), _p(), _p(), _p(), _p(), None, need, None) == -3
    bad = L.IndexDesc(0, 2, 12, 64, 4, 8, L.CSA_BF16, 100)  # 12 heads: not a kernel shape
    assert sc(ctypes.byref(bad), _p(), _p(), _p(), _p(), _p(), need, None) in (-1, -2)


def test_backward_calls_reject(lib):
    """The attention backward takes fp32 only, the supported head shapes and
    a full workspace, checked before anything is enqueued."""
    d = L.attn_desc(n=64, nh=8, c=128, k=16, n_entries=16, dtype=L.CSA_F32)
    need = L.workspace_bytes("sparse_mqa_backward", d)
    assert need > 0 and need == L.workspace_bytes("dense_mqa_backward", d)
    sb, db = lib.csa_sparse_mqa_backward, lib.hca_dense_mqa_backward
    assert sb(ctypes.byref(d), *([_p()] * 11), need - 1, None) == -3
    assert sb(ctypes.byref(d), None, *([_p()] * 10), need, None) == -1
    assert sb(ctypes.byref(d), _p(), _p(), _p(), None, *([_p()] * 7), need, None) == -1
    assert db(ctypes.byref(d), *([_p()] * 10), need - 1, None) == -3
    assert db(ctypes.byref(d), _p(), _p(), _p(), _p(), _p(), _p(), _p(), _p(), None, _p(),
              need, None) == -1  # dsink missing
    bf = L.attn_desc(n=64, nh=8, c=128, k=16, n_entries=16, dtype=L.CSA_BF16)
    assert sb(ctypes.byref(bf), *([_p()] * 11), need, None) == -2
    wide = L.attn_desc(n=64, nh=64, c=512, k=16, n_entries=16, dtype=L.CSA_F32)
    assert sb(ctypes.byref(wide), *([_p()] * 11), 1 << 40, None) == -2
    chunk = L.attn_desc(n=64, nh=8, c=128, k=16, n_entries=16, dtype=L.CSA_F32, t0=128)
    assert sb(ctypes.byref(chunk), *([_p()] * 11), 1 << 40, None) == -2


def test_fp8_calls_reject(lib):
    """FP8 rows: the row size, and the quantiser and decode attention calls
    reject unsupported shapes, a fp32 query and missing pointers."""
    assert lib.csa_kv_fp8_row_bytes(512, 64) == 592
    assert lib.csa_kv_fp8_row_bytes(512, 0) == 528
    assert lib.csa_kv_fp8_row_bytes(512, 448) == 976  # 64 codes, 448 bf16, 1 scale byte
    for c, r in ((512, 32), (512, 512), (256, 64), (512, -64)):
        assert lib.csa_kv_fp8_row_bytes(c, r) == 0
    d = L.Kv8Desc(4, 512, 64, L.CSA_BF16)
    assert lib.csa_kv_fp8_quant(ctypes.byref(d), None, _p(), None) == -1
    assert lib.csa_kv_fp8_quant(None, _p(), _p(), None) == -1
    assert lib.csa_kv_fp8_quant(ctypes.byref(L.Kv8Desc(4, 256, 64, L.CSA_BF16)), _p(), _p(),
                                None) == -2
    assert lib.csa_kv_fp8_quant(ctypes.byref(L.Kv8Desc(0, 512, 64, L.CSA_BF16)), None, None,
                                None) == 0  # nothing to do
    qd = lib.csa_kv_fp8_quant_decode
    assert qd(ctypes.byref(d), _p(), 8, _p(), 0, 0, _p(), None) == -1  # entries need m > 0
    assert qd(ctypes.byref(d), _p(), 0, _p(), 4, 0, _p(), None) == -1  # no rows
    assert qd(ctypes.byref(d), _p(), 8, None, 4, 0, _p(), None) == -1
    a = L.attn_desc(batch=2, nh=64, c=512, k=64, n_win=128, n_entries=256, dtype=L.CSA_BF16,
                    rope_dims=64)
    need = L.workspace_bytes("sparse_mqa_decode", a)
    sd, dd = lib.csa_sparse_mqa_decode_fp8, lib.hca_dense_mqa_decode_fp8
    assert sd(ctypes.byref(a), *([_p()] * 8), need - 1, None) == -3
    assert sd(ctypes.byref(a), _p(), _p(), _p(), None, *([_p()] * 4), need, None) == -1
    assert dd(ctypes.byref(a), _p(), _p(), None, *([_p()] * 4), 1 << 40, None) == -1
    for bad in (dict(dtype=L.CSA_F32), dict(c=256), dict(rope_dims=32)):
        kw = dict(batch=2, nh=64, c=512, k=64, n_win=128, n_entries=256, dtype=L.CSA_BF16,
                  rope_dims=64)
        kw.update(bad)
        b = L.attn_desc(**kw)
        assert sd(ctypes.byref(b), *([_p()] * 8), 1 << 40, None) == -2, bad
