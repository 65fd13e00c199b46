"""MI355X-native CSA / HCA hybrid compressed attention.

Thin ctypes binding to libcsa.so (HIP kernels for gfx950).  Every function
here only checks and marshals arguments -- shapes, dtypes, devices, the
current HIP stream -- and calls the C entry point of the same name; all
computation happens in the library's kernels.  torch supplies device memory
(outputs and workspaces) and streams.  If libcsa.so is missing or cannot be
loaded, every entry point raises: there is no fallback path.

The operations, layouts and conventions are documented in include/csa.h.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa.so")

CSA_F32, CSA_BF16 = 0, 1
ENTRY = dict(compress_prefill=0, compress_decode=1, index_topk_prefill=2, index_topk_decode=3,
             sparse_mqa_prefill=4, sparse_mqa_decode=5, dense_mqa_prefill=6, dense_mqa_decode=7,
             query_proj=8, output_proj=9, index_topk_decode_fp4=10, sparse_mqa_backward=11,
             dense_mqa_backward=12, index_topk_prefill_fp4=13)
EXPORTED = ["csa_compress_prefill", "csa_compress_decode", "csa_state_bytes", "csa_state_init",
            "csa_index_topk_prefill", "csa_index_topk_decode", "csa_sparse_mqa_prefill",
            "csa_sparse_mqa_decode", "hca_dense_mqa_prefill", "hca_dense_mqa_decode",
            "csa_query_proj", "csa_output_proj", "csa_indexer_fp4_quant",
            "csa_index_topk_decode_fp4", "csa_indexer_fp4_quant_decode", "csa_workspace_bytes",
            "csa_workspace_zero_bytes", "csa_status_string", "csa_abi_version",
            "csa_compress_decode_paged", "csa_index_topk_decode_paged",
            "csa_sparse_mqa_decode_paged", "hca_dense_mqa_decode_paged",
            "csa_indexer_fp4_quant_decode_paged", "csa_index_topk_decode_fp4_paged",
            "csa_index_topk_decode_noalloc", "csa_noalloc_scratch_bytes",
            "csa_index_topk_decode_score", "csa_index_topk_decode_select",
            "csa_sparse_mqa_backward", "hca_dense_mqa_backward", "csa_kv_fp8_row_bytes",
            "csa_kv_fp8_quant", "csa_kv_fp8_quant_decode", "csa_sparse_mqa_decode_fp8",
            "hca_dense_mqa_decode_fp8", "csa_index_topk_prefill_fp4",
            "csa_compress_prefill_paged"]


class CompressDesc(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("batch", ctypes.c_int32), ("d", ctypes.c_int32),
                ("c", ctypes.c_int32), ("m", ctypes.c_int32), ("overlap", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("qk_norm", ctypes.c_int32), ("eps", ctypes.c_float),
                ("rope_dims", ctypes.c_int32), ("rope_theta", ctypes.c_float),
                ("n_win", ctypes.c_int32), ("max_entries", ctypes.c_int64),
                ("pos0", ctypes.c_int64)]


class IndexDesc(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("batch", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("m", ctypes.c_int32), ("k", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("n_entries", ctypes.c_int64),
                ("score_dtype", ctypes.c_int32), ("t0", ctypes.c_int64)]


class Fp4Desc(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("width", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class Kv8Desc(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("c", ctypes.c_int32), ("rope_dims", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class QueryDesc(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("d", ctypes.c_int32), ("d_c", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("c", ctypes.c_int32), ("n_heads_i", ctypes.c_int32),
                ("c_i", ctypes.c_int32), ("dtype", ctypes.c_int32), ("eps", ctypes.c_float)]


class OprojDesc(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("n_heads", ctypes.c_int32), ("c", ctypes.c_int32),
                ("groups", ctypes.c_int32), ("d_g", ctypes.c_int32), ("d", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class AttnDesc(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("batch", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("c", ctypes.c_int32), ("k", ctypes.c_int32), ("m", ctypes.c_int32),
                ("n_win", ctypes.c_int32), ("dtype", ctypes.c_int32), ("scale", ctypes.c_float),
                ("qk_norm", ctypes.c_int32), ("eps", ctypes.c_float),
                ("rope_dims", ctypes.c_int32), ("rope_theta", ctypes.c_float),
                ("n_entries", ctypes.c_int64), ("t0", ctypes.c_int64)]


_lib = None


class CsaError(RuntimeError):
    pass


def load(path: str = LIB_PATH):
    """Load libcsa.so (once).  Raises if it is missing -- no fallback."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise CsaError(f"{path} not found: build it with `python -m long_context_attention_10_amd.build`")
    lib = ctypes.CDLL(path)
    P, S, I = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.csa_abi_version.restype = I
    lib.csa_status_string.restype = ctypes.c_char_p
    lib.csa_status_string.argtypes = [I]
    lib.csa_workspace_bytes.restype = S
    lib.csa_workspace_bytes.argtypes = [I, P]
    lib.csa_workspace_zero_bytes.restype = S
    lib.csa_workspace_zero_bytes.argtypes = [I, P]
    lib.csa_state_bytes.restype = S
    lib.csa_state_bytes.argtypes = [P]
    lib.csa_state_init.argtypes = [P, P, P]
    lib.csa_compress_prefill.argtypes = [P] * 11 + [S, P]
    lib.csa_compress_decode.argtypes = [P] * 11 + [S, P]
    lib.csa_index_topk_prefill.argtypes = [P] * 6 + [S, P]
    lib.csa_index_topk_decode.argtypes = [P] * 7 + [S, P]
    lib.csa_sparse_mqa_prefill.argtypes = [P] * 8 + [S, P]
    lib.csa_sparse_mqa_decode.argtypes = [P] * 9 + [S, P]
    lib.hca_dense_mqa_prefill.argtypes = [P] * 7 + [S, P]
    lib.hca_dense_mqa_decode.argtypes = [P] * 8 + [S, P]
    lib.csa_query_proj.argtypes = [P] * 11 + [S, P]
    lib.csa_output_proj.argtypes = [P] * 6 + [S, P]
    lib.csa_indexer_fp4_quant.argtypes = [P] * 5
    lib.csa_index_topk_decode_fp4.argtypes = [P] * 9 + [S, P]
    lib.csa_index_topk_prefill_fp4.argtypes = [P] * 8 + [S, P]
    lib.csa_indexer_fp4_quant_decode.argtypes = [P, P, ctypes.c_int64, P, I, P, P, P]
    I32 = ctypes.c_int32
    lib.csa_compress_decode_paged.argtypes = [P] * 10 + [I32] + [P] * 2 + [S, P]
    lib.csa_compress_prefill_paged.argtypes = [P] * 8 + [I32] + [P] * 4 + [S, P]
    lib.csa_index_topk_decode_paged.argtypes = [P] * 5 + [I32] + [P] * 3 + [S, P]
    lib.csa_sparse_mqa_decode_paged.argtypes = [P] * 5 + [I32] + [P] * 5 + [S, P]
    lib.hca_dense_mqa_decode_paged.argtypes = [P] * 5 + [I32] + [P] * 4 + [S, P]
    lib.csa_indexer_fp4_quant_decode_paged.argtypes = [P, P, ctypes.c_int64, P, I, P, P, P, I32, P]
    lib.csa_index_topk_decode_fp4_paged.argtypes = [P] * 7 + [I32] + [P] * 3 + [S, P]
    lib.csa_index_topk_decode_noalloc.argtypes = [P] * 7
    lib.csa_index_topk_decode_score.argtypes = [P] * 6 + [S, P]
    lib.csa_sparse_mqa_backward.argtypes = [P] * 12 + [S, P]
    lib.hca_dense_mqa_backward.argtypes = [P] * 11 + [S, P]
    lib.csa_index_topk_decode_select.argtypes = [P] * 7 + [S, P]
    lib.csa_kv_fp8_row_bytes.restype = S
    lib.csa_kv_fp8_row_bytes.argtypes = [I, I]
    lib.csa_kv_fp8_quant.argtypes = [P] * 4
    lib.csa_kv_fp8_quant_decode.argtypes = [P, P, ctypes.c_int64, P, I, I, P, P]
    lib.csa_sparse_mqa_decode_fp8.argtypes = [P] * 9 + [S, P]
    lib.hca_dense_mqa_decode_fp8.argtypes = [P] * 8 + [S, P]
    lib.csa_noalloc_scratch_bytes.restype = S
    lib.csa_noalloc_scratch_bytes.argtypes = []
    for f in EXPORTED:
        if f not in ("csa_abi_version", "csa_status_string", "csa_workspace_bytes",
                     "csa_workspace_zero_bytes", "csa_state_bytes", "csa_noalloc_scratch_bytes",
                     "csa_kv_fp8_row_bytes"):
            getattr(lib, f).restype = I
    _lib = lib
    return lib


# ----------------------------------------------------------------- helpers
def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return CSA_F32
    if t.dtype == torch.bfloat16:
        return CSA_BF16
    raise CsaError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise CsaError("all tensors must be on the GPU")
    if not t.is_contiguous():
        raise CsaError("all tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(status: int, what: str):
    if status != 0:
        msg = load().csa_status_string(status).decode()
        raise CsaError(f"{what} failed: {msg} ({status})")


def _expect(t, shape, dtype, name):
    if t is None:
        raise CsaError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise CsaError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise CsaError(f"{name}: expected {dtype}, got {t.dtype}")


_WS = {}
_WS_ZERO = {}  # (device, slot) -> leading bytes the last call left zero


def workspace(nbytes: int, device, slot: str = "default", zero_bytes: int = 0):
    """A cached device workspace of at least nbytes (torch-owned memory) whose
    first zero_bytes are zero: they are cleared (a fill kernel on the current
    stream) when the buffer is new or the previous call on it left fewer of
    them zero; a call that returns them to zero keeps that state."""
    if nbytes == 0:
        return None, 0
    key = (str(device), slot)
    t = _WS.get(key)
    if t is None or t.numel() < nbytes:
        t = torch.empty(nbytes, dtype=torch.uint8, device=device)
        _WS[key] = t
        _WS_ZERO.pop(key, None)
    if zero_bytes:
        if _WS_ZERO.get(key, 0) < zero_bytes:
            t[:zero_bytes].zero_()
        _WS_ZERO[key] = zero_bytes
    else:
        _WS_ZERO.pop(key, None)
    return t, t.numel()


def workspace_bytes(entry: str, desc) -> int:
    return load().csa_workspace_bytes(ENTRY[entry], ctypes.byref(desc))


def workspace_zero_bytes(entry: str, desc) -> int:
    return load().csa_workspace_zero_bytes(ENTRY[entry], ctypes.byref(desc))


# -------------------------------------------------------------- compressor
def compress_desc(n=0, batch=1, d=0, c=0, m=1, overlap=0, dtype=CSA_F32, qk_norm=True, eps=1e-6,
                  rope_dims=0, rope_theta=10000.0, n_win=128, max_entries=0, pos0=0):
    return CompressDesc(n, batch, d, c, m, int(overlap), dtype, int(qk_norm), eps, rope_dims,
                        rope_theta, n_win, max_entries, pos0)


def csa_state_bytes(desc) -> int:
    return load().csa_state_bytes(ctypes.byref(desc))


def csa_state_init(desc, state: torch.Tensor):
    _check(load().csa_state_init(ctypes.byref(desc), _ptr(state), _stream(state.device)), "csa_state_init")


def csa_compress_prefill(H, W_kv, W_z, ape, m, overlap, W_win=None, qk_norm=True, eps=1e-6,
                         rope_dims=0, rope_theta=10000.0, n_win=128, want_win=True,
                         want_ring=False, want_state=False, out_comp=None, out_win=None,
                         win_ring=None, state=None, ws_slot="default", pos0=0):
    """Compressed entries (and window rows / ring / decode state) of one
    sequence H [n, d].  Weights are output-major [(1+ov)c, d].  Calls that
    may run at the same time on different streams need distinct `ws_slot`
    names (each names its own cached workspace).  pos0 > 0 (a multiple of
    m): a chunk of new tokens at positions pos0.., whose H under overlap
    starts with the m tokens before pos0 (the halo)."""
    lib = load()
    n, d = H.shape
    if overlap and pos0 > 0:
        n -= m  # the halo rows are not new tokens
    w = W_kv.shape[0]
    c = w // (2 if overlap else 1)
    dt = _dt(H)
    _expect(W_kv, (w, d), H.dtype, "W_kv")
    _expect(W_z, (w, d), H.dtype, "W_z")
    _expect(ape, (m, w), torch.float32, "ape")
    desc = compress_desc(n=n, d=d, c=c, m=m, overlap=overlap, dtype=dt, qk_norm=qk_norm, eps=eps,
                         rope_dims=rope_dims, rope_theta=rope_theta, n_win=n_win, pos0=pos0)
    dev = H.device
    if out_comp is None:
        out_comp = torch.empty((n // m, c), dtype=H.dtype, device=dev)
    if W_win is not None:
        _expect(W_win, (c, d), H.dtype, "W_win")
        if want_win and out_win is None:
            out_win = torch.empty((n, c), dtype=H.dtype, device=dev)
        if want_ring and win_ring is None:
            win_ring = torch.empty((n_win, c), dtype=H.dtype, device=dev)
    if want_state and state is None:
        state = torch.empty(csa_state_bytes(desc) // 4, dtype=torch.float32, device=dev)
    ws, wsb = workspace(workspace_bytes("compress_prefill", desc), dev, ws_slot)
    st = lib.csa_compress_prefill(ctypes.byref(desc), _ptr(H), _ptr(W_kv), _ptr(W_z), _ptr(ape),
                                  _ptr(W_win), _ptr(out_comp) if out_comp.numel() else None,
                                  _ptr(out_win), _ptr(win_ring), _ptr(state), _ptr(ws), wsb,
                                  _stream(dev))
    _check(st, "csa_compress_prefill")
    return dict(comp=out_comp, win=out_win, ring=win_ring, state=state)


def csa_compress_prefill_paged(H, W_kv, W_z, ape, m, overlap, comp_pool, page_table,
                               page_entries, max_entries, W_win=None, qk_norm=True, eps=1e-6,
                               rope_dims=0, rope_theta=10000.0, n_win=128, out_win=None,
                               win_ring=None, state=None, ws_slot="default", pos0=0):
    """csa_compress_prefill with the entries written into a page pool
    comp_pool [P * page_entries, c] through one sequence's page table
    [ceil(max_entries / page_entries)] int32; window rows, ring and state as
    in csa_compress_prefill (given as tensors, or None)."""
    lib = load()
    n, d = H.shape
    if overlap and pos0 > 0:
        n -= m  # the halo rows are not new tokens
    w = W_kv.shape[0]
    c = w // (2 if overlap else 1)
    _expect(W_kv, (w, d), H.dtype, "W_kv")
    _expect(W_z, (w, d), H.dtype, "W_z")
    _expect(ape, (m, w), torch.float32, "ape")
    _expect(comp_pool, (comp_pool.shape[0], c), H.dtype, "comp_pool")
    _expect(page_table, (page_table.shape[0],), torch.int32, "page_table")
    if W_win is not None:
        _expect(W_win, (c, d), H.dtype, "W_win")
    desc = compress_desc(n=n, d=d, c=c, m=m, overlap=overlap, dtype=_dt(H), qk_norm=qk_norm,
                         eps=eps, rope_dims=rope_dims, rope_theta=rope_theta, n_win=n_win,
                         pos0=pos0, max_entries=max_entries)
    dev = H.device
    ws, wsb = workspace(workspace_bytes("compress_prefill", desc), dev, ws_slot)
    st = lib.csa_compress_prefill_paged(ctypes.byref(desc), _ptr(H), _ptr(W_kv), _ptr(W_z),
                                        _ptr(ape), _ptr(W_win), _ptr(comp_pool), _ptr(page_table),
                                        page_entries, _ptr(out_win), _ptr(win_ring), _ptr(state),
                                        _ptr(ws), wsb, _stream(dev))
    _check(st, "csa_compress_prefill_paged")
    return comp_pool


def csa_compress_decode(h, pos, W_kv, W_z, ape, m, overlap, state, cache, W_win=None,
                        win_ring=None, qk_norm=True, eps=1e-6, rope_dims=0, rope_theta=10000.0,
                        ws_slot="decode_proj"):
    """One new token per sequence: h [B, d], pos [B] int64; updates state,
    cache [B, max_entries, c] (on emission) and win_ring [B, n_win, c].
    Calls that may run at the same time on different streams need distinct
    `ws_slot` names (each names its own cached workspace)."""
    lib = load()
    B, d = h.shape
    w = W_kv.shape[0]
    c = w // (2 if overlap else 1)
    _expect(pos, (B,), torch.int64, "pos")
    _expect(cache, (B, cache.shape[1], c), h.dtype, "cache")
    n_win = win_ring.shape[1] if win_ring is not None else 0
    desc = compress_desc(batch=B, d=d, c=c, m=m, overlap=overlap, dtype=_dt(h), qk_norm=qk_norm,
                         eps=eps, rope_dims=rope_dims, rope_theta=rope_theta, n_win=n_win,
                         max_entries=cache.shape[1])
    if state.numel() * 4 < csa_state_bytes(desc):
        raise CsaError("state too small")
    ws, wsb = workspace(workspace_bytes("compress_decode", desc), h.device, ws_slot)
    st = lib.csa_compress_decode(ctypes.byref(desc), _ptr(h), _ptr(pos), _ptr(W_kv), _ptr(W_z),
                                 _ptr(ape), _ptr(W_win), _ptr(state), _ptr(cache), _ptr(win_ring),
                                 _ptr(ws), wsb, _stream(h.device))
    _check(st, "csa_compress_decode")


# -------------------------------------------------------- paged entry caches
def _paged(pool, page_table, page_entries, B, width, dtype, n_entries, name):
    """Checks a page pool [P * page_entries, width] and its table [B,
    ceil(n_entries / page_entries)] int32; returns n_entries (default: the
    table's capacity).  Page ids are not checked (that would synchronise)."""
    if page_entries < 1:
        raise CsaError("page_entries must be >= 1")
    if n_entries is None:
        n_entries = page_table.shape[1] * page_entries
    _expect(page_table, (B, -(-n_entries // page_entries)), torch.int32, "page_table")
    if pool.dim() != 2 or pool.shape[1] != width or pool.shape[0] % page_entries:
        raise CsaError(f"{name}: expected [pages * {page_entries}, {width}], got "
                       f"{tuple(pool.shape)}")
    if pool.dtype != dtype:
        raise CsaError(f"{name}: expected {dtype}, got {pool.dtype}")
    return n_entries


def csa_compress_decode_paged(h, pos, W_kv, W_z, ape, m, overlap, state, cache_pool, page_table,
                              page_entries, W_win=None, win_ring=None, n_entries=None,
                              qk_norm=True, eps=1e-6, rope_dims=0, rope_theta=10000.0,
                              ws_slot="decode_proj"):
    """csa_compress_decode with the entry cache in pages: entry e of sequence
    b is row page_table[b, e // page_entries] * page_entries + e %
    page_entries of cache_pool."""
    lib = load()
    B, d = h.shape
    w = W_kv.shape[0]
    c = w // (2 if overlap else 1)
    _expect(pos, (B,), torch.int64, "pos")
    ne = _paged(cache_pool, page_table, page_entries, B, c, h.dtype, n_entries, "cache_pool")
    n_win = win_ring.shape[1] if win_ring is not None else 0
    desc = compress_desc(batch=B, d=d, c=c, m=m, overlap=overlap, dtype=_dt(h), qk_norm=qk_norm,
                         eps=eps, rope_dims=rope_dims, rope_theta=rope_theta, n_win=n_win,
                         max_entries=ne)
    if state.numel() * 4 < csa_state_bytes(desc):
        raise CsaError("state too small")
    ws, wsb = workspace(workspace_bytes("compress_decode", desc), h.device, ws_slot)
    st = lib.csa_compress_decode_paged(ctypes.byref(desc), _ptr(h), _ptr(pos), _ptr(W_kv),
                                       _ptr(W_z), _ptr(ape), _ptr(W_win), _ptr(state),
                                       _ptr(cache_pool), _ptr(page_table), page_entries,
                                       _ptr(win_ring), _ptr(ws), wsb, _stream(h.device))
    _check(st, "csa_compress_decode_paged")


def csa_index_topk_decode_paged(qI, wI, KI_pool, page_table, page_entries, pos, m, k,
                                n_entries=None, out=None):
    lib = load()
    B, hI, cI = qI.shape
    ne = _paged(KI_pool, page_table, page_entries, B, cI, qI.dtype, n_entries, "KI_pool")
    _expect(pos, (B,), torch.int64, "pos")
    desc = IndexDesc(0, B, hI, cI, m, k, _dt(qI), ne)
    if out is None:
        out = torch.empty((B, k), dtype=torch.int32, device=qI.device)
    ws, wsb = workspace(workspace_bytes("index_topk_decode", desc), qI.device, "index_dec",
                        zero_bytes=workspace_zero_bytes("index_topk_decode", desc))
    st = lib.csa_index_topk_decode_paged(ctypes.byref(desc), _ptr(qI), _ptr(wI), _ptr(KI_pool),
                                         _ptr(page_table), page_entries, _ptr(pos), _ptr(out),
                                         _ptr(ws), wsb, _stream(qI.device))
    if st != 0:
        _WS_ZERO.pop((str(qI.device), "index_dec"), None)
    _check(st, "csa_index_topk_decode_paged")
    return out


def csa_sparse_mqa_decode_paged(q, win_ring, comp_pool, page_table, page_entries, idx, pos, sink,
                                n_entries=None, scale=None, qk_norm=True, eps=1e-6, rope_dims=0,
                                rope_theta=10000.0, out=None):
    lib = load()
    B, nh, c = q.shape
    n_win = win_ring.shape[1]
    k = idx.shape[1]
    _expect(win_ring, (B, n_win, c), q.dtype, "win_ring")
    ne = _paged(comp_pool, page_table, page_entries, B, c, q.dtype, n_entries, "comp_pool")
    _expect(idx, (B, k), torch.int32, "idx")
    _expect(pos, (B,), torch.int64, "pos")
    desc = attn_desc(batch=B, nh=nh, c=c, k=k, n_win=n_win, dtype=_dt(q), scale=scale,
                     qk_norm=qk_norm, eps=eps, rope_dims=rope_dims, rope_theta=rope_theta,
                     n_entries=ne)
    if out is None:
        out = torch.empty_like(q)
    ws, wsb = workspace(workspace_bytes("sparse_mqa_decode", desc), q.device, "attn_dec_s")
    st = lib.csa_sparse_mqa_decode_paged(ctypes.byref(desc), _ptr(q), _ptr(win_ring),
                                         _ptr(comp_pool), _ptr(page_table), page_entries,
                                         _ptr(idx), _ptr(pos), _ptr(sink), _ptr(out), _ptr(ws),
                                         wsb, _stream(q.device))
    _check(st, "csa_sparse_mqa_decode_paged")
    return out


def hca_dense_mqa_decode_paged(q, win_ring, comp_pool, page_table, page_entries, pos, sink, m,
                               n_entries=None, scale=None, qk_norm=True, eps=1e-6, rope_dims=0,
                               rope_theta=10000.0, out=None):
    lib = load()
    B, nh, c = q.shape
    n_win = win_ring.shape[1]
    _expect(win_ring, (B, n_win, c), q.dtype, "win_ring")
    ne = _paged(comp_pool, page_table, page_entries, B, c, q.dtype, n_entries, "comp_pool")
    _expect(pos, (B,), torch.int64, "pos")
    desc = attn_desc(batch=B, nh=nh, c=c, m=m, n_win=n_win, dtype=_dt(q), scale=scale,
                     qk_norm=qk_norm, eps=eps, rope_dims=rope_dims, rope_theta=rope_theta,
                     n_entries=ne)
    if out is None:
        out = torch.empty_like(q)
    ws, wsb = workspace(workspace_bytes("dense_mqa_decode", desc), q.device, "attn_dec_d")
    st = lib.hca_dense_mqa_decode_paged(ctypes.byref(desc), _ptr(q), _ptr(win_ring),
                                        _ptr(comp_pool), _ptr(page_table), page_entries,
                                        _ptr(pos), _ptr(sink), _ptr(out), _ptr(ws), wsb,
                                        _stream(q.device))
    _check(st, "hca_dense_mqa_decode_paged")
    return out


# ----------------------------------------------------------------- indexer
def csa_index_topk_prefill(qI, wI, KI, m, k, out=None, scores="f32", t0=0):
    """idx [n, k] int32: per token, the top-k visible entries (ascending), -1
    padded.  scores="bf16" selects on index scores rounded to bf16.  t0:
    position of row 0 (a chunk of a chunked prefill)."""
    lib = load()
    n, hI, cI = qI.shape
    _expect(wI, (n, hI), qI.dtype, "wI")
    ne = KI.shape[0]
    _expect(KI, (ne, cI), qI.dtype, "KI")
    sdt = {"f32": CSA_F32, "bf16": CSA_BF16}[scores]
    desc = IndexDesc(n, 1, hI, cI, m, k, _dt(qI), ne, sdt, t0)
    if out is None:
        out = torch.empty((n, k), dtype=torch.int32, device=qI.device)
    ws, wsb = workspace(workspace_bytes("index_topk_prefill", desc), qI.device, "index",
                        zero_bytes=workspace_zero_bytes("index_topk_prefill", desc))
    st = lib.csa_index_topk_prefill(ctypes.byref(desc), _ptr(qI), _ptr(wI),
                                    _ptr(KI) if ne else None, _ptr(out), _ptr(ws), wsb,
                                    _stream(qI.device))
    if st != 0:
        _WS_ZERO.pop((str(qI.device), "index"), None)
    _check(st, "csa_index_topk_prefill")
    return out


def csa_index_topk_decode(qI, wI, KI_cache, pos, m, k, out=None):
    lib = load()
    B, hI, cI = qI.shape
    ne = KI_cache.shape[1]
    _expect(KI_cache, (B, ne, cI), qI.dtype, "KI_cache")
    _expect(pos, (B,), torch.int64, "pos")
    desc = IndexDesc(0, B, hI, cI, m, k, _dt(qI), ne)
    if out is None:
        out = torch.empty((B, k), dtype=torch.int32, device=qI.device)
    ws, wsb = workspace(workspace_bytes("index_topk_decode", desc), qI.device, "index_dec",
                        zero_bytes=workspace_zero_bytes("index_topk_decode", desc))
    st = lib.csa_index_topk_decode(ctypes.byref(desc), _ptr(qI), _ptr(wI), _ptr(KI_cache),
                                   _ptr(pos), _ptr(out), _ptr(ws), wsb, _stream(qI.device))
    if st != 0:
        _WS_ZERO.pop((str(qI.device), "index_dec"), None)
    _check(st, "csa_index_topk_decode")
    return out


def csa_index_topk_decode_score(qI, wI, KI_cache, pos, m, k, ws_slot="index_dec"):
    """First half of csa_index_topk_decode: scores the cached keys that precede
    each sequence's step; csa_index_topk_decode_select with the same
    arguments and ws_slot must follow."""
    lib = load()
    B, hI, cI = qI.shape
    ne = KI_cache.shape[1]
    _expect(KI_cache, (B, ne, cI), qI.dtype, "KI_cache")
    _expect(pos, (B,), torch.int64, "pos")
    desc = IndexDesc(0, B, hI, cI, m, k, _dt(qI), ne)
    ws, wsb = workspace(workspace_bytes("index_topk_decode", desc), qI.device, ws_slot,
                        zero_bytes=workspace_zero_bytes("index_topk_decode", desc))
    # the histograms stay in use until the select call returns them to zero
    _WS_ZERO.pop((str(qI.device), ws_slot), None)
    st = lib.csa_index_topk_decode_score(ctypes.byref(desc), _ptr(qI), _ptr(wI), _ptr(KI_cache),
                                         _ptr(pos), _ptr(ws), wsb, _stream(qI.device))
    _check(st, "csa_index_topk_decode_score")


def csa_index_topk_decode_select(qI, wI, KI_cache, pos, m, k, out=None, ws_slot="index_dec"):
    """Second half: scores the step's new entries and selects."""
    lib = load()
    B, hI, cI = qI.shape
    ne = KI_cache.shape[1]
    desc = IndexDesc(0, B, hI, cI, m, k, _dt(qI), ne)
    if out is None:
        out = torch.empty((B, k), dtype=torch.int32, device=qI.device)
    ws = _WS.get((str(qI.device), ws_slot))
    need = workspace_bytes("index_topk_decode", desc)
    if ws is None or ws.numel() < need:
        raise CsaError("csa_index_topk_decode_select: no matching _score call on this workspace")
    st = lib.csa_index_topk_decode_select(ctypes.byref(desc), _ptr(qI), _ptr(wI), _ptr(KI_cache),
                                          _ptr(pos), _ptr(out), _ptr(ws), ws.numel(),
                                          _stream(qI.device))
    _check(st, "csa_index_topk_decode_select")
    _WS_ZERO[(str(qI.device), ws_slot)] = workspace_zero_bytes("index_topk_decode", desc)
    return out


def csa_index_topk_decode_noalloc(qI, wI, KI_cache, pos, m, k, out=None):
    """csa_index_topk_decode on the library's own per-device scratch (no
    workspace; `out` may be preallocated so that the call allocates nothing)."""
    lib = load()
    B, hI, cI = qI.shape
    ne = KI_cache.shape[1]
    _expect(KI_cache, (B, ne, cI), qI.dtype, "KI_cache")
    _expect(pos, (B,), torch.int64, "pos")
    desc = IndexDesc(0, B, hI, cI, m, k, _dt(qI), ne)
    if out is None:
        out = torch.empty((B, k), dtype=torch.int32, device=qI.device)
    st = lib.csa_index_topk_decode_noalloc(ctypes.byref(desc), _ptr(qI), _ptr(wI),
                                           _ptr(KI_cache), _ptr(pos), _ptr(out),
                                           _stream(qI.device))
    _check(st, "csa_index_topk_decode_noalloc")
    return out


# --------------------------------------------------------------- attention
def attn_desc(n=0, batch=1, nh=1, c=0, k=0, m=1, n_win=128, dtype=CSA_F32, scale=None,
              qk_norm=True, eps=1e-6, rope_dims=0, rope_theta=10000.0, n_entries=0, t0=0):
    if scale is None:
        scale = c ** -0.5
    return AttnDesc(n, batch, nh, c, k, m, n_win, dtype, scale, int(qk_norm), eps, rope_dims,
                    rope_theta, n_entries, t0)


def _mqa_backward(sparse, q, win_kv, comp, idx, sink, dout, m, n_win, scale, qk_norm, eps,
                  rope_dims, rope_theta):
    lib = load()
    n, nh, c = q.shape
    ne = comp.shape[0]
    k = idx.shape[1] if sparse else 0
    _expect(win_kv, (n, c), q.dtype, "win_kv")
    _expect(dout, (n, nh, c), q.dtype, "dout")
    _expect(comp, (ne, c), q.dtype, "comp")
    _expect(sink, (nh,), torch.float32, "sink")
    if sparse:
        _expect(idx, (n, k), torch.int32, "idx")
    desc = attn_desc(n=n, nh=nh, c=c, k=k, m=m, n_win=n_win, dtype=_dt(q), scale=scale,
                     qk_norm=qk_norm, eps=eps, rope_dims=rope_dims, rope_theta=rope_theta,
                     n_entries=ne)
    dq = torch.empty_like(q)
    dwin = torch.empty_like(win_kv)
    dcomp = torch.empty_like(comp)
    dsink = torch.empty(nh, dtype=torch.float32, device=q.device)
    name = "sparse_mqa_backward" if sparse else "dense_mqa_backward"
    ws, wsb = workspace(workspace_bytes(name, desc), q.device, "mqa_bwd")
    if sparse:
        st = lib.csa_sparse_mqa_backward(ctypes.byref(desc), _ptr(q), _ptr(win_kv), _ptr(comp),
                                         _ptr(idx), _ptr(sink), _ptr(dout), _ptr(dq), _ptr(dwin),
                                         _ptr(dcomp), _ptr(dsink), _ptr(ws), wsb,
                                         _stream(q.device))
    else:
        st = lib.hca_dense_mqa_backward(ctypes.byref(desc), _ptr(q), _ptr(win_kv), _ptr(comp),
                                        _ptr(sink), _ptr(dout), _ptr(dq), _ptr(dwin), _ptr(dcomp),
                                        _ptr(dsink), _ptr(ws), wsb, _stream(q.device))
    _check(st, "csa_" + name if sparse else "hca_" + name)
    return dq, dwin, dcomp, dsink


def csa_sparse_mqa_backward(q, win_kv, comp, idx, sink, dout, n_win=128, scale=None,
                            qk_norm=True, eps=1e-6, rope_dims=0, rope_theta=10000.0):
    """Gradients (dq, dwin, dcomp, dsink) of csa_sparse_mqa_prefill's output
    for the upstream gradient dout (fp32 tensors)."""
    return _mqa_backward(True, q, win_kv, comp, idx, sink, dout, 1, n_win,
                         scale if scale is not None else q.shape[2] ** -0.5, qk_norm, eps,
                         rope_dims, rope_theta)


def hca_dense_mqa_backward(q, win_kv, comp, sink, dout, m, n_win=128, scale=None, qk_norm=True,
                           eps=1e-6, rope_dims=0, rope_theta=10000.0):
    """Gradients (dq, dwin, dcomp, dsink) of hca_dense_mqa_prefill's output."""
    return _mqa_backward(False, q, win_kv, comp, None, sink, dout, m, n_win,
                         scale if scale is not None else q.shape[2] ** -0.5, qk_norm, eps,
                         rope_dims, rope_theta)


def _win_rows(n, n_win, t0):
    """Window rows a prefill chunk at t0 takes: positions max(0, t0-n_win+1)
    .. t0+n-1."""
    return t0 + n - max(0, t0 - n_win + 1)


def csa_sparse_mqa_prefill(q, win_kv, comp, idx, sink, n_win=128, scale=None, qk_norm=True,
                           eps=1e-6, rope_dims=0, rope_theta=10000.0, out=None, t0=0):
    """t0: position of row 0 (a chunk of a chunked prefill); win_kv then holds
    the window rows of positions max(0, t0-n_win+1) .. t0+n-1."""
    lib = load()
    n, nh, c = q.shape
    k = idx.shape[1]
    _expect(win_kv, (_win_rows(n, n_win, t0), c), q.dtype, "win_kv")
    _expect(idx, (n, k), torch.int32, "idx")
    _expect(sink, (nh,), torch.float32, "sink")
    desc = attn_desc(n=n, nh=nh, c=c, k=k, n_win=n_win, dtype=_dt(q), scale=scale, qk_norm=qk_norm,
                     eps=eps, rope_dims=rope_dims, rope_theta=rope_theta, n_entries=comp.shape[0],
                     t0=t0)
    if out is None:
        out = torch.empty_like(q)
    st = lib.csa_sparse_mqa_prefill(ctypes.byref(desc), _ptr(q), _ptr(win_kv),
                                    _ptr(comp) if comp.numel() else None, _ptr(idx), _ptr(sink),
                                    _ptr(out), None, 0, _stream(q.device))
    _check(st, "csa_sparse_mqa_prefill")
    return out


def hca_dense_mqa_prefill(q, win_kv, comp, sink, m, n_win=128, scale=None, qk_norm=True, eps=1e-6,
                          rope_dims=0, rope_theta=10000.0, out=None, t0=0):
    lib = load()
    n, nh, c = q.shape
    _expect(win_kv, (_win_rows(n, n_win, t0), c), q.dtype, "win_kv")
    _expect(sink, (nh,), torch.float32, "sink")
    desc = attn_desc(n=n, nh=nh, c=c, m=m, n_win=n_win, dtype=_dt(q), scale=scale, qk_norm=qk_norm,
                     eps=eps, rope_dims=rope_dims, rope_theta=rope_theta, n_entries=comp.shape[0],
                     t0=t0)
    if out is None:
        out = torch.empty_like(q)
    st = lib.hca_dense_mqa_prefill(ctypes.byref(desc), _ptr(q), _ptr(win_kv),
                                   _ptr(comp) if comp.numel() else None, _ptr(sink), _ptr(out),
                                   None, 0, _stream(q.device))
    _check(st, "hca_dense_mqa_prefill")
    return out


def csa_sparse_mqa_decode(q, win_ring, comp_cache, idx, pos, sink, scale=None, qk_norm=True,
                          eps=1e-6, rope_dims=0, rope_theta=10000.0, out=None):
    lib = load()
    B, nh, c = q.shape
    n_win = win_ring.shape[1]
    k = idx.shape[1]
    _expect(win_ring, (B, n_win, c), q.dtype, "win_ring")
    _expect(comp_cache, (B, comp_cache.shape[1], c), q.dtype, "comp_cache")
    _expect(idx, (B, k), torch.int32, "idx")
    _expect(pos, (B,), torch.int64, "pos")
    desc = attn_desc(batch=B, nh=nh, c=c, k=k, n_win=n_win, dtype=_dt(q), scale=scale,
                     qk_norm=qk_norm, eps=eps, rope_dims=rope_dims, rope_theta=rope_theta,
                     n_entries=comp_cache.shape[1])
    if out is None:
        out = torch.empty_like(q)
    ws, wsb = workspace(workspace_bytes("sparse_mqa_decode", desc), q.device, "attn_dec_s")
    st = lib.csa_sparse_mqa_decode(ctypes.byref(desc), _ptr(q), _ptr(win_ring), _ptr(comp_cache),
                                   _ptr(idx), _ptr(pos), _ptr(sink), _ptr(out), _ptr(ws), wsb,
                                   _stream(q.device))
    _check(st, "csa_sparse_mqa_decode")
    return out


def hca_dense_mqa_decode(q, win_ring, comp_cache, pos, sink, m, scale=None, qk_norm=True, eps=1e-6,
                         rope_dims=0, rope_theta=10000.0, out=None):
    lib = load()
    B, nh, c = q.shape
    n_win = win_ring.shape[1]
    _expect(win_ring, (B, n_win, c), q.dtype, "win_ring")
    _expect(comp_cache, (B, comp_cache.shape[1], c), q.dtype, "comp_cache")
    _expect(pos, (B,), torch.int64, "pos")
    desc = attn_desc(batch=B, nh=nh, c=c, m=m, n_win=n_win, dtype=_dt(q), scale=scale,
                     qk_norm=qk_norm, eps=eps, rope_dims=rope_dims, rope_theta=rope_theta,
                     n_entries=comp_cache.shape[1])
    if out is None:
        out = torch.empty_like(q)
    ws, wsb = workspace(workspace_bytes("dense_mqa_decode", desc), q.device, "attn_dec_d")
    st = lib.hca_dense_mqa_decode(ctypes.byref(desc), _ptr(q), _ptr(win_ring), _ptr(comp_cache),
                                  _ptr(pos), _ptr(sink), _ptr(out), _ptr(ws), wsb, _stream(q.device))
    _check(st, "hca_dense_mqa_decode")
    return out


# ------------------------------------------------------------ FP8 KV rows
def kv_fp8_row_bytes(c, rope_dims):
    """Bytes of one FP8 KV row of c channels whose last rope_dims stay bf16."""
    n = load().csa_kv_fp8_row_bytes(c, rope_dims)
    if n == 0:
        raise CsaError(f"no FP8 row format for c={c}, rope_dims={rope_dims}")
    return n


def csa_kv_fp8_quant(rows, rope_dims, out=None):
    """rows [..., c] (bf16 or fp32) -> their FP8 rows, uint8 [..., row_bytes]."""
    lib = load()
    c = rows.shape[-1]
    rb = kv_fp8_row_bytes(c, rope_dims)
    shape = tuple(rows.shape[:-1]) + (rb,)
    if out is None:
        out = torch.empty(shape, dtype=torch.uint8, device=rows.device)
    _expect(out, shape, torch.uint8, "out")
    desc = Kv8Desc(rows.numel() // c if c else 0, c, rope_dims, _dt(rows))
    _check(lib.csa_kv_fp8_quant(ctypes.byref(desc), _ptr(rows), _ptr(out), _stream(rows.device)),
           "csa_kv_fp8_quant")
    return out


def csa_kv_fp8_quant_decode(src, pos, dst, rope_dims, m=1, ring=False):
    """The rows one decode step wrote into src [B, n_rows, c] (a window ring
    when `ring`, else an entry cache of ratio m), converted in place into
    their FP8 copy dst [B, n_rows, row_bytes]."""
    lib = load()
    B, n_rows, c = src.shape
    rb = kv_fp8_row_bytes(c, rope_dims)
    _expect(dst, (B, n_rows, rb), torch.uint8, "dst")
    _expect(pos, (B,), torch.int64, "pos")
    desc = Kv8Desc(B, c, rope_dims, _dt(src))
    _check(lib.csa_kv_fp8_quant_decode(ctypes.byref(desc), _ptr(src), n_rows, _ptr(pos), m,
                                       1 if ring else 0, _ptr(dst), _stream(src.device)),
           "csa_kv_fp8_quant_decode")
    return dst


def _fp8_rows(t, B, rb, name):
    if t.dtype != torch.uint8 or t.dim() != 3 or t.shape[0] != B or t.shape[2] != rb:
        raise CsaError(f"{name}: expected uint8 [{B}, n, {rb}], got {t.dtype} {tuple(t.shape)}")


def csa_sparse_mqa_decode_fp8(q, win_ring8, cache8, idx, pos, sink, rope_dims, scale=None,
                              qk_norm=True, eps=1e-6, rope_theta=10000.0, out=None):
    """csa_sparse_mqa_decode over FP8 rows: win_ring8 [B, n_win, row_bytes],
    cache8 [B, n_entries, row_bytes] (uint8, csa_kv_fp8_quant's format)."""
    lib = load()
    B, nh, c = q.shape
    rb = kv_fp8_row_bytes(c, rope_dims)
    _fp8_rows(win_ring8, B, rb, "win_ring8")
    _fp8_rows(cache8, B, rb, "cache8")
    k = idx.shape[1]
    _expect(idx, (B, k), torch.int32, "idx")
    _expect(pos, (B,), torch.int64, "pos")
    desc = attn_desc(batch=B, nh=nh, c=c, k=k, n_win=win_ring8.shape[1], dtype=_dt(q),
                     scale=scale, qk_norm=qk_norm, eps=eps, rope_dims=rope_dims,
                     rope_theta=rope_theta, n_entries=cache8.shape[1])
    if out is None:
        out = torch.empty_like(q)
    ws, wsb = workspace(workspace_bytes("sparse_mqa_decode", desc), q.device, "attn_dec_s")
    st = lib.csa_sparse_mqa_decode_fp8(ctypes.byref(desc), _ptr(q), _ptr(win_ring8), _ptr(cache8),
                                       _ptr(idx), _ptr(pos), _ptr(sink), _ptr(out), _ptr(ws), wsb,
                                       _stream(q.device))
    _check(st, "csa_sparse_mqa_decode_fp8")
    return out


def hca_dense_mqa_decode_fp8(q, win_ring8, cache8, pos, sink, m, rope_dims, scale=None,
                             qk_norm=True, eps=1e-6, rope_theta=10000.0, out=None):
    """hca_dense_mqa_decode over FP8 rows (formats as csa_sparse_mqa_decode_fp8)."""
    lib = load()
    B, nh, c = q.shape
    rb = kv_fp8_row_bytes(c, rope_dims)
    _fp8_rows(win_ring8, B, rb, "win_ring8")
    _fp8_rows(cache8, B, rb, "cache8")
    _expect(pos, (B,), torch.int64, "pos")
    desc = attn_desc(batch=B, nh=nh, c=c, m=m, n_win=win_ring8.shape[1], dtype=_dt(q),
                     scale=scale, qk_norm=qk_norm, eps=eps, rope_dims=rope_dims,
                     rope_theta=rope_theta, n_entries=cache8.shape[1])
    if out is None:
        out = torch.empty_like(q)
    ws, wsb = workspace(workspace_bytes("dense_mqa_decode", desc), q.device, "attn_dec_d")
    st = lib.hca_dense_mqa_decode_fp8(ctypes.byref(desc), _ptr(q), _ptr(win_ring8), _ptr(cache8),
                                      _ptr(pos), _ptr(sink), _ptr(out), _ptr(ws), wsb,
                                      _stream(q.device))
    _check(st, "hca_dense_mqa_decode_fp8")
    return out


# ------------------------------------------------- query path / output proj
def csa_query_proj(H, W_DQ, W_UQ, n_heads, W_IUQ=None, W_w=None, n_heads_i=0, g_q=None, eps=1e-6,
                   out=None, ws_slot="query"):
    """Low-rank query path of n rows of H [n, d] (bf16): returns q [n, n_heads,
    c], and, with the indexer weights, q^I [n, n_heads_i, c_i] and w^I [n,
    n_heads_i].  Weights are output-major: W_DQ [d_c, d], W_UQ [n_heads*c,
    d_c], W_IUQ [n_heads_i*c_i, d_c], W_w [n_heads_i, d]; g_q [d_c] fp32 or
    None (unit latent-norm weight).  `out` may give the (q, q^I, w^I) buffers."""
    lib = load()
    n, d = H.shape
    dc = W_DQ.shape[0]
    c = W_UQ.shape[0] // n_heads
    ci = W_IUQ.shape[0] // n_heads_i if n_heads_i else 0
    _expect(W_DQ, (dc, d), H.dtype, "W_DQ")
    _expect(W_UQ, (n_heads * c, dc), H.dtype, "W_UQ")
    if n_heads_i:
        _expect(W_IUQ, (n_heads_i * ci, dc), H.dtype, "W_IUQ")
        _expect(W_w, (n_heads_i, d), H.dtype, "W_w")
    if g_q is not None:
        _expect(g_q, (dc,), torch.float32, "g_q")
    desc = QueryDesc(n, d, dc, n_heads, c, n_heads_i, ci, _dt(H), eps)
    if out is not None:
        q, qI, wI = out
        _expect(q, (n, n_heads, c), H.dtype, "q out")
        if n_heads_i:
            _expect(qI, (n, n_heads_i, ci), H.dtype, "qI out")
            _expect(wI, (n, n_heads_i), H.dtype, "wI out")
    else:
        q = torch.empty((n, n_heads, c), dtype=H.dtype, device=H.device)
        qI = torch.empty((n, n_heads_i, ci), dtype=H.dtype, device=H.device) if n_heads_i else None
        wI = torch.empty((n, n_heads_i), dtype=H.dtype, device=H.device) if n_heads_i else None
    ws, wsb = workspace(workspace_bytes("query_proj", desc), H.device, ws_slot)
    st = lib.csa_query_proj(ctypes.byref(desc), _ptr(H), _ptr(W_DQ), _ptr(g_q), _ptr(W_w),
                            _ptr(W_UQ), _ptr(W_IUQ), _ptr(q), _ptr(qI), _ptr(wI), _ptr(ws), wsb,
                            _stream(H.device))
    _check(st, "csa_query_proj")
    return q, qI, wI


def csa_output_proj(o, wo_a, wo_b, out=None, ws_slot="oproj"):
    """Grouped output projection of an attention output o [n, n_heads, c]
    (bf16): wo_a [groups, d_g, n_heads*c/groups], wo_b [d, groups*d_g];
    returns out [n, d]."""
    lib = load()
    n, nh, c = o.shape
    g, dg, kg = wo_a.shape
    d = wo_b.shape[0]
    if g * kg != nh * c:
        raise CsaError(f"wo_a: {g} groups of {kg} channels do not cover {nh}x{c}")
    _expect(wo_b, (d, g * dg), o.dtype, "wo_b")
    desc = OprojDesc(n, nh, c, g, dg, d, _dt(o))
    if out is None:
        out = torch.empty((n, d), dtype=o.dtype, device=o.device)
    ws, wsb = workspace(workspace_bytes("output_proj", desc), o.device, ws_slot)
    st = lib.csa_output_proj(ctypes.byref(desc), _ptr(o), _ptr(wo_a), _ptr(wo_b), _ptr(out),
                             _ptr(ws), wsb, _stream(o.device))
    _check(st, "csa_output_proj")
    return out


# ------------------------------------------------------ quantised indexer
def csa_indexer_fp4_quant(x, out=None):
    """Rotation + FP4 of the rows of x [..., W] (W = 64 or 128): returns
    (codes uint8 [..., W/2], exps uint8 [..., W/32]); `out` may give them."""
    lib = load()
    W = x.shape[-1]
    rows = x.numel() // W if W else 0
    if out is not None:
        codes, exps = out
        _expect(codes, tuple(x.shape[:-1]) + (W // 2,), torch.uint8, "codes")
        _expect(exps, tuple(x.shape[:-1]) + (W // 32,), torch.uint8, "exps")
    else:
        codes = torch.empty(x.shape[:-1] + (W // 2,), dtype=torch.uint8, device=x.device)
        exps = torch.empty(x.shape[:-1] + (W // 32,), dtype=torch.uint8, device=x.device)
    desc = Fp4Desc(rows, W, _dt(x))
    st = lib.csa_indexer_fp4_quant(ctypes.byref(desc), _ptr(x), _ptr(codes), _ptr(exps),
                                   _stream(x.device))
    _check(st, "csa_indexer_fp4_quant")
    return codes, exps


def csa_index_topk_decode_fp4(q_codes, q_exps, wI, k_codes, k_exps, pos, m, k, out=None):
    """csa_index_topk_decode on FP4 q^I [B, hI, cI/2] (+ exps [B, hI, cI/32])
    and FP4 keys [B, n_entries, cI/2] (+ exps); wI [B, hI] bf16."""
    lib = load()
    B, hI, half = q_codes.shape
    cI = 2 * half
    ne = k_codes.shape[1]
    _expect(q_exps, (B, hI, cI // 32), torch.uint8, "q_exps")
    _expect(k_codes, (B, ne, half), torch.uint8, "k_codes")
    _expect(k_exps, (B, ne, cI // 32), torch.uint8, "k_exps")
    _expect(wI, (B, hI), None, "wI")
    _expect(pos, (B,), torch.int64, "pos")
    desc = IndexDesc(0, B, hI, cI, m, k, _dt(wI), ne)
    if out is None:
        out = torch.empty((B, k), dtype=torch.int32, device=q_codes.device)
    ws, wsb = workspace(workspace_bytes("index_topk_decode_fp4", desc), q_codes.device,
                        "index_dec_fp4",
                        zero_bytes=workspace_zero_bytes("index_topk_decode_fp4", desc))
    st = lib.csa_index_topk_decode_fp4(ctypes.byref(desc), _ptr(q_codes), _ptr(q_exps), _ptr(wI),
                                       _ptr(k_codes), _ptr(k_exps), _ptr(pos), _ptr(out),
                                       _ptr(ws), wsb, _stream(q_codes.device))
    if st != 0:
        _WS_ZERO.pop((str(q_codes.device), "index_dec_fp4"), None)
    _check(st, "csa_index_topk_decode_fp4")
    return out


def csa_index_topk_prefill_fp4(q_codes, q_exps, wI, k_codes, k_exps, m, k, out=None,
                               scores="f32", t0=0):
    """csa_index_topk_prefill on FP4 q^I [n, hI, cI/2] (+ exps [n, hI,
    cI/32]) and FP4 keys [n_entries, cI/2] (+ exps [n_entries, cI/32]); wI
    [n, hI] bf16."""
    lib = load()
    n, hI, half = q_codes.shape
    cI = 2 * half
    ne = k_codes.shape[0]
    _expect(q_exps, (n, hI, cI // 32), torch.uint8, "q_exps")
    _expect(k_codes, (ne, half), torch.uint8, "k_codes")
    _expect(k_exps, (ne, cI // 32), torch.uint8, "k_exps")
    _expect(wI, (n, hI), None, "wI")
    sdt = {"f32": CSA_F32, "bf16": CSA_BF16}[scores]
    desc = IndexDesc(n, 1, hI, cI, m, k, _dt(wI), ne, sdt, t0)
    if out is None:
        out = torch.empty((n, k), dtype=torch.int32, device=q_codes.device)
    ws, wsb = workspace(workspace_bytes("index_topk_prefill_fp4", desc), q_codes.device, "index")
    st = lib.csa_index_topk_prefill_fp4(ctypes.byref(desc), _ptr(q_codes), _ptr(q_exps), _ptr(wI),
                                        _ptr(k_codes) if ne else None,
                                        _ptr(k_exps) if ne else None, _ptr(out), _ptr(ws), wsb,
                                        _stream(q_codes.device))
    _check(st, "csa_index_topk_prefill_fp4")
    return out


def csa_indexer_fp4_quant_decode(cache, pos, m, codes, exps):
    """Quantise, into the FP4 cache (codes [B, n_entries, W/2], exps [B,
    n_entries, W/32]), the entry each sequence's decode step has just emitted
    into the key cache [B, n_entries, W]."""
    lib = load()
    B, ne, W = cache.shape
    _expect(pos, (B,), torch.int64, "pos")
    _expect(codes, (B, ne, W // 2), torch.uint8, "codes")
    _expect(exps, (B, ne, W // 32), torch.uint8, "exps")
    desc = Fp4Desc(B, W, _dt(cache))
    st = lib.csa_indexer_fp4_quant_decode(ctypes.byref(desc), _ptr(cache), ne, _ptr(pos), m,
                                          _ptr(codes), _ptr(exps), _stream(cache.device))
    _check(st, "csa_indexer_fp4_quant_decode")


def csa_indexer_fp4_quant_decode_paged(cache_pool, pos, m, codes_pool, exps_pool, page_table,
                                       page_entries, n_entries=None):
    """csa_indexer_fp4_quant_decode over paged caches: the key pool [P * page,
    W] and the FP4 pools (codes [P * page, W/2], exps [P * page, W/32]) share
    page_table [B, ceil(n_entries / page)]."""
    lib = load()
    B = pos.shape[0]
    W = cache_pool.shape[1]
    ne = _paged(cache_pool, page_table, page_entries, B, W, cache_pool.dtype, n_entries,
                "cache_pool")
    _expect(codes_pool, (cache_pool.shape[0], W // 2), torch.uint8, "codes_pool")
    _expect(exps_pool, (cache_pool.shape[0], W // 32), torch.uint8, "exps_pool")
    desc = Fp4Desc(B, W, _dt(cache_pool))
    st = lib.csa_indexer_fp4_quant_decode_paged(ctypes.byref(desc), _ptr(cache_pool), ne, _ptr(pos),
                                                m, _ptr(codes_pool), _ptr(exps_pool),
                                                _ptr(page_table), page_entries,
                                                _stream(cache_pool.device))
    _check(st, "csa_indexer_fp4_quant_decode_paged")


def csa_index_topk_decode_fp4_paged(q_codes, q_exps, wI, k_codes_pool, k_exps_pool, page_table,
                                    page_entries, pos, m, k, n_entries=None, out=None):
    lib = load()
    B, hI, half = q_codes.shape
    cI = 2 * half
    _expect(q_exps, (B, hI, cI // 32), torch.uint8, "q_exps")
    ne = _paged(k_codes_pool, page_table, page_entries, B, half, torch.uint8, n_entries,
                "k_codes_pool")
    _expect(k_exps_pool, (k_codes_pool.shape[0], cI // 32), torch.uint8, "k_exps_pool")
    _expect(wI, (B, hI), None, "wI")
    _expect(pos, (B,), torch.int64, "pos")
    desc = IndexDesc(0, B, hI, cI, m, k, _dt(wI), ne)
    if out is None:
        out = torch.empty((B, k), dtype=torch.int32, device=q_codes.device)
    ws, wsb = workspace(workspace_bytes("index_topk_decode_fp4", desc), q_codes.device,
                        "index_dec_fp4",
                        zero_bytes=workspace_zero_bytes("index_topk_decode_fp4", desc))
    st = lib.csa_index_topk_decode_fp4_paged(ctypes.byref(desc), _ptr(q_codes), _ptr(q_exps),
                                             _ptr(wI), _ptr(k_codes_pool), _ptr(k_exps_pool),
                                             _ptr(page_table), page_entries, _ptr(pos), _ptr(out),
                                             _ptr(ws), wsb, _stream(q_codes.device))
    if st != 0:
        _WS_ZERO.pop((str(q_codes.device), "index_dec_fp4"), None)
    _check(st, "csa_index_topk_decode_fp4_paged")
    return out
