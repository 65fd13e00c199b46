// C ABI of libcsa: argument validation on the host, then kernel launches on
// the caller's stream.  Nothing here allocates, frees or synchronises.
// The operations and their definitions are documented in include/csa.h.
#include <hip/hip_runtime.h>

#include "../../include/csa.h"
#include "csa_launch.h"

using namespace csa;

namespace {

size_t al(size_t x) { return (x + 255) & ~(size_t)255; }

bool dtype_ok(int dt) { return dt == CSA_F32 || dt == CSA_BF16; }
size_t esize(int dt) { return dt == CSA_BF16 ? 2 : 4; }
bool pow2_c(int c) { return c == 32 || c == 64 || c == 128 || c == 256 || c == 512; }

// ------------------------------------------------------------- compressor
int check_compress(const csa_compress_desc* d, bool decode) {
  if (!d) return CSA_ERR_INVALID_ARG;
  if (!dtype_ok(d->dtype)) return CSA_ERR_UNSUPPORTED;
  if (d->d <= 0 || d->c <= 0 || d->m <= 0 || (d->overlap != 0 && d->overlap != 1))
    return CSA_ERR_INVALID_ARG;
  if (!pow2_c(d->c)) return CSA_ERR_UNSUPPORTED;
  if (d->m > 1024) return CSA_ERR_UNSUPPORTED;
  if (d->d % 64 != 0) return CSA_ERR_UNSUPPORTED;  // 128-byte K slices in the GEMMs
  if (d->rope_dims < 0 || d->rope_dims > d->c || (d->rope_dims & 1)) return CSA_ERR_INVALID_ARG;
  if (d->rope_dims > 0 && !(d->rope_theta > 0.f)) return CSA_ERR_INVALID_ARG;
  if (d->qk_norm && !(d->eps >= 0.f)) return CSA_ERR_INVALID_ARG;
  if (decode) {
    if (d->batch <= 0 || d->max_entries < 0) return CSA_ERR_INVALID_ARG;
  } else {
    if (d->n < 0 || d->pos0 < 0) return CSA_ERR_INVALID_ARG;
    if (d->pos0 % d->m) return CSA_ERR_UNSUPPORTED;  // chunks start at a block boundary
  }
  return CSA_OK;
}

// Rows of H a prefill projects: under overlap a chunk (pos0 > 0) also
// projects the previous block (the halo) for its b-series.
int64_t prefill_halo(const csa_compress_desc* d) { return d->overlap && d->pos0 > 0 ? d->m : 0; }

size_t ws_compress_prefill(const csa_compress_desc* d, bool has_win) {
  const int w = (1 + d->overlap) * d->c;
  return al((size_t)(d->n + prefill_halo(d)) * (size_t)(2 * w + (has_win ? d->c : 0)) * 4);
}

size_t ws_compress_decode(const csa_compress_desc* d, bool has_win) {
  const int w = (1 + d->overlap) * d->c;
  const int N = 2 * w + (has_win ? d->c : 0);
  const int ks = decode_proj_ksplit(N, d->d, d->dtype);
  return al((size_t)ks * d->batch * N * 4);
}

// ---------------------------------------------------------------- indexer
constexpr int64_t kRegRowMax = 256 * 64;  // visible entries a prefill row holds in registers

int check_index(const csa_index_desc* d, bool decode) {
  if (!d) return CSA_ERR_INVALID_ARG;
  if (!dtype_ok(d->dtype)) return CSA_ERR_UNSUPPORTED;
  if (d->m <= 0 || d->k <= 0 || d->n_entries < 0) return CSA_ERR_INVALID_ARG;
  if (!(d->n_heads == 4 || d->n_heads == 8 || d->n_heads == 16)) return CSA_ERR_UNSUPPORTED;
  if (!(d->head_dim == 64 || d->head_dim == 128)) return CSA_ERR_UNSUPPORTED;
  if (d->k > 2048) return CSA_ERR_UNSUPPORTED;
  if (d->score_dtype != CSA_F32 && d->score_dtype != CSA_BF16) return CSA_ERR_UNSUPPORTED;
  if (decode) {
    if (d->score_dtype != CSA_F32) return CSA_ERR_UNSUPPORTED;
    if (d->batch <= 0) return CSA_ERR_INVALID_ARG;
    if (d->n_entries >= (int64_t)1 << 31) return CSA_ERR_UNSUPPORTED;
  } else {
    if (d->n < 0 || d->t0 < 0) return CSA_ERR_INVALID_ARG;
    const int64_t last = (d->t0 + d->n) / d->m;  // visible entries of the last row
    const int64_t vis = last < d->n_entries ? last : d->n_entries;
    // rows past the register selector take the decode top-k (fp32 scores only)
    if (vis > kRegRowMax && (d->score_dtype != CSA_F32 || vis >= (int64_t)1 << 31))
      return CSA_ERR_UNSUPPORTED;
  }
  return CSA_OK;
}

// A prefill call whose last row sees more entries than the register selector
// holds: it runs the decode top-k over batches of rows.
bool index_prefill_long(const csa_index_desc* d) {
  const int64_t last = (d->t0 + d->n) / d->m;
  return (last < d->n_entries ? last : d->n_entries) > kRegRowMax;
}

// Row stride of the prefill score workspace (a multiple of 4 floats).
int64_t index_prefill_ld(const csa_index_desc* d) {
  const int64_t last = (d->t0 + d->n) / d->m;
  const int64_t vis = last < d->n_entries ? last : d->n_entries;
  return (vis + 3) & ~(int64_t)3;
}

// -------------------------------------------------------------- attention
int check_attn(const csa_attn_desc* d, bool decode, bool sparse) {
  if (!d) return CSA_ERR_INVALID_ARG;
  if (!dtype_ok(d->dtype)) return CSA_ERR_UNSUPPORTED;
  if (d->n_heads <= 0 || d->n_win <= 0 || d->n_entries < 0) return CSA_ERR_INVALID_ARG;
  if (d->n_heads > 64) return CSA_ERR_UNSUPPORTED;
  if (!(d->c == 128 || d->c == 256 || d->c == 512)) return CSA_ERR_UNSUPPORTED;
  if (sparse && d->k <= 0) return CSA_ERR_INVALID_ARG;
  if (!sparse && d->m <= 0) return CSA_ERR_INVALID_ARG;
  if (d->rope_dims < 0 || d->rope_dims > d->c || (d->rope_dims % 8)) return CSA_ERR_UNSUPPORTED;
  if (d->rope_dims > 0 && !(d->rope_theta > 0.f)) return CSA_ERR_INVALID_ARG;
  if (decode ? d->batch <= 0 : d->n < 0 || d->t0 < 0) return CSA_ERR_INVALID_ARG;
  return CSA_OK;
}

// ------------------------------------------------------- layer projections
int check_query(const csa_query_desc* d) {
  if (!d) return CSA_ERR_INVALID_ARG;
  if (d->dtype != CSA_BF16) return CSA_ERR_UNSUPPORTED;
  if (d->n < 0 || d->d <= 0 || d->d_c <= 0 || d->n_heads <= 0 || d->c <= 0 ||
      d->n_heads_i < 0 || d->c_i < 0 || !(d->eps >= 0.f))
    return CSA_ERR_INVALID_ARG;
  if (d->d % 64 || d->d_c % 64) return CSA_ERR_UNSUPPORTED;  // K of the two products
  if ((int64_t)d->n_heads * d->c + (int64_t)d->n_heads_i * d->c_i > (1 << 30))
    return CSA_ERR_UNSUPPORTED;
  return CSA_OK;
}

int check_oproj(const csa_oproj_desc* d) {
  if (!d) return CSA_ERR_INVALID_ARG;
  if (d->dtype != CSA_BF16) return CSA_ERR_UNSUPPORTED;
  if (d->n < 0 || d->n_heads <= 0 || d->c <= 0 || d->groups <= 0 || d->d_g <= 0 || d->d <= 0)
    return CSA_ERR_INVALID_ARG;
  const int64_t width = (int64_t)d->n_heads * d->c;
  if (width % d->groups) return CSA_ERR_INVALID_ARG;
  if ((width / d->groups) % 64 || ((int64_t)d->groups * d->d_g) % 64) return CSA_ERR_UNSUPPORTED;
  if (d->groups > 65535) return CSA_ERR_UNSUPPORTED;
  return CSA_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? CSA_OK : CSA_ERR_HIP; }

// A paged cache: entry e of sequence b is pool row
// page_table[b * max_pages + e / page] * page + e % page, with max_pages the
// pages that `capacity` entries per sequence need.
int entry_map(const int32_t* table, int32_t page, int64_t capacity, EntryMap* em) {
  if (!table || page <= 0 || capacity < 0) return CSA_ERR_INVALID_ARG;
  if (capacity > INT32_MAX) return CSA_ERR_UNSUPPORTED;  // entry numbers stay 32-bit
  const int64_t np = (capacity + page - 1) / page;
  em->table = table;
  em->page = page;
  em->max_pages = (int32_t)np;
  return CSA_OK;
}

int compress_decode(const csa_compress_desc* d, const void* h, const int64_t* pos,
                    const void* W_kv, const void* W_z, const float* ape, const void* W_win,
                    float* state, void* cache, void* win_ring, void* ws, size_t ws_bytes,
                    void* stream, EntryMap em) {
  int s = check_compress(d, true);
  if (s) return s;
  if (!h || !pos || !W_kv || !W_z || !ape || !state || !cache) return CSA_ERR_INVALID_ARG;
  const bool has_win = W_win != nullptr;
  if (has_win != (win_ring != nullptr)) return CSA_ERR_INVALID_ARG;
  if (has_win && d->n_win <= 0) return CSA_ERR_INVALID_ARG;
  const size_t need = ws_compress_decode(d, has_win);
  if (!ws || ws_bytes < need) return CSA_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const int w = (1 + d->overlap) * d->c;
  const int N = 2 * w + (has_win ? d->c : 0);
  const int ks = decode_proj_ksplit(N, d->d, d->dtype);
  WeightStack stack = {{W_kv, W_z, W_win}, {w, w, has_win ? d->c : 0}};
  hipError_t e = launch_decode_proj(d->dtype, h, d->batch, d->d, stack, (float*)ws, ks, st);
  if (e != hipSuccess) return CSA_ERR_HIP;
  e = launch_decode_update(d->dtype, (const float*)ws, ks, d->batch, N, d->c, d->m, d->overlap,
                           has_win, ape, pos, state, cache, d->max_entries, win_ring, d->n_win,
                           d->qk_norm, d->eps, d->rope_dims, d->rope_theta, st, em);
  return hip_status(e);
}

int index_topk_decode(const csa_index_desc* d, const void* qI, const void* wI,
                      const void* KI_cache, const int64_t* pos, int32_t* idx_out, void* ws,
                      size_t ws_bytes, void* stream, EntryMap em) {
  int s = check_index(d, true);
  if (s) return s;
  if (!qI || !wI || !KI_cache || !pos || !idx_out) return CSA_ERR_INVALID_ARG;
  const size_t need = index_decode_ws_bytes(*d);
  if (!ws || ws_bytes < need) return CSA_ERR_WORKSPACE;
  return hip_status(launch_index_topk_decode(*d, qI, wI, KI_cache, pos, idx_out, ws,
                                             (hipStream_t)stream, em));
}

int mqa_decode(const csa_attn_desc* d, int mode, const void* q, const void* win_ring,
               const void* comp_cache, const int32_t* idx, const int64_t* pos, const float* sink,
               void* out, void* ws, size_t ws_bytes, void* stream, EntryMap em) {
  const bool sparse = mode == ATTN_SPARSE;
  int s = check_attn(d, true, sparse);
  if (s) return s;
  if (!q || !win_ring || !comp_cache || (sparse && !idx) || !pos || !sink || !out)
    return CSA_ERR_INVALID_ARG;
  if (em.table && d->dtype != CSA_BF16) return CSA_ERR_UNSUPPORTED;
  const size_t need = mqa_decode_ws_bytes(*d, mode);
  if (!ws || ws_bytes < need) return CSA_ERR_WORKSPACE;
  return hip_status(launch_mqa_decode(*d, mode, q, win_ring, comp_cache, sparse ? idx : nullptr,
                                      pos, sink, out, ws, (hipStream_t)stream, em));
}

}  // namespace

extern "C" {

int csa_abi_version(void) { return CSA_ABI_VERSION; }

const char* csa_status_string(int s) {
  switch (s) {
    case CSA_OK: return "ok";
    case CSA_ERR_INVALID_ARG: return "invalid argument (null pointer or inconsistent sizes)";
    case CSA_ERR_UNSUPPORTED: return "unsupported shape or dtype for these kernels";
    case CSA_ERR_WORKSPACE: return "workspace smaller than csa_workspace_bytes()";
    case CSA_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

size_t csa_state_bytes(const csa_compress_desc* d) {
  if (!d || d->c <= 0) return 0;
  const int b = d->batch > 0 ? d->batch : 1;
  return (size_t)b * (d->overlap ? 3 : 1) * 3 * d->c * 4;
}

size_t csa_workspace_zero_bytes(int entry, const void* desc) {
  if (desc && entry == CSA_ENTRY_INDEX_TOPK_PREFILL) {
    const csa_index_desc* d = (const csa_index_desc*)desc;
    if (d->m <= 0 || d->n <= 0 || !index_prefill_long(d)) return 0;
    return index_prefill_long_zero_bytes(*d);
  }
  if (!desc || (entry != CSA_ENTRY_INDEX_TOPK_DECODE && entry != CSA_ENTRY_INDEX_TOPK_DECODE_FP4))
    return 0;
  const csa_index_desc* d = (const csa_index_desc*)desc;
  if (d->batch <= 0) return 0;
  return index_decode_zero_bytes(*d);
}

size_t csa_workspace_bytes(int entry, const void* desc) {
  if (!desc) return 0;
  switch (entry) {
    case CSA_ENTRY_COMPRESS_PREFILL: {
      const csa_compress_desc* d = (const csa_compress_desc*)desc;
      if (d->n + prefill_halo(d) <= 0 || d->c <= 0) return 0;
      return ws_compress_prefill(d, true);
    }
    case CSA_ENTRY_COMPRESS_DECODE: {
      const csa_compress_desc* d = (const csa_compress_desc*)desc;
      if (d->batch <= 0 || d->c <= 0 || d->d <= 0) return 0;
      return ws_compress_decode(d, true);
    }
    case CSA_ENTRY_INDEX_TOPK_PREFILL: {
      const csa_index_desc* d = (const csa_index_desc*)desc;
      if (d->m <= 0 || d->n <= 0) return 0;
      if (index_prefill_long(d)) return index_prefill_long_ws_bytes(*d);
      return al((size_t)d->n * index_prefill_ld(d) * (d->score_dtype == CSA_BF16 ? 2 : 4));
    }
    case CSA_ENTRY_INDEX_TOPK_PREFILL_FP4: {
      const csa_index_desc* d = (const csa_index_desc*)desc;
      if (d->m <= 0 || d->n <= 0 || index_prefill_long(d)) return 0;
      return al((size_t)d->n * index_prefill_ld(d) * (d->score_dtype == CSA_BF16 ? 2 : 4));
    }
    case CSA_ENTRY_INDEX_TOPK_DECODE:
    case CSA_ENTRY_INDEX_TOPK_DECODE_FP4: {
      const csa_index_desc* d = (const csa_index_desc*)desc;
      if (d->batch <= 0) return 0;
      return index_decode_ws_bytes(*d);
    }
    case CSA_ENTRY_SPARSE_MQA_PREFILL:
    case CSA_ENTRY_DENSE_MQA_PREFILL: return 0;
    case CSA_ENTRY_SPARSE_MQA_BACKWARD:
    case CSA_ENTRY_DENSE_MQA_BACKWARD: {
      const csa_attn_desc* d = (const csa_attn_desc*)desc;
      if (d->n < 0 || d->c <= 0 || d->n_heads <= 0 || d->n_win <= 0 || d->n_entries < 0)
        return 0;
      return mqa_backward_ws_bytes(*d);
    }
    case CSA_ENTRY_QUERY_PROJ: {
      const csa_query_desc* d = (const csa_query_desc*)desc;
      if (d->n <= 0 || d->d_c <= 0) return 0;
      return query_proj_ws_bytes(*d);
    }
    case CSA_ENTRY_OUTPUT_PROJ: {
      const csa_oproj_desc* d = (const csa_oproj_desc*)desc;
      if (d->n <= 0 || d->groups <= 0 || d->d_g <= 0) return 0;
      return output_proj_ws_bytes(*d);
    }
    case CSA_ENTRY_SPARSE_MQA_DECODE:
    case CSA_ENTRY_DENSE_MQA_DECODE: {
      const csa_attn_desc* d = (const csa_attn_desc*)desc;
      if (d->batch <= 0 || d->n_heads <= 0 || d->c <= 0) return 0;
      return mqa_decode_ws_bytes(*d, entry == CSA_ENTRY_SPARSE_MQA_DECODE ? ATTN_SPARSE : ATTN_DENSE);
    }
    default: return 0;
  }
}

int csa_state_init(const csa_compress_desc* d, float* state, void* stream) {
  if (!d || !state || d->c <= 0 || d->batch <= 0) return CSA_ERR_INVALID_ARG;
  const int64_t per = (int64_t)(d->overlap ? 3 : 1) * 3 * d->c;
  return hip_status(launch_state_init(state, per, d->batch, d->c, (hipStream_t)stream));
}

// The prefill compressor; with em.table the entries go to pool rows of one
// sequence's page table instead of consecutive rows of out_comp.
static int compress_prefill(const csa_compress_desc* d, const void* H, const void* W_kv,
                     const void* W_z, const float* ape, const void* W_win, void* out_comp,
                     void* out_win, void* win_ring, float* state, void* ws, size_t ws_bytes,
                     void* stream, EntryMap em) {
  int s = check_compress(d, false);
  if (s) return s;
  const bool has_win = W_win != nullptr;
  if ((out_win || win_ring) && !has_win) return CSA_ERR_INVALID_ARG;
  if (win_ring && d->n_win <= 0) return CSA_ERR_INVALID_ARG;
  const int64_t nc = d->n / d->m;
  const int64_t halo = prefill_halo(d), rows = d->n + halo;
  if (rows > 0 && (!H || !W_kv || !W_z || !ape)) return CSA_ERR_INVALID_ARG;
  if (nc > 0 && !out_comp) return CSA_ERR_INVALID_ARG;
  const size_t need = rows > 0 ? ws_compress_prefill(d, has_win) : 0;
  if (need > 0 && (!ws || ws_bytes < need)) return CSA_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const int w = (1 + d->overlap) * d->c;
  const int64_t ld = 2 * w + (has_win ? d->c : 0);
  float* P = (float*)ws;
  float* Pn = P + halo * ld;  // the new tokens' rows
  if (rows > 0) {
    WeightStack stack = {{W_kv, W_z, W_win}, {w, w, has_win ? d->c : 0}};
    hipError_t e = launch_proj_gemm(d->dtype, H, rows, d->d, stack, P, ld, st);
    if (e != hipSuccess) return CSA_ERR_HIP;
    e = launch_pool_entries(d->dtype, Pn, ld, d->n, d->c, d->m, d->overlap, ape, d->qk_norm,
                            d->eps, d->rope_dims, d->rope_theta, out_comp, d->pos0, st,
                            halo > 0, em);
    if (e != hipSuccess) return CSA_ERR_HIP;
    if (has_win && (out_win || win_ring)) {
      e = launch_window_rows(d->dtype, Pn, ld, 2 * w, d->n, d->c, d->qk_norm, d->eps,
                             d->rope_dims, d->rope_theta, out_win, win_ring, d->n_win, d->pos0,
                             st);
      if (e != hipSuccess) return CSA_ERR_HIP;
    }
  }
  if (state) {  // block-aligned from P's first row, so the halo is one more block
    hipError_t e = launch_stash_state(P, ld, rows, d->c, d->m, d->overlap, ape, state, st);
    if (e != hipSuccess) return CSA_ERR_HIP;
  }
  return CSA_OK;
}

int csa_compress_decode(const csa_compress_desc* d, const void* h, const int64_t* pos,
                        const void* W_kv, const void* W_z, const float* ape, const void* W_win,
                        float* state, void* cache, void* win_ring, void* ws, size_t ws_bytes,
                        void* stream) {
  return compress_decode(d, h, pos, W_kv, W_z, ape, W_win, state, cache, win_ring, ws, ws_bytes,
                         stream, EntryMap());
}

int csa_compress_prefill(const csa_compress_desc* d, const void* H, const void* W_kv,
                         const void* W_z, const float* ape, const void* W_win, void* out_comp,
                         void* out_win, void* win_ring, float* state, void* ws, size_t ws_bytes,
                         void* stream) {
  return compress_prefill(d, H, W_kv, W_z, ape, W_win, out_comp, out_win, win_ring, state, ws,
                          ws_bytes, stream, EntryMap());
}

int csa_compress_prefill_paged(const csa_compress_desc* d, const void* H, const void* W_kv,
                               const void* W_z, const float* ape, const void* W_win,
                               void* comp_pool, const int32_t* page_table,
                               int32_t page_entries, void* out_win, void* win_ring, float* state,
                               void* ws, size_t ws_bytes, void* stream) {
  if (!d) return CSA_ERR_INVALID_ARG;
  EntryMap em;
  int s = entry_map(page_table, page_entries, d->max_entries, &em);
  if (s) return s;
  // the chunk's entries pos0/m .. (pos0+n)/m - 1 must lie within the table
  if (d->m > 0 && d->n >= 0 && d->pos0 >= 0 && (d->pos0 + d->n) / d->m > d->max_entries)
    return CSA_ERR_INVALID_ARG;
  return compress_prefill(d, H, W_kv, W_z, ape, W_win, comp_pool, out_win, win_ring, state, ws,
                          ws_bytes, stream, em);
}

int csa_compress_decode_paged(const csa_compress_desc* d, const void* h, const int64_t* pos,
                              const void* W_kv, const void* W_z, const float* ape,
                              const void* W_win, float* state, void* cache_pool,
                              const int32_t* page_table, int32_t page_entries, void* win_ring,
                              void* ws, size_t ws_bytes, void* stream) {
  if (!d) return CSA_ERR_INVALID_ARG;
  EntryMap em;
  int s = entry_map(page_table, page_entries, d->max_entries, &em);
  if (s) return s;
  return compress_decode(d, h, pos, W_kv, W_z, ape, W_win, state, cache_pool, win_ring, ws,
                         ws_bytes, stream, em);
}

int csa_index_topk_prefill(const csa_index_desc* d, const void* qI, const void* wI,
                           const void* KI, int32_t* idx_out, void* ws, size_t ws_bytes,
                           void* stream) {
  int s = check_index(d, false);
  if (s) return s;
  if (d->n == 0) return CSA_OK;
  if (!qI || !wI || !idx_out || (d->n_entries > 0 && !KI)) return CSA_ERR_INVALID_ARG;
  if (index_prefill_long(d)) {
    if (!ws || ws_bytes < index_prefill_long_ws_bytes(*d)) return CSA_ERR_WORKSPACE;
    return hip_status(
        launch_index_topk_prefill_long(*d, qI, wI, KI, idx_out, ws, (hipStream_t)stream));
  }
  const int64_t ld = index_prefill_ld(d);
  const size_t need = al((size_t)d->n * ld * (d->score_dtype == CSA_BF16 ? 2 : 4));
  if (ld > 0 && (!ws || ws_bytes < need)) return CSA_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (ld > 0) e = launch_index_scores_prefill(*d, qI, wI, KI, ws, ld, st);
  if (e != hipSuccess) return CSA_ERR_HIP;
  return hip_status(launch_topk_rows_prefill(*d, ws, ld, idx_out, st));
}

int csa_index_topk_decode(const csa_index_desc* d, const void* qI, const void* wI,
                          const void* KI_cache, const int64_t* pos, int32_t* idx_out, void* ws,
                          size_t ws_bytes, void* stream) {
  return index_topk_decode(d, qI, wI, KI_cache, pos, idx_out, ws, ws_bytes, stream, EntryMap());
}

int csa_index_topk_decode_score(const csa_index_desc* d, const void* qI, const void* wI,
                                const void* KI_cache, const int64_t* pos, void* ws,
                                size_t ws_bytes, void* stream) {
  int s = check_index(d, true);
  if (s) return s;
  if (!qI || !wI || !KI_cache || !pos) return CSA_ERR_INVALID_ARG;
  if (!ws || ws_bytes < index_decode_ws_bytes(*d)) return CSA_ERR_WORKSPACE;
  return hip_status(launch_index_topk_decode_score(*d, qI, wI, KI_cache, pos, ws,
                                                   (hipStream_t)stream, EntryMap()));
}

int csa_index_topk_decode_select(const csa_index_desc* d, const void* qI, const void* wI,
                                 const void* KI_cache, const int64_t* pos, int32_t* idx_out,
                                 void* ws, size_t ws_bytes, void* stream) {
  int s = check_index(d, true);
  if (s) return s;
  if (!qI || !wI || !KI_cache || !pos || !idx_out) return CSA_ERR_INVALID_ARG;
  if (!ws || ws_bytes < index_decode_ws_bytes(*d)) return CSA_ERR_WORKSPACE;
  return hip_status(launch_index_topk_decode_select(*d, qI, wI, KI_cache, pos, idx_out, ws,
                                                    (hipStream_t)stream, EntryMap()));
}

int csa_index_topk_decode_noalloc(const csa_index_desc* d, const void* qI, const void* wI,
                                  const void* KI_cache, const int64_t* pos, int32_t* idx_out,
                                  void* stream) {
  int s = check_index(d, true);
  if (s) return s;
  if (index_decode_ws_bytes(*d) > noalloc_scratch_bytes()) return CSA_ERR_WORKSPACE;
  if (!qI || !wI || !KI_cache || !pos || !idx_out) return CSA_ERR_INVALID_ARG;
  return index_topk_decode_noalloc(*d, qI, wI, KI_cache, pos, idx_out, (hipStream_t)stream);
}

size_t csa_noalloc_scratch_bytes(void) { return noalloc_scratch_bytes(); }

int csa_index_topk_decode_paged(const csa_index_desc* d, const void* qI, const void* wI,
                                const void* KI_pool, const int32_t* page_table,
                                int32_t page_entries, const int64_t* pos, int32_t* idx_out,
                                void* ws, size_t ws_bytes, void* stream) {
  if (!d) return CSA_ERR_INVALID_ARG;
  EntryMap em;
  int s = entry_map(page_table, page_entries, d->n_entries, &em);
  if (s) return s;
  return index_topk_decode(d, qI, wI, KI_pool, pos, idx_out, ws, ws_bytes, stream, em);
}

int csa_query_proj(const csa_query_desc* d, const void* H, const void* W_DQ, const float* g_q,
                   const void* W_w, const void* W_UQ, const void* W_IUQ, void* q_out,
                   void* qI_out, void* wI_out, void* ws, size_t ws_bytes, void* stream) {
  int s = check_query(d);
  if (s) return s;
  const bool idx = d->n_heads_i > 0 && d->c_i > 0;
  if (!H || !W_DQ || !W_UQ || !q_out) return CSA_ERR_INVALID_ARG;
  if (d->n_heads_i > 0 && (!W_w || !wI_out)) return CSA_ERR_INVALID_ARG;
  if (idx && (!W_IUQ || !qI_out)) return CSA_ERR_INVALID_ARG;
  if (d->n == 0) return CSA_OK;
  if (!ws || ws_bytes < query_proj_ws_bytes(*d)) return CSA_ERR_WORKSPACE;
  return hip_status(launch_query_proj(*d, H, W_DQ, g_q, W_w, W_UQ, W_IUQ, q_out, qI_out, wI_out,
                                      ws, (hipStream_t)stream));
}

int csa_output_proj(const csa_oproj_desc* d, const void* o, const void* wo_a, const void* wo_b,
                    void* out, void* ws, size_t ws_bytes, void* stream) {
  int s = check_oproj(d);
  if (s) return s;
  if (!o || !wo_a || !wo_b || !out) return CSA_ERR_INVALID_ARG;
  if (d->n == 0) return CSA_OK;
  if (!ws || ws_bytes < output_proj_ws_bytes(*d)) return CSA_ERR_WORKSPACE;
  return hip_status(launch_output_proj(*d, o, wo_a, wo_b, out, ws, (hipStream_t)stream));
}

int csa_indexer_fp4_quant(const csa_fp4_desc* d, const void* x, uint8_t* codes, uint8_t* exps,
                          void* stream) {
  if (!d) return CSA_ERR_INVALID_ARG;
  if (!dtype_ok(d->dtype)) return CSA_ERR_UNSUPPORTED;
  if (d->rows < 0) return CSA_ERR_INVALID_ARG;
  if (d->width != 64 && d->width != 128) return CSA_ERR_UNSUPPORTED;
  if (d->rows == 0) return CSA_OK;
  if (!x || !codes || !exps) return CSA_ERR_INVALID_ARG;
  return hip_status(launch_fp4_rotate_quant(d->dtype, x, d->rows, d->width, codes, exps, nullptr,
                                            0, 1, (hipStream_t)stream));
}

int csa_indexer_fp4_quant_decode(const csa_fp4_desc* d, const void* cache, int64_t n_entries,
                                 const int64_t* pos, int m, uint8_t* codes, uint8_t* exps,
                                 void* stream) {
  if (!d) return CSA_ERR_INVALID_ARG;
  if (!dtype_ok(d->dtype)) return CSA_ERR_UNSUPPORTED;
  if (d->rows < 0 || n_entries < 0 || m <= 0) return CSA_ERR_INVALID_ARG;
  if (d->width != 64 && d->width != 128) return CSA_ERR_UNSUPPORTED;
  if (d->rows == 0 || n_entries == 0) return CSA_OK;
  if (!cache || !pos || !codes || !exps) return CSA_ERR_INVALID_ARG;
  return hip_status(launch_fp4_rotate_quant(d->dtype, cache, d->rows, d->width, codes, exps, pos,
                                            n_entries, m, (hipStream_t)stream));
}

int csa_indexer_fp4_quant_decode_paged(const csa_fp4_desc* d, const void* cache_pool,
                                       int64_t n_entries, const int64_t* pos, int m,
                                       uint8_t* codes_pool, uint8_t* exps_pool,
                                       const int32_t* page_table, int32_t page_entries,
                                       void* stream) {
  if (!d) return CSA_ERR_INVALID_ARG;
  if (!dtype_ok(d->dtype)) return CSA_ERR_UNSUPPORTED;
  if (d->rows < 0 || n_entries < 0 || m <= 0) return CSA_ERR_INVALID_ARG;
  if (d->width != 64 && d->width != 128) return CSA_ERR_UNSUPPORTED;
  EntryMap em;
  int s = entry_map(page_table, page_entries, n_entries, &em);
  if (s) return s;
  if (d->rows == 0 || n_entries == 0) return CSA_OK;
  if (!cache_pool || !pos || !codes_pool || !exps_pool) return CSA_ERR_INVALID_ARG;
  return hip_status(launch_fp4_rotate_quant(d->dtype, cache_pool, d->rows, d->width, codes_pool,
                                            exps_pool, pos, n_entries, m, (hipStream_t)stream,
                                            em));
}

// The FP4 scorer reads 16 code bytes per lane: both code arrays start on a
// 16-byte boundary (rows are 16-byte multiples, so every row does).
static bool codes_aligned(const uint8_t* q, const uint8_t* k) {
  return (((uintptr_t)q | (uintptr_t)k) & 15u) == 0;
}

int csa_index_topk_decode_fp4_paged(const csa_index_desc* d, const uint8_t* qI_codes,
                                    const uint8_t* qI_exps, const void* wI,
                                    const uint8_t* K_codes_pool, const uint8_t* K_exps_pool,
                                    const int32_t* page_table, int32_t page_entries,
                                    const int64_t* pos, int32_t* idx_out, void* ws,
                                    size_t ws_bytes, void* stream) {
  int s = check_index(d, true);
  if (s) return s;
  if (d->dtype != CSA_BF16) return CSA_ERR_UNSUPPORTED;
  EntryMap em;
  s = entry_map(page_table, page_entries, d->n_entries, &em);
  if (s) return s;
  if (!qI_codes || !qI_exps || !wI || !K_codes_pool || !K_exps_pool || !pos || !idx_out)
    return CSA_ERR_INVALID_ARG;
  if (!ws || ws_bytes < index_decode_ws_bytes(*d)) return CSA_ERR_WORKSPACE;
  if (!codes_aligned(qI_codes, K_codes_pool)) return CSA_ERR_INVALID_ARG;
  return hip_status(launch_index_topk_decode_fp4(*d, qI_codes, qI_exps, wI, K_codes_pool,
                                                 K_exps_pool, pos, idx_out, ws,
                                                 (hipStream_t)stream, em));
}

int csa_index_topk_decode_fp4(const csa_index_desc* d, const uint8_t* qI_codes,
                              const uint8_t* qI_exps, const void* wI, const uint8_t* K_codes,
                              const uint8_t* K_exps, const int64_t* pos, int32_t* idx_out,
                              void* ws, size_t ws_bytes, void* stream) {
  int s = check_index(d, true);
  if (s) return s;
  if (d->dtype != CSA_BF16) return CSA_ERR_UNSUPPORTED;
  if (!qI_codes || !qI_exps || !wI || !K_codes || !K_exps || !pos || !idx_out)
    return CSA_ERR_INVALID_ARG;
  if (!ws || ws_bytes < index_decode_ws_bytes(*d)) return CSA_ERR_WORKSPACE;
  if (!codes_aligned(qI_codes, K_codes)) return CSA_ERR_INVALID_ARG;
  return hip_status(launch_index_topk_decode_fp4(*d, qI_codes, qI_exps, wI, K_codes, K_exps, pos,
                                                 idx_out, ws, (hipStream_t)stream));
}

int csa_index_topk_prefill_fp4(const csa_index_desc* d, const uint8_t* qI_codes,
                               const uint8_t* qI_exps, const void* wI, const uint8_t* K_codes,
                               const uint8_t* K_exps, int32_t* idx_out, void* ws, size_t ws_bytes,
                               void* stream) {
  int s = check_index(d, false);
  if (s) return s;
  if (d->dtype != CSA_BF16 || index_prefill_long(d)) return CSA_ERR_UNSUPPORTED;
  if (d->n == 0) return CSA_OK;
  if (!qI_codes || !qI_exps || !wI || !idx_out || (d->n_entries > 0 && (!K_codes || !K_exps)))
    return CSA_ERR_INVALID_ARG;
  const int64_t ld = index_prefill_ld(d);
  const size_t need = al((size_t)d->n * ld * (d->score_dtype == CSA_BF16 ? 2 : 4));
  if (ld > 0 && (!ws || ws_bytes < need)) return CSA_ERR_WORKSPACE;
  if (!codes_aligned(qI_codes, d->n_entries > 0 ? K_codes : nullptr)) return CSA_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (ld > 0)
    e = launch_index_scores_prefill_fp4(*d, qI_codes, qI_exps, wI, K_codes, K_exps, ws, ld, st);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(launch_topk_rows_prefill(*d, ws, ld, idx_out, st));
}

int csa_sparse_mqa_prefill(const csa_attn_desc* d, const void* q, const void* win_kv,
                           const void* comp, const int32_t* idx, const float* sink, void* out,
                           void* ws, size_t ws_bytes, void* stream) {
  (void)ws; (void)ws_bytes;
  int s = check_attn(d, false, true);
  if (s) return s;
  if (d->n == 0) return CSA_OK;
  if (!q || !win_kv || !idx || !sink || !out || (d->n_entries > 0 && !comp))
    return CSA_ERR_INVALID_ARG;
  return hip_status(launch_mqa_prefill(*d, ATTN_SPARSE, q, win_kv, comp, idx, sink, out,
                                       (hipStream_t)stream));
}

static bool kv8_shape_ok(int c, int r) { return c == 512 && r >= 0 && r < c && r % 64 == 0; }

static int mqa_decode_fp8(const csa_attn_desc* d, int mode, const void* q, const void* ring8,
                          const void* cache8, const int32_t* idx, const int64_t* pos,
                          const float* sink, void* out, void* ws, size_t ws_bytes,
                          void* stream) {
  const bool sparse = mode == ATTN_SPARSE;
  int s = check_attn(d, true, sparse);
  if (s) return s;
  if (d->dtype != CSA_BF16 || !kv8_shape_ok(d->c, d->rope_dims)) return CSA_ERR_UNSUPPORTED;
  if (!q || !ring8 || !cache8 || (sparse && !idx) || !pos || !sink || !out)
    return CSA_ERR_INVALID_ARG;
  if (!ws || ws_bytes < mqa_decode_ws_bytes(*d, mode)) return CSA_ERR_WORKSPACE;
  return hip_status(launch_mqa_decode(*d, mode, q, ring8, cache8, sparse ? idx : nullptr, pos,
                                      sink, out, ws, (hipStream_t)stream, EntryMap(), true));
}

size_t csa_kv_fp8_row_bytes(int c, int rope_dims) {
  return kv8_shape_ok(c, rope_dims) ? (size_t)kv8_row_bytes(c, rope_dims) : 0;
}

int csa_kv_fp8_quant(const csa_kv8_desc* d, const void* src, uint8_t* dst, void* stream) {
  if (!d) return CSA_ERR_INVALID_ARG;
  if (!dtype_ok(d->dtype) || !kv8_shape_ok(d->c, d->rope_dims)) return CSA_ERR_UNSUPPORTED;
  if (d->rows < 0) return CSA_ERR_INVALID_ARG;
  if (d->rows == 0) return CSA_OK;
  if (!src || !dst) return CSA_ERR_INVALID_ARG;
  return hip_status(launch_kv_fp8_quant(d->dtype, src, d->rows, d->rope_dims, dst, nullptr, 0,
                                        1, 0, (hipStream_t)stream));
}

int csa_kv_fp8_quant_decode(const csa_kv8_desc* d, const void* src, int64_t n_rows,
                            const int64_t* pos, int m, int ring, uint8_t* dst, void* stream) {
  if (!d) return CSA_ERR_INVALID_ARG;
  if (!dtype_ok(d->dtype) || !kv8_shape_ok(d->c, d->rope_dims)) return CSA_ERR_UNSUPPORTED;
  if (d->rows < 0 || n_rows <= 0 || (!ring && m <= 0)) return CSA_ERR_INVALID_ARG;
  if (d->rows == 0) return CSA_OK;
  if (!src || !pos || !dst) return CSA_ERR_INVALID_ARG;
  return hip_status(launch_kv_fp8_quant(d->dtype, src, d->rows, d->rope_dims, dst, pos, n_rows,
                                        ring ? 1 : m, ring ? 1 : 0, (hipStream_t)stream));
}

int csa_sparse_mqa_decode_fp8(const csa_attn_desc* d, const void* q, const void* win_ring8,
                              const void* cache8, const int32_t* idx, const int64_t* pos,
                              const float* sink, void* out, void* ws, size_t ws_bytes,
                              void* stream) {
  return mqa_decode_fp8(d, ATTN_SPARSE, q, win_ring8, cache8, idx, pos, sink, out, ws, ws_bytes,
                        stream);
}

int hca_dense_mqa_decode_fp8(const csa_attn_desc* d, const void* q, const void* win_ring8,
                             const void* cache8, const int64_t* pos, const float* sink, void* out,
                             void* ws, size_t ws_bytes, void* stream) {
  return mqa_decode_fp8(d, ATTN_DENSE, q, win_ring8, cache8, nullptr, pos, sink, out, ws,
                        ws_bytes, stream);
}

static int mqa_backward(const csa_attn_desc* d, int mode, const void* q, const void* win_kv,
                        const void* comp, const int32_t* idx, const float* sink,
                        const void* dout, void* dq, void* dwin, void* dcomp, float* dsink,
                        void* ws, size_t ws_bytes, void* stream) {
  const bool sparse = mode == ATTN_SPARSE;
  int s = check_attn(d, false, sparse);
  if (s) return s;
  if (!mqa_backward_supported(*d)) return CSA_ERR_UNSUPPORTED;
  if (!q || !win_kv || (sparse && !idx) || !sink || !dout || !dq || !dwin || !dsink ||
      (d->n_entries > 0 && (!comp || !dcomp)))
    return CSA_ERR_INVALID_ARG;
  if (!ws || ws_bytes < mqa_backward_ws_bytes(*d)) return CSA_ERR_WORKSPACE;
  return hip_status(launch_mqa_backward(*d, mode, (const float*)q, (const float*)win_kv,
                                        (const float*)comp, idx, sink, (const float*)dout,
                                        (float*)dq, (float*)dwin, (float*)dcomp, dsink, ws,
                                        (hipStream_t)stream));
}

int csa_sparse_mqa_backward(const csa_attn_desc* d, const void* q, const void* win_kv,
                            const void* comp, const int32_t* idx, const float* sink,
                            const void* dout, void* dq, void* dwin, void* dcomp, float* dsink,
                            void* ws, size_t ws_bytes, void* stream) {
  return mqa_backward(d, ATTN_SPARSE, q, win_kv, comp, idx, sink, dout, dq, dwin, dcomp, dsink,
                      ws, ws_bytes, stream);
}

int hca_dense_mqa_backward(const csa_attn_desc* d, const void* q, const void* win_kv,
                           const void* comp, const float* sink, const void* dout, void* dq,
                           void* dwin, void* dcomp, float* dsink, void* ws, size_t ws_bytes,
                           void* stream) {
  return mqa_backward(d, ATTN_DENSE, q, win_kv, comp, nullptr, sink, dout, dq, dwin, dcomp,
                      dsink, ws, ws_bytes, stream);
}

int csa_sparse_mqa_decode(const csa_attn_desc* d, const void* q, const void* win_ring,
                          const void* comp_cache, const int32_t* idx, const int64_t* pos,
                          const float* sink, void* out, void* ws, size_t ws_bytes, void* stream) {
  return mqa_decode(d, ATTN_SPARSE, q, win_ring, comp_cache, idx, pos, sink, out, ws, ws_bytes,
                    stream, EntryMap());
}

int csa_sparse_mqa_decode_paged(const csa_attn_desc* d, const void* q, const void* win_ring,
                                const void* comp_pool, const int32_t* page_table,
                                int32_t page_entries, const int32_t* idx, const int64_t* pos,
                                const float* sink, void* out, void* ws, size_t ws_bytes,
                                void* stream) {
  if (!d) return CSA_ERR_INVALID_ARG;
  EntryMap em;
  int s = entry_map(page_table, page_entries, d->n_entries, &em);
  if (s) return s;
  return mqa_decode(d, ATTN_SPARSE, q, win_ring, comp_pool, idx, pos, sink, out, ws, ws_bytes,
                    stream, em);
}

int hca_dense_mqa_prefill(const csa_attn_desc* d, const void* q, const void* win_kv,
                          const void* comp, const float* sink, void* out, void* ws,
                          size_t ws_bytes, void* stream) {
  (void)ws; (void)ws_bytes;
  int s = check_attn(d, false, false);
  if (s) return s;
  if (d->n == 0) return CSA_OK;
  if (!q || !win_kv || !sink || !out || (d->n_entries > 0 && !comp)) return CSA_ERR_INVALID_ARG;
  return hip_status(launch_mqa_prefill(*d, ATTN_DENSE, q, win_kv, comp, nullptr, sink, out,
                                       (hipStream_t)stream));
}

int hca_dense_mqa_decode(const csa_attn_desc* d, const void* q, const void* win_ring,
                         const void* comp_cache, const int64_t* pos, const float* sink, void* out,
                         void* ws, size_t ws_bytes, void* stream) {
  return mqa_decode(d, ATTN_DENSE, q, win_ring, comp_cache, nullptr, pos, sink, out, ws, ws_bytes,
                    stream, EntryMap());
}

int hca_dense_mqa_decode_paged(const csa_attn_desc* d, const void* q, const void* win_ring,
                               const void* comp_pool, const int32_t* page_table,
                               int32_t page_entries, const int64_t* pos, const float* sink,
                               void* out, void* ws, size_t ws_bytes, void* stream) {
  if (!d) return CSA_ERR_INVALID_ARG;
  EntryMap em;
  int s = entry_map(page_table, page_entries, d->n_entries, &em);
  if (s) return s;
  return mqa_decode(d, ATTN_DENSE, q, win_ring, comp_pool, nullptr, pos, sink, out, ws, ws_bytes,
                    stream, em);
}

}  // extern "C"
