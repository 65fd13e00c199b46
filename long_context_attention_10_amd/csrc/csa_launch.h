// Host-side launchers of the libcsa kernels.  Each returns hipSuccess or the
// launch error; arguments were validated by the C ABI layer before the call.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/csa.h"
#include "csa_common.h"  // EntryMap

namespace csa {

// A stacked set of up to three output-major weight matrices [rows_i, K]
// that one projection multiplies with the same left operand.
struct WeightStack {
  const void* w[3];
  int rows[3];
  int total() const { return rows[0] + rows[1] + rows[2]; }
};

// Outputs of a stacked product: matrix i writes its columns to p[i] with row
// stride ld[i] (elements of the output type).
struct GemmOuts {
  void* p[3];
  int64_t ld[3];
};

// bf16 operands: for each group z < groups, out_i = A_z[M, K] . W_i^T where
// A_z = A + z * a_zoff (row stride lda), W_0 is offset by z * w_zoff and
// output 0 by z * o_zoff; fp32 or bf16 (rounded once) outputs.  K % 64 == 0.
hipError_t launch_gemm_bf16(const void* A, int64_t lda, int64_t M, int K, const WeightStack& w,
                            const GemmOuts& outs, bool bf16_out, int groups, int64_t a_zoff,
                            int64_t w_zoff, int64_t o_zoff, hipStream_t st);

// out[M, ldo] (fp32, columns [0, stack.total())) = A[M, K] . stack^T
hipError_t launch_proj_gemm(int dtype, const void* A, int64_t M, int K, const WeightStack& ws,
                            float* out, int64_t ldo, hipStream_t st);

// Pool complete blocks of a projected scratch [n, ld] (C at col 0, Z at col w)
// into entries, apply the epilogue and store.  Row 0 of P is position pos0;
// prev0: P[-m, 0) holds the previous block (its b-series joins entry 0).
// With em.table, entry i goes to the pool row of entry pos0 / m + i of one
// sequence; otherwise to row i of out.
hipError_t launch_pool_entries(int dtype, const float* P, int64_t ld, int64_t n, int c, int m,
                               int ov, const float* ape, int qk_norm, float eps, int rope_dims,
                               float theta, void* out, int64_t pos0, hipStream_t st,
                               int prev0 = 0, EntryMap em = EntryMap());

// Window rows from scratch column `col` (width c) -> out [n, c] and/or ring.
hipError_t launch_window_rows(int dtype, const float* P, int64_t ld, int col, int64_t n, int c,
                              int qk_norm, float eps, int rope_dims, float theta, void* out,
                              void* ring, int n_win, int64_t pos0, hipStream_t st);

// Decode state after the last prefill token (fold tail rows / last block).
hipError_t launch_stash_state(const float* P, int64_t ld, int64_t n, int c, int m, int ov,
                              const float* ape, float* state, hipStream_t st);

hipError_t launch_state_init(float* state, int64_t floats_per_seq, int batch, int c,
                             hipStream_t st);

// Decode projection partials: ws[ks][B][N] over K-splits.
hipError_t launch_decode_proj(int dtype, const void* h, int B, int K, const WeightStack& w,
                              float* part, int ksplit, hipStream_t st);

hipError_t launch_decode_update(int dtype, const float* part, int ksplit, int B, int N, int c,
                                int m, int ov, int has_win, const float* ape, const int64_t* pos,
                                float* state, void* cache, int64_t max_entries, void* ring,
                                int n_win, int qk_norm, float eps, int rope_dims, float theta,
                                hipStream_t st, EntryMap em = EntryMap());

int decode_proj_ksplit(int N, int K, int dtype);

// ------------------------------------------------------------- indexer
// scores: [n, ld] of d.score_dtype (fp32, or bf16 rounded once)
hipError_t launch_index_scores_prefill(const csa_index_desc& d, const void* qI, const void* wI,
                                       const void* KI, void* scores, int64_t ld,
                                       hipStream_t st);
hipError_t launch_topk_rows_prefill(const csa_index_desc& d, const void* scores, int64_t ld,
                                    int32_t* idx_out, hipStream_t st);

size_t index_decode_ws_bytes(const csa_index_desc& d);
// prefill rows beyond the register selector (decode top-k over row batches)
size_t index_prefill_long_ws_bytes(const csa_index_desc& d);
size_t index_prefill_long_zero_bytes(const csa_index_desc& d);
hipError_t launch_index_topk_prefill_long(const csa_index_desc& d, const void* qI,
                                          const void* wI, const void* KI, int32_t* idx_out,
                                          void* ws, hipStream_t st);
size_t index_decode_zero_bytes(const csa_index_desc& d);
hipError_t launch_index_scores_prefill_fp4(const csa_index_desc& d, const uint8_t* qc,
                                           const uint8_t* qe, const void* wI, const uint8_t* kc,
                                           const uint8_t* ke, void* scores, int64_t ld,
                                           hipStream_t st);
hipError_t launch_index_topk_decode_fp4(const csa_index_desc& d, const uint8_t* qc,
                                        const uint8_t* qe, const void* wI, const uint8_t* kc,
                                        const uint8_t* ke, const int64_t* pos, int32_t* idx_out,
                                        void* wsp, hipStream_t st, EntryMap em = EntryMap());
// pos == nullptr: rows 0..rows-1; else row b * n_entries + pos[b] / m of each
// of `rows` sequences, when (pos[b] + 1) % m == 0.
hipError_t launch_fp4_rotate_quant(int dtype, const void* x, int64_t rows, int width,
                                   uint8_t* codes, uint8_t* exps, const int64_t* pos,
                                   int64_t n_entries, int m, hipStream_t st,
                                   EntryMap em = EntryMap());
hipError_t launch_index_topk_decode(const csa_index_desc& d, const void* qI, const void* wI,
                                    const void* KI, const int64_t* pos, int32_t* idx_out,
                                    void* ws, hipStream_t st, EntryMap em = EntryMap());
// The same in two parts: scoring of the entries that precede each position's
// step (may run while that step's compressor emits its entry), then the
// selection, which scores the emitted entry itself.
hipError_t launch_index_topk_decode_score(const csa_index_desc& d, const void* qI,
                                          const void* wI, const void* KI, const int64_t* pos,
                                          void* ws, hipStream_t st, EntryMap em = EntryMap());
hipError_t launch_index_topk_decode_select(const csa_index_desc& d, const void* qI,
                                           const void* wI, const void* KI, const int64_t* pos,
                                           int32_t* idx_out, void* ws, hipStream_t st,
                                           EntryMap em = EntryMap());

// The no-allocation variant (noalloc.hip): the same launches on a
// library-owned static scratch of noalloc_scratch_bytes() per device.
size_t noalloc_scratch_bytes();
int index_topk_decode_noalloc(const csa_index_desc& d, const void* qI, const void* wI,
                              const void* KI, const int64_t* pos, int32_t* idx_out,
                              hipStream_t st);

// ------------------------------------------------------------- attention
enum AttnMode { ATTN_SPARSE = 0, ATTN_DENSE = 1 };

hipError_t launch_mqa_prefill(const csa_attn_desc& d, int mode, const void* q, const void* win,
                              const void* comp, const int32_t* idx, const float* sink, void* out,
                              hipStream_t st);
// bf16 fast path (head dims 128/256/512, up to 1024 index slots)
hipError_t launch_mqa_prefill_bf16(const csa_attn_desc& d, int mode, const void* q, const void* win,
                                   const void* comp, const int32_t* idx, const float* sink,
                                   void* out, hipStream_t st);

size_t mqa_decode_ws_bytes(const csa_attn_desc& d, int mode);
// bf16 decode: split-K chunk width (candidates) and the split-K launcher
int mqa_decode_bf16_split(int mode);
hipError_t launch_mqa_decode_bf16(const csa_attn_desc& d, int mode, const void* q,
                                  const void* ring, const void* cache, const int32_t* idx,
                                  const int64_t* pos, const float* sink, void* out, float* ws_o,
                                  float2* ws_ml, int nsplit, hipStream_t st,
                                  EntryMap em = EntryMap(), bool kv8 = false);
// kv8: ring and cache hold FP8 rows (kv8_row_bytes; bf16 queries and output)
hipError_t launch_mqa_decode(const csa_attn_desc& d, int mode, const void* q, const void* ring,
                             const void* cache, const int32_t* idx, const int64_t* pos,
                             const float* sink, void* out, void* ws, hipStream_t st,
                             EntryMap em = EntryMap(), bool kv8 = false);
// FP8 KV rows (kvfp8.hip): rows of width 512 with r RoPE channels.  pos ==
// nullptr: rows 0..rows-1; else one row per sequence b < rows: ring != 0 the
// window slot b * n + pos % n, ring == 0 the entry pos / m of sequence b
// (through em) when (pos + 1) % m == 0.
hipError_t launch_kv_fp8_quant(int dtype, const void* src, int64_t rows, int r, uint8_t* dst,
                               const int64_t* pos, int64_t n, int m, int ring, hipStream_t st,
                               EntryMap em = EntryMap());

// Deterministic fp32 attention backward (backward.hip).
bool mqa_backward_supported(const csa_attn_desc& d);
size_t mqa_backward_ws_bytes(const csa_attn_desc& d);
hipError_t launch_mqa_backward(const csa_attn_desc& d, int mode, const float* q, const float* win,
                               const float* comp, const int32_t* idx, const float* sink,
                               const float* dout, float* dq, float* dwin, float* dcomp,
                               float* dsink, void* ws, hipStream_t st);

// The layer around the attention calls (layer.hip).
size_t query_proj_ws_bytes(const csa_query_desc& d);
hipError_t launch_query_proj(const csa_query_desc& d, const void* H, const void* W_DQ,
                             const float* g_q, const void* W_w, const void* W_UQ,
                             const void* W_IUQ, void* q_out, void* qI_out, void* wI_out,
                             void* ws, hipStream_t st);
size_t output_proj_ws_bytes(const csa_oproj_desc& d);
hipError_t launch_output_proj(const csa_oproj_desc& d, const void* o, const void* wo_a,
                              const void* wo_b, void* out, void* ws, hipStream_t st);

}  // namespace csa
