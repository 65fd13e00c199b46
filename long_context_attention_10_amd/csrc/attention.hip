// Shared-KV multi-query core attention over (window rows + compressed
// entries) with a per-head attention sink.
//
// Citation keys: [R] = page "DeepSeek-V4 技术解读报告" (juejin.cn), section
// 2.3.1 eq 18-19 (each entry is both key and value), 2.3.3 (QK RMSNorm,
// partial RoPE with the output rotated back, sliding window, sink logits,
// eq 27), 4.3 (batch-invariant, deterministic attention); [A] = page
// "DeepSeek-V4：算法架构" (1zeryu.github.io), Sparse Attention candidate
// assembly (window ++ selected entries), HCA selection rule, and the output
// projection's inverse RoPE.
//
// Workgroup layout (256 threads = 4 waves): the waves split the head dim c
// into four slices of CW = c/4 channels.  For each tile of 32 candidates:
//   1. the candidate rows are gathered into LDS (one copy serves as K and V);
//   2. each wave forms the partial logits S_w = Q[:, slice] K[:, slice]^T on
//      16x16 matrix-core blocks (heads x candidates), Q kept in registers;
//   3. the four partials are summed in LDS, and an online softmax per head
//      (seeded with the sink: running max = sink, running sum = 1) produces
//      P (rounded to the operand type) and the rescale factor alpha;
//   4. each wave rescales its O slice and accumulates O += P V[:, slice].
// Prefill: one workgroup per query token, all heads.  Decode: one workgroup
// per (sequence, 16-head group, fixed-size candidate chunk); the chunk
// partials (max, sum, unnormalised O) are merged by a second kernel in a fixed
// order, adding the sink exactly once -- the chunk size does not depend on
// the batch, so a sequence's result does not either.
#include "csa_common.h"
#include "csa_launch.h"

namespace csa {

constexpr int kTile = 32;        // candidates per tile
constexpr int kDecSplit = 256;   // candidates per decode chunk (fixed)

enum { MODE_PREFILL_SPARSE = 0, MODE_PREFILL_DENSE = 1, MODE_DECODE_SPARSE = 2,
       MODE_DECODE_DENSE = 3 };

template <class T, int C, int MB>
struct MqaSmem {
  typedef typename T::S S;
  static constexpr int ROWB = C * (int)sizeof(S) + 16;      // KV tile row bytes
  static constexpr int PROWB = kTile * (int)sizeof(S) + 16; // P row bytes
  static constexpr int SROW = kTile + 1;                    // S partial row floats
  uint8_t kv[kTile * ROWB];
  float spart[4][MB * 16][SROW];
  uint8_t p[MB * 16 * PROWB];
  float alpha[MB * 16];
  float red[4][MB * 16];
  int valid[kTile];
};

template <class T, int C, int MB, int MODE>
__global__ __launch_bounds__(256) void mqa_kernel(
    const typename T::S* __restrict__ q, const typename T::S* __restrict__ win,
    const typename T::S* __restrict__ comp, const int32_t* __restrict__ idx,
    const int64_t* __restrict__ posv, const float* __restrict__ sink, typename T::S* __restrict__ out,
    float* __restrict__ ws_o, float* __restrict__ ws_ml, int64_t n, int nh, int k, int m,
    int n_win, float scale, int qk_norm, float eps, int r, float theta, int64_t n_entries,
    int nsplit, int64_t t0) {
  typedef typename T::S S;
  typedef MqaSmem<T, C, MB> Sm;
  constexpr int E = 16 / (int)sizeof(S);
  constexpr int KGE = 4 * E;          // reduction elements per 16x16 k-group
  constexpr int CW = C / 4;           // channels per wave
  constexpr int NGQ = CW / KGE;       // k-groups per wave slice (QK^T)
  constexpr int NCB = CW / 16;        // 16-channel output blocks per wave (PV)
  constexpr int NH = MB * 16;         // head rows in this workgroup
  constexpr int TPH = 256 / NH;       // softmax threads per head
  constexpr int CPT = kTile / TPH;    // candidates per softmax thread
  constexpr bool DECODE = MODE >= MODE_DECODE_SPARSE;
  constexpr bool SPARSE = MODE == MODE_PREFILL_SPARSE || MODE == MODE_DECODE_SPARSE;
  static_assert(NGQ >= 1 && NCB >= 1, "head dim too small for 4 waves");
  __shared__ __align__(16) Sm sm;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lg = lane >> 4;

  // ---------------------------------------------------------------- task
  int64_t t, b = 0, pos;
  int h0 = 0, split = 0;
  if (!DECODE) {
    t = blockIdx.x;
    pos = t0 + t;  // win row 0 is position max(t0 - n_win + 1, 0)
  } else {
    b = blockIdx.y;
    h0 = blockIdx.z * 16;
    split = blockIdx.x;
    pos = posv[b];
    t = b;  // query row
  }
  const int nwin = (int)max64(0, min64(n_win, pos + 1));  // no window before position 0
  int64_t ncomp;
  if (SPARSE) ncomp = k;
  else ncomp = min64((pos + 1) / m, n_entries);
  const int64_t ncand = nwin + ncomp;
  int64_t cbeg = 0, cend = ncand;
  if (DECODE) {
    cbeg = (int64_t)split * kDecSplit;
    cend = min64(cbeg + kDecSplit, ncand);
    if (cbeg >= ncand && split > 0) {
      // nothing in this chunk: publish an empty partial
      if (tid < NH) {
        const int h = h0 + tid;
        if (h < nh) {
          float* ml = ws_ml + (((int64_t)b * nsplit + split) * nh + h) * 2;
          ml[0] = -INFINITY;
          ml[1] = 0.f;
        }
      }
      return;
    }
  }
  const S* qrow = q + t * (int64_t)nh * C;
  const S* crow_base = comp + (DECODE ? b * n_entries * C : 0);
  const S* wbase = win + (DECODE ? b * (int64_t)n_win * C : 0);
  const int32_t* irow = SPARSE ? idx + t * (int64_t)k : nullptr;

  // ------------------------------------------------ query prologue (regs)
  uint4 qf[MB][NGQ];
  {
    float qv[MB][NGQ][E];
    float ss[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int h = h0 + mb * 16 + (lane & 15);
      ss[mb] = 0.f;
#pragma unroll
      for (int g = 0; g < NGQ; ++g) {
        uint4 raw = make_uint4(0, 0, 0, 0);
        if (h < nh) raw = *(const uint4*)(qrow + (int64_t)h * C + wave * CW + g * KGE + lg * E);
        chunk_to_f32<T>(raw, qv[mb][g]);
#pragma unroll
        for (int e = 0; e < E; ++e) ss[mb] += qv[mb][g][e] * qv[mb][g][e];
      }
    }
    if (qk_norm) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        float s = ss[mb];
        s += __shfl_xor(s, 16, 64);
        s += __shfl_xor(s, 32, 64);
        if (lg == 0) sm.red[wave][mb * 16 + (lane & 15)] = s;
      }
      __syncthreads();
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int hr = mb * 16 + (lane & 15);
        const float tot = sm.red[0][hr] + sm.red[1][hr] + sm.red[2][hr] + sm.red[3][hr];
        const float inv = rsqrtf(tot / (float)C + eps);
#pragma unroll
        for (int g = 0; g < NGQ; ++g)
#pragma unroll
          for (int e = 0; e < E; ++e) qv[mb][g][e] *= inv;
      }
    }
    if (r > 0) {
#pragma unroll
      for (int g = 0; g < NGQ; ++g) {
        const int ch0 = wave * CW + g * KGE + lg * E;
#pragma unroll
        for (int e = 0; e < E; e += 2) {
          const int ch = ch0 + e;
          if (ch >= C - r) {
            float cs, sn;
            rope_cs(pos, (ch - (C - r)) / 2, r, theta, &cs, &sn);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
              const float x0 = qv[mb][g][e], x1 = qv[mb][g][e + 1];
              qv[mb][g][e] = x0 * cs - x1 * sn;
              qv[mb][g][e + 1] = x0 * sn + x1 * cs;
            }
          }
        }
      }
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int g = 0; g < NGQ; ++g) qf[mb][g] = f32_to_chunk<T>(qv[mb][g]);
  }

  // ----------------------------------------------- softmax state per head
  const int sh_head = tid / TPH;         // head row handled in the softmax phase
  const int sh_sub = tid % TPH;
  float run_m, run_l;
  if (!DECODE) {
    const int h = h0 + sh_head;
    run_m = h < nh ? sink[h] : 0.f;       // the sink seeds the running max/sum
    run_l = 1.f;
  } else {
    run_m = -INFINITY;
    run_l = 0.f;
  }

  f32x4_t oacc[MB][NCB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) oacc[mb][cb] = f32x4_t{};

  constexpr int CHUNKS_PER_ROW = C * (int)sizeof(S) / 16;
  constexpr int THR_PER_ROW = 256 / kTile;                 // 8
  constexpr int LOADS = CHUNKS_PER_ROW / THR_PER_ROW;
  const int my_row = tid / THR_PER_ROW, my_sub = tid % THR_PER_ROW;

  for (int64_t c0 = cbeg; c0 < cend; c0 += kTile) {
    // ------------------------------------------------------------ gather
    const int64_t j = c0 + my_row;
    const S* src = nullptr;
    if (j < cend) {
      if (j < nwin) {
        const int64_t p = pos - nwin + 1 + j;
        src = DECODE ? wbase + (p % n_win) * C : wbase + (p - max64(t0 - n_win + 1, 0)) * C;
      } else {
        const int64_t jj = j - nwin;
        int64_t e;
        if (SPARSE) e = irow[jj];
        else e = jj;
        if (e >= 0 && e < n_entries) src = crow_base + e * C;
      }
    }
    uint4 ld[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i)
      ld[i] = src ? *(const uint4*)((const uint8_t*)src + (my_sub + i * THR_PER_ROW) * 16)
                  : make_uint4(0, 0, 0, 0);
    __syncthreads();  // previous tile fully consumed
#pragma unroll
    for (int i = 0; i < LOADS; ++i)
      *(uint4*)(sm.kv + my_row * Sm::ROWB + (my_sub + i * THR_PER_ROW) * 16) = ld[i];
    if (my_sub == 0) sm.valid[my_row] = src != nullptr;
    __syncthreads();

    // ------------------------------------------- partial logits per wave
    f32x4_t sacc[MB][2];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) { sacc[mb][0] = f32x4_t{}; sacc[mb][1] = f32x4_t{}; }
#pragma unroll
    for (int cbk = 0; cbk < 2; ++cbk) {
#pragma unroll
      for (int g = 0; g < NGQ; ++g) {
        const uint4 kb = *(const uint4*)(sm.kv + (cbk * 16 + (lane & 15)) * Sm::ROWB +
                                         (wave * CW + g * KGE + lg * E) * (int)sizeof(S));
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) mma16<T>(sacc[mb][cbk], qf[mb][g], kb);
      }
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int cbk = 0; cbk < 2; ++cbk)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sm.spart[wave][mb * 16 + 4 * lg + i][cbk * 16 + (lane & 15)] = sacc[mb][cbk][i];
    __syncthreads();

    // --------------------------------------------------- online softmax
    {
      float s[CPT];
      float tmax = -INFINITY;
#pragma unroll
      for (int u = 0; u < CPT; ++u) {
        const int cc = sh_sub * CPT + u;
        float v = sm.spart[0][sh_head][cc] + sm.spart[1][sh_head][cc] + sm.spart[2][sh_head][cc] +
                  sm.spart[3][sh_head][cc];
        v = sm.valid[cc] ? v * scale : -INFINITY;
        s[u] = v;
        tmax = fmaxf(tmax, v);
      }
#pragma unroll
      for (int o = 1; o < TPH; o <<= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, o, 64));
      const float nm = fmaxf(run_m, tmax);
      const float alpha = (nm == -INFINITY) ? 1.f : __expf(run_m - nm);
      float psum = 0.f;
      float pv[CPT];
#pragma unroll
      for (int u = 0; u < CPT; ++u) {
        pv[u] = (nm == -INFINITY) ? 0.f : __expf(s[u] - nm);
        psum += pv[u];
      }
#pragma unroll
      for (int o = 1; o < TPH; o <<= 1) psum += __shfl_xor(psum, o, 64);
      run_l = run_l * alpha + psum;
      run_m = nm;
      S* prow = (S*)(sm.p + sh_head * Sm::PROWB) + sh_sub * CPT;
#pragma unroll
      for (int u = 0; u < CPT; ++u) prow[u] = T::cvt(pv[u]);
      if (sh_sub == 0) sm.alpha[sh_head] = alpha;
    }
    __syncthreads();

    // ------------------------------------------------- O += P V (slice)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = sm.alpha[mb * 16 + 4 * lg + i];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) oacc[mb][cb][i] *= a;
      }
    }
#pragma unroll
    for (int kg = 0; kg < kTile / KGE; ++kg) {
      uint4 pa[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        pa[mb] = *(const uint4*)(sm.p + (mb * 16 + (lane & 15)) * Sm::PROWB +
                                 (kg * KGE + lg * E) * (int)sizeof(S));
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        S vv[E];
        const int ch = wave * CW + cb * 16 + (lane & 15);
#pragma unroll
        for (int e = 0; e < E; ++e)
          vv[e] = *(const S*)(sm.kv + (kg * KGE + lg * E + e) * Sm::ROWB + ch * (int)sizeof(S));
        uint4 vb;
        __builtin_memcpy(&vb, vv, 16);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) mma16<T>(oacc[mb][cb], pa[mb], vb);
      }
    }
  }

  // ------------------------------------------------------------ epilogue
  if (!DECODE) {
    __syncthreads();
    if (sh_sub == 0) sm.red[0][sh_head] = 1.f / run_l;
    __syncthreads();
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hr = mb * 16 + 4 * lg + i;
        const int h = h0 + hr;
        const float inv = sm.red[0][hr];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const int ch = wave * CW + cb * 16 + (lane & 15);
          float v = oacc[mb][cb][i] * inv;
          if (r > 0 && ch >= C - r) {  // inverse RoPE at the query position
            const float other = __shfl_xor(v, 1, 64);
            float cs, sn;
            rope_cs(pos, (ch - (C - r)) / 2, r, theta, &cs, &sn);
            v = (ch & 1) ? (v * cs - other * sn) : (v * cs + other * sn);
          }
          if (h < nh) T::st(out, (t * nh + h) * (int64_t)C + ch, v);
        }
      }
    }
  } else {
    // partial state of this chunk: unnormalised O, running max and sum
    const int64_t base = ((int64_t)b * nsplit + split) * nh;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = h0 + mb * 16 + 4 * lg + i;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const int ch = wave * CW + cb * 16 + (lane & 15);
          if (h < nh) ws_o[(base + h) * C + ch] = oacc[mb][cb][i];
        }
      }
    if (sh_sub == 0) {
      const int h = h0 + sh_head;
      if (h < nh) {
        ws_ml[(base + h) * 2 + 0] = run_m;
        ws_ml[(base + h) * 2 + 1] = run_l;
      }
    }
  }
}

// Fixed-order merge of the decode chunk partials with the sink, then the
// inverse RoPE at the query position.  One workgroup per (sequence, head),
// thread j owning channels (2j, 2j+1).
template <class T>
__global__ __launch_bounds__(256) void mqa_combine_kernel(const float* __restrict__ ws_o,
                                                          const float* __restrict__ ws_ml,
                                                          const int64_t* __restrict__ posv,
                                                          const float* __restrict__ sink,
                                                          typename T::S* __restrict__ out, int nh,
                                                          int C, int nsplit, int r, float theta) {
  const int b = blockIdx.x, h = blockIdx.y;
  const int j = threadIdx.x;
  if (2 * j >= C) return;
  const int64_t base = (int64_t)b * nsplit * nh;
  float M = sink[h];
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, ws_ml[((base + (int64_t)s * nh) + h) * 2]);
  float den = __expf(sink[h] - M);
  float o0 = 0.f, o1 = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const int64_t row = base + (int64_t)s * nh + h;
    const float ms = ws_ml[row * 2];
    if (ms == -INFINITY) continue;
    const float f = __expf(ms - M);
    den += f * ws_ml[row * 2 + 1];
    const float2 ov = *(const float2*)(ws_o + row * C + 2 * j);
    o0 += f * ov.x;
    o1 += f * ov.y;
  }
  o0 /= den;
  o1 /= den;
  const int64_t pos = posv[b];
  if (r > 0 && 2 * j >= C - r) {
    float cs, sn;
    rope_cs(pos, j - (C - r) / 2, r, theta, &cs, &sn);
    const float x0 = o0, x1 = o1;
    o0 = x0 * cs + x1 * sn;   // rotation by -pos
    o1 = -x0 * sn + x1 * cs;
  }
  T::st(out, ((int64_t)b * nh + h) * C + 2 * j, o0);
  T::st(out, ((int64_t)b * nh + h) * C + 2 * j + 1, o1);
}

// ===========================================================================
// Host launchers
// ===========================================================================
template <class T, int MODE>
static hipError_t dispatch_prefill(const csa_attn_desc& d, const void* q, const void* win,
                                   const void* comp, const int32_t* idx, const float* sink,
                                   void* out, hipStream_t st) {
  typedef typename T::S S;
  const int mb = d.n_heads <= 16 ? 1 : d.n_heads <= 32 ? 2 : 4;
#define CSA_MQA_P(CC, MBB)                                                                      \
  if (d.c == CC && mb == MBB) {                                                                \
    mqa_kernel<T, CC, MBB, MODE><<<(unsigned)d.n, 256, 0, st>>>(                               \
        (const S*)q, (const S*)win, (const S*)comp, idx, nullptr, sink, (S*)out, nullptr,       \
        nullptr, d.n, d.n_heads, d.k, d.m, d.n_win, d.scale, d.qk_norm, d.eps, d.rope_dims,     \
        d.rope_theta, d.n_entries, 1, d.t0);                                                    \
    return hipGetLastError();                                                                   \
  }
  CSA_MQA_P(128, 1) CSA_MQA_P(128, 2) CSA_MQA_P(128, 4)
  CSA_MQA_P(256, 1) CSA_MQA_P(256, 2) CSA_MQA_P(256, 4)
  CSA_MQA_P(512, 1) CSA_MQA_P(512, 2) CSA_MQA_P(512, 4)
#undef CSA_MQA_P
  return hipErrorInvalidValue;
}

hipError_t launch_mqa_prefill(const csa_attn_desc& d, int mode, const void* q, const void* win,
                              const void* comp, const int32_t* idx, const float* sink, void* out,
                              hipStream_t st) {
  if (d.n == 0) return hipSuccess;
  if (d.dtype == CSA_BF16 && (mode == ATTN_DENSE || d.k <= 1024))
    return launch_mqa_prefill_bf16(d, mode, q, win, comp, idx, sink, out, st);
  if (d.dtype == CSA_BF16)
    return mode == ATTN_SPARSE
               ? dispatch_prefill<BF16, MODE_PREFILL_SPARSE>(d, q, win, comp, idx, sink, out, st)
               : dispatch_prefill<BF16, MODE_PREFILL_DENSE>(d, q, win, comp, idx, sink, out, st);
  return mode == ATTN_SPARSE
             ? dispatch_prefill<F32, MODE_PREFILL_SPARSE>(d, q, win, comp, idx, sink, out, st)
             : dispatch_prefill<F32, MODE_PREFILL_DENSE>(d, q, win, comp, idx, sink, out, st);
}

static int decode_nsplit(const csa_attn_desc& d, int mode) {
  const int64_t maxc = (int64_t)d.n_win + (mode == ATTN_SPARSE ? d.k : d.n_entries);
  const int spl = d.dtype == CSA_BF16 ? mqa_decode_bf16_split(mode) : kDecSplit;
  return (int)((maxc + spl - 1) / spl);
}

size_t mqa_decode_ws_bytes(const csa_attn_desc& d, int mode) {
  const size_t S = decode_nsplit(d, mode);
  const size_t rows = (size_t)d.batch * S * d.n_heads;
  return ((rows * d.c * 4 + 255) & ~(size_t)255) + rows * 2 * 4;
}

template <class T, int MODE>
static hipError_t dispatch_decode(const csa_attn_desc& d, const void* q, const void* ring,
                                  const void* cache, const int32_t* idx, const int64_t* pos,
                                  const float* sink, void* out, void* ws, int mode,
                                  hipStream_t st) {
  typedef typename T::S S;
  const int S_ = decode_nsplit(d, mode);
  const size_t rows = (size_t)d.batch * S_ * d.n_heads;
  float* ws_o = (float*)ws;
  float* ws_ml = (float*)((uint8_t*)ws + ((rows * d.c * 4 + 255) & ~(size_t)255));
  dim3 grid(S_, d.batch, (d.n_heads + 15) / 16);
#define CSA_MQA_D(CC)                                                                           \
  if (d.c == CC) {                                                                             \
    mqa_kernel<T, CC, 1, MODE><<<grid, 256, 0, st>>>(                                          \
        (const S*)q, (const S*)ring, (const S*)cache, idx, pos, sink, nullptr, ws_o, ws_ml, 0,  \
        d.n_heads, d.k, d.m, d.n_win, d.scale, d.qk_norm, d.eps, d.rope_dims, d.rope_theta,     \
        d.n_entries, S_, (int64_t)0);                                                           \
  } else
  CSA_MQA_D(128) CSA_MQA_D(256) CSA_MQA_D(512) { return hipErrorInvalidValue; }
#undef CSA_MQA_D
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  mqa_combine_kernel<T><<<dim3(d.batch, d.n_heads), d.c / 2, 0, st>>>(
      ws_o, ws_ml, pos, sink, (S*)out, d.n_heads, d.c, S_, d.rope_dims, d.rope_theta);
  return hipGetLastError();
}

hipError_t launch_mqa_decode(const csa_attn_desc& d, int mode, const void* q, const void* ring,
                             const void* cache, const int32_t* idx, const int64_t* pos,
                             const float* sink, void* out, void* ws, hipStream_t st,
                             EntryMap em, bool kv8) {
  if (d.batch == 0) return hipSuccess;
  if (d.dtype == CSA_BF16) {
    const int S_ = decode_nsplit(d, mode);
    const size_t rows = (size_t)d.batch * S_ * d.n_heads;
    float* ws_o = (float*)ws;
    float2* ws_ml = (float2*)((uint8_t*)ws + ((rows * d.c * 4 + 255) & ~(size_t)255));
    return launch_mqa_decode_bf16(d, mode, q, ring, cache, idx, pos, sink, out, ws_o, ws_ml, S_,
                                  st, em, kv8);
  }
  if (kv8) return hipErrorInvalidValue;
  if (d.dtype == CSA_BF16)
    return mode == ATTN_SPARSE
               ? dispatch_decode<BF16, MODE_DECODE_SPARSE>(d, q, ring, cache, idx, pos, sink, out, ws, mode, st)
               : dispatch_decode<BF16, MODE_DECODE_DENSE>(d, q, ring, cache, idx, pos, sink, out, ws, mode, st);
  return mode == ATTN_SPARSE
             ? dispatch_decode<F32, MODE_DECODE_SPARSE>(d, q, ring, cache, idx, pos, sink, out, ws, mode, st)
             : dispatch_decode<F32, MODE_DECODE_DENSE>(d, q, ring, cache, idx, pos, sink, out, ws, mode, st);
}

}  // namespace csa
