// Deterministic backward of the core sparse (CSA) and dense (HCA) shared-KV
// attention, fp32 ([R] section 4.3: the attention backward gives every unit
// its own accumulation buffer and sums them in a fixed order -- no atomic
// adds; the gradients are the chain rule through eq 19 and 27 with the query
// RMSNorm and RoPE and the output's inverse RoPE of section 2.3.3).
//
// S "slots" (S = min(256, n), fixed by n) each own a contiguous block of query
// tokens and one workgroup.  A slot walks its tokens in order; per token it
//   1. forms the rotated, normalised query q^ and the rotated upstream
//      gradient do' = R(t) dout (the output was rotated back by -t),
//   2. passes once over the candidates (window rows, then selected or visible
//      entries) for the softmax statistics (running max M from the sink,
//      sum D with the sink's term) and the unnormalised output o',
//   3. passes again: p = e^(z-M)/D, dp = do'.kv_j, dz = p (dp - do'.o'/D),
//      dq^ += scale dz kv_j, and each candidate row's gradient
//      sum_h (p_hj do'_h + scale dz_hj q^_h), added into the slot's own buffer
//      (read, add, write: the slot's workgroup is its only writer),
//   4. turns dq^ into dq through the inverse rotation and the RMSNorm's
//      backward, and adds -p_sink (do'.o'/D) to the slot's sink gradients.
// A second kernel sums the slot buffers in slot order.  Nothing depends on
// timing, so results are bitwise repeatable.
#include "csa_common.h"
#include "csa_launch.h"

namespace csa {

namespace {

constexpr int kBT = 32;       // candidates per tile
constexpr int kMaxSlots = 256;

template <int C, int NH>
struct BwdGeo {
  static constexpr int TPH = 256 / NH;  // threads per head (a power of two <= 64)
  static constexpr int DPT = C / TPH;   // channels per thread, even
  static constexpr int LD = C + 4;      // padded LDS row (floats)
  static_assert(TPH <= 64 && DPT >= 2 && DPT % 2 == 0, "unsupported head shape");
};

template <int TPH>
CSA_DEV float head_sum(float v) {
#pragma unroll
  for (int o = TPH / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Candidate j of token t (j < nwin: window position t - nwin + 1 + j; else
// entry slot j - nwin of idx, or entry j - nwin when dense): its row pointer
// and gradient target (window position, or -1 - entry), -1 ... when empty.
struct Cand {
  const float* row;
  int64_t target;  // >= 0: window position; <= -2: entry -(target + 2); -1: none
};

}  // namespace

template <int C, int NH, bool SPARSE>
__global__ __launch_bounds__(256) void mqa_backward_kernel(
    const float* __restrict__ q, const float* __restrict__ win, const float* __restrict__ comp,
    const int32_t* __restrict__ idx, const float* __restrict__ sink,
    const float* __restrict__ dout, float* __restrict__ dq, float* __restrict__ slot_win,
    float* __restrict__ slot_comp, float* __restrict__ slot_sink, int64_t n, int k, int m,
    int n_win, int64_t n_entries, float scale, int qk_norm, float eps, int r, float theta,
    int nslots, int64_t wrows) {
  typedef BwdGeo<C, NH> G;
  constexpr int TPH = G::TPH, DPT = G::DPT, LD = G::LD;
  __shared__ float qh_s[NH * C];   // q^ (rotated, normalised query), all heads
  __shared__ float do_s[NH * C];   // do' = R(t) dout
  __shared__ __align__(16) float tile[kBT * LD];
  __shared__ float zs[NH * kBT];   // logits, then p
  __shared__ float dzs[NH * kBT];  // dz
  __shared__ Cand cands[kBT];
  __shared__ float2 rope_tab[C / 2];
  __shared__ float hstat[NH][3];  // per head: M, 1/D, do'.o'

  const int tid = threadIdx.x;
  const int h = tid / TPH, l = tid % TPH;
  const int d0 = l * DPT;  // this thread's channels of head h
  const int slot = blockIdx.x;
  const int64_t t_beg = n * slot / nslots, t_end = n * (slot + 1) / nslots;
  const int64_t wbase = max64(0, t_beg - n_win + 1);  // first window row of the slot buffer
  float* my_win = slot_win + (int64_t)slot * wrows * C;
  float* my_comp = slot_comp + (int64_t)slot * n_entries * C;
  const float sl = sink[h];
  float dsink_acc = 0.f;

  for (int64_t t = t_beg; t < t_end; ++t) {
    // ---- 1. q^ and do' for this thread's channels
    for (int p = tid; p < r / 2; p += 256) {
      float cs, sn;
      rope_cs(t, p, r, theta, &cs, &sn);
      rope_tab[p] = make_float2(cs, sn);
    }
    float qv[DPT], nq[DPT], dv[DPT];
    const float* qrow = q + (t * NH + h) * C + d0;
    const float* grow = dout + (t * NH + h) * C + d0;
#pragma unroll
    for (int i = 0; i < DPT; ++i) {
      qv[i] = qrow[i];
      dv[i] = grow[i];
    }
    float rr = 1.f;
    if (qk_norm) {
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < DPT; ++i) ss += qv[i] * qv[i];
      ss = head_sum<TPH>(ss);
      rr = sqrtf(ss / (float)C + eps);
    }
#pragma unroll
    for (int i = 0; i < DPT; ++i) nq[i] = qv[i] / rr;
    __syncthreads();  // rope_tab
    float qh[DPT], dov[DPT];
#pragma unroll
    for (int i = 0; i < DPT; i += 2) {
      const int ch = d0 + i;
      float cs = 1.f, sn = 0.f;
      if (ch >= C - r) {
        const float2 v = rope_tab[(ch - (C - r)) >> 1];
        cs = v.x;
        sn = v.y;
      }
      qh[i] = nq[i] * cs - nq[i + 1] * sn;  // rotate by +t
      qh[i + 1] = nq[i] * sn + nq[i + 1] * cs;
      dov[i] = dv[i] * cs - dv[i + 1] * sn;
      dov[i + 1] = dv[i] * sn + dv[i + 1] * cs;
    }
#pragma unroll
    for (int i = 0; i < DPT; ++i) {
      qh_s[h * C + d0 + i] = qh[i];
      do_s[h * C + d0 + i] = dov[i];
    }
    // ---- candidate list geometry
    const int64_t nwin = min64(n_win, t + 1);
    const int64_t ncomp = SPARSE ? (int64_t)k : min64((t + 1) / m, n_entries);
    const int64_t ncand = nwin + ncomp;
    const int ntiles = (int)((ncand + kBT - 1) / kBT);

    auto load_tile = [&](int ti) {
      if (tid < kBT) {
        const int64_t j = (int64_t)ti * kBT + tid;
        Cand c{win, -1};
        if (j < nwin) {
          const int64_t pos = t - nwin + 1 + j;
          c.row = win + pos * C;
          c.target = pos;
        } else if (j < ncand) {
          const int64_t e = SPARSE ? (int64_t)idx[t * k + (j - nwin)] : j - nwin;
          if (e >= 0 && e < n_entries) {
            c.row = comp + e * C;
            c.target = -2 - e;
          }
        }
        cands[tid] = c;
      }
      __syncthreads();
      constexpr int F4 = kBT * C / 4;  // float4s in a tile
      for (int f = tid; f < F4; f += 256) {
        const int j = f / (C / 4), c4 = f % (C / 4);
        const float4 v = cands[j].target != -1 ? *(const float4*)(cands[j].row + 4 * c4)
                                               : make_float4(0.f, 0.f, 0.f, 0.f);
        *(float4*)(tile + j * LD + 4 * c4) = v;
      }
      __syncthreads();
    };
    // logits of (head hp, candidate jp) pairs: thread tid covers pairs
    // tid, tid + 256, ... of the NH x kBT grid
    auto pair_dot = [&](const float* a_s, int hp, int jp) {
      const float* a = a_s + hp * C;
      const float* b = tile + jp * LD;
      float s = 0.f;
#pragma unroll 8
      for (int c = 0; c < C; ++c) s = fmaf(a[c], b[c], s);
      return s;
    };

    // ---- 2. statistics and o'
    float M = sl, Dsum = 1.f;  // the sink's term e^(sink - M)
    float o[DPT];
#pragma unroll
    for (int i = 0; i < DPT; ++i) o[i] = 0.f;
    for (int ti = 0; ti < ntiles; ++ti) {
      load_tile(ti);
      for (int pr = tid; pr < NH * kBT; pr += 256) {
        const int hp = pr / kBT, jp = pr % kBT;
        zs[pr] = cands[jp].target != -1 ? scale * pair_dot(qh_s, hp, jp) : -INFINITY;
      }
      __syncthreads();
      float tm = M;
      for (int j = 0; j < kBT; ++j) tm = fmaxf(tm, zs[h * kBT + j]);
      const float a = __expf(M - tm);
      Dsum *= a;
#pragma unroll
      for (int i = 0; i < DPT; ++i) o[i] *= a;
      for (int j = 0; j < kBT; ++j) {
        const float e = __expf(zs[h * kBT + j] - tm);  // 0 for an empty slot
        Dsum += e;
#pragma unroll
        for (int i = 0; i < DPT; ++i) o[i] = fmaf(e, tile[j * LD + d0 + i], o[i]);
      }
      M = tm;
      __syncthreads();  // before the next tile overwrites tile / zs
    }
    const float invD = 1.f / Dsum;
    float dd = 0.f;  // do' . o' (o' normalised)
#pragma unroll
    for (int i = 0; i < DPT; ++i) dd = fmaf(dov[i], o[i] * invD, dd);
    dd = head_sum<TPH>(dd);
    // every thread of head h holds M, invD, dd; publish them per head
    if (l == 0) {
      hstat[h][0] = M;
      hstat[h][1] = invD;
      hstat[h][2] = dd;
    }
    dsink_acc -= __expf(sl - M) * invD * dd;

    // ---- 3. gradients
    float dqh[DPT];
#pragma unroll
    for (int i = 0; i < DPT; ++i) dqh[i] = 0.f;
    for (int ti = 0; ti < ntiles; ++ti) {
      load_tile(ti);  // its barriers also publish hstat
      for (int pr = tid; pr < NH * kBT; pr += 256) {
        const int hp = pr / kBT, jp = pr % kBT;
        float p = 0.f, dz = 0.f;
        if (cands[jp].target != -1) {
          const float z = scale * pair_dot(qh_s, hp, jp);
          p = __expf(z - hstat[hp][0]) * hstat[hp][1];
          const float dp = pair_dot(do_s, hp, jp);
          dz = p * (dp - hstat[hp][2]);
        }
        zs[pr] = p;
        dzs[pr] = dz;
      }
      __syncthreads();
      for (int j = 0; j < kBT; ++j) {
        const float g = scale * dzs[h * kBT + j];
#pragma unroll
        for (int i = 0; i < DPT; ++i) dqh[i] = fmaf(g, tile[j * LD + d0 + i], dqh[i]);
      }
      // candidate rows' gradients: thread tid takes channels of row tid / 8
      {
        constexpr int CPT8 = C / 8;
        const int j = tid / 8, c0 = (tid % 8) * CPT8;
        const Cand cj = cands[j];
        if (cj.target != -1) {
          float* dst = cj.target >= 0 ? my_win + (cj.target - wbase) * C
                                      : my_comp + (-2 - cj.target) * C;
#pragma unroll 4
          for (int c = c0; c < c0 + CPT8; ++c) {
            float g = 0.f;
#pragma unroll
            for (int hh = 0; hh < NH; ++hh)
              g = fmaf(zs[hh * kBT + j], do_s[hh * C + c], fmaf(scale * dzs[hh * kBT + j],
                                                               qh_s[hh * C + c], g));
            dst[c] += g;
          }
        }
      }
      __syncthreads();  // the slot buffer rows and LDS before the next tile
    }
    // ---- 4. dq through the inverse rotation and the RMSNorm backward
    float dn[DPT];
#pragma unroll
    for (int i = 0; i < DPT; i += 2) {
      const int ch = d0 + i;
      float cs = 1.f, sn = 0.f;
      if (ch >= C - r) {
        const float2 v = rope_tab[(ch - (C - r)) >> 1];
        cs = v.x;
        sn = v.y;
      }
      dn[i] = dqh[i] * cs + dqh[i + 1] * sn;  // rotate by -t
      dn[i + 1] = -dqh[i] * sn + dqh[i + 1] * cs;
    }
    float* dqrow = dq + (t * NH + h) * C + d0;
    if (qk_norm) {
      float dm = 0.f;
#pragma unroll
      for (int i = 0; i < DPT; ++i) dm = fmaf(dn[i], nq[i], dm);
      dm = head_sum<TPH>(dm) / (float)C;
#pragma unroll
      for (int i = 0; i < DPT; ++i) dqrow[i] = (dn[i] - nq[i] * dm) / rr;
    } else {
#pragma unroll
      for (int i = 0; i < DPT; ++i) dqrow[i] = dn[i];
    }
    __syncthreads();  // qh_s / do_s / rope_tab are rewritten by the next token
  }
  if (l == 0) slot_sink[slot * NH + h] = dsink_acc;
}

__global__ void bwd_zero_kernel(float4* __restrict__ p, int64_t n4) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// Fixed slot order: window row j sums the slots whose token blocks reach it.
__global__ void bwd_reduce_kernel(const float* __restrict__ slot_win,
                                  const float* __restrict__ slot_comp,
                                  const float* __restrict__ slot_sink, float* __restrict__ dwin,
                                  float* __restrict__ dcomp, float* __restrict__ dsink, int64_t n,
                                  int64_t n_entries, int C, int NH, int n_win, int nslots,
                                  int64_t wrows) {
  const int64_t tot_w = n * C, tot_c = n_entries * C;
  for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < tot_w + tot_c + NH;
       x += (int64_t)gridDim.x * blockDim.x) {
    float s = 0.f;
    if (x < tot_w) {
      const int64_t j = x / C, c = x % C;
      for (int sl = 0; sl < nslots; ++sl) {
        const int64_t tb = n * sl / nslots, te = n * (sl + 1) / nslots;
        const int64_t wb = max64(0, tb - n_win + 1);
        if (te > tb && j >= wb && j < te) s += slot_win[((int64_t)sl * wrows + (j - wb)) * C + c];
      }
      dwin[x] = s;
    } else if (x < tot_w + tot_c) {
      const int64_t y = x - tot_w;
      for (int sl = 0; sl < nslots; ++sl) s += slot_comp[(int64_t)sl * tot_c + y];
      dcomp[y] = s;
    } else {
      const int hh = (int)(x - tot_w - tot_c);
      for (int sl = 0; sl < nslots; ++sl) s += slot_sink[sl * NH + hh];
      dsink[hh] = s;
    }
  }
}

static int bwd_slots(int64_t n) { return (int)(n < kMaxSlots ? (n > 0 ? n : 1) : kMaxSlots); }
static int64_t bwd_wrows(const csa_attn_desc& d) {
  const int S = bwd_slots(d.n);
  return (d.n + S - 1) / S + d.n_win - 1;
}

bool mqa_backward_supported(const csa_attn_desc& d) {
  const int64_t w = (int64_t)d.n_heads * d.c;
  return d.dtype == CSA_F32 && (d.c == 128 || d.c == 256 || d.c == 512) &&
         (d.n_heads == 4 || d.n_heads == 8 || d.n_heads == 16) && w >= 512 && w <= 2048 &&
         d.t0 == 0;
}

size_t mqa_backward_ws_bytes(const csa_attn_desc& d) {
  const size_t S = bwd_slots(d.n);
  const size_t a = S * bwd_wrows(d) * d.c * 4, b = S * d.n_entries * d.c * 4,
               c = S * d.n_heads * 4;
  return ((a + 255) & ~(size_t)255) + ((b + 255) & ~(size_t)255) + ((c + 255) & ~(size_t)255);
}

hipError_t launch_mqa_backward(const csa_attn_desc& d, int mode, const float* q, const float* win,
                               const float* comp, const int32_t* idx, const float* sink,
                               const float* dout, float* dq, float* dwin, float* dcomp,
                               float* dsink, void* ws, hipStream_t st) {
  const int S = bwd_slots(d.n);
  const int64_t wrows = bwd_wrows(d);
  const size_t a = (size_t)S * wrows * d.c * 4, b = (size_t)S * d.n_entries * d.c * 4;
  float* slot_win = (float*)ws;
  float* slot_comp = (float*)((uint8_t*)ws + ((a + 255) & ~(size_t)255));
  float* slot_sink =
      (float*)((uint8_t*)ws + ((a + 255) & ~(size_t)255) + ((b + 255) & ~(size_t)255));
  const int64_t zero4 = (int64_t)(((a + 255) & ~(size_t)255) + ((b + 255) & ~(size_t)255)) / 16;
  bwd_zero_kernel<<<1024, 256, 0, st>>>((float4*)ws, zero4);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (d.n == 0) return hipSuccess;
#define CSA_BWD(CC, HH)                                                                        \
  if (d.c == CC && d.n_heads == HH) {                                                          \
    if (mode == ATTN_SPARSE)                                                                   \
      mqa_backward_kernel<CC, HH, true><<<S, 256, 0, st>>>(                                    \
          q, win, comp, idx, sink, dout, dq, slot_win, slot_comp, slot_sink, d.n, d.k, d.m,     \
          d.n_win, d.n_entries, d.scale, d.qk_norm, d.eps, d.rope_dims, d.rope_theta, S, wrows); \
    else                                                                                       \
      mqa_backward_kernel<CC, HH, false><<<S, 256, 0, st>>>(                                   \
          q, win, comp, idx, sink, dout, dq, slot_win, slot_comp, slot_sink, d.n, d.k, d.m,     \
          d.n_win, d.n_entries, d.scale, d.qk_norm, d.eps, d.rope_dims, d.rope_theta, S, wrows); \
  } else
  CSA_BWD(128, 4) CSA_BWD(128, 8) CSA_BWD(128, 16) CSA_BWD(256, 4) CSA_BWD(256, 8)
  CSA_BWD(512, 4) { return hipErrorInvalidValue; }
#undef CSA_BWD
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t tot = d.n * d.c + d.n_entries * d.c + d.n_heads;
  const unsigned g = (unsigned)((tot + 255) / 256 < 8192 ? (tot + 255) / 256 : 8192);
  bwd_reduce_kernel<<<g, 256, 0, st>>>(slot_win, slot_comp, slot_sink, dwin, dcomp, dsink, d.n,
                                       d.n_entries, d.c, d.n_heads, d.n_win, S, wrows);
  return hipGetLastError();
}

}  // namespace csa
