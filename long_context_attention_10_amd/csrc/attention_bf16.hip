// bf16 shared-KV MQA prefill on gfx950 (the dominant kernel of CSA prefill).
//
// Citation keys: [R] = page "DeepSeek-V4 技术解读报告" (juejin.cn), section
// 2.3.1 eq 18-19 (shared KV: each entry is both key and value), 2.3.3 (QK
// RMSNorm, partial RoPE with the output rotated back, sliding window, sink
// logits of eq 27); [A] = page "DeepSeek-V4：算法架构" (1zeryu.github.io),
// Sparse Attention candidate assembly and HCA selection rule.
//
// One workgroup per query token (4 waves x 16 heads = 64 heads, head dim C).
// Each wave owns its 16 heads over the FULL head dim, so logits, the online
// softmax and P never leave the wave's registers:
//   S^T[cand, head] = K[cand, :] . Q[head, :]^T      16x16x32 MFMA, A = K rows
//   O^T[ch, head]  += V^T[ch, cand] . P^T[cand, head] 16x16x32 MFMA, B = P
// The candidate rows (K = V) are staged in LDS once per 32-candidate tile by
// direct global->LDS loads into a double buffer (the next tile streams in while
// the current one is consumed); K fragments are plain 16-byte LDS reads and V
// fragments use the LDS transpose read, so no copy is transposed by hand.
// q and the output go through LDS so that HBM sees whole-row transfers.
// The running max starts at the sink logit and the running sum at 1, which
// adds exp(sink) to the denominator exactly once.  The max is only raised
// (and O rescaled) when a tile's logits exceed it by more than 8 in log2
// units, which keeps the rescale off the common path without overflow risk.
#include "csa_common.h"
#include "csa_launch.h"

namespace csa {


namespace {

constexpr int kT = 32;            // candidates per tile
constexpr int kPad = 32;          // bytes of padding per 1 KiB LDS burst
constexpr int kMaxK = 1024;       // index slots staged in LDS

template <int C>
struct Geo {
  static constexpr int ROW = C * 2;                       // bytes per row
  static constexpr int RPI = 1024 / ROW;                  // rows per 1 KiB DMA burst
  static constexpr int BURST = 1024 + kPad;               // LDS bytes per burst
  static constexpr int TILE = (kT / RPI) * BURST;         // LDS bytes per tile
  static constexpr int QBYTES = (64 / RPI) * BURST;       // q / output staging
  static constexpr int BUF = (2 * TILE > QBYTES) ? 2 * TILE : QBYTES;
  CSA_DEV static int off(int r) { return (r / RPI) * BURST + (r % RPI) * ROW; }
};


}  // namespace


// O accumulators are split in two halves of at most 16 blocks: the compiler
// keeps fully unrolled 16-entry arrays in registers, not 32-entry ones.
template <int C>
struct OAcc {
  static constexpr int NCB = C / 16;  // 16-channel output blocks
  static constexpr int NLO = NCB > 16 ? 16 : NCB;
  static constexpr int NHI = NCB > 16 ? NCB - 16 : 1;
  f32x4_t lo[NLO], hi[NHI];
};

// Candidate slot permutation.  Lane group lg (lanes 16*lg..16*lg+15) holds,
// after the logits, the 8 tile rows pi(lg, h, i) = 16*(lg/2) + 8*h + 4*(lg%2) + i
// (h = 0, 1; i = 0..3); those rows are also its PV reduction slots 8*lg+4*h+i.
// With 1056-byte LDS rows (8 banks apart) both the 16-byte K reads (rows
// pi(lc/4, b, lc%4) for lanes lc) and the transpose reads (4 consecutive
// rows per 16-lane group) touch distinct banks.
CSA_DEV int slot_pi(int g, int h, int i) { return 16 * (g >> 1) + 8 * h + 4 * (g & 1) + i; }

// Logits of one 32-candidate tile for this wave's 16 heads, S^T = K Q^T, in
// log2 units; z[4b+i] is tile row pi(lg, b, i) for head lc, -inf where the
// row is masked.  Returns the per-head maximum over the tile.
template <int C>
CSA_DEV float tile_logits(const uint8_t* kv, const int* vflags, const bf16x8_t* qf, float sl2,
                          int koff0, int koff1, int lg, float (&z)[8]) {
  constexpr int NKG = C / 32;
  // block b's A rows are K rows pi(lc/4, b, lc%4).  The fragments of the
  // next D-1 k-groups are read while a k-group's products issue, so the LDS
  // latency overlaps the matrix cores.
  constexpr int D = 3;  // k-groups of fragments in flight
  f32x4_t s[2] = {f32x4_t{}, f32x4_t{}};
  bf16x8_t a0[D], a1[D];
#pragma unroll
  for (int g = 0; g < D - 1; ++g) {
    a0[g] = *(const bf16x8_t*)(kv + koff0 + g * 64);
    a1[g] = *(const bf16x8_t*)(kv + koff1 + g * 64);
  }
#pragma unroll
  for (int g = 0; g < NKG; ++g) {
    if (g + D - 1 < NKG) {
      a0[(g + D - 1) % D] = *(const bf16x8_t*)(kv + koff0 + (g + D - 1) * 64);
      a1[(g + D - 1) % D] = *(const bf16x8_t*)(kv + koff1 + (g + D - 1) * 64);
    }
    s[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[g % D], qf[g], s[0], 0, 0, 0);
    s[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[g % D], qf[g], s[1], 0, 0, 0);
  }
  float mx = -INFINITY;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int4 vf = *(const int4*)&vflags[slot_pi(lg, b, 0)];  // rows pi(lg, b, 0..3)
    const int vfl[4] = {vf.x, vf.y, vf.z, vf.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float zz = vfl[i] ? s[b][i] * sl2 : -INFINITY;
      z[4 * b + i] = zz;
      mx = fmaxf(mx, zz);
    }
  }
  return xlane_max(mx);
}

// One 32-candidate tile for this wave's 16 heads over the full head dim: the
// logits, the online softmax update (log2 units), O^T += V^T P^T.
template <int C>
CSA_DEV void mqa_tile(const uint8_t* kv, const int* vflags, const bf16x8_t* qf, OAcc<C>& o,
                      float& run_m, float& run_l, float sl2, int koff0, int koff1, int troff0,
                      int troff1, int lg) {
  typedef OAcc<C> A;
  float z[8];
  const float mx = tile_logits<C>(kv, vflags, qf, sl2, koff0, koff1, lg, z);
  if (__any(mx > run_m + 8.f)) {  // wave-uniform rescale of O
    const float nm = fmaxf(run_m, mx);
    const float alpha = __builtin_amdgcn_exp2f(run_m - nm);
    run_l *= alpha;
    run_m = nm;
#pragma unroll
    for (int cb = 0; cb < A::NLO; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) o.lo[cb][i] *= alpha;
    if constexpr (A::NCB > 16) {
#pragma unroll
      for (int cb = 0; cb < A::NHI; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i) o.hi[cb][i] *= alpha;
    }
  }
  f32x8_t p;
  float ps = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    p[j] = __builtin_amdgcn_exp2f(z[j] - run_m);
    ps += p[j];
  }
  run_l += xlane_sum(ps);
  const bf16x8_t pb = __builtin_convertvector(p, bf16x8_t);  // B operand, slots 8*lg+j

  // O^T += V^T P^T over the 16-channel blocks; V^T fragments by transpose read:
  // lane (lg, lc) reads row pi(lg, h, lc/4), channels cb*16 + 4*(lc%4) .. +3,
  // and receives V[pi(lg, h, j)][cb*16 + lc] for j = 0..3.
  auto pv = [&](int cb, f32x4_t& acc) {
    const bf16x4_t x0 =
        __builtin_amdgcn_ds_read_tr16_b64_v4bf16((CSA_LDS bf16x4_t*)(kv + troff0 + cb * 32));
    const bf16x4_t x1 =
        __builtin_amdgcn_ds_read_tr16_b64_v4bf16((CSA_LDS bf16x4_t*)(kv + troff1 + cb * 32));
    const bf16x8_t a = __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, acc, 0, 0, 0);
  };
#pragma unroll
  for (int cb = 0; cb < A::NLO; ++cb) pv(cb, o.lo[cb]);
  if constexpr (A::NCB > 16) {
#pragma unroll
    for (int cb = 0; cb < A::NHI; ++cb) pv(A::NLO + cb, o.hi[cb]);
  }
}

// Channel-split variant for one query's 64 heads in a workgroup.  Wave w
// still forms the logits and the softmax of heads 16w..16w+15, but the PV
// product of the tile is split by channels: wave w accumulates O^T for its
// C/4 channels and all 64 heads.  Every wave's P^T operand (and, when a
// wave raised its running max, the rescale factors of its heads) goes
// through LDS, so each wave transposes a quarter of the tile instead of all
// of it; the logits still read each K row once per wave.
struct Xchg {
  bf16x8_t p[4][64];  // P^T B operands, [wave][lane]
  float alpha[64];    // O rescale factor per head, valid where flag is set
  int flag[4];        // wave w raised the running max of its heads
  float l[64];        // running sums at the end
};

template <int C>
struct OSplit {
  static constexpr int NCB = C / 64;  // 16-channel blocks per wave
  f32x4_t h[4][NCB];                  // [head block][channel block]
};

// Logit side of a channel-split tile: this wave's logits and online softmax
// (heads 16*sw..16*sw+15), published to `xc` as the P^T operand, with the
// rescale factors when the running max was raised.
template <int C>
CSA_DEV void publish_p(const uint8_t* kv, const int* vflags, const bf16x8_t* qf, float& run_m,
                       float& run_l, float sl2, int koff0, int koff1, int lane, int lg, int sw,
                       Xchg& xc) {
  float z[8];
  const float mx = tile_logits<C>(kv, vflags, qf, sl2, koff0, koff1, lg, z);
  const bool resc = __any(mx > run_m + 8.f);
  if (resc) {  // wave-uniform
    const float nm = fmaxf(run_m, mx);
    const float alpha = __builtin_amdgcn_exp2f(run_m - nm);
    run_l *= alpha;
    run_m = nm;
    if (lg == 0) xc.alpha[sw * 16 + lane] = alpha;
  }
  if (lane == 0) xc.flag[sw] = resc;
  f32x8_t p;
  float ps = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    p[j] = __builtin_amdgcn_exp2f(z[j] - run_m);
    ps += p[j];
  }
  run_l += xlane_sum(ps);
  xc.p[sw][lane] = __builtin_convertvector(p, bf16x8_t);
}

// PV side of a channel-split tile: rescale where a logit wave raised its
// max, then O^T += V^T P^T over channel quarter cq for all 64 heads
// (transpose reads as in mqa_tile, offset to the quarter); one V^T fragment
// serves the four head blocks, and the next DV-1 fragments are in flight.
template <int C>
CSA_DEV void pv_quarter(const uint8_t* kv, const Xchg& xc, OSplit<C>& o, int troff0, int troff1,
                        int lane, int cq) {
  typedef OSplit<C> A;
  const int4 fl = *(const int4*)xc.flag;
  const int fla[4] = {fl.x, fl.y, fl.z, fl.w};
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    if (__builtin_amdgcn_readfirstlane(fla[hb])) {
      const float a = xc.alpha[hb * 16 + (lane & 15)];
#pragma unroll
      for (int cb = 0; cb < A::NCB; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i) o.h[hb][cb][i] *= a;
    }
  }
  bf16x8_t pb[4];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) pb[hb] = xc.p[hb][lane];
  const int cofs = cq * A::NCB * 32;
  constexpr int DV = 3;
  bf16x8_t va[DV];
  auto vread = [&](int cb) {
    const bf16x4_t x0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (CSA_LDS bf16x4_t*)(kv + troff0 + cofs + cb * 32));
    const bf16x4_t x1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (CSA_LDS bf16x4_t*)(kv + troff1 + cofs + cb * 32));
    return __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
  };
#pragma unroll
  for (int cb = 0; cb < DV - 1 && cb < A::NCB; ++cb) va[cb] = vread(cb);
#pragma unroll
  for (int cb = 0; cb < A::NCB; ++cb) {
    if (cb + DV - 1 < A::NCB) va[(cb + DV - 1) % DV] = vread(cb + DV - 1);
#pragma unroll
    for (int hb = 0; hb < 4; ++hb)
      o.h[hb][cb] =
          __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[cb % DV], pb[hb], o.h[hb][cb], 0, 0, 0);
  }
}

template <int C>
CSA_DEV void mqa_tile_split(const uint8_t* kv, const int* vflags, const bf16x8_t* qf,
                            OSplit<C>& o, float& run_m, float& run_l, float sl2, int koff0,
                            int koff1, int troff0, int troff1, int lane, int lg, int wave,
                            Xchg& xc) {
  publish_p<C>(kv, vflags, qf, run_m, run_l, sl2, koff0, koff1, lane, lg, wave, xc);
  __syncthreads();  // P^T operands and rescale factors of all heads
  pv_quarter<C>(kv, xc, o, troff0, troff1, lane, wave);
}

// q prologue: per-head RMSNorm over the row held by the 4 lane groups, RoPE
// of the last r channels from the token's angle table, bf16 MFMA operands.
template <int C>
CSA_DEV void q_prologue(const uint4* qraw, bf16x8_t* qf, const float2* rtab, int qk_norm, float eps,
                        int r, int lg) {
  constexpr int NKG = C / 32;
  float ss = 0.f;
#pragma unroll
  for (int g = 0; g < NKG; ++g) {
    float v[8];
    chunk_to_f32<BF16>(qraw[g], v);
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += v[e] * v[e];
  }
  ss = xlane_sum(ss);
  const float inv = qk_norm ? rsqrtf(ss / (float)C + eps) : 1.f;
#pragma unroll
  for (int g = 0; g < NKG; ++g) {
    float v[8];
    chunk_to_f32<BF16>(qraw[g], v);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] *= inv;
    if (r > 0) {
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const int ch = g * 32 + lg * 8 + e;
        if (ch >= C - r) {
          const float2 cs = rtab[(ch - (C - r)) >> 1];
          const float x0 = v[e], x1 = v[e + 1];
          v[e] = x0 * cs.x - x1 * cs.y;
          v[e + 1] = x0 * cs.y + x1 * cs.x;
        }
      }
    }
    qf[g] = __builtin_bit_cast(bf16x8_t, f32_to_chunk<BF16>(v));
  }
}

// Lane L < 8 of wave w resolves tile row (w + 4*(L / RPI)) * RPI + L % RPI
// (address and validity flag); each 1 KiB burst's DMA then takes its row
// address from that lane (readlane), so the gather costs one LDS index read
// and a few scalar moves per row.  `row_of(j)` gives (row pointer, valid) for
// candidate j of the tile's range.
template <int C, class RowOf>
CSA_DEV void issue_tile_rows(uint8_t* base, int* vflags, int lane, int wave, int64_t j0,
                             RowOf row_of) {
  typedef Geo<C> G;
  constexpr int BPW = kT / G::RPI / 4;  // bursts (1 KiB each) per wave
  constexpr int LPR = 64 / G::RPI;      // lanes per row within a burst
  const uint16_t* rp = nullptr;
  if (lane < BPW * G::RPI) {
    const int row = (wave + 4 * (lane / G::RPI)) * G::RPI + lane % G::RPI;
    bool ok;
    rp = row_of(j0 + row, ok);
    vflags[row] = ok;
  }
  const uint32_t ra_lo = (uint32_t)(size_t)rp, ra_hi = (uint32_t)((size_t)rp >> 32);
#pragma unroll
  for (int u = 0; u < BPW; ++u) {
    uint32_t lo, hi;
    if constexpr (G::RPI == 1) {
      lo = __builtin_amdgcn_readlane(ra_lo, u);
      hi = __builtin_amdgcn_readlane(ra_hi, u);
    } else {
      const int src = u * G::RPI + lane / LPR;
      lo = __shfl((int)ra_lo, src, 64);
      hi = __shfl((int)ra_hi, src, 64);
    }
    const uint8_t* g = (const uint8_t*)(size_t)(((uint64_t)hi << 32) | lo) + (lane % LPR) * 16;
    lds_dma16(g, base + (wave + 4 * u) * G::BURST);
  }
}

// ---------------------------------------------------------------------------
// Prefill: one workgroup per query token.  XCD-aware order (workgroup b runs
// on die b % 8): the tokens form 16 contiguous ranges and die x takes ranges
// x and 15 - x, so a die's L2 keeps the window rows its consecutive tokens
// share, and every die gets early tokens (fewer visible entries) and late
// ones alike.  The first tile holds only window rows whenever
// the window covers it; its gather then starts before the index row is in.
// The running max starts at the sink logit and the running sum at 1, which
// adds exp(sink) to the denominator exactly once.  The output goes through
// LDS so that HBM sees whole-row stores.
// ---------------------------------------------------------------------------
template <int C, bool SPARSE>
__global__ __launch_bounds__(256, 2) void mqa_prefill_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ win,
    const uint16_t* __restrict__ comp, const int32_t* __restrict__ idx,
    const float* __restrict__ sink, uint16_t* __restrict__ out, int64_t n, int nh, int k, int m,
    int n_win, float scale, int qk_norm, float eps, int r, float theta, int64_t n_entries,
    int64_t t0) {
  typedef Geo<C> G;
  typedef OSplit<C> A;
  constexpr int NKG = C / 32;
  __shared__ __align__(16) uint8_t smem[G::BUF];
  __shared__ __align__(16) Xchg xc;
  __shared__ __align__(16) int valid[2][kT];
  __shared__ int sidx[SPARSE ? kMaxK : 1];
  __shared__ float2 rope_tab[C / 2];  // (cos, sin) of this token's RoPE pairs

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int lc = lane & 15, lg = lane >> 4;
  const int head = wave * 16 + lc;
  const int64_t per = (n + 15) >> 4;  // tokens per range
  const int die = blockIdx.x & 7;
  const int64_t bi = blockIdx.x >> 3;
  const int64_t t = bi < per ? die * per + bi : (15 - die) * per + (bi - per);
  if (t >= n) return;

  // q rows first, so that the first tile's gather overlaps their load
  uint4 qraw[NKG];
  {
    const uint16_t* qh = q + (t * nh + (head < nh ? head : 0)) * C + lg * 8;
#pragma unroll
    for (int g = 0; g < NKG; ++g) qraw[g] = *(const uint4*)(qh + g * 32);
  }
  // row t is the token at position pt = t0 + t; win row 0 is position w0
  const int64_t pt = t0 + t, w0 = max64(t0 - n_win + 1, 0);
  const int nwin = (int)min64(n_win, pt + 1);
  const int64_t ncand = nwin + (SPARSE ? (int64_t)k : min64((pt + 1) / m, n_entries));
  const int ntiles = (int)((ncand + kT - 1) / kT);
  auto issue_tile = [&](int ti, int buf) {
    issue_tile_rows<C>(smem + buf * G::TILE, valid[buf], lane, wave, (int64_t)ti * kT,
                       [&](int64_t j, bool& ok) -> const uint16_t* {
                         ok = false;
                         if (j >= ncand) return win;  // a valid row for masked candidates
                         if (j < nwin) { ok = true; return win + (pt - nwin + 1 + j - w0) * C; }
                         const int64_t e = SPARSE ? (int64_t)sidx[j - nwin] : j - nwin;
                         if (e < 0 || e >= n_entries) return win;
                         ok = true;
                         return comp + e * C;
                       });
  };
  const bool early0 = nwin >= kT;  // tile 0 is window rows only
  if (early0) issue_tile(0, 0);
  if (SPARSE)
    for (int j = tid; j < k; j += 256) sidx[j] = idx[t * k + j];
  for (int p = tid; p < r / 2; p += 256) {
    float cs, sn;
    rope_cs(pt, p, r, theta, &cs, &sn);
    rope_tab[p] = make_float2(cs, sn);
  }
  __syncthreads();  // sidx and rope_tab are visible
  if (!early0) issue_tile(0, 0);

  bf16x8_t qf[NKG];
  q_prologue<C>(qraw, qf, rope_tab, qk_norm, eps, r, lg);
  constexpr float LOG2E = 1.4426950408889634f;
  float run_m = (head < nh ? sink[head] : 0.f) * LOG2E, run_l = 1.f;
  A o;
#pragma unroll
  for (int hb = 0; hb < 4; ++hb)
#pragma unroll
    for (int cb = 0; cb < A::NCB; ++cb) o.h[hb][cb] = f32x4_t{};
  const int koff0 = G::off(slot_pi(lc >> 2, 0, lc & 3)) + lg * 16;
  const int koff1 = G::off(slot_pi(lc >> 2, 1, lc & 3)) + lg * 16;
  const int troff0 = G::off(slot_pi(lg, 0, lc >> 2)) + 8 * (lc & 3);
  const int troff1 = G::off(slot_pi(lg, 1, lc >> 2)) + 8 * (lc & 3);
  wait_vmem();  // tile 0 (and q) have landed
  __syncthreads();
  for (int ti = 0; ti < ntiles; ++ti) {
    const int buf = ti & 1;
    if (ti + 1 < ntiles) issue_tile(ti + 1, buf ^ 1);
    mqa_tile_split<C>(smem + buf * G::TILE, valid[buf], qf, o, run_m, run_l, scale * LOG2E,
                      koff0, koff1, troff0, troff1, lane, lg, wave, xc);
    wait_vmem();
    __syncthreads();
  }

  // epilogue: block (hb, cb), element i = O[16*hb + lc][wave*C/4 + cb*16 + 4*lg + i]
  if (lg == 0) xc.l[head] = run_l;
  __syncthreads();
  uint8_t* ostage = smem;  // [head][C] bf16, padded like the tiles
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    const float inv = 1.f / xc.l[hb * 16 + lc];
#pragma unroll
    for (int cb = 0; cb < A::NCB; ++cb) {
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = o.h[hb][cb][i] * inv;
      const int ch0 = wave * (C / 4) + cb * 16 + 4 * lg;
      if (r > 0 && ch0 >= C - r) {
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          const float2 cs = rope_tab[(ch0 + i - (C - r)) >> 1];
          const float x0 = v[i], x1 = v[i + 1];
          v[i] = x0 * cs.x + x1 * cs.y;  // rotate by -t
          v[i + 1] = -x0 * cs.y + x1 * cs.x;
        }
      }
      const uint32_t w0 = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
      const uint32_t w1 = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
      *(uint2*)(ostage + G::off(hb * 16 + lc) + ch0 * 2) = make_uint2(w0, w1);
    }
  }
  __syncthreads();
  uint16_t* orow = out + t * (int64_t)nh * C;
  const int chunks = nh * C / 8;  // 16-byte chunks of this token's output
  for (int ci = tid; ci < chunks; ci += 256) {
    const int h = ci / (C / 8), cc = ci % (C / 8);
    *(uint4*)(orow + (int64_t)h * C + cc * 8) = *(const uint4*)(ostage + G::off(h) + cc * 16);
  }
}

// ---------------------------------------------------------------------------
// Dense prefill for 128-channel rows and 64 heads (HCA, [R] 2.3.2): one
// workgroup per block of kDenseTB consecutive tokens, two waves per token,
// each with 32 of its heads (kDenseHG 16-head groups: their O accumulators,
// queries and probabilities fit the vector registers, two waves per SIMD).  The block's tokens
// share nearly all their candidates: their windows differ in a few rows, and
// the entries visible to the last token include every other token's.  So
// each 32-row tile is gathered into LDS once, each K and V fragment read from
// it feeds four head groups, and each wave masks the tile by its own token's
// window and visible entries.  Tiles are fixed by absolute position: window
// tile a holds positions 32a .. 32a+31, entry tile e entries 32e .. 32e+31;
// a block visits the window tiles its tokens' windows touch, then the entry
// tiles its last token sees.  A token thus meets the same tiles in the same
// order whatever block or chunk it is computed in (tiles it does not see are
// all masked: they add exact zeros), so chunked and one-shot calls agree bit
// for bit.  The per-head softmax is the one-token kernel's: running max from
// the sink logit, running sum from 1, the O rescale only when a max rises by
// more than 2^8.  The output goes through LDS so that HBM sees whole-row
// stores.
// ---------------------------------------------------------------------------
constexpr int kDenseTB = 2;  // tokens per workgroup (two workgroups per CU)
constexpr int kDenseHG = 2;  // 16-head groups per wave: two waves per token

// Its tiles have a layout of their own: 32 rows of 256 bytes back to back, and
// 16-byte granule g of row r at slot g ^ dense_key(r).  A K read touches one
// granule of 16 rows, whose keys are distinct; a transposed V read touches two
// adjacent granules of 8 rows, whose keys differ above bit 0: both read
// patterns then cover distinct LDS banks.  The gather fetches, for slot s of
// row r, global granule s ^ dense_key(r).
CSA_DEV int dense_key(int r) { return ((r & 7) << 1) | ((r >> 4) & 1); }

// A compile-time int for generic lambdas.
template <int N> struct IntC { static constexpr int value = N; };

template <int C>
__global__ __launch_bounds__(64 * kDenseTB * 4 / kDenseHG, 8 / (kDenseTB * 4 / kDenseHG)) void
mqa_dense_tokblock_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ win,
    const uint16_t* __restrict__ comp, const float* __restrict__ sink,
    uint16_t* __restrict__ out, int64_t n, int m, int n_win, float scale, int qk_norm, float eps,
    int r, float theta, int64_t n_entries, int64_t t0) {
  static_assert(C == 128, "the tile layout is that of 256-byte rows");
  constexpr int NH = 64, HG = kDenseHG;    // heads; 16-head groups per wave
  constexpr int WPT = 4 / HG;              // waves per token
  constexpr int NKG = C / 32, NCB = C / 16;
  constexpr int OST = C * 2 + 16;          // staged output row stride (bytes)
  constexpr int NBUF = 4, AHEAD = NBUF - 1;  // tile ring; gathers run 3 tiles ahead
  constexpr int TROW = C * 2, TBYTES = kT * TROW;  // 256 B rows, 8 KiB tiles
  constexpr int BPW = TBYTES / 1024 / 4;     // 1 KiB DMA bursts per gathering wave and tile
  __shared__ __align__(16) uint8_t smem[NBUF * TBYTES];
  __shared__ __align__(16) uint8_t ostage[kDenseTB][NH * OST];
  __shared__ float2 rope_tab[kDenseTB][C / 2];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tw = wave / WPT, hw = wave % WPT;  // token of the block; head range 16 HG hw ..
  const int h0 = 16 * HG * hw;
  const int lc = lane & 15, lg = lane >> 4;
  // XCD-aware order: workgroup b runs on die b % 8.  The blocks form 16
  // contiguous ranges and die x takes ranges x and 15 - x: a token's work
  // grows with its position (its visible entries), so every die gets early
  // and late tokens alike, and each range's window rows and entries stay in
  // that die's L2
  const int64_t nblk = (n + kDenseTB - 1) / kDenseTB;
  const int64_t per = (nblk + 15) >> 4;  // blocks per range
  const int die = blockIdx.x & 7;
  const int64_t bi = blockIdx.x >> 3;
  const int64_t blk = bi < per ? die * per + bi : (15 - die) * per + (bi - per);
  if (blk >= nblk) return;  // the whole workgroup
  const int64_t tb = blk * kDenseTB, tl = min64(tb + kDenseTB - 1, n - 1);
  const bool live = tb + tw < n;
  const int64_t t = live ? tb + tw : tl;  // a wave past n repeats the last token, unstored
  const int64_t pt = t0 + t, ptb = t0 + tb, ptl = t0 + tl;
  const int64_t w0 = max64(t0 - n_win + 1, 0);           // position of win row 0
  const int64_t wt0 = max64(ptb - n_win + 1, 0) / kT;    // first window tile
  const int64_t nwr = (ptl / kT - wt0 + 1) * kT;         // window tile rows
  const int64_t neu = min64((ptl + 1) / m, n_entries);   // entries of the last token
  const int64_t pw0 = wt0 * kT;                          // position of window tile row 0
  const int ntiles = (int)(nwr / kT + (neu + kT - 1) / kT);
  // this token's candidates: window tile rows [wbeg, wend], entries < vis
  const int64_t wbeg = max64(pt - n_win + 1, 0) - pw0, wend = pt - pw0;
  const int64_t vis = min64((pt + 1) / m, n_entries);

  uint4 qraw[HG][NKG];
  {
    const uint16_t* qt = q + t * (int64_t)NH * C + lg * 8;
#pragma unroll
    for (int hg = 0; hg < HG; ++hg)
#pragma unroll
      for (int g = 0; g < NKG; ++g)
        qraw[hg][g] = *(const uint4*)(qt + (h0 + 16 * hg + lc) * C + g * 32);
  }
  float sink_h[HG];
#pragma unroll
  for (int hg = 0; hg < HG; ++hg) sink_h[hg] = sink[h0 + 16 * hg + lc];

  auto issue_tile = [&](int ti, int buf) {
    auto row_of = [&](int64_t j, bool& ok) -> const uint16_t* {
      // rows no token of the block sees load a valid row
      const uint16_t* dummy = win + (ptl - w0) * C;
      if (j < nwr) {
        const int64_t p = pw0 + j;
        ok = p >= w0 && p <= ptl;
        return ok ? win + (p - w0) * C : dummy;
      }
      ok = j - nwr < neu;
      return ok ? comp + (j - nwr) * C : dummy;
    };
    // lane L < 8 resolves row 4 (wave + 4 (L / 4)) + L % 4; burst u of the
    // wave (rows 4 (wave + 4u) .. + 3) takes its lanes' rows from lanes
    // 4u + L / 16
    const uint16_t* rp = win;
    if (lane < 8) {
      bool ok;
      rp = row_of((int64_t)ti * kT + 4 * (wave + 4 * (lane >> 2)) + (lane & 3), ok);
    }
    const uint32_t lo_a = (uint32_t)(size_t)rp, hi_a = (uint32_t)((size_t)rp >> 32);
#pragma unroll
    for (int u = 0; u < BPW; ++u) {
      const int src = 4 * u + (lane >> 4);
      const uint32_t lo = (uint32_t)__shfl((int)lo_a, src, 64);
      const uint32_t hi = (uint32_t)__shfl((int)hi_a, src, 64);
      const int rr = 4 * (wave + 4 * u) + (lane >> 4);
      const uint8_t* g =
          (const uint8_t*)(size_t)(((uint64_t)hi << 32) | lo) + ((lane & 15) ^ dense_key(rr)) * 16;
      lds_dma16(g, smem + buf * TBYTES + (wave + 4 * u) * 1024);
    }
  };
  // the gather: the first four waves (eight 1 KiB bursts of a tile)
  if (wave < 4) issue_tile(0, 0);  // eight 1 KiB bursts per tile
  if (hw == 0)
    for (int p = lane; p < r / 2; p += 64) {
      float cs, sn;
      rope_cs(pt, p, r, theta, &cs, &sn);
      rope_tab[tw][p] = make_float2(cs, sn);
    }
  __syncthreads();  // rope_tab is visible

  bf16x8_t qf[HG][NKG];
#pragma unroll
  for (int hg = 0; hg < HG; ++hg)
    q_prologue<C>(qraw[hg], qf[hg], rope_tab[tw], qk_norm, eps, r, lg);
  constexpr float LOG2E = 1.4426950408889634f;
  const float sl2 = scale * LOG2E;
  float run_m[HG], run_l[HG];
  f32x4_t o[HG][NCB];
#pragma unroll
  for (int hg = 0; hg < HG; ++hg) {
    run_m[hg] = sink_h[hg] * LOG2E;  // the sink enters the sum once, as 1
    run_l[hg] = 1.f;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) o[hg][cb] = f32x4_t{};
  }
  // the next gathers only now: the compiler's waits for q and the sink count
  // its own loads only, and would drain gathers issued before them
#pragma unroll
  for (int a = 1; a < AHEAD; ++a)
    if (wave < 4 && a < ntiles) issue_tile(a, a);
  // fragment addresses: K rows pi(lc >> 2, b, lc & 3), granule 4 g + lg;
  // transposed-read rows pi(lg, h, lc >> 2), granule 2 cb + (lc & 3) / 2,
  // half lc & 1
  int kofs[2][NKG], tofs[2][NCB];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int rk = slot_pi(lc >> 2, b, lc & 3), rt = slot_pi(lg, b, lc >> 2);
#pragma unroll
    for (int g = 0; g < NKG; ++g) kofs[b][g] = rk * TROW + (((4 * g + lg) ^ dense_key(rk)) << 4);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
      tofs[b][cb] = rt * TROW + (((2 * cb + ((lc & 3) >> 1)) ^ dense_key(rt)) << 4) + 8 * (lc & 1);
  }
  int slot[8];  // tile rows pi(lg, b, i) of this lane's logits z[4b + i]
#pragma unroll
  for (int e = 0; e < 8; ++e) slot[e] = slot_pi(lg, e >> 2, e & 3);
  // the token's rows relative to the block's tiles, in 32 bits (the launch
  // keeps the window and the entry count below 2^30, so tile rows, window
  // bounds and visible entries all fit)
  const int nwr32 = (int)nwr, wbeg32 = (int)wbeg, wend32 = (int)wend, vis32 = (int)vis;
  // tile 0 has landed once at most the later prologue gathers are in flight
  if (min(AHEAD - 1, ntiles - 1) >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * BPW));
  else if (min(AHEAD - 1, ntiles - 1) == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(BPW));
  else wait_vmem();
  __syncthreads();
  // One tile: its ring buffer is a compile-time constant, so every LDS read
  // takes the buffer offset as an immediate and only the per-lane offsets
  // above occupy registers.
  auto step = [&](int ti, auto bufc) {
    constexpr int buf = decltype(bufc)::value;  // buffer (buf + AHEAD) % NBUF held tile ti - 1
    if (wave < 4 && ti + AHEAD < ntiles) issue_tile(ti + AHEAD, (buf + AHEAD) % NBUF);
    const uint8_t* kv = smem + buf * TBYTES;
    // S^T = K Q^T for the wave's head groups; each K fragment read once
    f32x4_t sc[HG][2];
#pragma unroll
    for (int hg = 0; hg < HG; ++hg) sc[hg][0] = sc[hg][1] = f32x4_t{};
#pragma unroll
    for (int g = 0; g < NKG; ++g) {
      const bf16x8_t a0 = *(const bf16x8_t*)(kv + kofs[0][g]);
      const bf16x8_t a1 = *(const bf16x8_t*)(kv + kofs[1][g]);
#pragma unroll
      for (int hg = 0; hg < HG; ++hg) {
        sc[hg][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qf[hg][g], sc[hg][0], 0, 0, 0);
        sc[hg][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qf[hg][g], sc[hg][1], 0, 0, 0);
      }
    }
    // raw logits; this token's rows of the tile are [lo, hi] (wave-uniform),
    // and only a tile it does not see whole is masked (rows outside -> -inf)
    float z[HG][8];
#pragma unroll
    for (int hg = 0; hg < HG; ++hg)
#pragma unroll
      for (int e = 0; e < 8; ++e) z[hg][e] = sc[hg][e >> 2][e & 3];
    const int j0 = ti * kT;
    const int lo = min(max(j0 < nwr32 ? wbeg32 - j0 : 0, 0), kT);
    const int hi = max(min(j0 < nwr32 ? wend32 - j0 : vis32 - (j0 - nwr32) - 1, kT - 1), -1);
    if (!(lo == 0 && hi == kT - 1)) {
      const bool none = hi < lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bool in = !none && (unsigned)(slot[e] - lo) <= (unsigned)(hi - lo);
#pragma unroll
        for (int hg = 0; hg < HG; ++hg) z[hg][e] = in ? z[hg][e] : -INFINITY;
      }
    }
    bf16x8_t pb[HG];
#pragma unroll
    for (int hg = 0; hg < HG; ++hg) {
      float mx = z[hg][0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, z[hg][e]);
      // in log2 units: the maximum commutes with the positive scale
      mx = xlane_max(mx) * sl2;
      if (__any(mx > run_m[hg] + 8.f)) {  // wave-uniform rescale of this group's O
        const float nm = fmaxf(run_m[hg], mx);
        const float alpha = __builtin_amdgcn_exp2f(run_m[hg] - nm);
        run_l[hg] *= alpha;
        run_m[hg] = nm;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
          for (int i = 0; i < 4; ++i) o[hg][cb][i] *= alpha;
      }
      const float nm = -run_m[hg];
      f32x8_t p;
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(fmaf(z[hg][e], sl2, nm));
      const float ps = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      run_l[hg] += xlane_sum(ps);
      pb[hg] = __builtin_convertvector(p, bf16x8_t);
    }
    // O^T += V^T P^T; each V^T fragment (transpose read) feeds every group
    bf16x8_t vt[NCB];  // every V^T fragment of the tile, read before the products
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const bf16x4_t x0 =
          __builtin_amdgcn_ds_read_tr16_b64_v4bf16((CSA_LDS bf16x4_t*)(kv + tofs[0][cb]));
      const bf16x4_t x1 =
          __builtin_amdgcn_ds_read_tr16_b64_v4bf16((CSA_LDS bf16x4_t*)(kv + tofs[1][cb]));
      vt[cb] = __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
    }
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const bf16x8_t a = vt[cb];
#pragma unroll
      for (int hg = 0; hg < HG; ++hg)
        o[hg][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[hg], o[hg][cb], 0, 0, 0);
    }
    // tile ti+1 must have landed; the gathers of ti+2 .. ti+AHEAD may run
    const int later = min(ntiles - 1, ti + AHEAD) - (ti + 1);
    if (later >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * BPW));
    else if (later == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(BPW));
    else wait_vmem();
    __syncthreads();
  };
  static_assert(NBUF == 4, "the loop below visits the ring's four buffers in turn");
  for (int ti = 0; ti < ntiles; ti += NBUF) {
    step(ti, IntC<0>{});
    if (ti + 1 < ntiles) step(ti + 1, IntC<1>{});
    if (ti + 2 < ntiles) step(ti + 2, IntC<2>{});
    if (ti + 3 < ntiles) step(ti + 3, IntC<3>{});
  }

  // epilogue: o[hg][cb][i] = O[16 hg + lc][16 cb + 4 lg + i]; normalise,
  // rotate back by -t, stage this token's [64][C] rows, store them whole
  uint8_t* st = ostage[tw];
#pragma unroll
  for (int hg = 0; hg < HG; ++hg) {
    const float inv = 1.f / run_l[hg];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = o[hg][cb][i] * inv;
      const int ch0 = cb * 16 + 4 * lg;
      if (r > 0 && ch0 >= C - r) {
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          const float2 cs = rope_tab[tw][(ch0 + i - (C - r)) >> 1];
          const float x0 = v[i], x1 = v[i + 1];
          v[i] = x0 * cs.x + x1 * cs.y;  // rotate by -t
          v[i + 1] = -x0 * cs.y + x1 * cs.x;
        }
      }
      const uint32_t u0 = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
      const uint32_t u1 = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
      *(uint2*)(st + (h0 + 16 * hg + lc) * OST + ch0 * 2) = make_uint2(u0, u1);
    }
  }
  __syncthreads();
  if (live) {
    uint16_t* orow = out + t * (int64_t)NH * C;
    constexpr int CH = C / 8;  // 16-byte chunks per head row; this wave's heads
#pragma unroll 4
    for (int ci = h0 * CH + lane; ci < (h0 + 16 * HG) * CH; ci += 64) {
      const int h = ci / CH, cc = ci % CH;
      *(uint4*)(orow + (int64_t)h * C + cc * 8) = *(const uint4*)(st + h * OST + cc * 16);
    }
  }
}

hipError_t launch_mqa_prefill_bf16(const csa_attn_desc& d, int mode, const void* q, const void* win,
                                   const void* comp, const int32_t* idx, const float* sink,
                                   void* out, hipStream_t st) {
  // HCA's shape; the kernel's per-tile row bounds are 32-bit, exact while the
  // window and the entry count stay below 2^30
  if (mode != ATTN_SPARSE && d.c == 128 && d.n_heads == 64 && d.n_entries < (1 << 30) &&
      d.n_win < (1 << 30)) {
    const int64_t nblk = (d.n + kDenseTB - 1) / kDenseTB;
    mqa_dense_tokblock_kernel<128><<<(unsigned)(((nblk + 15) / 16) * 16), 64 * kDenseTB * 4 / kDenseHG, 0,
                                     st>>>(
        (const uint16_t*)q, (const uint16_t*)win, (const uint16_t*)comp, sink, (uint16_t*)out,
        d.n, d.m, d.n_win, d.scale, d.qk_norm, d.eps, d.rope_dims, d.rope_theta, d.n_entries,
        d.t0);
    return hipGetLastError();
  }
  const unsigned grid = (unsigned)(((d.n + 15) / 16) * 16);
#define CSA_FAST(CC)                                                                          \
  if (d.c == CC) {                                                                           \
    if (mode == ATTN_SPARSE)                                                                 \
      mqa_prefill_bf16_kernel<CC, true><<<grid, 256, 0, st>>>(                              \
          (const uint16_t*)q, (const uint16_t*)win, (const uint16_t*)comp, idx, sink,         \
          (uint16_t*)out, d.n, d.n_heads, d.k, d.m, d.n_win, d.scale, d.qk_norm, d.eps,       \
          d.rope_dims, d.rope_theta, d.n_entries, d.t0);                                      \
    else                                                                                     \
      mqa_prefill_bf16_kernel<CC, false><<<grid, 256, 0, st>>>(                             \
          (const uint16_t*)q, (const uint16_t*)win, (const uint16_t*)comp, idx, sink,         \
          (uint16_t*)out, d.n, d.n_heads, d.k, d.m, d.n_win, d.scale, d.qk_norm, d.eps,       \
          d.rope_dims, d.rope_theta, d.n_entries, d.t0);                                      \
    return hipGetLastError();                                                                \
  }
  CSA_FAST(128) CSA_FAST(256) CSA_FAST(512)
#undef CSA_FAST
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Decode split-K: one workgroup per (candidate chunk `spl` wide, sequence);
// the query of sequence b sits at position posv[b], window rows come from the
// ring (position p in slot p % n_win), and the workgroup writes its
// unnormalised partial O with (running max in log2 units, running sum), the
// sink left to the combine.  PAGED: the entry cache is a page pool; each
// chunk looks its entries' pool rows up once, into LDS, before its first
// tile, so no tile load waits on a page-table read.
// ---------------------------------------------------------------------------
constexpr int kDecSplitMax = 256;  // candidates per chunk, at most

// KV8: the ring and the cache hold FP8 rows (kv8_row_bytes(C, r) bytes each,
// C = 512): wave w's 8 rows of a tile are loaded into registers while the
// previous tile is computed, then decoded to bf16 into the same LDS layout.
template <int C, bool SPARSE, bool PAGED, bool KV8>
__global__ __launch_bounds__(256, 2) void mqa_decode_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ ring,
    const uint16_t* __restrict__ cache, const int32_t* __restrict__ idx,
    const float* __restrict__ sink, int nh, int k, int m, int n_win, float scale, int qk_norm,
    float eps, int r, float theta, int64_t n_entries, const int64_t* __restrict__ posv,
    float* __restrict__ ws_o, float2* __restrict__ ws_ml, int nsplit, int spl, EntryMap em) {
  typedef Geo<C> G;
  typedef OAcc<C> A;
  constexpr int NKG = C / 32;
  __shared__ __align__(16) uint8_t smem[2 * G::TILE];
  __shared__ __align__(16) int valid[2][kT];
  __shared__ int sidx[SPARSE ? kMaxK : 1];
  __shared__ int64_t srow[PAGED ? kDecSplitMax : 1];  // pool row per staged entry slot
  __shared__ float2 rope_tab[C / 2];
  constexpr int kRaw8 = kv8_row_bytes(512, 448);  // the widest FP8 row (r < 512)
  __shared__ __align__(16) uint8_t raw8[KV8 ? 2 * kT * kRaw8 : 16];  // tiles ti & 1

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lc = lane & 15, lg = lane >> 4;
  const int head = wave * 16 + lc;
  const int64_t b = blockIdx.y;
  const int split = blockIdx.x;

  // q and the sink first: their addresses do not depend on the position
  uint4 qraw[NKG];
  {
    const uint16_t* qh = q + (b * nh + (head < nh ? head : 0)) * C + lg * 8;
#pragma unroll
    for (int g = 0; g < NKG; ++g) qraw[g] = *(const uint4*)(qh + g * 32);
  }
  const float sink_h = head < nh ? sink[head] : 0.f;
  // This chunk's first index slots, loaded before the position is known on
  // the guess that the window is full (t + 1 >= n_win); used if it is.
  const int64_t cbeg = (int64_t)split * spl;
  const int64_t js = max64(cbeg - n_win, 0) + tid;
  const bool pre_ok = SPARSE && js < cbeg + spl - n_win && js < k;
  const int32_t pre = pre_ok ? idx[b * k + js] : -1;
  const int64_t t = posv[b];
  const int nwin = (int)max64(0, min64(n_win, t + 1));
  const int64_t ncomp = SPARSE ? (int64_t)k : max64(0, min64((t + 1) / m, n_entries));
  const int64_t ncand = nwin + ncomp;
  const int64_t cend = min64(cbeg + spl, ncand);
  if (cbeg >= cend) return;  // nothing in this chunk; the combine skips it
  const int ntiles = (int)((cend - cbeg + kT - 1) / kT);
  const uint16_t* wbase = ring + b * (int64_t)n_win * C;
  const int64_t s0 = max64(cbeg - nwin, 0);  // first index slot staged
  // ring slot of the oldest window position (candidate j at w0 + j mod n_win)
  const int w0 = nwin > 0 ? (int)((t - nwin + 1) % n_win) : 0;

  auto issue_tile = [&](int ti, int buf) {
    issue_tile_rows<C>(smem + buf * G::TILE, valid[buf], lane, wave, cbeg + (int64_t)ti * kT,
                       [&](int64_t j, bool& ok) -> const uint16_t* {
                         ok = false;
                         if (j >= cend) return wbase;  // a valid row for masked candidates
                         if (j < nwin) {
                           int slot = w0 + (int)j;
                           if (slot >= n_win) slot -= n_win;
                           ok = true;
                           return wbase + (int64_t)slot * C;
                         }
                         const int64_t e = SPARSE ? (int64_t)sidx[j - nwin - s0] : j - nwin;
                         if (e < 0 || e >= n_entries) return wbase;
                         ok = true;
                         return cache + (PAGED ? srow[j - nwin - s0] : b * n_entries + e) * C;
                       });
  };
  // ---- FP8 rows (C = 512): each wave gathers its own rows w, w + 4, ...,
  // w + 28 of a tile as raw bytes into LDS with DMA, two tiles ahead of the
  // one computing (no registers held meanwhile), then decodes them to the
  // bf16 tile layout.  Every gather is exactly kT / 4 DMA instructions per
  // wave (a masked row loads a row of this sequence's ring that is then
  // ignored), so a wait for all but the newest gather is vmcnt(kT / 4).  A
  // masked row's bf16 row is written as zeros, so that P = 0 never meets a
  // non-finite V.
  static_assert(!KV8 || C == 512, "FP8 rows are 512 channels wide");
  const int RB8 = kv8_row_bytes(C, r);
  const int nf8 = C - r;
  const uint8_t* cache8 = (const uint8_t*)cache;
  const uint8_t* wbase8 = (const uint8_t*)ring + b * (int64_t)n_win * RB8;
  int ok8 = 0;  // lanes 0..7, bit p: row wave + 4 * lane of the tile of parity p is live
  auto row8_of = [&](int64_t j, int& ok) -> const uint8_t* {
    ok = 0;
    if (j >= cend) return wbase8;
    if (j < nwin) {
      int slot = w0 + (int)j;
      if (slot >= n_win) slot -= n_win;
      ok = 1;
      return wbase8 + (int64_t)slot * RB8;
    }
    const int64_t e = SPARSE ? (int64_t)sidx[j - nwin - s0] : j - nwin;
    if (e < 0 || e >= n_entries) return wbase8;
    ok = 1;
    return cache8 + (PAGED ? srow[j - nwin - s0] : b * n_entries + e) * RB8;
  };
  auto dma8 = [&](int ti) {  // raw bytes of this wave's rows of tile ti
    const int par = ti & 1;
    const uint8_t* rp = wbase8;
    if (lane < kT / 4) {
      int ok;
      rp = row8_of(cbeg + (int64_t)ti * kT + wave + 4 * lane, ok);
      ok8 = (ok8 & ~(1 << par)) | (ok << par);
    }
    const uint32_t lo_a = (uint32_t)(size_t)rp, hi_a = (uint32_t)((size_t)rp >> 32);
    const int nl = RB8 / 16;  // 16-byte pieces per row
    uint8_t* dst = raw8 + par * (kT * kRaw8);
#pragma unroll
    for (int u = 0; u < kT / 4; ++u) {
      // readlane returns int: both halves as uint32 (no sign extension)
      const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane(lo_a, u);
      const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane(hi_a, u);
      const uint8_t* g = (const uint8_t*)(size_t)(((uint64_t)hi << 32) | lo);
      if (lane < nl) lds_dma16(g + 16 * lane, dst + (wave + 4 * u) * kRaw8);
    }
  };
  auto decode8 = [&](int ti) {  // this wave's raw rows of tile ti -> bf16 tile ti & 1
    const int par = ti & 1;
    if (lane < kT / 4) valid[par][wave + 4 * lane] = (ok8 >> par) & 1;
    // Branch-free, four rows at a time, so that their LDS reads issue back to
    // back: a code lane (8 * lane < c - r) reads its 8 codes and its block's
    // scale byte, a RoPE lane its 8 bf16 channels (two 8-byte reads); every
    // lane converts, and selects keep the right result (zero for a masked row).
    const bool code_lane = 8 * lane < nf8;
    const int off0 = code_lane ? 8 * lane : nf8 + 16 * (lane - nf8 / 8);
    const int offs = code_lane ? nf8 + 2 * r + lane / 8 : 0;
    const uint8_t* raw0 = raw8 + par * (kT * kRaw8);
    uint8_t* dst0 = smem + par * G::TILE + 16 * lane;
#pragma unroll
    for (int u0 = 0; u0 < kT / 4; u0 += 4) {
      uint2 w0[4], w1[4];
      uint32_t sb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint8_t* raw = raw0 + (wave + 4 * (u0 + i)) * kRaw8;
        w0[i] = *(const uint2*)(raw + off0);
        w1[i] = *(const uint2*)(raw + off0 + 8);
        sb[i] = raw[offs];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // the matrix cores' OCP E4M3 conversion times the block's 2^e (byte
        // e + 127 is the exponent field of 2^e as fp32); every product is
        // exact in bf16
        const float sc = __uint_as_float(sb[i] << 23);
        const uint32_t c0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0[i].x, sc, false));
        const uint32_t c1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0[i].x, sc, true));
        const uint32_t c2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0[i].y, sc, false));
        const uint32_t c3 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0[i].y, sc, true));
        // all-ones when the row is live (a wave-uniform mask, no branch)
        const uint32_t km = 0u - (uint32_t)((__builtin_amdgcn_readlane(ok8, u0 + i) >> par) & 1);
        uint4 o;
        o.x = (code_lane ? c0 : w0[i].x) & km;
        o.y = (code_lane ? c1 : w0[i].y) & km;
        o.z = (code_lane ? c2 : w1[i].x) & km;
        o.w = (code_lane ? c3 : w1[i].y) & km;
        *(uint4*)(dst0 + (wave + 4 * (u0 + i)) * G::BURST) = o;
      }
    }
  };
  // wait until the gather of tile ti has landed, the next one (issued
  // later) still in flight when `newer`
  auto wait8 = [&](bool newer) {
    if (newer)
      wait_vmem_fence_n<kT / 4>();
    else
      wait_vmem_fence_n<0>();
  };

  const bool early0 = !KV8 && cbeg + kT <= nwin;  // tile 0 is window rows only
  if (early0) issue_tile(0, 0);
  // entry slot j (index slot j of idx, or entry j) of this chunk -> pool row
  auto stage_row = [&](int64_t j, int64_t e) {
    if (PAGED) srow[j - s0] = e >= 0 && e < n_entries ? em.row(b, e, n_entries) : 0;
  };
  if (SPARSE) {
    int64_t j = s0 + tid;
    if (nwin == n_win) {  // the guess held: js == j
      if (j < cend - nwin) {
        sidx[j - s0] = pre;
        stage_row(j, pre);
      }
      j += 256;
    }
    for (; j < cend - nwin; j += 256) {
      const int32_t e = idx[b * k + j];
      sidx[j - s0] = e;
      stage_row(j, e);
    }
  } else if (PAGED) {
    for (int64_t j = s0 + tid; j < cend - nwin; j += 256) stage_row(j, j);
  }
  for (int p = tid; p < r / 2; p += 256) {
    float cs, sn;
    rope_cs(t, p, r, theta, &cs, &sn);
    rope_tab[p] = make_float2(cs, sn);
  }
  __syncthreads();
  if constexpr (KV8) {
    // the compiler counts only its own loads: settle them (q, the sink) so
    // that none of its waits later drains the gathers, which land while the
    // query prologue runs
    wait_vmem();
    dma8(0);
    if (ntiles > 1) dma8(1);
  } else if (!early0) {
    issue_tile(0, 0);
  }

  bf16x8_t qf[NKG];
  q_prologue<C>(qraw, qf, rope_tab, qk_norm, eps, r, lg);
  constexpr float LOG2E = 1.4426950408889634f;
  float run_m = sink_h * LOG2E;  // a finite start, log2 units
  float run_l = 0.f;                                     // the sink is the combine's
  A o;
#pragma unroll
  for (int cb = 0; cb < A::NLO; ++cb) o.lo[cb] = f32x4_t{};
#pragma unroll
  for (int cb = 0; cb < A::NHI; ++cb) o.hi[cb] = f32x4_t{};
  const int koff0 = G::off(slot_pi(lc >> 2, 0, lc & 3)) + lg * 16;
  const int koff1 = G::off(slot_pi(lc >> 2, 1, lc & 3)) + lg * 16;
  const int troff0 = G::off(slot_pi(lg, 0, lc >> 2)) + 8 * (lc & 3);
  const int troff1 = G::off(slot_pi(lg, 1, lc >> 2)) + 8 * (lc & 3);
  if constexpr (KV8) {
    wait8(ntiles > 1);
    decode8(0);
    if (ntiles > 2) dma8(2);
  } else {
    wait_vmem();
  }
  __syncthreads();
  for (int ti = 0; ti < ntiles; ++ti) {
    const int buf = ti & 1;
    if constexpr (KV8) {
      // tile ti+1's rows landed while tile ti-1 computed (tile ti+2's gather
      // may still run); bf16 buffer buf^1 was last read before the previous
      // barrier.  The decode is straight-line code ahead of the tile's
      // matrix work, which the compiler may interleave with it.
      if (ti + 1 < ntiles) {
        wait8(ti + 2 < ntiles);
        decode8(ti + 1);
      }
    } else {
      if (ti + 1 < ntiles) issue_tile(ti + 1, buf ^ 1);
    }
    mqa_tile<C>(smem + buf * G::TILE, valid[buf], qf, o, run_m, run_l, scale * LOG2E, koff0,
                koff1, troff0, troff1, lg);
    if constexpr (KV8) {
      if (ti + 3 < ntiles) dma8(ti + 3);  // raw buffer (ti+1) & 1 is decoded
    } else {
      wait_vmem();
    }
    __syncthreads();
  }
  // partial O^T: block cb, element i = O[head][cb*16 + 4*lg + i]
  if (head < nh) {
    const int64_t row = (b * nsplit + split) * nh + head;
    float* po = ws_o + row * C + 4 * lg;
#pragma unroll
    for (int cb = 0; cb < A::NLO; ++cb) *(f32x4_t*)(po + cb * 16) = o.lo[cb];
    if constexpr (A::NCB > 16) {
#pragma unroll
      for (int cb = 0; cb < A::NHI; ++cb) *(f32x4_t*)(po + (A::NLO + cb) * 16) = o.hi[cb];
    }
    if (lg == 0) ws_ml[row] = make_float2(run_m, run_l);
  }
}

// Fixed-order merge of the chunk partials of one sequence with the sink, then
// normalisation and the inverse RoPE at the query position.  WPH waves per
// (sequence, head), 4 / WPH heads per workgroup: wave j of a head folds chunks
// j, j+WPH, ... in index order (eight loads in flight, a running max), lane l
// owning channels [CPL*l, CPL*l + CPL); the head's wave states are then
// merged in wave order through LDS, the sink entering once.  Few chunks take
// one wave per head; many take four, so that their loads overlap.
template <int C, int WPH>
__global__ __launch_bounds__(256) void mqa_decode_combine_kernel(
    const float* __restrict__ ws_o, const float2* __restrict__ ws_ml,
    const int64_t* __restrict__ posv, const float* __restrict__ sink, uint16_t* __restrict__ out,
    int nh, int nsplit, int spl, int sparse, int k, int m, int n_win, int64_t n_entries, int r,
    float theta) {
  constexpr int CPL = C / 64;
  constexpr int U = 8;
  constexpr float LOG2E = 1.4426950408889634f;
  __shared__ float sacc[4][C];
  __shared__ float2 smd[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = wave % WPH;
  const int h0 = blockIdx.y * (4 / WPH) + wave / WPH;
  const bool live = h0 < nh;  // uniform per wave; every wave reaches the barrier
  const int h = live ? h0 : 0;
  const int64_t b = blockIdx.x;
  const int64_t pos = posv[b];
  const int64_t nwin = max64(0, min64(n_win, pos + 1));
  const int64_t ncomp = sparse ? (int64_t)k : max64(0, min64((pos + 1) / m, n_entries));
  const int ns = live ? (int)((nwin + ncomp + spl - 1) / spl) : 0;  // chunks with candidates
  const float2* ml = ws_ml + (int64_t)b * nsplit * nh + h;
  const float* po = ws_o + ((int64_t)b * nsplit * nh + h) * C + lane * CPL;
  const float sl2 = sink[h] * LOG2E;
  float M = sl2;    // a finite start; the sink itself is added in the merge
  float den = 0.f;
  float acc[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) acc[i] = 0.f;
  for (int s0 = sub; s0 < ns; s0 += WPH * U) {
    float2 mv[U];
    float ov[U][CPL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + WPH * u;
      mv[u] = make_float2(-INFINITY, 0.f);
#pragma unroll
      for (int i = 0; i < CPL; ++i) ov[u][i] = 0.f;
      if (s < ns) {
        mv[u] = ml[(int64_t)s * nh];
        const float* p = po + (int64_t)s * nh * C;
#pragma unroll
        for (int i = 0; i < CPL; i += 2) {
          const float2 v = *(const float2*)(p + i);
          ov[u][i] = v.x;
          ov[u][i + 1] = v.y;
        }
      }
    }
    float cm = M;
#pragma unroll
    for (int u = 0; u < U; ++u) cm = fmaxf(cm, mv[u].x);
    const float a = __builtin_amdgcn_exp2f(M - cm);
    den *= a;
#pragma unroll
    for (int i = 0; i < CPL; ++i) acc[i] *= a;
    M = cm;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float f = __builtin_amdgcn_exp2f(mv[u].x - M);
      den += f * mv[u].y;
#pragma unroll
      for (int i = 0; i < CPL; ++i) acc[i] += f * ov[u][i];
    }
  }
  float v[CPL];
  if constexpr (WPH == 1) {  // the wave's own state is the head's (M >= the sink's logit)
    if (!live) return;
    const float inv = 1.f / (den + __builtin_amdgcn_exp2f(sl2 - M));
#pragma unroll
    for (int i = 0; i < CPL; ++i) v[i] = acc[i] * inv;
  } else {
#pragma unroll
    for (int i = 0; i < CPL; ++i) sacc[wave][lane * CPL + i] = acc[i];
    if (lane == 0) smd[wave] = make_float2(M, den);
    __syncthreads();
    if (sub != 0 || !live) return;
    float Mt = sl2;
#pragma unroll
    for (int w = 0; w < WPH; ++w) Mt = fmaxf(Mt, smd[wave + w].x);
    float sc[WPH];
    float dt = __builtin_amdgcn_exp2f(sl2 - Mt);  // the sink's term
#pragma unroll
    for (int w = 0; w < WPH; ++w) {
      sc[w] = __builtin_amdgcn_exp2f(smd[wave + w].x - Mt);
      dt += sc[w] * smd[wave + w].y;
    }
    const float inv = 1.f / dt;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      float x = 0.f;
#pragma unroll
      for (int w = 0; w < WPH; ++w) x += sc[w] * sacc[wave + w][lane * CPL + i];
      v[i] = x * inv;
    }
  }
  const int ch0 = lane * CPL;
  if (r > 0 && ch0 >= C - r) {
#pragma unroll
    for (int i = 0; i < CPL; i += 2) {
      float cs, sn;
      rope_cs(pos, (ch0 + i - (C - r)) >> 1, r, theta, &cs, &sn);
      const float x0 = v[i], x1 = v[i + 1];
      v[i] = x0 * cs + x1 * sn;  // rotate by -pos
      v[i + 1] = -x0 * sn + x1 * cs;
    }
  }
  uint16_t* o = out + (b * nh + h) * C + ch0;
#pragma unroll
  for (int i = 0; i < CPL; i += 2)
    *(uint32_t*)(o + i) = (uint32_t)f32_to_bf16(v[i]) | ((uint32_t)f32_to_bf16(v[i + 1]) << 16);
}

int mqa_decode_bf16_split(int mode) { return mode == ATTN_SPARSE ? 128 : 256; }

hipError_t launch_mqa_decode_bf16(const csa_attn_desc& d, int mode, const void* q,
                                  const void* ring, const void* cache, const int32_t* idx,
                                  const int64_t* pos, const float* sink, void* out, float* ws_o,
                                  float2* ws_ml, int nsplit, hipStream_t st, EntryMap em,
                                  bool kv8) {
  const int spl = mqa_decode_bf16_split(mode);
  if (spl > kDecSplitMax) return hipErrorInvalidValue;  // the LDS row table's size
  if (kv8 && d.c != 512) return hipErrorInvalidValue;
  const dim3 grid((unsigned)nsplit, (unsigned)d.batch);
  const bool wide = nsplit > 8;  // more chunks than one wave's loads in flight
  const dim3 cgrid((unsigned)d.batch, (unsigned)(wide ? d.n_heads : (d.n_heads + 3) / 4));
#define CSA_DEC_K(CC, SP, PG, K8)                                                              \
  mqa_decode_bf16_kernel<CC, SP, PG, K8><<<grid, 256, 0, st>>>(                                \
      (const uint16_t*)q, (const uint16_t*)ring, (const uint16_t*)cache, idx, sink, d.n_heads,   \
      d.k, d.m, d.n_win, d.scale, d.qk_norm, d.eps, d.rope_dims, d.rope_theta, d.n_entries, pos, \
      ws_o, ws_ml, nsplit, spl, em);
#define CSA_DEC_MODES(CC, K8)                                                                  \
  if (mode == ATTN_SPARSE && em.table)                                                        \
    CSA_DEC_K(CC, true, true, K8)                                                             \
  else if (mode == ATTN_SPARSE)                                                               \
    CSA_DEC_K(CC, true, false, K8)                                                            \
  else if (em.table)                                                                          \
    CSA_DEC_K(CC, false, true, K8)                                                            \
  else                                                                                        \
    CSA_DEC_K(CC, false, false, K8)
#define CSA_DEC(CC, ...)                                                                       \
  if (d.c == CC) {                                                                            \
    __VA_ARGS__                                                                               \
    hipError_t e = hipGetLastError();                                                         \
    if (e != hipSuccess) return e;                                                            \
    if (wide)                                                                                 \
      mqa_decode_combine_kernel<CC, 4><<<cgrid, 256, 0, st>>>(                                \
          ws_o, ws_ml, pos, sink, (uint16_t*)out, d.n_heads, nsplit, spl, mode == ATTN_SPARSE,  \
          d.k, d.m, d.n_win, d.n_entries, d.rope_dims, d.rope_theta);                          \
    else                                                                                      \
      mqa_decode_combine_kernel<CC, 1><<<cgrid, 256, 0, st>>>(                                \
          ws_o, ws_ml, pos, sink, (uint16_t*)out, d.n_heads, nsplit, spl, mode == ATTN_SPARSE,  \
          d.k, d.m, d.n_win, d.n_entries, d.rope_dims, d.rope_theta);                          \
    return hipGetLastError();                                                                 \
  }
  CSA_DEC(128, CSA_DEC_MODES(128, false))
  CSA_DEC(256, CSA_DEC_MODES(256, false))
  CSA_DEC(512, if (kv8) { CSA_DEC_MODES(512, true) } else { CSA_DEC_MODES(512, false) })
#undef CSA_DEC
#undef CSA_DEC_MODES
#undef CSA_DEC_K
  return hipErrorInvalidValue;
}

}  // namespace csa
