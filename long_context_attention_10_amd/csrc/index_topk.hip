// Lightning indexer scoring and exact top-k selection.
//
// Citation keys: [R] = page "DeepSeek-V4 技术解读报告" (juejin.cn), section
// 2.3.1 eq 16 (I[t,s] = sum_h w[t,h] ReLU(q[t,h] . K[s])) and eq 17 (top-k);
// [A] = page "DeepSeek-V4：算法架构" (1zeryu.github.io), Indexer class:
// causal mask s < (t+1)//m, top-min(k, visible), -1 padding.
//
// Selection is exact: scores are fp32, mapped to order-preserving uint32 keys,
// and the k-th largest key is found by radix selection; equal scores are
// broken toward the smaller entry index.  Output rows list the chosen
// indices in ascending order, then -1.
#include "csa_common.h"
#include "csa_launch.h"

namespace csa {

// ===========================================================================
// Prefill scoring: scores[t][s] for a tile of queries x all keys of a chunk.
// One 256-thread workgroup owns 16*HI... (query, head) rows: each wave holds
// two 32-row blocks of them as matrix-core A operands for the whole chunk.
// Keys stream through LDS in blocks of KB by direct global->LDS loads into a
// double buffer (the next block loads while the current one is consumed).
// Key rows are stored unpadded with their 16-byte granules XOR-permuted, so
// the 16 lanes of a B-fragment read (16 keys, one granule each) hit distinct
// banks.  The head reduction with the ReLU and weights happens in registers.
// ===========================================================================
template <class T, int HI, int CI, class SC>
__global__ __launch_bounds__(256) void index_scores_prefill_kernel(
    const typename T::S* __restrict__ qI, const typename T::S* __restrict__ wI,
    const typename T::S* __restrict__ KI, int64_t n, int64_t n_entries, int m, int key_chunk,
    SC* __restrict__ scores, int64_t ld, int64_t t0) {
  typedef typename T::S S;
  constexpr int E = 16 / (int)sizeof(S);
  constexpr int KGE = 2 * E;        // elements per 32x32 k-group
  constexpr int NG = CI / KGE;      // k-groups per key
  constexpr int RB = 2;             // 32-row blocks per wave
  constexpr int ROWS = 4 * RB * 32; // (query, head) rows per workgroup
  constexpr int TQ = ROWS / HI;     // queries per workgroup
  constexpr int RBYTES = CI * (int)sizeof(S);   // bytes per key row
  constexpr int GR = RBYTES / 16;               // granules per key row
  constexpr int KB = RBYTES <= 128 ? 128 : 64;  // keys per staged block
  constexpr int KPI = 1024 / RBYTES;            // keys per 64-lane DMA
  constexpr int DPW = KB / KPI / 4;             // DMA instructions per wave per block
  static_assert(GR >= 8 && DPW >= 1, "key row layout");
  __shared__ __align__(16) uint8_t sK[2][KB * RBYTES];
  auto swz = [](int key) { return GR == 8 ? (key >> 1) & 7 : key & 15; };

  const int tid = threadIdx.x, lane = tid & 63, hl = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t q0 = (int64_t)blockIdx.x * TQ;
  const int64_t tlast = min64(q0 + TQ, n) - 1;
  // query row t is the token at position t0 + t
  const int64_t kend =
      min64(min64((t0 + tlast + 1) / m, n_entries), (int64_t)(blockIdx.y + 1) * key_chunk);
  const int64_t kbeg = (int64_t)blockIdx.y * key_chunk;
  if (kbeg >= kend) return;

  // keys past kend are read from the last key; their scores are not stored
  auto issue_block = [&](int64_t k0, int buf) {
#pragma unroll
    for (int u = 0; u < DPW; ++u) {
      const int d = wave + 4 * u;             // DMA index within the block
      const int key = d * KPI + lane / GR;    // key within the block
      const int pos = lane % GR;              // LDS granule position
      const int64_t sidx = min64(k0 + key, kend - 1);
      const uint8_t* src = (const uint8_t*)(KI + sidx * CI) + 16 * (pos ^ swz(key));
      lds_dma16(src, &sK[buf][d * 1024]);
    }
  };
  issue_block(kbeg, 0);

  // A fragments (query rows) and per-row weights, held for the whole chunk.
  uint4 qa[RB][NG];
  float wv[RB][16];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = wave * (RB * 32) + rb * 32 + (lane & 31);
    const int64_t t = q0 + row / HI;
    const int h = row % HI;
    const bool ok = t < n;
#pragma unroll
    for (int g = 0; g < NG; ++g)
      qa[rb][g] = ok ? *(const uint4*)(qI + (t * HI + h) * CI + g * KGE + hl * E) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int rr = wave * (RB * 32) + rb * 32 + 8 * (i >> 2) + 4 * hl + (i & 3);
      const int64_t tt = q0 + rr / HI;
      wv[rb][i] = tt < n ? T::ld(wI, tt * HI + rr % HI) : 0.f;
    }
  }
  // per stored query: its visible-entry count (0 past the last token), so the
  // causal test in the loop is one compare
  int vis[RB][4];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int64_t tb = q0 + (wave * (RB * 32) + rb * 32) / HI;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t t = HI == 4 ? tb + 2 * j + hl : HI == 8 ? tb + 2 * hl + (j & 1) : tb + hl;
      vis[rb][j] = t < n ? (int)min64((t0 + t + 1) / m, n_entries) : 0;
    }
  }
  wait_vmem();
  __syncthreads();
  // rows of this workgroup's queries: one uniform base, 32-bit offsets
  SC* srow0 = scores + q0 * ld;
  const int ld32 = (int)ld;

  const int nblk = (int)((kend - kbeg + KB - 1) / KB);
  for (int bi = 0; bi < nblk; ++bi) {
    const int buf = bi & 1;
    const int64_t kb0 = kbeg + (int64_t)bi * KB;
    if (bi + 1 < nblk) issue_block(kb0 + KB, buf ^ 1);
    const int nsub = (int)min64(KB / 32, (kend - kb0 + 31) / 32);
    for (int sb = 0; sb < nsub; ++sb) {
      const int kk = sb * 32 + (lane & 31);  // this lane's key within the block
      const uint8_t* krow = &sK[buf][kk * RBYTES];
      f32x16_t acc[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) acc[rb] = f32x16_t{};
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const uint4 kb = *(const uint4*)(krow + 16 * ((2 * g + hl) ^ swz(kk)));
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) mma32<T>(acc[rb], qa[rb][g], kb);
      }
      const int si = (int)(kb0 + kk);  // entry index (< 2^31)
      const bool sok = si < kend;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        float part[4];
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          float p = 0.f;
#pragma unroll
          for (int r = 0; r < 4; ++r) p += wv[rb][gq * 4 + r] * relu(acc[rb][gq * 4 + r]);
          part[gq] = p;
        }
        // rows of this block's first query relative to the workgroup's first
        const int tr = (wave * (RB * 32) + rb * 32) / HI;
        auto put = [&](int tq, int vq, float v) {  // query q0 + tq, visible count vq
          if (sok && si < vq) {
            if constexpr (sizeof(SC) == 2) srow0[(uint32_t)(tq * ld32 + si)] = f32_to_bf16(v);
            else srow0[(uint32_t)(tq * ld32 + si)] = v;
          }
        };
        if (HI == 4) {  // each group of 4 rows is one whole query
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) put(tr + 2 * gq + hl, vis[rb][gq], part[gq]);
        } else if (HI == 8) {  // rows 8q..8q+7 are query q; lanes < 32 keep 0, 1, the rest 2, 3
          const float v0 = swap32_pair_add(part[0], part[2]);
          const float v1 = swap32_pair_add(part[1], part[3]);
          put(tr + 2 * hl, vis[rb][0], v0);
          put(tr + 2 * hl + 1, vis[rb][1], v1);
        } else {  // HI == 16: rows 0-15 query 0 (lanes < 32), rows 16-31 query 1
          put(tr + hl, vis[rb][0], swap32_pair_add(part[0] + part[1], part[2] + part[3]));
        }
      }
    }
    wait_vmem();
    __syncthreads();
  }
}

// ===========================================================================
// Block-wide helpers (256 threads)
// ===========================================================================
// Exclusive prefix sum over the 256 threads in thread order; returns the total
// in *total.  `tmp` is LDS scratch of >= 4 ints.
CSA_DEV int block_excl_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  __syncthreads();
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += tmp[w];
  *total = tmp[0] + tmp[1] + tmp[2] + tmp[3];
  return base + x - v;
}

// Given a 256-bin histogram in LDS and `need` >= 1, find the digit d such
// that (#items with digit > d) < need <= (#items with digit >= d).  Wave 0
// computes; results are broadcast through `out` (digit, items above d).
CSA_DEV void find_digit(const int* hist, int need, int* out) {
  if (threadIdx.x < 64) {
    const int l = threadIdx.x;
    const int c4 = hist[4 * l] + hist[4 * l + 1] + hist[4 * l + 2] + hist[4 * l + 3];
    int suf = c4;  // inclusive suffix sum over lanes >= l
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_down(suf, o, 64);
      if (l + o < 64) suf += y;
    }
    const int above = suf - c4;  // items in lanes > l
    if (suf >= need && above < need) {
      int acc = above;
      for (int b = 3; b >= 0; --b) {
        const int hcount = hist[4 * l + b];
        if (acc + hcount >= need) { out[0] = 4 * l + b; out[1] = acc; break; }
        acc += hcount;
      }
    }
  }
}

// Threshold bin from a histogram (suffix search from the top): the bin T with
// (#items in bins > T) < need <= (#items in bins >= T); every thread gets
// res = (T, #items above T).  `h` holds NB bins (global memory or LDS), `sh`
// is LDS scratch of 4 ints; 256 threads.
template <int NB>
CSA_DEV void bin_threshold_vals(const int (&loc)[NB / 256], int need, int* sh, int* res) {
  constexpr int PER = NB / 256;  // consecutive bins per thread
  const int tid = threadIdx.x;
  int cs = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) cs += loc[i];
  // inclusive suffix sum over threads
  const int lane = tid & 63, wave = tid >> 6;
  int suf = cs;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_down(suf, o, 64);
    if (lane + o < 64) suf += y;
  }
  __syncthreads();
  if (lane == 0) sh[wave] = suf;
  __syncthreads();
  int above_w = 0;
  for (int w = wave + 1; w < 4; ++w) above_w += sh[w];
  suf += above_w;
  const int above = suf - cs;
  if (suf >= need && above < need) {
    int acc = above;
    for (int i = PER - 1; i >= 0; --i) {
      if (acc + loc[i] >= need) { res[0] = tid * PER + i; res[1] = acc; break; }
      acc += loc[i];
    }
  }
  __syncthreads();
}

template <int NB>
CSA_DEV void bin_threshold(const int* __restrict__ h, int need, int* sh, int* res) {
  int loc[NB / 256];
#pragma unroll
  for (int i = 0; i < NB / 256; ++i) loc[i] = h[threadIdx.x * (NB / 256) + i];
  bin_threshold_vals<NB>(loc, need, sh, res);
}


// ===========================================================================
// Prefill row selection: one workgroup per query row over its v <= 16384
// visible scores, held in registers as order-preserving uint32 keys (thread
// j owns entries 4(j + 256 i) + 0..3).  Entries are ordered by the composite
// (key << 32 | ~index): higher score first, ties to the smaller index.
//   0. a lower bound of the k-th largest key: each thread offers its Q-th
//      largest key (256 Q >= k); when the offering threads' top-Q sets hold
//      at least k keys, the smallest offer is such a bound, and keys below it
//      take no further part (else the bound is the row minimum);
//   1. keys from the bound up are binned linearly by score VALUE between
//      the bound and the row maximum (1024 bins; the map is monotone, so each
//      bin is a key interval) and the bin T holding the k-th largest is found
//      from the histogram -- raw float bits would pile most of a row into the
//      few bins of its common exponent;
//   2. in one more pass over the keys, entries of bins above T are marked
//      as winners in an LDS bitmap over the row and the composites of T are
//      gathered and ranked (at most 256; else T's need-th largest composite
//      is found by an 8-bit radix and a last pass marks T's winners);
//   3. the bitmap is emitted in ascending index order.
// ===========================================================================
constexpr int kSelBins = 1024;
constexpr int kRankMax = 256;

CSA_DEV float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
CSA_DEV uint64_t composite(uint32_t key, uint32_t idx) {
  return ((uint64_t)key << 32) | (uint32_t)~idx;
}

template <int MAXIT, int Q, class SC>
__global__ __launch_bounds__(256) void topk_rows_prefill_kernel(const SC* __restrict__ scores,
                                                                int64_t ld, int64_t n,
                                                                int64_t n_entries, int m, int k,
                                                                int32_t* __restrict__ idx_out,
                                                                int64_t row0, int64_t t0) {
  constexpr int NQ = MAXIT / 4;  // 4-entry groups per thread
  __shared__ int hist[kSelBins];
  __shared__ uint32_t bits[MAXIT * 256 / 32];
  __shared__ uint64_t cand[kRankMax];
  __shared__ int tmp[8];
  __shared__ int res[2];
  __shared__ uint32_t red[8];
  __shared__ int ncand;
  const int t = (int)(row0 + blockIdx.x);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int v = (int)min64((t0 + t + 1) / m, n_entries);  // row t: position t0 + t
  const int kt = min(k, v);
  int32_t* orow = idx_out + (int64_t)t * k;
  if (v <= k) {
    for (int j = tid; j < k; j += 256) orow[j] = j < v ? j : -1;
    return;
  }
  // keys (coalesced 16-byte loads, all in flight together; the row start is
  // 16-byte aligned and ld % 4 == 0).  Entries past v get key 0, below every
  // real key.
  const SC* srow = scores + (int64_t)t * ld;
  uint32_t u[MAXIT];
  if constexpr (sizeof(SC) == 4) {
    float4 xs[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int e = 4 * (tid + 256 * q);
      if (e < v) xs[q] = *(const float4*)(srow + e);
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int e = 4 * (tid + 256 * q);
      const float x4[4] = {xs[q].x, xs[q].y, xs[q].z, xs[q].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) u[4 * q + j] = e + j < v ? float_key(x4[j]) : 0u;
    }
  } else {  // bf16 scores: 8-byte loads of 4 entries, widened exactly to fp32
    uint2 xs[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int e = 4 * (tid + 256 * q);
      if (e < v) xs[q] = *(const uint2*)(srow + e);
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int e = 4 * (tid + 256 * q);
      const uint32_t b4[4] = {xs[q].x << 16, xs[q].x & 0xffff0000u, xs[q].y << 16,
                              xs[q].y & 0xffff0000u};
#pragma unroll
      for (int j = 0; j < 4; ++j) u[4 * q + j] = e + j < v ? float_key(__uint_as_float(b4[j])) : 0u;
    }
  }
  auto idx_of = [&](int i) { return 4 * (tid + 256 * (i >> 2)) + (i & 3); };
  for (int i = tid; i < kSelBins; i += 256) hist[i] = 0;
  for (int w = tid; w < MAXIT * 256 / 32; w += 256) bits[w] = 0u;
  if (tid == 0) ncand = 0;
  // Lower bound of the kt-th key: every thread holding at least Q real keys
  // offers its Q-th largest; when those threads' top-Q sets hold >= kt keys,
  // the smallest offer is <= the kt-th largest key of the row, and keys below
  // it can never be selected -- they skip the histogram and the marking.
  // (Q = 0: no bound; the bins span the row's minimum to its maximum.)
  uint32_t lo = 0xffffffffu, hi = 0u;
  int offers = 0;
  if constexpr (Q > 0) {
    uint32_t a[Q];
#pragma unroll
    for (int j = 0; j < Q; ++j) a[j] = 0u;
#pragma unroll
    for (int i = 0; i < MAXIT; ++i) {
      uint32_t x = u[i];
#pragma unroll
      for (int j = 0; j < Q; ++j) {  // insertion into the descending top-Q
        const uint32_t y = max(a[j], x);
        x = min(a[j], x);
        a[j] = y;
      }
    }
    hi = a[0];
    if (a[Q - 1]) { lo = a[Q - 1]; offers = Q; }
  } else {
#pragma unroll
    for (int i = 0; i < MAXIT; ++i)
      if (u[i]) { lo = min(lo, u[i]); hi = max(hi, u[i]); }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    lo = min(lo, (uint32_t)__shfl_xor((int)lo, o, 64));
    hi = max(hi, (uint32_t)__shfl_xor((int)hi, o, 64));
    if constexpr (Q > 0) offers += __shfl_xor(offers, o, 64);
  }
  if (lane == 0) { red[wave] = lo; red[4 + wave] = hi; if (Q > 0) tmp[wave] = offers; }
  __syncthreads();
  lo = min(min(red[0], red[1]), min(red[2], red[3]));
  hi = max(max(red[4], red[5]), max(red[6], red[7]));
  uint32_t lk = 1u;  // keys >= lk take part (real keys are >= 1)
  if constexpr (Q > 0) {
    if (tmp[0] + tmp[1] + tmp[2] + tmp[3] >= kt) lk = lo;
    else {  // too few offers: bins over the whole row
      lo = 0xffffffffu;
#pragma unroll
      for (int i = 0; i < MAXIT; ++i)
        if (u[i]) lo = min(lo, u[i]);
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) lo = min(lo, (uint32_t)__shfl_xor((int)lo, o, 64));
      __syncthreads();
      if (lane == 0) red[wave] = lo;
      __syncthreads();
      lo = min(min(red[0], red[1]), min(red[2], red[3]));
    }
  }
  const float fmin = key_float(lo), fmax = key_float(hi);
  float scale = (float)kSelBins / (fmax - fmin);
  if (!(scale < INFINITY)) scale = 0.f;  // equal or non-finite range: one bin
  // bin of a real key (>= 1): monotone in the key, so bins are key intervals
  // and membership is recomputed exactly wherever it is needed
  auto vbin_with = [&](uint32_t key, float f0, float sc) {
    const float f = (key_float(key) - f0) * sc;
    return f >= (float)(kSelBins - 1) ? kSelBins - 1 : (f > 0.f ? (int)f : 0);
  };
  auto vbin = [&](uint32_t key) { return vbin_with(key, fmin, scale); };
  auto mark = [&](int e) { atomicOr(&bits[e >> 5], 1u << (e & 31)); };

  // 1. value histogram; threshold bin T
#pragma unroll
  for (int i = 0; i < MAXIT; ++i)
    if (u[i] >= lk) atomicAdd(&hist[vbin(u[i])], 1);
  __syncthreads();
  bin_threshold<kSelBins>(hist, kt, tmp, res);
  const int T = res[0];
  int need = kt - res[1];  // to take from bin T (>= 1)
  const int nT = hist[T];

  // 2. bins above T win outright; bin T's composites (key << 32 | ~index) are
  //    ranked when few (the winners of T are the need largest), else their
  //    need-th largest is found by an 8-bit radix.  The bins are recomputed
  //    (from copies the compiler cannot see through), not kept from pass 1:
  //    keeping 64 of them would cost as many registers.
  float fmin2 = fmin, scale2 = scale;
  asm volatile("" : "+v"(fmin2), "+v"(scale2));
  if (nT <= kRankMax) {
#pragma unroll
    for (int i = 0; i < MAXIT; ++i)
      if (u[i] >= lk) {
        const int b = vbin_with(u[i], fmin2, scale2);
        if (b > T) mark(idx_of(i));
        else if (b == T) cand[atomicAdd(&ncand, 1)] = composite(u[i], idx_of(i));
      }
    __syncthreads();
    if (tid < nT) {
      const uint64_t c = cand[tid];
      int rank = 0;
      for (int j = 0; j < nT; ++j) rank += cand[j] > c;
      if (rank < need) mark((int)~(uint32_t)c);  // composites are distinct
    }
  } else {
    uint64_t prefix = 0, pmask = 0;
    for (int pass = 0; pass < 8; ++pass) {
      const int shift = 56 - 8 * pass;
      __syncthreads();
      hist[tid] = 0;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < MAXIT; ++i) {
        const uint64_t c = composite(u[i], idx_of(i));
        if (u[i] >= lk && vbin_with(u[i], fmin2, scale2) == T && (c & pmask) == prefix)
          atomicAdd(&hist[(c >> shift) & 255], 1);
      }
      __syncthreads();
      bin_threshold<256>(hist, need, tmp, res);
      need -= res[1];
      prefix |= (uint64_t)res[0] << shift;
      pmask |= (uint64_t)0xff << shift;
    }
    const uint64_t thr = prefix;  // the need-th largest composite of bin T
#pragma unroll
    for (int i = 0; i < MAXIT; ++i) {
      uint32_t ui = u[i];
      asm volatile("" : "+v"(ui));  // recomputed here, not held from the passes above
      if (ui >= lk) {
        const int b = vbin_with(ui, fmin2, scale2);
        if (b > T || (b == T && composite(ui, idx_of(i)) >= thr)) mark(idx_of(i));
      }
    }
  }

  // 3. bitmap -> ascending indices
  __syncthreads();
  const int W = (v + 31) / 32;
  const int WPT = (W + 255) / 256;
  const int w0 = tid * WPT, w1 = min(w0 + WPT, W);
  int cnt = 0;
  for (int w = w0; w < w1; ++w) cnt += __popc(bits[w]);
  int tot;
  int p = block_excl_scan(cnt, tmp + 4, &tot);
  for (int w = w0; w < w1; ++w) {
    uint32_t b = bits[w];
    while (b) {
      orow[p++] = w * 32 + __ffs(b) - 1;
      b &= b - 1;
    }
  }
  for (int j = kt + tid; j < k; j += 256) orow[j] = -1;
}

// ===========================================================================
// Decode: one query per sequence over up to ~10^6 cached keys.
//   D1 score chunks of keys (16x16 matrix-core tiles, keys streamed straight
//      from memory -- this pass moves the step's dominant bytes) and build a
//      2048-bin histogram of the keys' top 11 bits, added into one of R
//      copies per sequence (chunk mod R, R = chunks / 32 clamped to [1, 8]):
//      atomics on one cache line are serialised, so at most ~32 workgroups
//      add into the same lines;
//   D2 per chunk: find the coarse threshold bin T of the k-th key from the
//      summed copies (scanning down from the top bin), then store the
//      chunk's entries of bins above T (the "sure" entries) at the front of
//      the chunk's own slice of the list buffer and those of T (the ties) at
//      its back, with the two counts per chunk -- no atomics;
//   D3 per sequence: gather the chunks' lists, resolve the ties exactly on
//      (score, -index) from their fine histogram (a radix select over the
//      whole tie list when the fine bin is crowded), and merge the two
//      ascending lists into the output row, and zero the sequence's
//      histograms for the next call.
// The histograms lead the workspace: they must be zero when a call starts
// (the caller clears them once) and every call leaves them zero, so no
// clearing launch precedes the scoring.  Nothing depends on the order in
// which workgroups run.
// ===========================================================================
constexpr int kDecChunk = 1024;    // keys per scoring workgroup
constexpr int kCoarseBins = 2048;  // top 11 bits
constexpr int kHistCopies = 8;     // most histogram copies per sequence
constexpr int kChunkLds = 1024;    // chunk counts staged in LDS by the finalize
constexpr int kTieLds = 6144;      // tie candidates resolved in LDS

struct DecWs {  // carve-up of the decode workspace
  int* hist;      // [B][copies][kCoarseBins], then fine [B][kCoarseBins] (tie bits 20..10)
  int* fine;
  float* scores;  // [B][n_entries]
  int2* ccnt;     // [B][chunks]: (sure, tie) counts per chunk
  uint2* lists;   // [B][n_entries] (key, index): chunk slices, sure first, ties last
  uint2* flat;    // [B][n_entries]: tie lists too long for LDS, contiguous
};

static size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

static int64_t dec_chunks(const csa_index_desc& d) {
  return (d.n_entries + kDecChunk - 1) / kDecChunk;
}

static int dec_hist_copies(int64_t nchunks) {
  return nchunks >= 32 * kHistCopies ? kHistCopies : nchunks >= 64 ? (int)(nchunks / 32) : 1;
}

static DecWs carve(void* ws, const csa_index_desc& d) {
  uint8_t* p = (uint8_t*)ws;
  DecWs w;
  const size_t B = d.batch, ne = d.n_entries, nc = dec_chunks(d);
  w.hist = (int*)p;
  w.fine = w.hist + B * dec_hist_copies(nc) * kCoarseBins;
  p += align_up(B * (dec_hist_copies(nc) + 1) * kCoarseBins * 4);
  w.scores = (float*)p; p += align_up(B * ne * 4);
  w.ccnt = (int2*)p; p += align_up(B * nc * 8);
  w.lists = (uint2*)p; p += align_up(B * ne * 8);
  w.flat = (uint2*)p; p += align_up(B * ne * 8);
  return w;
}

size_t index_decode_zero_bytes(const csa_index_desc& d) {
  return align_up((size_t)d.batch * (dec_hist_copies(dec_chunks(d)) + 1) * kCoarseBins * 4);
}

size_t index_decode_ws_bytes(const csa_index_desc& d) {
  const size_t B = d.batch, ne = d.n_entries, nc = dec_chunks(d);
  return align_up(B * ne * 4) + align_up(B * (dec_hist_copies(nc) + 1) * kCoarseBins * 4) +
         align_up(B * nc * 8) + 2 * align_up(B * ne * 8);
}

// PAGED: KI is a page pool.  The page-table slots of the chunk's entries are
// read first, before the position (they lie in the table whether or not the
// entries are visible; only the visible ones' values are used), and turned
// into pool rows in LDS, so no key load waits on a table read.
template <class T, int HI, int CI, bool PAGED>
__global__ __launch_bounds__(256) void dec_score_kernel(
    const typename T::S* __restrict__ qI, const typename T::S* __restrict__ wI,
    const typename T::S* __restrict__ KI, const int64_t* __restrict__ posv, int64_t n_entries,
    int m, int k, float* __restrict__ scores, int* __restrict__ hist, int ncopies, EntryMap em) {
  typedef typename T::S S;
  constexpr int E = 16 / (int)sizeof(S);
  constexpr int KGE = 4 * E;      // elements per 16x16 k-group
  constexpr int NG = CI / KGE;
  __shared__ int lh[kCoarseBins];
  __shared__ int64_t srow[PAGED ? kDecChunk : 1];
  const int b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lg = lane >> 4;
  const int64_t c0 = (int64_t)blockIdx.x * kDecChunk;
  constexpr int NS = kDecChunk / 256;  // entries per thread in the row table
  int32_t tslot[PAGED ? NS : 1];
  if (PAGED) {
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int64_t s = c0 + tid + 256 * i;
      tslot[i] = s < n_entries ? em.table[(int64_t)b * em.max_pages + (uint32_t)s / (uint32_t)em.page]
                               : 0;
    }
  }
  const int64_t vis = min64((posv[b] + 1) / m, n_entries);
  if (vis <= k) return;  // everything visible is selected
  if (c0 >= vis) return;
  const int64_t c1 = min64(c0 + kDecChunk, vis);
  for (int i = tid; i < kCoarseBins; i += 256) lh[i] = 0;
  if (PAGED) {
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int64_t s = c0 + tid + 256 * i;
      if (s < c1) srow[s - c0] = (int64_t)tslot[i] * em.page + (uint32_t)s % (uint32_t)em.page;
    }
  }

  // A = indexer queries: row = head (lane % 16), padded with zero rows
  uint4 qa[NG];
  float wv[4];
  const int hrow = lane & 15;
#pragma unroll
  for (int g = 0; g < NG; ++g)
    qa[g] = hrow < HI ? *(const uint4*)(qI + ((int64_t)b * HI + hrow) * CI + g * KGE + lg * E)
                      : make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * lg + i;
    wv[i] = h < HI ? T::ld(wI, (int64_t)b * HI + h) : 0.f;
  }
  __syncthreads();
  // Each wave scores a contiguous quarter of the chunk, 64 keys (4 steps of
  // 16) at a time; the next 64 keys load while the current ones are scored.
  const int64_t w0 = c0 + (int64_t)wave * (kDecChunk / 4);
  const int64_t w1 = min64(w0 + kDecChunk / 4, c1);
  auto load64 = [&](int64_t s0, uint4 (&dst)[4][NG]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t s = min64(s0 + u * 16 + (lane & 15), c1 - 1);  // past c1: not stored
      const S* krow = KI + (PAGED ? srow[s - c0] : (int64_t)b * n_entries + s) * CI;
#pragma unroll
      for (int g = 0; g < NG; ++g) dst[u][g] = *(const uint4*)(krow + g * KGE + lg * E);
    }
  };
  auto score64 = [&](int64_t s0, const uint4 (&src)[4][NG]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      f32x4_t acc = f32x4_t{};
#pragma unroll
      for (int g = 0; g < NG; ++g) mma16<T>(acc, qa[g], src[u][g]);
      float p = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) p += wv[i] * relu(acc[i]);
      p = xlane_sum(p);
      const int64_t s = s0 + u * 16 + (lane & 15);
      if (lg == 0 && s < w1) {
        scores[(int64_t)b * n_entries + s] = p;
        atomicAdd(&lh[float_key(p) >> 21], 1);
      }
    }
  };
  // two register buffers, used alternately (static indices keep them in VGPRs)
  uint4 ka[4][NG], kc[4][NG];
  if (w0 < w1) load64(w0, ka);
  for (int64_t s0 = w0; s0 < w1; s0 += 128) {
    if (s0 + 64 < w1) load64(s0 + 64, kc);
    score64(s0, ka);
    if (s0 + 64 >= w1) break;
    if (s0 + 128 < w1) load64(s0 + 128, ka);
    score64(s0 + 64, kc);
  }
  __syncthreads();
  int* gh = hist + ((int64_t)b * ncopies + blockIdx.x % ncopies) * kCoarseBins;
  for (int i = tid; i < kCoarseBins; i += 256)
    if (lh[i]) atomicAdd(&gh[i], lh[i]);
}

// ---------------------------------------------------------------------------
// The quantised indexer path ([A] Compressor with rotate=True and the Indexer
// forward: rotate_activation then fp4_act_quant; [R] section 4.4: the QK path
// cached, loaded and multiplied in FP4).  A row of width CI is rotated by the
// normalised Walsh-Hadamard transform and stored as E2M1 codes (two per byte,
// the even element in the low nibble) with one power-of-two scale per block
// of 32 values (its exponent e as the byte e + 127), the smallest e with
// max |x| <= 6 * 2^e; values round to the nearest E2M1 value, ties to the
// even mantissa.
// ---------------------------------------------------------------------------
CSA_DEV uint32_t e2m1_code(float x, float inv_scale) {
  const float a = fabsf(x) * inv_scale;  // in [0, 6]
  const uint32_t i = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) +
                     (a >= 3.5f) + (a > 5.0f);
  return i | ((x < 0.f && i) ? 8u : 0u);
}

CSA_DEV int e2m1_block_exp(float amax) {
  if (!(amax > 0.f)) return 0;
  int k;
  const float f = frexpf(amax, &k);  // amax = f * 2^k, 0.5 <= f < 1
  return f <= 0.75f ? k - 3 : k - 2;
}

// One wave per row: lane l holds elements l (and l + 64); butterflies over
// the strides 64 (in the lane), 32 .. 1 (across lanes), then 1/sqrt(CI).
// With posv (decode): wave b quantises row b * n_entries + pos[b] / m of
// the cache, the entry the step has just emitted, when (pos[b] + 1) % m == 0.
template <class T, int CI>
__global__ __launch_bounds__(256) void fp4_rotate_quant_kernel(const typename T::S* __restrict__ x,
                                                               int64_t rows,
                                                               uint8_t* __restrict__ codes,
                                                               uint8_t* __restrict__ exps,
                                                               const int64_t* __restrict__ posv,
                                                               int64_t n_entries, int m,
                                                               EntryMap em) {
  constexpr int NV = CI / 64;
  const int lane = threadIdx.x & 63;
  int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;  // whole wave
  if (posv) {
    const int64_t p = posv[r];
    if (p < 0 || (p + 1) % m != 0 || p / m >= n_entries) return;
    r = em.row(r, p / m, n_entries);  // the same row of the key cache and the FP4 caches
  }
  float v[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) v[j] = T::ld(x, r * CI + j * 64 + lane);
  if constexpr (NV == 2) {
    const float a = v[0], b = v[1];
    v[0] = a + b;
    v[1] = a - b;
  }
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1)
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const float p = __shfl_xor(v[j], s, 64);
      v[j] = (lane & s) ? p - v[j] : v[j] + p;
    }
  const float norm = CI == 64 ? 0.125f : 0.0883883476483184406f;  // 1/sqrt(CI)
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const float y = v[j] * norm;
    float am = fabsf(y);
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) am = fmaxf(am, __shfl_xor(am, o, 64));  // 32-value block
    const int e = e2m1_block_exp(am);
    const uint32_t c = e2m1_code(y, ldexpf(1.f, -e));
    const uint32_t c1 = __shfl_xor(c, 1, 64);
    const int elem = j * 64 + lane;
    if (!(lane & 1)) codes[r * (CI / 2) + elem / 2] = (uint8_t)(c | (c1 << 4));
    if ((lane & 31) == 0) exps[r * (CI / 32) + elem / 32] = (uint8_t)(e + 127);
  }
}

// 8 consecutive E2M1 values (4 code bytes) with the block scale 2^(eb - 127)
// as one bf16 matrix-core fragment.
CSA_DEV uint4 fp4x8_to_bf16(uint32_t cw, uint32_t eb) {
  const float sc = __uint_as_float(eb << 23);  // 2^(eb - 127)
  uint4 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, sc, 0));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, sc, 1));
  r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, sc, 2));
  r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, sc, 3));
  return r;
}

// D1 over FP4 keys: dec_score_kernel with q^I and the keys read as E2M1 codes
// and block exponents (a quarter of the bf16 bytes) and widened to bf16
// fragments in registers; the products, head sum and histogram are the same.
template <int HI, int CI, bool PAGED>
__global__ __launch_bounds__(256) void dec_score_fp4_kernel(
    const uint8_t* __restrict__ qc, const uint8_t* __restrict__ qe, const uint16_t* __restrict__ wI,
    const uint8_t* __restrict__ kc, const uint8_t* __restrict__ ke,
    const int64_t* __restrict__ posv, int64_t n_entries, int m, int k, float* __restrict__ scores,
    int* __restrict__ hist, int ncopies, EntryMap em) {
  constexpr int NG = CI / 32;  // 32-value k-groups (= scale blocks) per row
  constexpr int RB = CI / 2;   // code bytes per row
  __shared__ int lh[kCoarseBins];
  __shared__ int64_t srow[PAGED ? kDecChunk : 1];  // pool rows (as in dec_score_kernel)
  const int b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lg = lane >> 4;
  const int64_t c0 = (int64_t)blockIdx.x * kDecChunk;
  constexpr int NS = kDecChunk / 256;
  int32_t tslot[PAGED ? NS : 1];
  if (PAGED) {
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int64_t s = c0 + tid + 256 * i;
      tslot[i] = s < n_entries ? em.table[(int64_t)b * em.max_pages + (uint32_t)s / (uint32_t)em.page]
                               : 0;
    }
  }
  const int64_t vis = min64((posv[b] + 1) / m, n_entries);
  if (vis <= k) return;  // everything visible is selected
  if (c0 >= vis) return;
  const int64_t c1 = min64(c0 + kDecChunk, vis);
  for (int i = tid; i < kCoarseBins; i += 256) lh[i] = 0;
  if (PAGED) {
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int64_t s = c0 + tid + 256 * i;
      if (s < c1) srow[s - c0] = (int64_t)tslot[i] * em.page + (uint32_t)s % (uint32_t)em.page;
    }
  }

  uint4 qa[NG];
  float wv[4];
  const int hrow = lane & 15;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int64_t row = (int64_t)b * HI + hrow;
    qa[g] = hrow < HI ? fp4x8_to_bf16(*(const uint32_t*)(qc + row * RB + g * 16 + lg * 4),
                                      qe[row * NG + g])
                      : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * lg + i;
    wv[i] = h < HI ? BF16::ld(wI, (int64_t)b * HI + h) : 0.f;
  }
  __syncthreads();
  const int64_t rb0 = PAGED ? 0 : (int64_t)b * n_entries;  // row of entry 0 (contiguous)
  const int64_t w0 = c0 + (int64_t)wave * (kDecChunk / 4);
  const int64_t w1 = min64(w0 + kDecChunk / 4, c1);
  // 64 keys per step: each lane loads 4 code bytes and the scale byte per
  // k-group for its 4 keys (16 keys per MFMA, 4 MFMA steps)
  auto load64 = [&](int64_t s0, uint32_t (&dc)[4][NG], uint32_t (&de)[4][NG]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t s = min64(s0 + u * 16 + (lane & 15), c1 - 1);  // past c1: not stored
      const int64_t row = PAGED ? srow[s - c0] : rb0 + s;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        dc[u][g] = *(const uint32_t*)(kc + row * RB + g * 16 + lg * 4);
        de[u][g] = ke[row * NG + g];
      }
    }
  };
  auto score64 = [&](int64_t s0, const uint32_t (&dc)[4][NG], const uint32_t (&de)[4][NG]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      f32x4_t acc = f32x4_t{};
#pragma unroll
      for (int g = 0; g < NG; ++g) mma16<BF16>(acc, qa[g], fp4x8_to_bf16(dc[u][g], de[u][g]));
      float p = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) p += wv[i] * relu(acc[i]);
      p = xlane_sum(p);
      const int64_t s = s0 + u * 16 + (lane & 15);
      if (lg == 0 && s < w1) {
        scores[(int64_t)b * n_entries + s] = p;
        atomicAdd(&lh[float_key(p) >> 21], 1);
      }
    }
  };
  uint32_t ka[4][NG], kae[4][NG], kb[4][NG], kbe[4][NG];
  if (w0 < w1) load64(w0, ka, kae);
  for (int64_t s0 = w0; s0 < w1; s0 += 128) {
    if (s0 + 64 < w1) load64(s0 + 64, kb, kbe);
    score64(s0, ka, kae);
    if (s0 + 64 >= w1) break;
    if (s0 + 128 < w1) load64(s0 + 128, ka, kae);
    score64(s0 + 64, kb, kbe);
  }
  __syncthreads();
  int* gh = hist + ((int64_t)b * ncopies + blockIdx.x % ncopies) * kCoarseBins;
  for (int i = tid; i < kCoarseBins; i += 256)
    if (lh[i]) atomicAdd(&gh[i], lh[i]);
}

// The coarse threshold bin T of the `need`-th largest key from a sequence's
// histogram copies: blocks of 256 bins are summed over the copies from the
// top bin down until they hold `need` keys.  Every thread gets res = (T,
// #keys in bins above T).  Requires at least `need` keys in the histogram.
CSA_DEV void dec_threshold(const int* __restrict__ h, int ncopies, int need, int* sh, int* res) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int above = 0;
  for (int blk = kCoarseBins / 256 - 1; blk >= 0; --blk) {
    const int bin = blk * 256 + tid;
    int v[kHistCopies];
#pragma unroll
    for (int r = 0; r < kHistCopies; ++r) v[r] = r < ncopies ? h[r * kCoarseBins + bin] : 0;
    int c = 0;
#pragma unroll
    for (int r = 0; r < kHistCopies; ++r) c += v[r];
    int suf = c;  // inclusive suffix sum over the wave's lanes
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_down(suf, o, 64);
      if (lane + o < 64) suf += y;
    }
    __syncthreads();
    if (lane == 0) sh[wave] = suf;
    __syncthreads();
    for (int w = wave + 1; w < 4; ++w) suf += sh[w];
    const int tot = sh[0] + sh[1] + sh[2] + sh[3];
    if (above + suf >= need && above + suf - c < need) {
      res[0] = bin;
      res[1] = above + suf - c;
    }
    if (above + tot >= need) break;  // uniform
    above += tot;
  }
  __syncthreads();
}

// D2: classify a chunk against T.  Thread j owns entries c0 + PER*j + u; one
// block-wide prefix sum per list gives each entry its slot in the chunk's
// slice of `lists` (sure from the front, ties from the back, both in index
// order).  Ties are also counted by their next 11 key bits (the fine
// histogram; few per chunk, spread over the bins).
__global__ __launch_bounds__(256) void dec_collect_kernel(const int64_t* __restrict__ posv,
                                                          int64_t n_entries, int m, int k,
                                                          const float* __restrict__ scores,
                                                          const int* __restrict__ hist,
                                                          int* __restrict__ fine,
                                                          int2* __restrict__ ccnt,
                                                          uint2* __restrict__ lists,
                                                          int64_t nchunks, int ncopies) {
  __shared__ int sh[8];
  __shared__ int res[2];
  const int b = blockIdx.y;
  const int64_t vis = min64((posv[b] + 1) / m, n_entries);
  if (vis <= k) return;
  const int64_t c0 = (int64_t)blockIdx.x * kDecChunk;
  if (c0 >= vis) return;
  const int64_t c1 = min64(c0 + kDecChunk, vis);
  const int tid = threadIdx.x;
  constexpr int PER = kDecChunk / 256;
  const float* sc = scores + (int64_t)b * n_entries;
  float v[PER];  // loads in flight during the threshold search
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int64_t s = c0 + tid * PER + u;
    v[u] = s < c1 ? sc[s] : 0.f;
  }
  dec_threshold(hist + (int64_t)b * ncopies * kCoarseBins, ncopies, k, sh, res);
  const uint32_t T = (uint32_t)res[0];
  uint32_t key[PER];
  int ns = 0, nt = 0;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int64_t s = c0 + tid * PER + u;
    key[u] = float_key(v[u]);
    const uint32_t bin = key[u] >> 21;
    ns += (s < c1 && bin > T);
    nt += (s < c1 && bin == T);
  }
  int totS, totT;
  int os = block_excl_scan(ns, sh, &totS);
  int ot = block_excl_scan(nt, sh + 4, &totT);
  const int cap = (int)(c1 - c0);
  uint2* L = lists + (int64_t)b * n_entries + c0;
  ot += cap - totT;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int64_t s = c0 + tid * PER + u;
    if (s >= c1) continue;
    const uint32_t bin = key[u] >> 21;
    if (bin > T) L[os++] = make_uint2(key[u], (uint32_t)s);
    else if (bin == T) {
      L[ot++] = make_uint2(key[u], (uint32_t)s);
      atomicAdd(&fine[(int64_t)b * kCoarseBins + ((key[u] >> 10) & (kCoarseBins - 1))], 1);
    }
  }
  if (tid == 0) ccnt[(int64_t)b * nchunks + blockIdx.x] = make_int2(totS, totT);
}

// Radix selection over a list in global memory of `cnt` (key, index) pairs,
// ordered by (key desc, index asc): marks how many to take via the composite
// 64-bit value (key << 32) | ~index.  Returns through res the composite
// threshold (hi, lo); items >= threshold are the `need` best.
CSA_DEV void list_select(const uint2* __restrict__ L, int cnt, int need, int* hist, int* res,
                         uint32_t* thr_hi, uint32_t* thr_lo) {
  uint64_t prefix = 0, pmask = 0;
  const int tid = threadIdx.x;
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < cnt; i += 256) {
      const uint2 e = L[i];
      const uint64_t ck = ((uint64_t)e.x << 32) | (uint64_t)(~e.y);
      if ((ck & pmask) == prefix) atomicAdd(&hist[(ck >> shift) & 255], 1);
    }
    __syncthreads();
    find_digit(hist, need, res);
    __syncthreads();
    need -= res[1];
    prefix |= (uint64_t)res[0] << shift;
    pmask |= (uint64_t)0xff << shift;
    __syncthreads();
  }
  *thr_hi = (uint32_t)(prefix >> 32);
  *thr_lo = (uint32_t)prefix;
}

// The same selection over n <= kTieLds pairs held in LDS whose keys share
// their top 11 bits (composite bits 63..53): digits of 8 bits from composite
// bit 52 down (the last one 5 bits wide), stopping at the first digit whose
// bucket is taken whole.
CSA_DEV uint64_t lds_list_select(const uint2* L, int n, int need, int* hist, int* res) {
  const int tid = threadIdx.x;
  uint64_t pmask = ~0ull << 53;
  uint64_t prefix = composite(L[0].x, L[0].y) & pmask;
  for (int shift = 45;; shift = shift > 5 ? shift - 8 : 0) {
    const uint32_t dmask = shift ? 255u : 31u;
    hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += 256) {
      const uint64_t ck = composite(L[i].x, L[i].y);
      if ((ck & pmask) == prefix) atomicAdd(&hist[(ck >> shift) & dmask], 1);
    }
    __syncthreads();
    find_digit(hist, need, res);
    __syncthreads();
    const int d = res[0];
    need -= res[1];
    prefix |= (uint64_t)d << shift;
    pmask |= (uint64_t)dmask << shift;
    const bool whole = hist[d] == need;  // uniform: LDS values after the barrier
    __syncthreads();
    if (whole || shift == 0) break;
  }
  return prefix;
}

// Position of v in the ascending list a[0, n): how many elements are below it.
CSA_DEV int lower_rank(const int32_t* a, int n, int32_t v) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < v) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// Output positions of a contiguous run a[j0, j1) of one ascending list merged
// with the ascending list o[0, no) (disjoint values): one binary search for the
// first element, then a walk, since the ranks grow along the run.
CSA_DEV void merge_run(const int32_t* a, int j0, int j1, const int32_t* o, int no,
                       int32_t* __restrict__ out) {
  if (j0 >= j1) return;
  int r = lower_rank(o, no, a[j0]);
  for (int j = j0; j < j1; ++j) {
    const int32_t x = a[j];
    while (r < no && o[r] < x) ++r;
    out[j + r] = x;
  }
}

// D3: one workgroup per sequence.  The chunks' sure entries and ties are
// gathered in chunk order, so both lists are in ascending index order.  The
// ties' fine histogram (bits 20..10 of the key, counted by D2) gives the fine
// bin F holding the last winner: ties above F are taken, those in F are
// ranked exactly (or, past 256 of them, the whole tie list is radix-selected);
// the winners are compacted in order and merged with the sure list.
__global__ __launch_bounds__(256) void dec_finalize_kernel(
    const int64_t* __restrict__ posv, int64_t n_entries, int m, int k,
    int* __restrict__ hist, int ncopies, int* __restrict__ fine, const int2* __restrict__ ccnt,
    const uint2* __restrict__ lists, uint2* __restrict__ flat, int64_t nchunks,
    int32_t* __restrict__ idx_out) {
  __shared__ int sh[8];
  __shared__ int res[2];
  __shared__ int h256[256];
  __shared__ int32_t surev[2048];
  __shared__ int32_t tsel[2048];
  __shared__ int ncand, ncand_f;
  __shared__ uint64_t fk[256];
  __shared__ uint64_t fk64_thr;
  __shared__ uint2 tls[kTieLds];
  __shared__ int2 ccs[kChunkLds];
  __shared__ int slotS[2048];
  __shared__ int slotT[kTieLds];
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t vis = min64((posv[b] + 1) / m, n_entries);
  int32_t* orow = idx_out + (int64_t)b * k;
  if (vis <= k) {
    for (int j = tid; j < k; j += 256) orow[j] = j < vis ? j : -1;
    return;
  }
  // the ties' fine histogram, loaded now so that its latency overlaps the
  // gather (thread j holds bins 8j .. 8j+7)
  int fl[kCoarseBins / 256];
  {
    int4* f4 = (int4*)(fine + (int64_t)b * kCoarseBins) + 2 * tid;
    const int4 x = f4[0], y = f4[1];
    fl[0] = x.x; fl[1] = x.y; fl[2] = x.z; fl[3] = x.w;
    fl[4] = y.x; fl[5] = y.y; fl[6] = y.z; fl[7] = y.w;
    f4[0] = make_int4(0, 0, 0, 0);  // after this thread's own loads of them
    f4[1] = make_int4(0, 0, 0, 0);
  }
  {  // the coarse copies were read by the collect pass, which has finished
    int4* h4 = (int4*)(hist + (int64_t)b * ncopies * kCoarseBins);
    for (int i = tid; i < ncopies * kCoarseBins / 4; i += 256) h4[i] = make_int4(0, 0, 0, 0);
  }
  // gather: thread j takes a contiguous run of chunks and writes the slice
  // slot of each of their entries into per-list slot tables in LDS (list
  // position -> slot), then every thread fetches a share of the entries, so
  // that the loads of many entries are in flight together
  const int nch = (int)((vis + kDecChunk - 1) / kDecChunk);
  const int CPT = (nch + 255) / 256;
  const int ch0 = min(tid * CPT, nch), ch1 = min(ch0 + CPT, nch);
  const int2* cg = ccnt + (int64_t)b * nchunks;
  for (int c = tid; c < nch && c < kChunkLds; c += 256) ccs[c] = cg[c];
  if (tid == 0) ncand = 0;
  __syncthreads();
  const int2* cc = nch <= kChunkLds ? ccs : cg;
  int my_s = 0, my_t = 0;
  for (int c = ch0; c < ch1; ++c) {
    const int2 v = cc[c];
    my_s += v.x;
    my_t += v.y;
  }
  int ns, nt;
  int ps = block_excl_scan(my_s, sh, &ns);
  int pt = block_excl_scan(my_t, sh + 4, &nt);
  const int need = k - ns;  // >= 1 by the threshold construction
  const bool in_lds = nt <= kTieLds;
  uint2* tdst = in_lds ? tls : flat + (int64_t)b * n_entries;
  const uint2* lb = lists + (int64_t)b * n_entries;
  for (int c = ch0; c < ch1; ++c) {
    const int2 v = cc[c];
    const int base = c * kDecChunk;
    const int tb = base + (int)min64(kDecChunk, vis - base) - v.y;  // the chunk's ties
    for (int i = 0; i < v.x; ++i) slotS[ps++] = base + i;
    if (in_lds)
      for (int i = 0; i < v.y; ++i) slotT[pt++] = tb + i;
    else
      for (int i = 0; i < v.y; ++i) tdst[pt++] = lb[tb + i];  // long lists: slow path
  }
  __syncthreads();
  constexpr int U = 8;
  for (int p0 = 0; p0 < ns; p0 += 256 * U) {
    uint32_t e[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = p0 + u * 256 + tid;
      e[u] = p < ns ? lb[slotS[p]].y : 0u;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = p0 + u * 256 + tid;
      if (p < ns) surev[p] = (int32_t)e[u];
    }
  }
  if (in_lds) {
    for (int p0 = 0; p0 < nt; p0 += 256 * U) {
      uint2 e[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int p = p0 + u * 256 + tid;
        e[u] = p < nt ? lb[slotT[p]] : make_uint2(0, 0);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int p = p0 + u * 256 + tid;
        if (p < nt) tls[p] = e[u];
      }
    }
  }
  // fine threshold bin F of the ties (the histogram holds exactly the nt ties)
  bin_threshold_vals<kCoarseBins>(fl, need, sh, res);
  const uint32_t F = (uint32_t)res[0];
  const int need2 = need - res[1];  // winners among the ties of fine bin F (>= 1)
  if (tid == (int)(F >> 3)) {
    int v = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) v = (int)(F & 7) == i ? fl[i] : v;
    ncand_f = v;
  }
  __syncthreads();
  const int nF = ncand_f;  // ties in fine bin F
  const uint2* tl = tdst;
  // composite key (score key << 32 | ~index): larger is better, all distinct;
  // thr = the need-th largest composite among the ties
  uint64_t thr;
  if (nF == need2) {  // fine bin F is taken whole
    const uint32_t kf = (tl[0].x & ~0x1fffffu) | (F << 10);
    thr = (uint64_t)kf << 32;
  } else if (nF <= 256) {  // rank the ties of F directly
    for (int i = tid; i < nt; i += 256) {
      const uint2 e = tl[i];
      if (((e.x >> 10) & (kCoarseBins - 1)) == F) fk[atomicAdd(&ncand, 1)] = composite(e.x, e.y);
    }
    __syncthreads();
    uint64_t ck = 0;
    int rank = 0;
    if (tid < nF) {
      ck = fk[tid];
      for (int j = 0; j < nF; ++j) rank += fk[j] > ck;
    }
    if (tid < nF && rank == need2 - 1) fk64_thr = ck;
    __syncthreads();
    thr = fk64_thr;
  } else if (in_lds) {
    thr = lds_list_select(tls, nt, need, h256, res);
  } else {
    uint32_t thi = 0, tlo = 0;
    list_select(tl, nt, need, h256, res, &thi, &tlo);
    thr = ((uint64_t)thi << 32) | tlo;
  }
  // winners in list (= index) order: each thread takes a contiguous run of the
  // ties, and one prefix sum over the threads' counts places them
  {
    const int TPT = (nt + 255) / 256;
    const int i0 = min(tid * TPT, nt), i1 = min(i0 + TPT, nt);
    int cnt = 0;
    for (int i = i0; i < i1; ++i) cnt += composite(tl[i].x, tl[i].y) >= thr;
    int tot;
    int off = block_excl_scan(cnt, sh, &tot);
    for (int i = i0; i < i1; ++i) {
      const uint2 e = tl[i];
      if (composite(e.x, e.y) >= thr) tsel[off++] = (int32_t)e.y;
    }
  }
  __syncthreads();
  // merge the two ascending lists (disjoint index sets): an element's output
  // position is its own rank plus its rank in the other list; each thread
  // places a contiguous run of each list
  {
    const int RS = (ns + 255) / 256, RT = (need + 255) / 256;
    merge_run(surev, min(tid * RS, ns), min(tid * RS + RS, ns), tsel, need, orow);
    merge_run(tsel, min(tid * RT, need), min(tid * RT + RT, need), surev, ns, orow);
  }
}

// ===========================================================================
// Host launchers
// ===========================================================================
#define CSA_INDEX_DISPATCH(HIv, CIv, ...)                                        \
  if (HIv == 4 && CIv == 64) { constexpr int HI = 4, CI = 64; __VA_ARGS__; }         \
  else if (HIv == 8 && CIv == 64) { constexpr int HI = 8, CI = 64; __VA_ARGS__; }    \
  else if (HIv == 16 && CIv == 64) { constexpr int HI = 16, CI = 64; __VA_ARGS__; }  \
  else if (HIv == 4 && CIv == 128) { constexpr int HI = 4, CI = 128; __VA_ARGS__; }  \
  else if (HIv == 8 && CIv == 128) { constexpr int HI = 8, CI = 128; __VA_ARGS__; }  \
  else if (HIv == 16 && CIv == 128) { constexpr int HI = 16, CI = 128; __VA_ARGS__; } \
  else return hipErrorInvalidValue;

hipError_t launch_index_scores_prefill(const csa_index_desc& d, const void* qI, const void* wI,
                                       const void* KI, void* scores, int64_t ld,
                                       hipStream_t st) {
  const int key_chunk = 2048;
  const int64_t nvis = (d.t0 + d.n) / d.m < d.n_entries ? (d.t0 + d.n) / d.m : d.n_entries;
  if (nvis == 0) return hipSuccess;
  CSA_INDEX_DISPATCH(d.n_heads, d.head_dim, {
    constexpr int TQ = 256 / HI;
    // the kernel addresses a workgroup's TQ score rows with 32-bit offsets
    if ((int64_t)TQ * ld >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    dim3 grid((unsigned)((d.n + TQ - 1) / TQ), (unsigned)((nvis + key_chunk - 1) / key_chunk));
    const bool sb = d.score_dtype == CSA_BF16;
    if (d.dtype == CSA_BF16 && sb)
      index_scores_prefill_kernel<BF16, HI, CI, uint16_t><<<grid, 256, 0, st>>>(
          (const BF16::S*)qI, (const BF16::S*)wI, (const BF16::S*)KI, d.n, d.n_entries, d.m,
          key_chunk, (uint16_t*)scores, ld, d.t0);
    else if (d.dtype == CSA_BF16)
      index_scores_prefill_kernel<BF16, HI, CI, float><<<grid, 256, 0, st>>>(
          (const BF16::S*)qI, (const BF16::S*)wI, (const BF16::S*)KI, d.n, d.n_entries, d.m,
          key_chunk, (float*)scores, ld, d.t0);
    else if (sb)
      index_scores_prefill_kernel<F32, HI, CI, uint16_t><<<grid, 256, 0, st>>>(
          (const float*)qI, (const float*)wI, (const float*)KI, d.n, d.n_entries, d.m, key_chunk,
          (uint16_t*)scores, ld, d.t0);
    else
      index_scores_prefill_kernel<F32, HI, CI, float><<<grid, 256, 0, st>>>(
          (const float*)qI, (const float*)wI, (const float*)KI, d.n, d.n_entries, d.m, key_chunk,
          (float*)scores, ld, d.t0);
  });
  return hipGetLastError();
}

// Rows are launched in bands by their visible-entry count (it grows with t):
// each band's kernel holds 16, 32, 48 or 64 entries per thread, so short rows do
// not pay for the longest one's registers and loops.
hipError_t launch_topk_rows_prefill(const csa_index_desc& d, const void* scores, int64_t ld,
                                    int32_t* idx_out, hipStream_t st) {
  // first row whose visible count exceeds `cap` entries
  auto band_end = [&](int64_t cap) {
    if (d.n_entries <= cap) return d.n;
    const int64_t e = (cap + 1) * d.m - 1 - d.t0;  // row of position (cap + 1) m - 1
    return e < 0 ? (int64_t)0 : e < d.n ? e : d.n;
  };
  const int64_t e16 = band_end(16 * 256), e32 = band_end(32 * 256), e48 = band_end(48 * 256);
  // Q: keys per thread offered for the lower bound, 256 * Q >= k
  const int q = d.k <= 512 ? 2 : d.k <= 1024 ? 4 : 0;
  auto band_t = [&](auto maxit, auto sc, int64_t r0, int64_t r1) {
    constexpr int MI = decltype(maxit)::value;
    typedef decltype(sc) SC;
    const SC* sp = (const SC*)scores;
    if (r1 <= r0) return;
    const unsigned g = (unsigned)(r1 - r0);
    if (q == 2)
      topk_rows_prefill_kernel<MI, 2, SC><<<g, 256, 0, st>>>(sp, ld, d.n, d.n_entries, d.m, d.k,
                                                             idx_out, r0, d.t0);
    else if (q == 4)
      topk_rows_prefill_kernel<MI, 4, SC><<<g, 256, 0, st>>>(sp, ld, d.n, d.n_entries, d.m, d.k,
                                                             idx_out, r0, d.t0);
    else
      topk_rows_prefill_kernel<MI, 0, SC><<<g, 256, 0, st>>>(sp, ld, d.n, d.n_entries, d.m, d.k,
                                                             idx_out, r0, d.t0);
  };
  auto band = [&](auto maxit, int64_t r0, int64_t r1) {
    if (d.score_dtype == CSA_BF16) band_t(maxit, uint16_t(), r0, r1);
    else band_t(maxit, float(), r0, r1);
  };
  band(std::integral_constant<int, 16>(), 0, e16);
  band(std::integral_constant<int, 32>(), e16, e32);
  band(std::integral_constant<int, 48>(), e32, e48);
  band(std::integral_constant<int, 64>(), e48, d.n);
  return hipGetLastError();
}

// D2 and D3 after the scores and histograms of a decode call are in place.
static hipError_t dec_select(const csa_index_desc& d, const DecWs& w, int64_t nch, int ncopies,
                             const int64_t* pos, int32_t* idx_out, hipStream_t st) {
  const dim3 grid((unsigned)nch, (unsigned)d.batch);
  dec_collect_kernel<<<grid, 256, 0, st>>>(pos, d.n_entries, d.m, d.k, w.scores, w.hist, w.fine,
                                           w.ccnt, w.lists, nch, ncopies);
  dec_finalize_kernel<<<d.batch, 256, 0, st>>>(pos, d.n_entries, d.m, d.k, w.hist, ncopies, w.fine,
                                               w.ccnt, w.lists, w.flat, nch, idx_out);
  return hipGetLastError();
}

hipError_t launch_index_topk_decode(const csa_index_desc& d, const void* qI, const void* wI,
                                    const void* KI, const int64_t* pos, int32_t* idx_out,
                                    void* wsp, hipStream_t st, EntryMap em) {
  DecWs w = carve(wsp, d);
  const int B = d.batch;
  const int64_t nch = dec_chunks(d);
  const int ncopies = dec_hist_copies(nch);
  const dim3 grid((unsigned)nch, (unsigned)B);
#define CSA_DSCORE(TT, PG)                                                                    \
  dec_score_kernel<TT, HI, CI, PG><<<grid, 256, 0, st>>>(                                     \
      (const TT::S*)qI, (const TT::S*)wI, (const TT::S*)KI, pos, d.n_entries, d.m, d.k,        \
      w.scores, w.hist, ncopies, em)
  CSA_INDEX_DISPATCH(d.n_heads, d.head_dim, {
    if (d.dtype == CSA_BF16) {
      if (em.table) CSA_DSCORE(BF16, true);
      else CSA_DSCORE(BF16, false);
    } else {
      if (em.table) CSA_DSCORE(F32, true);
      else CSA_DSCORE(F32, false);
    }
  });
#undef CSA_DSCORE
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return dec_select(d, w, nch, ncopies, pos, idx_out, st);
}

// ---------------------------------------------------------------------------
// Prefill rows with more visible entries than the register selector holds
// (long chunks of a chunked prefill): sub-batches of rows run the decode
// top-k, each row a "sequence" at position t0 + row, all rows sharing the
// one key table through an entry map of a single page (max_pages = 0, so
// every row reads slot 0, which holds page 0).
// ---------------------------------------------------------------------------
__global__ void long_rows_prep_kernel(int64_t* __restrict__ pos, int64_t first, int rows,
                                      int32_t* __restrict__ table) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < rows) pos[i] = first + i;
  if (i == 0) table[0] = 0;
}

static csa_index_desc long_rows_desc(const csa_index_desc& d) {
  csa_index_desc dd = d;
  const int64_t last = (d.t0 + d.n) / d.m;  // visible entries of the last row
  dd.n_entries = last < d.n_entries ? last : d.n_entries;
  // rows per sub-batch: about 2 GiB of decode workspace (20 B per entry and row)
  const int64_t r = ((int64_t)1 << 31) / (20 * (dd.n_entries > 0 ? dd.n_entries : 1));
  dd.batch = (int32_t)(r < 1 ? 1 : r > 1024 ? 1024 : r);
  if (dd.batch > d.n) dd.batch = (int32_t)(d.n > 0 ? d.n : 1);
  return dd;
}

size_t index_prefill_long_zero_bytes(const csa_index_desc& d) {
  return index_decode_zero_bytes(long_rows_desc(d));
}

size_t index_prefill_long_ws_bytes(const csa_index_desc& d) {
  const csa_index_desc dd = long_rows_desc(d);
  return index_decode_ws_bytes(dd) + align_up((size_t)dd.batch * 8) + 256;
}

hipError_t launch_index_topk_prefill_long(const csa_index_desc& d, const void* qI,
                                          const void* wI, const void* KI, int32_t* idx_out,
                                          void* ws, hipStream_t st) {
  const csa_index_desc dd = long_rows_desc(d);
  uint8_t* extra = (uint8_t*)ws + index_decode_ws_bytes(dd);
  int64_t* pos = (int64_t*)extra;
  int32_t* table = (int32_t*)(extra + align_up((size_t)dd.batch * 8));
  EntryMap em;
  em.table = table;
  em.page = (int32_t)(dd.n_entries > 0 ? dd.n_entries : 1);
  em.max_pages = 0;
  const size_t es = d.dtype == CSA_BF16 ? 2 : 4;
  for (int64_t r0 = 0; r0 < d.n; r0 += dd.batch) {
    csa_index_desc db = dd;
    db.batch = (int32_t)(d.n - r0 < dd.batch ? d.n - r0 : dd.batch);
    long_rows_prep_kernel<<<(db.batch + 255) / 256, 256, 0, st>>>(pos, d.t0 + r0, db.batch, table);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_index_topk_decode(db, (const uint8_t*)qI + r0 * d.n_heads * d.head_dim * es,
                                 (const uint8_t*)wI + r0 * d.n_heads * es, KI, pos,
                                 idx_out + r0 * d.k, ws, st, em);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_index_topk_decode_fp4(const csa_index_desc& d, const uint8_t* qc,
                                        const uint8_t* qe, const void* wI, const uint8_t* kc,
                                        const uint8_t* ke, const int64_t* pos, int32_t* idx_out,
                                        void* wsp, hipStream_t st, EntryMap em) {
  DecWs w = carve(wsp, d);
  const int64_t nch = dec_chunks(d);
  const int ncopies = dec_hist_copies(nch);
  const dim3 grid((unsigned)nch, (unsigned)d.batch);
  CSA_INDEX_DISPATCH(d.n_heads, d.head_dim, {
    if (em.table)
      dec_score_fp4_kernel<HI, CI, true><<<grid, 256, 0, st>>>(
          qc, qe, (const uint16_t*)wI, kc, ke, pos, d.n_entries, d.m, d.k, w.scores, w.hist,
          ncopies, em);
    else
      dec_score_fp4_kernel<HI, CI, false><<<grid, 256, 0, st>>>(
          qc, qe, (const uint16_t*)wI, kc, ke, pos, d.n_entries, d.m, d.k, w.scores, w.hist,
          ncopies, em);
  });
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return dec_select(d, w, nch, ncopies, pos, idx_out, st);
}

hipError_t launch_fp4_rotate_quant(int dtype, const void* x, int64_t rows, int width,
                                   uint8_t* codes, uint8_t* exps, const int64_t* pos,
                                   int64_t n_entries, int m, hipStream_t st, EntryMap em) {
  if (rows == 0) return hipSuccess;
  const unsigned g = (unsigned)((rows + 3) / 4);
#define CSA_FP4Q(TT, WW)                                                                      \
  fp4_rotate_quant_kernel<TT, WW><<<g, 256, 0, st>>>((const TT::S*)x, rows, codes, exps, pos, \
                                                     n_entries, m, em)
  if (width == 64) {
    if (dtype == CSA_BF16) CSA_FP4Q(BF16, 64);
    else CSA_FP4Q(F32, 64);
  } else {
    if (dtype == CSA_BF16) CSA_FP4Q(BF16, 128);
    else CSA_FP4Q(F32, 128);
  }
#undef CSA_FP4Q
  return hipGetLastError();
}

}  // namespace csa
