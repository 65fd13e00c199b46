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
// Prefill scoring over FP4 q^I and keys (the E2M1 codes and block exponents
// of the quantised indexer path): the workgroup shape, key blocks and head
// reduction of index_scores_prefill_kernel, with the products on the scaled
// E2M1 matrix instruction, one per 64 channels for 32 keys and 32 rows.  A
// key block's codes are staged in LDS by direct loads (rows of CI/2 bytes,
// 16-byte granules XOR-permuted by key so that each 16-lane group of a read,
// 16 keys with one granule each, hits distinct banks); its exponent bytes
// come through registers into LDS with the block's prefetch.
// ===========================================================================
template <int HI, int CI, class SC>
__global__ __launch_bounds__(256) void index_scores_prefill_fp4_kernel(
    const uint8_t* __restrict__ qc, const uint8_t* __restrict__ qe, const uint16_t* __restrict__ wI,
    const uint8_t* __restrict__ kc, const uint8_t* __restrict__ ke, int64_t n, int64_t n_entries,
    int m, int key_chunk, SC* __restrict__ scores, int64_t ld, int64_t t0) {
  constexpr int NG = CI / 32;       // scale blocks per row
  constexpr int NH = CI / 64;       // 64-channel k-groups: one instruction each
  constexpr int RBC = CI / 2;       // code bytes per row
  constexpr int GR = RBC / 16;      // 16-byte granules per row
  constexpr int KPR = 256 / RBC;    // rows per 256 bytes (one 16-lane read group)
  constexpr int RB = 2;             // 32-row blocks per wave
  constexpr int ROWS = 4 * RB * 32; // (query, head) rows per workgroup
  constexpr int TQ = ROWS / HI;     // queries per workgroup
  constexpr int KB = 128;           // keys per staged block
  constexpr int KPI = 1024 / RBC;   // keys per 64-lane DMA
  constexpr int DPW = KB / KPI / 4; // DMA instructions per wave per block
  constexpr int EB = KB * NG;       // exponent bytes per block
  constexpr int EPT = EB / 256;     // exponent bytes per thread
  static_assert(DPW >= 1 && EB % 256 == 0, "key block layout");
  __shared__ __align__(16) uint8_t sK[2][KB * RBC];
  __shared__ uint8_t sE[2][EB];
  auto swz = [](int key) { return (key / KPR) % GR; };

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
      const int d = wave + 4 * u;           // DMA index within the block
      const int key = d * KPI + lane / GR;  // key within the block
      const int pos = lane % GR;            // LDS granule position
      const int64_t sidx = min64(k0 + key, kend - 1);
      lds_dma16(kc + sidx * RBC + 16 * (pos ^ swz(key)), &sK[buf][d * 1024]);
    }
  };
  auto load_exps = [&](int64_t k0, uint32_t (&e)[EPT]) {
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const int bi = tid + 256 * j;  // byte of the block: key bi / NG, scale block bi % NG
      e[j] = ke[min64(k0 + bi / NG, kend - 1) * NG + bi % NG];
    }
  };
  auto store_exps = [&](int buf, const uint32_t (&e)[EPT]) {
#pragma unroll
    for (int j = 0; j < EPT; ++j) sE[buf][tid + 256 * j] = (uint8_t)e[j];
  };
  issue_block(kbeg, 0);
  uint32_t en[EPT];
  load_exps(kbeg, en);

  // A operands (query rows: codes and scale per lane) and per-row weights,
  // held for the whole chunk; a row past n is zero with scale 1
  uint4 qa[RB][NH];
  uint32_t qs[RB][NH];
  float wv[RB][16];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = wave * (RB * 32) + rb * 32 + (lane & 31);
    const int64_t t = q0 + row / HI;
    const int h = row % HI;
    const bool ok = t < n;
#pragma unroll
    for (int g = 0; g < NH; ++g) {
      const int blk = 2 * g + hl;
      qa[rb][g] = ok ? *(const uint4*)(qc + (t * HI + h) * RBC + blk * 16) : make_uint4(0, 0, 0, 0);
      qs[rb][g] = ok ? (uint32_t)qe[(t * HI + h) * NG + blk] : 127u;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int rr = wave * (RB * 32) + rb * 32 + 8 * (i >> 2) + 4 * hl + (i & 3);
      const int64_t tt = q0 + rr / HI;
      wv[rb][i] = tt < n ? BF16::ld(wI, tt * HI + rr % HI) : 0.f;
    }
  }
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
  store_exps(0, en);
  wait_vmem();
  __syncthreads();
  SC* srow0 = scores + q0 * ld;
  const int ld32 = (int)ld;

  const int nblk = (int)((kend - kbeg + KB - 1) / KB);
  for (int bi = 0; bi < nblk; ++bi) {
    const int buf = bi & 1;
    const int64_t kb0 = kbeg + (int64_t)bi * KB;
    const bool more = bi + 1 < nblk;
    if (more) {
      issue_block(kb0 + KB, buf ^ 1);
      load_exps(kb0 + KB, en);
    }
    const int nsub = (int)min64(KB / 32, (kend - kb0 + 31) / 32);
    for (int sb = 0; sb < nsub; ++sb) {
      const int kk = sb * 32 + (lane & 31);  // this lane's key within the block
      const uint8_t* krow = &sK[buf][kk * RBC];
      f32x16_t acc[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) acc[rb] = f32x16_t{};
#pragma unroll
      for (int g = 0; g < NH; ++g) {
        const int gi = 2 * g + hl;
        const uint4 kb = *(const uint4*)(krow + 16 * (gi ^ swz(kk)));
        const uint32_t ks = sE[buf][kk * NG + gi];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) mma32_fp4(acc[rb], qa[rb][g], qs[rb][g], kb, ks);
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
        const int tr = (wave * (RB * 32) + rb * 32) / HI;
        auto put = [&](int tq, int vq, float v) {  // query q0 + tq, visible count vq
          if (sok && si < vq) {
            if constexpr (sizeof(SC) == 2) srow0[(uint32_t)(tq * ld32 + si)] = f32_to_bf16(v);
            else srow0[(uint32_t)(tq * ld32 + si)] = v;
          }
        };
        if (HI == 4) {
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) put(tr + 2 * gq + hl, vis[rb][gq], part[gq]);
        } else if (HI == 8) {
          const float v0 = swap32_pair_add(part[0], part[2]);
          const float v1 = swap32_pair_add(part[1], part[3]);
          put(tr + 2 * hl, vis[rb][0], v0);
          put(tr + 2 * hl + 1, vis[rb][1], v1);
        } else {
          put(tr + hl, vis[rb][0], swap32_pair_add(part[0] + part[1], part[2] + part[3]));
        }
      }
    }
    if (more) store_exps(buf ^ 1, en);
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

// The 48-key band runs at four waves per SIMD (128 registers, one spilled
// value) instead of three: its rows are latency-bound, and the fourth resident
// workgroup hides more of that latency.  The 64-key band would spill heavily
// at that bound; the shorter bands gained nothing measurable from one more wave.
template <int MAXIT, int Q, class SC>
__global__ __launch_bounds__(256, MAXIT == 48 ? 4 : 1) void topk_rows_prefill_kernel(const SC* __restrict__ scores,
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
//   D1 one workgroup per chunk of 1024 keys scores them (16x16 matrix-core
//      tiles, keys streamed straight from memory -- this pass moves the
//      step's dominant bytes), stores the scores, and keeps the chunk's L
//      best entries as its candidates, in index order, with the L-th best.
//      Entries are ranked by the composite (key << 32 | ~index): higher score
//      first, ties to the smaller index, all distinct.
//   D2 one workgroup per sequence gathers every chunk's candidates into LDS
//      (adding the step's own new entry when D1 left it out), finds the k-th
//      best composite by a radix selection in LDS and emits the winners in
//      index order.  A chunk that offered L candidates and whose L-th best
//      still beats that threshold may hold more winners than it offered;
//      then the workgroup selects exactly over all the row's stored scores
//      instead (slow, and rare: L is twice a chunk's expected share of the k,
//      plus 16).
// No state carries from one call to the next: the workspace needs no
// clearing, and nothing depends on the order in which workgroups run.
// ===========================================================================
constexpr int kDecChunk = 1024;  // keys per scoring workgroup
constexpr int kCandLds = 8192;   // candidates D2 holds in LDS (64 KiB)

struct DecWs {  // carve-up of the decode workspace
  float* scores;  // [B][n_entries]
  uint2* cand;    // [B][chunks][L] (key, index), index order
  uint4* cmeta;   // [B][chunks]: (count, full, L-th key, L-th index)
};

static size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

static int64_t dec_chunks(const csa_index_desc& d) {
  return (d.n_entries + kDecChunk - 1) / kDecChunk;
}

// Candidates per chunk: twice a chunk's expected share of the k winners,
// plus 16, within what D2 holds in LDS (one slot kept for the new entry).
static int dec_cand_per_chunk(const csa_index_desc& d) {
  const int64_t nch = dec_chunks(d) > 0 ? dec_chunks(d) : 1;
  int64_t L = 2 * (int64_t)d.k / nch + 16;
  L = (L + 7) & ~(int64_t)7;
  if (L > kDecChunk) L = kDecChunk;
  const int64_t cap = (kCandLds - 1) / nch;
  if (L > cap) L = cap;  // D2 then falls back for rows with more chunks
  return (int)(L < 1 ? 1 : L);
}

static DecWs carve(void* ws, const csa_index_desc& d) {
  uint8_t* p = (uint8_t*)ws;
  DecWs w;
  const size_t B = d.batch, ne = d.n_entries, nc = dec_chunks(d), L = dec_cand_per_chunk(d);
  w.scores = (float*)p; p += align_up(B * ne * 4);
  w.cand = (uint2*)p; p += align_up(B * nc * L * 8);
  w.cmeta = (uint4*)p;
  return w;
}

size_t index_decode_zero_bytes(const csa_index_desc&) { return 0; }

size_t index_decode_ws_bytes(const csa_index_desc& d) {
  const size_t B = d.batch, ne = d.n_entries, nc = dec_chunks(d), L = dec_cand_per_chunk(d);
  return align_up(B * ne * 4) + align_up(B * nc * L * 8) + align_up(B * nc * 16);
}

// Block-wide max / min of a uint32 over 256 threads (sh: 8 ints of LDS).
CSA_DEV uint32_t block_max_u32(uint32_t v, int* sh) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = (int)v;
  __syncthreads();
  return max(max((uint32_t)sh[0], (uint32_t)sh[1]), max((uint32_t)sh[2], (uint32_t)sh[3]));
}
CSA_DEV uint32_t block_min_u32(uint32_t v, int* sh) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o, 64));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[4 + (threadIdx.x >> 6)] = (int)v;
  __syncthreads();
  return min(min((uint32_t)sh[4], (uint32_t)sh[5]), min((uint32_t)sh[6], (uint32_t)sh[7]));
}

// D1's chunk-local selection.  ls[0, c) holds the chunk's keys in index order
// (entry c0 + i at i); thread j owns entries 4j .. 4j+3.  Keeps the L best
// by composite (all of them when c <= L) in cand, in index order, and
// records (count, full, L-th best key, its index) in *meta.  hist: 256 ints
// of LDS.
CSA_DEV void chunk_candidates(const uint32_t* ls, int c, int L, int64_t c0, int* hist, int* sh,
                              int* res, uint2* __restrict__ cand, uint4* __restrict__ meta) {
  const int tid = threadIdx.x;
  uint32_t key[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) key[u] = 4 * tid + u < c ? ls[4 * tid + u] : 0u;
  uint32_t V = 0;  // the L-th largest key
  int take = 0;    // how many entries of key V are kept (the smallest indices)
  if (c > L) {
    // the bits above the highest one where the keys differ are common: the
    // radix starts below them, so that its first digit spreads the keys
    uint32_t kmax = 0, kmin = 0xffffffffu;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (4 * tid + u < c) { kmax = max(kmax, key[u]); kmin = min(kmin, key[u]); }
    kmax = block_max_u32(kmax, sh);
    kmin = block_min_u32(kmin, sh);
    int hi = kmax == kmin ? -1 : 31 - __builtin_clz(kmax ^ kmin);  // highest undecided bit
    uint32_t mask = hi >= 31 ? 0u : ~((2u << hi) - 1u);
    uint32_t prefix = kmax & mask;
    int need = L;
    while (hi >= 0) {
      const int lo = hi >= 7 ? hi - 7 : 0;
      const uint32_t dm = (2u << (hi - lo)) - 1u;
      hist[tid] = 0;
      __syncthreads();
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (4 * tid + u < c && (key[u] & mask) == prefix) atomicAdd(&hist[(key[u] >> lo) & dm], 1);
      __syncthreads();
      find_digit(hist, need, res);
      __syncthreads();
      const int d = res[0];
      need -= res[1];
      prefix |= (uint32_t)d << lo;
      mask |= dm << lo;
      __syncthreads();
      hi = lo - 1;
    }
    V = prefix;  // the L-th largest key itself (every bit decided)
    take = need;
  }
  // tie ranks in index order, then output slots in index order
  int nt = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) nt += (c > L && 4 * tid + u < c && key[u] == V);
  int tot;
  int tr = block_excl_scan(nt, sh, &tot);
  bool keep[4];
  int nk = 0;
  int lth = -1;  // the L-th best entry, if this thread holds it (tie rank take - 1)
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = 4 * tid + u;
    bool kp = i < c;
    if (c > L && kp) {
      if (key[u] == V) {
        kp = tr < take;
        if (tr == take - 1) lth = i;
        ++tr;
      } else {
        kp = key[u] > V;
      }
    }
    keep[u] = kp;
    nk += kp;
  }
  int off = block_excl_scan(nk, sh + 4, &tot);
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (keep[u]) cand[off++] = make_uint2(key[u], (uint32_t)(c0 + 4 * tid + u));
  if (c <= L) {
    if (tid == 0) *meta = make_uint4((uint32_t)c, 0u, 0u, 0u);
  } else if (lth >= 0) {
    *meta = make_uint4((uint32_t)L, 1u, V, (uint32_t)(c0 + lth));
  }
}

// PAGED: KI is a page pool.  The page-table slots of the chunk's entries are
// read first, before the position (they lie in the table whether or not the
// entries are visible; only the visible ones' values are used), and turned
// into pool rows in LDS, so no key load waits on a table read.
template <class T, int HI, int CI, bool PAGED>
__global__ __launch_bounds__(256) void dec_score_kernel(
    const typename T::S* __restrict__ qI, const typename T::S* __restrict__ wI,
    const typename T::S* __restrict__ KI, const int64_t* __restrict__ posv, int64_t n_entries,
    int m, int k, float* __restrict__ scores, uint2* __restrict__ cand, uint4* __restrict__ cmeta,
    int L, int64_t nch, EntryMap em) {
  typedef typename T::S S;
  constexpr int E = 16 / (int)sizeof(S);
  constexpr int KGE = 4 * E;      // elements per 16x16 k-group
  constexpr int NG = CI / KGE;
  __shared__ uint32_t ls[kDecChunk];  // the chunk's keys, in index order
  __shared__ int hist[256];
  __shared__ int sh[8];
  __shared__ int res[2];
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
  const int64_t tpos = posv[b];
  const int64_t vis = min64((tpos + 1) / m, n_entries);
  if (vis <= k) return;  // everything visible is selected
  // Only the entries that exist before position tpos's own step: the one
  // that step emits (when (tpos + 1) % m == 0) is scored by the selection
  // pass, so this kernel may run while the compressor writes it.
  const int64_t vpre = min64(tpos / m, n_entries);
  if (c0 >= vpre) return;
  const int64_t c1 = min64(c0 + kDecChunk, vpre);
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
        ls[s - c0] = float_key(p);
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
  const int64_t slot = (int64_t)b * nch + blockIdx.x;
  chunk_candidates(ls, (int)(c1 - c0), L, c0, hist, sh, res, cand + slot * L, cmeta + slot);
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

// D1 over FP4 keys: q^I and the keys stay E2M1 codes and block exponents
// (a quarter of the bf16 bytes) and go straight into the scaled FP4 matrix
// instruction, one per 64 channels for 32 keys: A = q^I (row = head, rows
// past HI zero), B = 32 keys (column = key); lane l loads 16 code bytes and
// the scale byte of channel block (l / 32) of its key (l % 32).  Each product
// of two E2M1 values is exact and a block's 32 of them sum exactly, so a
// score differs from the dequantised dot product only by the fp32 rounding
// of the block sums' accumulation.  Head sum and histogram as dec_score_kernel.
template <int HI, int CI, bool PAGED>
__global__ __launch_bounds__(256) void dec_score_fp4_kernel(
    const uint8_t* __restrict__ qc, const uint8_t* __restrict__ qe, const uint16_t* __restrict__ wI,
    const uint8_t* __restrict__ kc, const uint8_t* __restrict__ ke,
    const int64_t* __restrict__ posv, int64_t n_entries, int m, int k, float* __restrict__ scores,
    uint2* __restrict__ cand, uint4* __restrict__ cmeta, int L, int64_t nch, EntryMap em) {
  constexpr int NG = CI / 32;  // 32-value scale blocks per row
  constexpr int NH = CI / 64;  // 64-channel k-groups per row: one instruction each
  constexpr int RB = CI / 2;   // code bytes per row
  constexpr int KW = kDecChunk / 4;  // keys per wave
  constexpr int NU = KW / 32;        // 32-key groups per wave
  constexpr int NQ = HI > 8 ? 8 : 4; // accumulators that hold heads < HI
  static_assert(HI <= 16, "heads 16..31 of the 32-row block are not summed");
  __shared__ uint32_t ls[kDecChunk];
  __shared__ int hist[256];
  __shared__ int sh[8];
  __shared__ int res[2];
  __shared__ int64_t srow[PAGED ? kDecChunk : 1];  // pool rows (as in dec_score_kernel)
  const int b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, kg = lane >> 5;
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
  if (PAGED) {
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int64_t s = c0 + tid + 256 * i;
      if (s < c1) srow[s - c0] = (int64_t)tslot[i] * em.page + (uint32_t)s % (uint32_t)em.page;
    }
  }

  // q^I rows as the A operand; a row past HI is zero with scale 1 (a finite
  // scale keeps its products zero)
  uint4 qa[NH];
  uint32_t qs[NH];
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    const int64_t row = (int64_t)b * HI + col;
    const int blk = 2 * h + kg;
    qa[h] = col < HI ? *(const uint4*)(qc + row * RB + blk * 16) : make_uint4(0, 0, 0, 0);
    qs[h] = col < HI ? (uint32_t)qe[row * NG + blk] : 127u;
  }
  // weights of the heads in this lane's accumulators: acc[4j+i] is head 8j + 4*kg + i
  float wv[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int h = 8 * (q / 4) + 4 * kg + (q % 4);
    wv[q] = h < HI ? BF16::ld(wI, (int64_t)b * HI + h) : 0.f;
  }
  __syncthreads();
  const int64_t rb0 = PAGED ? 0 : (int64_t)b * n_entries;  // row of entry 0 (contiguous)
  const int64_t w0 = c0 + (int64_t)wave * KW;
  const int64_t w1 = min64(w0 + KW, c1);
  if (w0 < w1) {
    // every load of the wave in flight at once; a key past c1 re-reads row
    // c1 - 1 and is not stored
    uint4 kw[NU][NH];
    uint32_t ks[NU][NH];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int64_t s = min64(w0 + u * 32 + col, c1 - 1);
      const int64_t row = PAGED ? srow[s - c0] : rb0 + s;
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        kw[u][h] = *(const uint4*)(kc + row * RB + (2 * h + kg) * 16);
        ks[u][h] = ke[row * NG + 2 * h + kg];
      }
    }
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      if (w0 + u * 32 >= w1) break;  // uniform
      f32x16_t acc = f32x16_t{};
#pragma unroll
      for (int h = 0; h < NH; ++h) mma32_fp4(acc, qa[h], qs[h], kw[u][h], ks[u][h]);
      float p = 0.f;
#pragma unroll
      for (int q = 0; q < NQ; ++q) p += wv[q] * relu(acc[q]);
      p += __shfl_xor(p, 32, 64);  // the other half of the heads
      const int64_t s = w0 + u * 32 + col;
      if (kg == 0 && s < w1) {
        scores[(int64_t)b * n_entries + s] = p;
        ls[s - c0] = float_key(p);
      }
    }
  }
  __syncthreads();
  const int64_t slot = (int64_t)b * nch + blockIdx.x;
  chunk_candidates(ls, (int)(c1 - c0), L, c0, hist, sh, res, cand + slot * L, cmeta + slot);
}

// Index score of one key row (eq 16 for one entry), computed by one wave:
// lane l takes head l / 4 and a quarter of the key's channels, in a fixed
// order, so every caller gets the same value bit for bit.
template <class T, int HI, int CI>
CSA_DEV float one_entry_score(const typename T::S* __restrict__ q,
                              const typename T::S* __restrict__ w,
                              const typename T::S* __restrict__ key, int lane) {
  constexpr int DPL = CI / 4;
  const int h = lane >> 2, part = lane & 3;
  float dot = 0.f;
  if (h < HI) {
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
      const int dch = part * DPL + i;
      dot = fmaf(T::ld(q, h * CI + dch), T::ld(key, dch), dot);
    }
  }
  dot += __shfl_xor(dot, 1, 64);
  dot += __shfl_xor(dot, 2, 64);
  const float p = (h < HI && part == 0) ? T::ld(w, h) * relu(dot) : 0.f;
  return wave_sum(p);
}

// Radix selection of the k-th best composite: digits of up to 8 bits from
// composite bit `hi` down (the bits above it are `prefix`, common to every
// item), stopping at the first digit whose bucket is taken whole (the lower
// bits are then zero in the result).  Items >= the result are exactly the
// `need` best.  get(i) gives item i's composite; hist: 256 ints of LDS.
template <class GET>
CSA_DEV uint64_t radix_select64(GET get, int64_t n, int need, int hi, uint64_t prefix,
                                int* hist, int* res) {
  const int tid = threadIdx.x;
  uint64_t pmask = hi >= 63 ? 0ull : ~((2ull << hi) - 1ull);
  while (hi >= 0) {
    const int lo = hi >= 7 ? hi - 7 : 0;
    const uint32_t dm = (2u << (hi - lo)) - 1u;
    hist[tid] = 0;
    __syncthreads();
    for (int64_t i = tid; i < n; i += 256) {
      const uint64_t ck = get(i);
      if ((ck & pmask) == prefix) atomicAdd(&hist[(uint32_t)(ck >> lo) & dm], 1);
    }
    __syncthreads();
    find_digit(hist, need, res);
    __syncthreads();
    const int d = res[0];
    need -= res[1];
    prefix |= (uint64_t)d << lo;
    pmask |= (uint64_t)dm << lo;
    const bool whole = hist[d] == need;  // uniform: LDS values after the barrier
    __syncthreads();
    if (whole) break;
    hi = lo - 1;
  }
  return prefix;
}

// The highest composite bit where items can differ, and the common bits above
// it, from the block-wide max and min of the items' keys.
CSA_DEV int common_prefix(uint32_t kmax, uint32_t kmin, uint64_t* prefix) {
  if (kmax == kmin) {  // every key equal: the indices decide
    *prefix = (uint64_t)kmax << 32;
    return 31;
  }
  const int hb = 31 - __builtin_clz(kmax ^ kmin);
  const uint32_t m = hb >= 31 ? 0u : ~((2u << hb) - 1u);
  *prefix = (uint64_t)(kmax & m) << 32;
  return 32 + hb;
}

constexpr int kSelThreads = 1024;  // one selection workgroup per sequence

// Block-wide helpers for a workgroup of NT threads (NT / 64 waves): the
// selection runs wider than the scorer, whose helpers above assume four.
template <int NT>
CSA_DEV int block_excl_scan_n(int v, int* tmp, int* total) {
  constexpr int NW = NT / 64;
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
  int base = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    base += w < wave ? tmp[w] : 0;
    all += tmp[w];
  }
  *total = all;
  return base + x - v;
}
// Block-wide max of `mx` and min of `mn` with one set of barriers (sh: 2 NT / 64
// ints of LDS).
template <int NT>
CSA_DEV void block_maxmin_u32(uint32_t& mx, uint32_t& mn, int* sh) {
  constexpr int NW = NT / 64;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, o, 64));
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, o, 64));
  }
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    sh[threadIdx.x >> 6] = (int)mx;
    sh[NW + (threadIdx.x >> 6)] = (int)mn;
  }
  __syncthreads();
  uint32_t a = (uint32_t)sh[0], b = (uint32_t)sh[NW];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    a = max(a, (uint32_t)sh[w]);
    b = min(b, (uint32_t)sh[NW + w]);
  }
  __syncthreads();  // sh is reused by the next call
  mx = a;
  mn = b;
}

// radix_select64 for NT threads (hist: two buffers of 256 ints of LDS).  The
// passes alternate between the buffers: a pass clears the next pass's buffer
// once its own counts are in (every read of that buffer, by the pass before,
// precedes that barrier), so a pass needs two barriers instead of four.
template <int NT, class GET>
CSA_DEV uint64_t radix_select64_n(GET get, int64_t n, int need, int hi, uint64_t prefix,
                                  int* hist, int* res) {
  const int tid = threadIdx.x;
  uint64_t pmask = hi >= 63 ? 0ull : ~((2ull << hi) - 1ull);
  for (int i = tid; i < 256; i += NT) hist[i] = 0;
  __syncthreads();
  int pb = 0;
  while (hi >= 0) {
    int* h = hist + 256 * pb;
    int* hn = hist + 256 * (pb ^ 1);
    const int lo = hi >= 7 ? hi - 7 : 0;
    const uint32_t dm = (2u << (hi - lo)) - 1u;
    for (int64_t i = tid; i < n; i += NT) {
      const uint64_t ck = get(i);
      if ((ck & pmask) == prefix) atomicAdd(&h[(uint32_t)(ck >> lo) & dm], 1);
    }
    __syncthreads();  // the counts are in; the pass before has read hn
    for (int i = tid; i < 256; i += NT) hn[i] = 0;
    find_digit(h, need, res);
    __syncthreads();  // res and the cleared hn are visible
    const int d = res[0];
    need -= res[1];
    prefix |= (uint64_t)d << lo;
    pmask |= (uint64_t)dm << lo;
    const bool whole = h[d] == need;  // uniform: LDS values after the barrier
    if (whole) break;
    hi = lo - 1;
    pb ^= 1;
  }
  return prefix;
}

// D2: one workgroup per sequence (see the section comment).  FOLD: the
// entry emitted by position t's own step (when (t + 1) % m == 0) was left
// out of D1; it is scored here and joins the candidates.
template <class TS, int HI, int CI, bool FOLD, int NT>
__global__ __launch_bounds__(NT) void dec_select_kernel(
    const int64_t* __restrict__ posv, int64_t n_entries, int m, int k,
    const float* __restrict__ scores, const uint2* __restrict__ cand,
    const uint4* __restrict__ cmeta, int64_t nchunks, int L, const typename TS::S* __restrict__ qI,
    const typename TS::S* __restrict__ wI, const typename TS::S* __restrict__ KI, EntryMap em,
    int32_t* __restrict__ idx_out) {
  __shared__ uint2 cl[kCandLds];
  __shared__ int coff[kCandLds];  // per chunk: its first slot in cl, or -1 past its count
  __shared__ int hist[2 * 256];
  __shared__ int sh[2 * NT / 64];
  __shared__ int res[2];
  __shared__ float snew;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t tpos = posv[b];
  const int64_t vis = min64((tpos + 1) / m, n_entries);
  int32_t* orow = idx_out + (int64_t)b * k;
  if (vis <= k) {
    for (int j = tid; j < k; j += NT) orow[j] = j < vis ? j : -1;
    return;
  }
  const int64_t e_new = (FOLD && (tpos + 1) % m == 0 && (tpos + 1) / m <= n_entries) ? vis - 1 : -1;
  const int64_t vsc = e_new >= 0 ? vis - 1 : vis;  // entries D1 scored
  const int nch = (int)((vsc + kDecChunk - 1) / kDecChunk);
  const float* sc = scores + (int64_t)b * n_entries;
  // chunk counts: thread j sums a contiguous run of chunks, one prefix sum
  // places the runs in chunk (= index) order
  const int CPT = (nch + NT - 1) / NT;
  const int ch0 = min(tid * CPT, nch), ch1 = min(ch0 + CPT, nch);
  const uint4* meta = cmeta + (int64_t)b * nchunks;
  int my = 0;
  bool full_any = false;  // one of this thread's chunks may hide winners
  uint4 m0 = make_uint4(0, 0, 0, 0);  // this thread's first chunk, kept for the vote
  for (int c = ch0; c < ch1; ++c) {
    const uint4 mt = meta[c];
    if (c == ch0) m0 = mt;
    my += (int)mt.x;
  }
  if (e_new >= 0) {  // uniform: one wave scores the new entry
    if (tid < 64) {
      const float p = one_entry_score<TS, HI, CI>(qI + (int64_t)b * HI * CI, wI + (int64_t)b * HI,
                                                  KI + em.row(b, e_new, n_entries) * CI, tid);
      if (tid == 0) snew = p;
    }
  }
  int tot;
  int off = block_excl_scan_n<NT>(my, sh, &tot);  // its barriers also publish snew
  const int ntot = tot + (e_new >= 0);
  const uint32_t new_key = e_new >= 0 ? float_key(snew) : 0u;
  bool fallback = ntot > kCandLds || ntot < k;  // (fewer than k: not reached, see L)
  uint64_t thr = 0;
  if (!fallback) {
    // slot p = c * L + i of the candidate buffer goes to cl[coff[c] + i] when
    // i < count(c): every thread loads independent slots, 8 in flight
    for (int c = ch0; c < ch1; ++c) {
      coff[c] = off;
      off += (int)meta[c].x;
    }
    __syncthreads();
    const uint2* cb = cand + (int64_t)b * nchunks * L;
    const int nslot = nch * L;
    for (int p0 = tid; p0 < nslot; p0 += NT * 8) {
      uint2 v[8];
      int dst[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int p = p0 + NT * u;
        dst[u] = -1;
        if (p < nslot) {
          const int c = p / L, i = p - c * L;
          const int lim = (c + 1 < nch ? coff[c + 1] : tot) - coff[c];  // count(c)
          if (i < lim) {
            dst[u] = coff[c] + i;
            v[u] = cb[p];
          }
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (dst[u] >= 0) cl[dst[u]] = v[u];
    }
    if (e_new >= 0 && tid == 0) cl[tot] = make_uint2(new_key, (uint32_t)e_new);
    __syncthreads();
    uint32_t kmax = 0, kmin = 0xffffffffu;
    for (int i = tid; i < ntot; i += NT) {
      kmax = max(kmax, cl[i].x);
      kmin = min(kmin, cl[i].x);
    }
    uint64_t pre;
    block_maxmin_u32<NT>(kmax, kmin, sh);
    const int hi = common_prefix(kmax, kmin, &pre);
    thr = radix_select64_n<NT>([&](int64_t i) { return composite(cl[i].x, cl[i].y); }, ntot, k, hi,
                               pre, hist, res);
    // a chunk that kept L entries whose L-th best beats thr may hide winners
    for (int c = ch0; c < ch1; ++c) {
      const uint4 mt = c == ch0 ? m0 : meta[c];
      full_any |= mt.y != 0 && composite(mt.z, mt.w) > thr;
    }
  }
  fallback = __syncthreads_or(fallback || full_any);
  if (!fallback) {
    // winners in list (= index) order: contiguous runs, one prefix sum
    const int TPT = (ntot + NT - 1) / NT;
    const int i0 = min(tid * TPT, ntot), i1 = min(i0 + TPT, ntot);
    int cnt = 0;
    for (int i = i0; i < i1; ++i) cnt += composite(cl[i].x, cl[i].y) >= thr;
    int o = block_excl_scan_n<NT>(cnt, sh, &tot);
    for (int i = i0; i < i1; ++i)
      if (composite(cl[i].x, cl[i].y) >= thr) orow[o++] = (int32_t)cl[i].y;
    return;
  }
  // exact selection over the whole row's scores, then the winners in index
  // order, tile by tile
  auto row_key = [&](int64_t i) { return i == e_new ? new_key : float_key(sc[i]); };
  {
    uint32_t kmax = 0, kmin = 0xffffffffu;
    for (int64_t i = tid; i < vis; i += NT) {
      const uint32_t kk = row_key(i);
      kmax = max(kmax, kk);
      kmin = min(kmin, kk);
    }
    uint64_t pre;
    block_maxmin_u32<NT>(kmax, kmin, sh);
    const int hi = common_prefix(kmax, kmin, &pre);
    thr = radix_select64_n<NT>([&](int64_t i) { return composite(row_key(i), (uint32_t)i); }, vis,
                               k, hi, pre, hist, res);
  }
  int base = 0;
  for (int64_t t0 = 0; t0 < vis; t0 += 4 * NT) {
    int cnt = 0;
    bool win[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i = t0 + 4 * tid + u;
      const uint32_t kk = i < vis ? row_key(i) : 0u;
      win[u] = i < vis && composite(kk, (uint32_t)i) >= thr;
      cnt += win[u];
    }
    int o = block_excl_scan_n<NT>(cnt, sh, &tot);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (win[u]) orow[base + o++] = (int32_t)(t0 + 4 * tid + u);
    base += tot;
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

hipError_t launch_index_scores_prefill_fp4(const csa_index_desc& d, const uint8_t* qc,
                                           const uint8_t* qe, const void* wI, const uint8_t* kc,
                                           const uint8_t* ke, void* scores, int64_t ld,
                                           hipStream_t st) {
  const int key_chunk = 2048;
  const int64_t nvis = (d.t0 + d.n) / d.m < d.n_entries ? (d.t0 + d.n) / d.m : d.n_entries;
  if (nvis == 0) return hipSuccess;
  CSA_INDEX_DISPATCH(d.n_heads, d.head_dim, {
    constexpr int TQ = 256 / HI;
    if ((int64_t)TQ * ld >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    dim3 grid((unsigned)((d.n + TQ - 1) / TQ), (unsigned)((nvis + key_chunk - 1) / key_chunk));
    if (d.score_dtype == CSA_BF16)
      index_scores_prefill_fp4_kernel<HI, CI, uint16_t><<<grid, 256, 0, st>>>(
          qc, qe, (const uint16_t*)wI, kc, ke, d.n, d.n_entries, d.m, key_chunk,
          (uint16_t*)scores, ld, d.t0);
    else
      index_scores_prefill_fp4_kernel<HI, CI, float><<<grid, 256, 0, st>>>(
          qc, qe, (const uint16_t*)wI, kc, ke, d.n, d.n_entries, d.m, key_chunk, (float*)scores,
          ld, d.t0);
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
// D2 (FOLD: with the position's own new entry, see dec_select_kernel).
template <class T, int HI, int CI, bool FOLD>
static hipError_t dec_select(const csa_index_desc& d, const DecWs& w, int64_t nch, int L,
                             const int64_t* pos, int32_t* idx_out, const void* qI,
                             const void* wI, const void* KI, EntryMap em, hipStream_t st) {
  typedef typename T::S S;
  dec_select_kernel<T, HI, CI, FOLD, kSelThreads><<<d.batch, kSelThreads, 0, st>>>(
      pos, d.n_entries, d.m, d.k, w.scores, w.cand, w.cmeta, nch, L, (const S*)qI, (const S*)wI,
      (const S*)KI, em, idx_out);
  return hipGetLastError();
}

// D1 over the entries that exist before each sequence's position steps
// (entries s < floor(pos / m)): it reads no row that step's compressor writes.
hipError_t launch_index_topk_decode_score(const csa_index_desc& d, const void* qI,
                                          const void* wI, const void* KI, const int64_t* pos,
                                          void* wsp, hipStream_t st, EntryMap em) {
  DecWs w = carve(wsp, d);
  const int64_t nch = dec_chunks(d);
  const int L = dec_cand_per_chunk(d);
  const dim3 grid((unsigned)nch, (unsigned)d.batch);
#define CSA_DSCORE(TT, PG)                                                                    \
  dec_score_kernel<TT, HI, CI, PG><<<grid, 256, 0, st>>>(                                     \
      (const TT::S*)qI, (const TT::S*)wI, (const TT::S*)KI, pos, d.n_entries, d.m, d.k,        \
      w.scores, w.cand, w.cmeta, L, nch, em)
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
  return hipGetLastError();
}

// D2 after launch_index_topk_decode_score on the same workspace, once the
// step's new entries are in the cache: the new entry of each sequence is
// scored here.
hipError_t launch_index_topk_decode_select(const csa_index_desc& d, const void* qI,
                                           const void* wI, const void* KI, const int64_t* pos,
                                           int32_t* idx_out, void* wsp, hipStream_t st,
                                           EntryMap em) {
  DecWs w = carve(wsp, d);
  const int64_t nch = dec_chunks(d);
  const int L = dec_cand_per_chunk(d);
  CSA_INDEX_DISPATCH(d.n_heads, d.head_dim, {
    if (d.dtype == CSA_BF16)
      return dec_select<BF16, HI, CI, true>(d, w, nch, L, pos, idx_out, qI, wI, KI, em, st);
    return dec_select<F32, HI, CI, true>(d, w, nch, L, pos, idx_out, qI, wI, KI, em, st);
  });
}

hipError_t launch_index_topk_decode(const csa_index_desc& d, const void* qI, const void* wI,
                                    const void* KI, const int64_t* pos, int32_t* idx_out,
                                    void* wsp, hipStream_t st, EntryMap em) {
  hipError_t e = launch_index_topk_decode_score(d, qI, wI, KI, pos, wsp, st, em);
  if (e != hipSuccess) return e;
  return launch_index_topk_decode_select(d, qI, wI, KI, pos, idx_out, wsp, st, em);
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

// Wave-level scans and reductions over the 64 lanes.
CSA_DEV int wave_excl_scan(int v) {
  const int lane = threadIdx.x & 63;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x - v;
}
CSA_DEV uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
  return v;
}
CSA_DEV uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o, 64));
  return v;
}

// chunk_candidates for one wave and no barriers: the chunk's c <= 1024 keys
// in registers, lane l holding entries 16l .. 16l+15 (so lane-major order is
// index order).  The L-th best key is found by the same radix over the bits
// below the keys' common prefix, each 8-bit digit from a histogram of this
// wave's own 256 LDS ints; the output (cand in index order, meta) is
// chunk_candidates' exactly.
CSA_DEV void chunk_candidates_wave(const uint32_t (&key)[16], int c, int L, int64_t c0,
                                   int* hist, uint2* __restrict__ cand, uint4* __restrict__ meta) {
  const int lane = threadIdx.x & 63;
  uint32_t V = 0;
  int take = 0;
  if (c > L) {
    uint32_t kmax = 0, kmin = 0xffffffffu;
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (16 * lane + u < c) { kmax = max(kmax, key[u]); kmin = min(kmin, key[u]); }
    kmax = wave_max_u32(kmax);
    kmin = wave_min_u32(kmin);
    int hi = kmax == kmin ? -1 : 31 - __builtin_clz(kmax ^ kmin);  // highest undecided bit
    uint32_t mask = hi >= 31 ? 0u : ~((2u << hi) - 1u);
    uint32_t prefix = kmax & mask;
    int need = L;
    while (hi >= 0) {
      const int lo = hi >= 7 ? hi - 7 : 0;
      const uint32_t dm = (2u << (hi - lo)) - 1u;
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");  // last pass's reads are done
#pragma unroll
      for (int b = 0; b < 4; ++b) hist[4 * lane + b] = 0;
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (16 * lane + u < c && (key[u] & mask) == prefix)
          __hip_atomic_fetch_add(&hist[(key[u] >> lo) & dm], 1, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_WAVEFRONT);
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      int h[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) h[b] = hist[4 * lane + b];
      // the digit d with (#keys above d) < need <= (#keys at or above d):
      // suffix sums over lanes from the top bins down
      const int c4 = h[0] + h[1] + h[2] + h[3];
      int suf = c4;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_down(suf, o, 64);
        if (lane + o < 64) suf += y;
      }
      const int above = suf - c4;  // keys in the bins of higher lanes
      int dig = -1, abv = 0;
      if (above < need && suf >= need) {
        int acc = above;
        for (int b = 3; b >= 0; --b) {
          if (acc + h[b] >= need) { dig = 4 * lane + b; abv = acc; break; }
          acc += h[b];
        }
      }
      const int src = __ffsll((long long)__ballot(dig >= 0)) - 1;  // exactly one lane
      const int d = __shfl(dig, src, 64);
      need -= __shfl(abv, src, 64);
      prefix |= (uint32_t)d << lo;
      mask |= dm << lo;
      hi = lo - 1;
    }
    V = prefix;
    take = need;
  }
  int nt = 0;
#pragma unroll
  for (int u = 0; u < 16; ++u) nt += (c > L && 16 * lane + u < c && key[u] == V);
  int tr = wave_excl_scan(nt);  // tie ranks in index order
  bool keep[16];
  int nk = 0, lth = -1;
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int i = 16 * lane + u;
    bool kp = i < c;
    if (c > L && kp) {
      if (key[u] == V) {
        kp = tr < take;
        if (tr == take - 1) lth = i;
        ++tr;
      } else {
        kp = key[u] > V;
      }
    }
    keep[u] = kp;
    nk += kp;
  }
  int off = wave_excl_scan(nk);
#pragma unroll
  for (int u = 0; u < 16; ++u)
    if (keep[u]) cand[off++] = make_uint2(key[u], (uint32_t)(c0 + 16 * lane + u));
  if (c <= L) {
    if (lane == 0) *meta = make_uint4((uint32_t)c, 0u, 0u, 0u);
  } else if (lth >= 0) {
    *meta = make_uint4((uint32_t)L, 1u, V, (uint32_t)(c0 + lth));
  }
}

// Candidates of (row, chunk)s from stored scores: the chunk-local selection
// of dec_score_kernel without its scoring, for rows whose scores the prefill
// scorer wrote into the decode workspace (row stride n_entries, every
// visible entry scored).  Each wave takes one chunk of one row, four chunks
// per workgroup.
__global__ __launch_bounds__(256) void dec_cand_from_scores_kernel(
    const float* __restrict__ scores, const int64_t* __restrict__ posv, int64_t n_entries, int m,
    int k, uint2* __restrict__ cand, uint4* __restrict__ cmeta, int L, int64_t nch) {
  __shared__ int hist[4][256];
  const int b = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t ch = (int64_t)blockIdx.x * 4 + wave;
  const int64_t c0 = ch * kDecChunk;
  const int64_t vis = min64((posv[b] + 1) / m, n_entries);
  if (vis <= k) return;  // everything visible is selected
  if (ch >= nch || c0 >= vis) return;  // the whole wave
  const int c = (int)(min64(c0 + kDecChunk, vis) - c0);
  const float* sc = scores + (int64_t)b * n_entries + c0;
  uint32_t key[16];
  if (16 * lane + 16 <= c && (n_entries & 3) == 0) {  // four 16-byte loads
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 v = *(const float4*)(sc + 16 * lane + 4 * q);
      key[4 * q] = float_key(v.x);
      key[4 * q + 1] = float_key(v.y);
      key[4 * q + 2] = float_key(v.z);
      key[4 * q + 3] = float_key(v.w);
    }
  } else {
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int i = 16 * lane + u;
      key[u] = i < c ? float_key(sc[i]) : 0u;
    }
  }
  const int64_t slot = (int64_t)b * nch + ch;
  chunk_candidates_wave(key, c, L, c0, hist[wave], cand + slot * L, cmeta + slot);
}

static csa_index_desc long_rows_desc(const csa_index_desc& d) {
  csa_index_desc dd = d;
  const int64_t last = (d.t0 + d.n) / d.m;  // visible entries of the last row
  dd.n_entries = last < d.n_entries ? last : d.n_entries;
  // rows per sub-batch: about 2 GiB of decode workspace
  dd.batch = 1;
  const int64_t r = ((int64_t)1 << 31) / (int64_t)index_decode_ws_bytes(dd);
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
    const uint8_t* qb = (const uint8_t*)qI + r0 * d.n_heads * d.head_dim * es;
    const uint8_t* wb = (const uint8_t*)wI + r0 * d.n_heads * es;
    // the batch's scores by the prefill scorer (every visible entry, the
    // decode workspace's rows of stride n_entries), then each chunk's
    // candidates, then the per-row selection over them
    DecWs w = carve(ws, db);
    csa_index_desc ds = d;
    ds.n = db.batch;
    ds.t0 = d.t0 + r0;
    ds.n_entries = dd.n_entries;
    ds.score_dtype = CSA_F32;
    e = launch_index_scores_prefill(ds, qb, wb, KI, w.scores, dd.n_entries, st);
    if (e != hipSuccess) return e;
    const int64_t nch = dec_chunks(db);
    const int L = dec_cand_per_chunk(db);
    dec_cand_from_scores_kernel<<<dim3((unsigned)((nch + 3) / 4), (unsigned)db.batch), 256, 0, st>>>(
        w.scores, pos, db.n_entries, db.m, db.k, w.cand, w.cmeta, L, nch);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    CSA_INDEX_DISPATCH(d.n_heads, d.head_dim, {
      if (d.dtype == CSA_BF16)
        e = dec_select<BF16, HI, CI, false>(db, w, nch, L, pos, idx_out + r0 * d.k, qb, wb, KI,
                                            em, st);
      else
        e = dec_select<F32, HI, CI, false>(db, w, nch, L, pos, idx_out + r0 * d.k, qb, wb, KI,
                                           em, st);
    });
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
  const int L = dec_cand_per_chunk(d);
  const dim3 grid((unsigned)nch, (unsigned)d.batch);
  CSA_INDEX_DISPATCH(d.n_heads, d.head_dim, {
    if (em.table)
      dec_score_fp4_kernel<HI, CI, true><<<grid, 256, 0, st>>>(
          qc, qe, (const uint16_t*)wI, kc, ke, pos, d.n_entries, d.m, d.k, w.scores, w.cand,
          w.cmeta, L, nch, em);
    else
      dec_score_fp4_kernel<HI, CI, false><<<grid, 256, 0, st>>>(
          qc, qe, (const uint16_t*)wI, kc, ke, pos, d.n_entries, d.m, d.k, w.scores, w.cand,
          w.cmeta, L, nch, em);
  });
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the FP4 scorer scores every visible entry, the new one included
  return dec_select<BF16, 4, 64, false>(d, w, nch, L, pos, idx_out, nullptr, nullptr, nullptr, em,
                                        st);
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
