// Compressor kernels: projection GEMM, block softmax pooling with the entry
// epilogue, window rows, and the decode-time online pooling state.
//
// Citation keys: [R] = page "DeepSeek-V4 技术解读报告" (juejin.cn), section
// 2.3.1 eq 9-12 (overlapped CSA compression), 2.3.2 eq 20-23 (HCA), 2.3.3
// (QK RMSNorm, partial RoPE); [A] = page "DeepSeek-V4：算法架构"
// (1zeryu.github.io), Compressor class (prefill and decode branches) and the
// attention's wkv -> kv_norm -> RoPE window path.
#include "csa_common.h"
#include "csa_launch.h"

namespace csa {

// Most K slices of a decode projection (the update sums them per column with
// all loads in flight at once).
constexpr int kMaxKSplit = 8;

// ===========================================================================
// Projection GEMM:  out[M, 0:N] (fp32) = A[M, K] . [W0; W1; W2]^T
// fp32 operands: 128x128 output tile per 256-thread workgroup (2x2 waves of
// 64x64), K staged through LDS in 128-byte slices, double buffered.  Both
// operands are K-major in memory (A rows = tokens, W rows = output channels),
// so every lane feeds the matrix cores with one 16-byte LDS read per operand
// and k-group.  (bf16 operands take proj_gemm_bf16_kernel below.)
// ===========================================================================
template <class T>
__global__ __launch_bounds__(256, 2) void proj_gemm_kernel(
    const typename T::S* __restrict__ A, int64_t M, int K, const typename T::S* __restrict__ W0,
    int r0, const typename T::S* __restrict__ W1, int r1, const typename T::S* __restrict__ W2,
    int r2, float* __restrict__ out, int64_t ldo) {
  typedef typename T::S S;
  constexpr int BM = 128, BN = 128, BKB = 128;
  constexpr int E = 16 / (int)sizeof(S);
  constexpr int BK = BKB / (int)sizeof(S);
  constexpr int LDB = BKB + 16;
  __shared__ __align__(16) uint8_t sA[2][BM * LDB];
  __shared__ __align__(16) uint8_t sB[2][BN * LDB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.y * BM;
  const int n0 = blockIdx.x * BN;
  const int ntot = r0 + r1 + r2;

  const S* a_ptr[4];
  const S* b_ptr[4];
  bool a_ok[4], b_ok[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = (tid >> 3) + 32 * q;
    const int64_t gm = m0 + row;
    a_ok[q] = gm < M;
    a_ptr[q] = A + (a_ok[q] ? gm : 0) * (int64_t)K + (tid & 7) * E;
    const int j = n0 + row;
    const S* wp = W0;
    int jr = j;
    if (jr >= r0) { jr -= r0; wp = W1; if (jr >= r1) { jr -= r1; wp = W2; } }
    b_ok[q] = j < ntot;
    b_ptr[q] = wp + (int64_t)(b_ok[q] ? jr : 0) * K + (tid & 7) * E;
    if (!b_ok[q]) b_ptr[q] = W0;
  }

  uint4 ra[4], rb[4];
  auto gload = [&](int kt) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ra[q] = a_ok[q] ? *(const uint4*)(a_ptr[q] + (int64_t)kt * BK) : make_uint4(0, 0, 0, 0);
      rb[q] = b_ok[q] ? *(const uint4*)(b_ptr[q] + (int64_t)kt * BK) : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = (tid >> 3) + 32 * q;
      *(uint4*)(sA[buf] + row * LDB + (tid & 7) * 16) = ra[q];
      *(uint4*)(sB[buf] + row * LDB + (tid & 7) * 16) = rb[q];
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};

  const int nk = K / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) gload(kt + 1);
    const uint8_t* As = sA[kt & 1];
    const uint8_t* Bs = sB[kt & 1];
#pragma unroll
    for (int kg = 0; kg < BKB / 32; ++kg) {
      uint4 a[2], b[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        a[mb] = *(const uint4*)(As + (wm * 64 + mb * 32 + (lane & 31)) * LDB + kg * 32 + (lane >> 5) * 16);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        b[nb] = *(const uint4*)(Bs + (wn * 64 + nb * 32 + (lane & 31)) * LDB + kg * 32 + (lane >> 5) * 16);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) mma32<T>(acc[mb][nb], a[mb], b[nb]);
    }
    if (kt + 1 < nk) sstore((kt + 1) & 1);
    __syncthreads();
  }

#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int col = n0 + wn * 64 + nb * 32 + (lane & 31);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int64_t row = m0 + wm * 64 + mb * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        if (row < M && col < ntot) out[row * ldo + col] = acc[mb][nb][i];
      }
    }
}

// ===========================================================================
// fp32 projection GEMM for narrow outputs (N <= kF32KSplitMaxN): a 64x64
// output tile per 256-thread workgroup, so a short token range still spreads
// over many CUs.  The four waves split each 32-wide K slice by k-group (wave
// w takes floats 8w .. 8w+7 of every slice), so each wave holds the whole
// tile as four 32x32 accumulator blocks (four independent matrix-core
// chains); the partial tiles are then added through LDS in wave order, a
// fixed order, so the result does not depend on M or on scheduling.  The
// choice of kernel depends on N only, so a chunked prefill and a one-shot
// prefill of the same weights sum every output in the same order.
// ===========================================================================
constexpr int kF32KSplitMaxN = 1024;

__global__ __launch_bounds__(256) void proj_gemm_f32_ksplit_kernel(
    const float* __restrict__ A, int64_t M, int K, const float* __restrict__ W0, int r0,
    const float* __restrict__ W1, int r1, const float* __restrict__ W2, int r2,
    float* __restrict__ out, int64_t ldo) {
  constexpr int BM = 64, BN = 64, BKB = 128, BK = BKB / 4, LDB = BKB + 16;
  // the K slices' double buffers, reused after the loop for the partial
  // tiles of two waves at a time ([block * 16 + i][lane] floats each)
  __shared__ __align__(16) uint8_t smem[2 * (BM + BN) * LDB];
  static_assert(2 * 16 * 4 * 64 * 4 <= 2 * (BM + BN) * LDB, "two partial tiles fit");
  uint8_t(*sA)[BM * LDB] = (uint8_t(*)[BM * LDB])smem;
  uint8_t(*sB)[BN * LDB] = (uint8_t(*)[BN * LDB])(smem + 2 * BM * LDB);
  float* red = (float*)smem;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t m0 = (int64_t)blockIdx.y * BM;
  const int n0 = blockIdx.x * BN;
  const int ntot = r0 + r1 + r2;

  const float* a_ptr[2];
  const float* b_ptr[2];
  bool a_ok[2], b_ok[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int row = (tid >> 3) + 32 * q;
    const int64_t gm = m0 + row;
    a_ok[q] = gm < M;
    a_ptr[q] = A + (a_ok[q] ? gm : 0) * (int64_t)K + (tid & 7) * 4;
    const int j = n0 + row;
    const float* wp = W0;
    int jr = j;
    if (jr >= r0) { jr -= r0; wp = W1; if (jr >= r1) { jr -= r1; wp = W2; } }
    b_ok[q] = j < ntot;
    b_ptr[q] = b_ok[q] ? wp + (int64_t)jr * K + (tid & 7) * 4 : W0;
  }
  uint4 ra[2], rb[2];
  auto gload = [&](int kt) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      ra[q] = a_ok[q] ? *(const uint4*)(a_ptr[q] + (int64_t)kt * BK) : make_uint4(0, 0, 0, 0);
      rb[q] = b_ok[q] ? *(const uint4*)(b_ptr[q] + (int64_t)kt * BK) : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int row = (tid >> 3) + 32 * q;
      *(uint4*)(sA[buf] + row * LDB + (tid & 7) * 16) = ra[q];
      *(uint4*)(sB[buf] + row * LDB + (tid & 7) * 16) = rb[q];
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};
  const int nk = K / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) gload(kt + 1);
    const uint8_t* As = sA[kt & 1];
    const uint8_t* Bs = sB[kt & 1];
    uint4 a[2], b[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
      a[mb] = *(const uint4*)(As + (mb * 32 + (lane & 31)) * LDB + wave * 32 + (lane >> 5) * 16);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
      b[nb] = *(const uint4*)(Bs + (nb * 32 + (lane & 31)) * LDB + wave * 32 + (lane >> 5) * 16);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) mma32<F32>(acc[mb][nb], a[mb], b[nb]);
    if (kt + 1 < nk) sstore((kt + 1) & 1);
    __syncthreads();
  }
  // wave 0 adds the other waves' partial tiles in wave order: waves 1 and 2
  // through the staging buffers, then wave 3 (the loop's last barrier has
  // released them)
  constexpr int PT = 16 * 4 * 64;  // floats of one partial tile
  auto put = [&](int slot) {
#pragma unroll
    for (int blk = 0; blk < 4; ++blk)
#pragma unroll
      for (int i = 0; i < 16; ++i) red[slot * PT + (blk * 16 + i) * 64 + lane] = acc[blk >> 1][blk & 1][i];
  };
  auto add = [&](int slot) {
#pragma unroll
    for (int blk = 0; blk < 4; ++blk)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[blk >> 1][blk & 1][i] += red[slot * PT + (blk * 16 + i) * 64 + lane];
  };
  if (wave == 1 || wave == 2) put(wave - 1);
  __syncthreads();
  if (wave == 0) {
    add(0);
    add(1);
  }
  __syncthreads();
  if (wave == 3) put(0);
  __syncthreads();
  if (wave != 0) return;
  add(0);
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
    const int mb = blk >> 1, nb = blk & 1;
    const int col = n0 + nb * 32 + (lane & 31);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t row = m0 + mb * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
      if (row < M && col < ntot) out[row * ldo + col] = acc[mb][nb][i];
    }
  }
}

// ===========================================================================
// bf16 projection GEMM: TM x TN output tile per 512-thread workgroup, 4x2
// waves of (TM/4) x (TN/2) (blocks of 32x32x16 MFMA; the 256x256 tile gives
// each wave 2x4 blocks, 128 accumulators, two waves per SIMD).  A and W
// panels stream into a ring of four LDS stages (32-wide K slices) by direct
// global->LDS loads issued three slices ahead, so a slice's loads have three
// slices of products to land in; the next k-group's fragments are read while
// a k-group's products run.  In LDS, 16-byte granule g of tile row r (64
// bytes per row) sits at column g ^ ((r >> 2) & 3), so every 16 consecutive
// rows of a fragment read cover all banks.  Tile order: die x (workgroup id
// mod 8) takes M blocks x, x+8, ... in groups that its workgroups run side
// by side, so the A and W slices they stream are shared in the die's L2.
// Each stacked weight matrix writes its columns to its own output (fp32 or
// bf16, rounded once); blockIdx.y selects a group of a grouped product (A,
// W0 and output 0 offset per group).  Smaller tiles serve products too
// narrow to give the 256x256 tile a workgroup per CU.
// ===========================================================================
constexpr int kGKB = 64;             // bytes of K per slice (32 bf16)
constexpr int kGemmBigTileMinWorkgroups = 256;  // one 256x256 tile per CU at least
constexpr int kGemmSmallTM = 256;               // rows of the narrow-product tile
constexpr int kGS = 4;               // LDS stages
constexpr int kGAhead = kGS - 1;     // slices in flight ahead of the one in use

template <class OUT, int TM, int TN>
__global__ __launch_bounds__(512, 1) void proj_gemm_bf16_kernel(
    const uint16_t* __restrict__ A, int64_t lda, int64_t M, int K,
    const uint16_t* __restrict__ W0, int r0, const uint16_t* __restrict__ W1, int r1,
    const uint16_t* __restrict__ W2, int r2, GemmOuts outs, int mblocks, int ntiles,
    int64_t a_zoff, int64_t w_zoff, int64_t o_zoff) {
  static_assert(TM % 128 == 0 && TN % 128 == 0, "tiles are multiples of 128");
  constexpr int WM = TM / 4, WN = TN / 2;     // wave tile
  constexpr int MB = WM / 32, NB = WN / 32;   // 32x32 blocks per wave
  constexpr int NA = TM / 128, NW = TN / 128; // 1 KiB load chunks per wave and slice
  constexpr int LPS = NA + NW;                // loads per wave and slice
  static_assert(LPS <= 2 * MB + 2, "every load of a slice has a product slot");
  __shared__ __align__(16) uint8_t sA[kGS][TM * kGKB];
  __shared__ __align__(16) uint8_t sB[kGS][TN * kGKB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;  // row band, column band
  // die x owns M blocks x, x+8, ...; it walks them in groups of 8, and
  // within a group over 8 x 4 tiles (8 M blocks, 4 N tiles) at a time, so the
  // 32 workgroups a die runs together share every A and W slice they load
  const int xcd = blockIdx.x & 7, seq = blockIdx.x >> 3;
  const int mg = seq / (8 * ntiles), rg = seq % (8 * ntiles);
  const int nfull = ntiles / 4;
  int mi, nt;
  if (rg < nfull * 32) {
    mi = (rg % 32) / 4;
    nt = 4 * (rg / 32) + rg % 4;
  } else {
    const int gs = ntiles - 4 * nfull, rr = rg - nfull * 32;
    mi = rr / gs;
    nt = 4 * nfull + rr % gs;
  }
  const int mbk = 8 * (8 * mg + mi) + xcd;
  if (mbk >= mblocks) return;
  const int64_t m0 = (int64_t)mbk * TM;
  const int n0 = nt * TN;
  const int ntot = r0 + r1 + r2;
  A += blockIdx.y * a_zoff;
  W0 += blockIdx.y * w_zoff;

  // Loads: wave w fills 1 KiB chunks w, w+8, ... (16 rows each) of both
  // panels; lane i of chunk c carries row 16c + i/4 into LDS column i%4,
  // which holds global granule (i%4) ^ ((row >> 2) & 3).
  const uint8_t* pa[NA];
  const uint8_t* pb[NW];
#pragma unroll
  for (int u = 0; u < NA; ++u) {
    const int row = 16 * (wave + 8 * u) + (lane >> 2);
    const int gran = (lane & 3) ^ ((row >> 2) & 3);
    const int64_t ar = min64(m0 + row, M - 1);  // rows past M read a valid row
    pa[u] = (const uint8_t*)(A + ar * lda) + gran * 16;
  }
#pragma unroll
  for (int u = 0; u < NW; ++u) {
    const int row = 16 * (wave + 8 * u) + (lane >> 2);
    const int gran = (lane & 3) ^ ((row >> 2) & 3);
    int n = n0 + row;
    const uint16_t* wp = W0;
    if (n >= ntot) n = 0;  // masked columns read a valid row
    else if (n >= r0 + r1) { wp = W2; n -= r0 + r1; }
    else if (n >= r0) { wp = W1; n -= r0; }
    pb[u] = (const uint8_t*)(wp + (int64_t)n * K) + gran * 16;
  }
  // load q (0 .. LPS-1) of slice kt: the A chunks, then the W chunks
  auto issue1 = [&](int kt, int q) {
    const int s = kt % kGS;
    if (q < NA) lds_dma16(pa[q] + (int64_t)kt * kGKB, sA[s] + (wave + 8 * q) * 1024);
    else lds_dma16(pb[q - NA] + (int64_t)kt * kGKB, sB[s] + (wave + 8 * (q - NA)) * 1024);
  };
  auto issue = [&](int kt) {
#pragma unroll
    for (int q = 0; q < LPS; ++q) issue1(kt, q);
  };

  f32x16_t acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x16_t{};
  // fragment rows (l & 31) of 32-row blocks, granule 2*kg + l/32
  const int frow = lane & 31, fhalf = lane >> 5, fsw = (frow >> 2) & 3;
  const int aoff = (wm * WM + frow) * kGKB;
  const int boff = (wn * WN + frow) * kGKB;
  bf16x8_t fa[2][MB], fb[2][NB];
  auto frags = [&](int s, int kg, int slot) {
    const int col = ((2 * kg + fhalf) ^ fsw) * 16;
#pragma unroll
    for (int i = 0; i < MB; ++i)
      fa[slot][i] = *(const bf16x8_t*)(sA[s] + aoff + i * 32 * kGKB + col);
#pragma unroll
    for (int j = 0; j < NB; ++j)
      fb[slot][j] = *(const bf16x8_t*)(sB[s] + boff + j * 32 * kGKB + col);
  };

  const int nk = K / 32;  // K is a multiple of 64, so nk >= 2
#pragma unroll
  for (int kt = 0; kt < kGAhead; ++kt)
    if (kt < nk) issue(kt);
  // slice 0 has landed once at most the later slices' loads are outstanding
  if (nk >= 3) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * LPS));
  else __builtin_amdgcn_s_waitcnt(vmcnt_imm(LPS));
  __syncthreads();
  frags(0, 0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    const int s = kt % kGS;
    const bool ahead = kt + kGAhead < nk;
    frags(s, 1, 1);
    // the loads of slice kt+3 go out between the products, so the load
    // pipe and the matrix cores work side by side
#pragma unroll
    for (int kg = 0; kg < 2; ++kg)
#pragma unroll
      for (int i = 0; i < MB; ++i) {
#pragma unroll
        for (int j = 0; j < NB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kg][i], fb[kg][j], acc[i][j],
                                                              0, 0, 0);
        if (ahead && kg * MB + i < LPS) issue1(kt + kGAhead, kg * MB + i);
      }
    if (ahead) {
#pragma unroll
      for (int q = 2 * MB; q < LPS; ++q) issue1(kt + kGAhead, q);
    }
    // slice kt+1 must have landed; the loads of kt+2 and kt+3 may still run
    const int later = min(nk - 1, kt + kGAhead) - (kt + 1);
    if (later >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * LPS));
    else if (later == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(LPS));
    else wait_vmem();
    __syncthreads();
    if (kt + 1 < nk) frags((kt + 1) % kGS, 0, 0);
  }

#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int col = n0 + wn * WN + j * 32 + frow;
    int cm = col;  // column within its weight matrix
    OUT* op = (OUT*)outs.p[0] + blockIdx.y * o_zoff;
    int64_t ld = outs.ld[0];
    if (cm >= r0 + r1) { cm -= r0 + r1; op = (OUT*)outs.p[2]; ld = outs.ld[2]; }
    else if (cm >= r0) { cm -= r0; op = (OUT*)outs.p[1]; ld = outs.ld[1]; }
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = m0 + wm * WM + i * 32 + 8 * (e >> 2) + 4 * fhalf + (e & 3);
        if (row < M && col < ntot) {
          if constexpr (sizeof(OUT) == 2) op[row * ld + cm] = f32_to_bf16(acc[i][j][e]);
          else op[row * ld + cm] = acc[i][j][e];
        }
      }
  }
}

// ===========================================================================
// Row epilogue shared by entries, window rows and decode emission: a group of
// G = c/2 threads owns one row of width c, thread j the channel pair
// (2j, 2j+1).  The pooled (or projected) values are first rounded to the
// storage type T, as [A] Compressor casts the pooled entry to the model dtype
// before its norm (and the attention's wkv is a model-dtype linear layer);
// then RMSNorm (unit weight) over the row, then RoPE of the last r channels
// at `pos` ([R] 2.3.3; pairs are adjacent channels).  The caller rounds the
// result to T once more at store.
// `red` is LDS scratch of at least (blockDim / 64) floats, used when G > 64.
// Every thread of the block must call this (it may synchronise).
// ===========================================================================
template <class T, int G>
CSA_DEV void row_finish(float& v0, float& v1, int j, int c, int64_t pos, int qk_norm, float eps,
                        int r, float theta, float* red) {
  v0 = T::f(T::cvt(v0));
  v1 = T::f(T::cvt(v1));
  if (qk_norm) {
    float s = v0 * v0 + v1 * v1;
    if (G <= 64) {
#pragma unroll
      for (int o = G / 2; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
    } else {
      s = wave_sum(s);
      const int w = threadIdx.x >> 6;
      __syncthreads();
      if ((threadIdx.x & 63) == 0) red[w] = s;
      __syncthreads();
      const int g0 = (w / (G / 64)) * (G / 64);
      s = 0.f;
#pragma unroll
      for (int i = 0; i < G / 64; ++i) s += red[g0 + i];
    }
    const float inv = rsqrtf(s / (float)c + eps);
    v0 *= inv;
    v1 *= inv;
  }
  if (r > 0 && 2 * j >= c - r) {
    float cs, sn;
    rope_cs(pos, j - (c - r) / 2, r, theta, &cs, &sn);
    const float x0 = v0, x1 = v1;
    v0 = x0 * cs - x1 * sn;
    v1 = x0 * sn + x1 * cs;
  }
}

// Online softmax accumulation of one (logit, value) pair.
CSA_DEV void osm_push(float& mx, float& sm, float& ac, float lg, float v) {
  const float nm = fmaxf(mx, lg);
  const float a = __expf(mx - nm);  // mx = -inf on first use -> 0
  const float b = __expf(lg - nm);
  sm = sm * a + b;
  ac = ac * a + v * b;
  mx = nm;
}
// Merge state 2 into state 1 (either may be empty: mx = -inf, sm = ac = 0).
CSA_DEV void osm_merge(float& m1, float& s1, float& a1, float m2, float s2, float a2) {
  const float nm = fmaxf(m1, m2);
  if (nm == -INFINITY) return;
  const float x = __expf(m1 - nm), y = __expf(m2 - nm);
  s1 = s1 * x + s2 * y;
  a1 = a1 * x + a2 * y;
  m1 = nm;
}

// ===========================================================================
// Pool complete blocks ([R] eq 11-12 / 22-23) and finish each entry.
// Scratch P[t][ld]: C at columns [0, w), Z at [w, 2w), w = (1+ov) c; under
// overlap columns [0, c) of each are the b-series and [c, 2c) the a-series.
// ===========================================================================
template <class T, int G>
__global__ __launch_bounds__(256) void pool_entries_kernel(
    const float* __restrict__ P, int64_t ld, int64_t n_entries, int c, int m, int ov,
    const float* __restrict__ ape, int qk_norm, float eps, int r, float theta,
    typename T::S* __restrict__ out, int64_t pos0, int prev0, EntryMap em) {
  // prev0: the m rows before P hold block -1 (a chunk's halo), whose
  // b-series joins entry 0 under overlap.  Entry i of the call is entry
  // pos0 / m + i of the sequence: row i of out, or its pool row under em.
  __shared__ float red[4];
  constexpr int GPW = 256 / G;
  const int g = threadIdx.x / G, j = threadIdx.x % G;
  const int64_t i = (int64_t)blockIdx.x * GPW + g;
  const bool live = i < n_entries;
  const int w = (1 + ov) * c;
  const int ca = ov ? c : 0;  // a-series column offset
  float v0 = 0.f, v1 = 0.f;
  if (live) {
    float mx0 = -INFINITY, s0 = 0.f, a0 = 0.f, mx1 = -INFINITY, s1 = 0.f, a1 = 0.f;
    for (int rr = 0; rr < m; ++rr) {
      const float* row = P + (i * m + rr) * ld;
      const float2 cv = *(const float2*)(row + ca + 2 * j);
      const float2 zv = *(const float2*)(row + w + ca + 2 * j);
      const float2 bv = *(const float2*)(ape + (int64_t)rr * w + ca + 2 * j);
      osm_push(mx0, s0, a0, zv.x + bv.x, cv.x);
      osm_push(mx1, s1, a1, zv.y + bv.y, cv.y);
    }
    if (ov && (i > 0 || prev0)) {  // block i-1's b-series joins the same softmax
      for (int rr = 0; rr < m; ++rr) {
        const float* row = P + ((i - 1) * m + rr) * ld;
        const float2 cv = *(const float2*)(row + 2 * j);
        const float2 zv = *(const float2*)(row + w + 2 * j);
        const float2 bv = *(const float2*)(ape + (int64_t)rr * w + 2 * j);
        osm_push(mx0, s0, a0, zv.x + bv.x, cv.x);
        osm_push(mx1, s1, a1, zv.y + bv.y, cv.y);
      }
    }
    v0 = a0 / s0;
    v1 = a1 / s1;
  }
  row_finish<T, G>(v0, v1, j, c, (int64_t)m * (pos0 / m + i), qk_norm, eps, r, theta, red);
  if (live) {
    const int64_t orow = em.table ? em.row(0, pos0 / m + i, 0) : i;
    T::st(out, orow * c + 2 * j, v0);
    T::st(out, orow * c + 2 * j + 1, v1);
  }
}

// The same pooling for long blocks (m >= kPoolSplitM, HCA's m' = 128): one
// workgroup per entry, its 256 / G thread groups each folding the rows
// rr = g, g + S, ... of the block (and of block i-1's b-series under
// overlap) into an online softmax state of their own; the S states are then
// merged in group order through LDS, so the result does not depend on
// scheduling.  Few long blocks would otherwise leave most of the chip idle
// while each thread walked m rows in sequence.
constexpr int kPoolSplitM = 32;

template <class T, int G>
__global__ __launch_bounds__(256) void pool_entries_split_kernel(
    const float* __restrict__ P, int64_t ld, int64_t n_entries, int c, int m, int ov,
    const float* __restrict__ ape, int qk_norm, float eps, int r, float theta,
    typename T::S* __restrict__ out, int64_t pos0, int prev0, EntryMap em) {
  constexpr int S = 256 / G;
  __shared__ float red[4];
  __shared__ float st[S][6][G];  // (max, sum, acc) of both channels, per group
  const int g = threadIdx.x / G, j = threadIdx.x % G;
  const int64_t i = blockIdx.x;  // grid = n_entries
  const int w = (1 + ov) * c;
  const int ca = ov ? c : 0;  // a-series column offset
  float mx0 = -INFINITY, s0 = 0.f, a0 = 0.f, mx1 = -INFINITY, s1 = 0.f, a1 = 0.f;
  auto fold = [&](int64_t row0, int col) {
#pragma unroll 4
    for (int rr = g; rr < m; rr += S) {
      const float* row = P + (row0 + rr) * ld;
      const float2 cv = *(const float2*)(row + col + 2 * j);
      const float2 zv = *(const float2*)(row + w + col + 2 * j);
      const float2 bv = *(const float2*)(ape + (int64_t)rr * w + col + 2 * j);
      osm_push(mx0, s0, a0, zv.x + bv.x, cv.x);
      osm_push(mx1, s1, a1, zv.y + bv.y, cv.y);
    }
  };
  fold(i * m, ca);
  if (ov && (i > 0 || prev0)) fold((i - 1) * m, 0);  // block i-1's b-series
  st[g][0][j] = mx0; st[g][1][j] = s0; st[g][2][j] = a0;
  st[g][3][j] = mx1; st[g][4][j] = s1; st[g][5][j] = a1;
  __syncthreads();
  mx0 = st[0][0][j]; s0 = st[0][1][j]; a0 = st[0][2][j];
  mx1 = st[0][3][j]; s1 = st[0][4][j]; a1 = st[0][5][j];
#pragma unroll
  for (int h = 1; h < S; ++h) {
    osm_merge(mx0, s0, a0, st[h][0][j], st[h][1][j], st[h][2][j]);
    osm_merge(mx1, s1, a1, st[h][3][j], st[h][4][j], st[h][5][j]);
  }
  float v0 = a0 / s0, v1 = a1 / s1;
  row_finish<T, G>(v0, v1, j, c, (int64_t)m * (pos0 / m + i), qk_norm, eps, r, theta, red);
  if (g == 0) {
    const int64_t orow = em.table ? em.row(0, pos0 / m + i, 0) : i;
    T::st(out, orow * c + 2 * j, v0);
    T::st(out, orow * c + 2 * j + 1, v1);
  }
}

// Window rows: V (scratch column `col`, width c) -> RMSNorm, RoPE at t.
template <class T, int G>
__global__ __launch_bounds__(256) void window_rows_kernel(
    const float* __restrict__ P, int64_t ld, int col, int64_t n, int c, int qk_norm, float eps,
    int r, float theta, typename T::S* __restrict__ out, typename T::S* __restrict__ ring,
    int n_win, int64_t pos0) {
  __shared__ float red[4];
  constexpr int GPW = 256 / G;
  const int g = threadIdx.x / G, j = threadIdx.x % G;
  const int64_t t = (int64_t)blockIdx.x * GPW + g;
  const bool live = t < n;
  float v0 = 0.f, v1 = 0.f;
  if (live) {
    const float2 v = *(const float2*)(P + t * ld + col + 2 * j);
    v0 = v.x;
    v1 = v.y;
  }
  row_finish<T, G>(v0, v1, j, c, pos0 + t, qk_norm, eps, r, theta, red);
  if (live) {
    if (out) {
      T::st(out, t * c + 2 * j, v0);
      T::st(out, t * c + 2 * j + 1, v1);
    }
    if (ring && t >= n - n_win) {
      const int64_t s = (pos0 + t) % n_win;
      T::st(ring, s * c + 2 * j, v0);
      T::st(ring, s * c + 2 * j + 1, v1);
    }
  }
}

// ===========================================================================
// Decode state (per sequence, fp32): NS series x {running max, sum, weighted
// sum} x c channels.  Series 0 = the current block's a-series (the only
// series without overlap), 1 = the current block's b-series, 2 = the previous
// (complete) block's b-series.
// ===========================================================================
__global__ void state_init_kernel(float* __restrict__ st, int64_t per_seq, int c, int batch) {
  const int64_t total = per_seq * batch;
  for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < total;
       x += (int64_t)gridDim.x * blockDim.x) {
    const int64_t within = (x % per_seq) / c;  // series*3 + field
    st[x] = (within % 3 == 0) ? -INFINITY : 0.f;
  }
}

// After a prefill of n tokens: series 0/1 fold the tail rows of block n/m,
// series 2 folds the b-series of the last complete block.
__global__ void stash_state_kernel(const float* __restrict__ P, int64_t ld, int64_t n, int c,
                                   int m, int ov, const float* __restrict__ ape,
                                   float* __restrict__ st) {
  const int w = (1 + ov) * c;
  const int64_t nc = n / m;
  const int tail = (int)(n - nc * m);
  const int ns = ov ? 3 : 1;
  for (int ch = threadIdx.x; ch < c; ch += blockDim.x) {
    for (int s = 0; s < ns; ++s) {
      float mx = -INFINITY, sm = 0.f, ac = 0.f;
      int64_t t0;
      int rows, coff;
      if (s == 0) { t0 = nc * m; rows = tail; coff = ov ? c : 0; }
      else if (s == 1) { t0 = nc * m; rows = tail; coff = 0; }
      else { t0 = (nc - 1) * m; rows = nc >= 1 ? m : 0; coff = 0; }
      for (int rr = 0; rr < rows; ++rr) {
        const float* row = P + (t0 + rr) * ld;
        osm_push(mx, sm, ac, row[w + coff + ch] + ape[(int64_t)rr * w + coff + ch], row[coff + ch]);
      }
      st[(s * 3 + 0) * c + ch] = mx;
      st[(s * 3 + 1) * c + ch] = sm;
      st[(s * 3 + 2) * c + ch] = ac;
    }
  }
}

// ===========================================================================
// Decode projection: part[ks][b][j] = sum over the ks-th K slice of
// h[b, :] . W_j.  One 32x32 (batch x channel) tile per workgroup and K slice;
// the four waves split the slice further and are summed in a fixed order, so
// results are bitwise reproducible.  The weights are the bytes that bound
// this step: each is read exactly once.
// ===========================================================================
template <class T>
__global__ __launch_bounds__(256) void decode_proj_kernel(
    const typename T::S* __restrict__ h, int B, int K, const typename T::S* __restrict__ W0,
    int r0, const typename T::S* __restrict__ W1, int r1, const typename T::S* __restrict__ W2,
    int r2, float* __restrict__ part, int ksplit) {
  typedef typename T::S S;
  constexpr int E = 16 / (int)sizeof(S);
  constexpr int KG = 2 * E;  // elements per 32x32 k-group
  __shared__ float red[4][32 * 33];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ntot = r0 + r1 + r2;
  const int j0 = blockIdx.x * 32;
  const int ks = blockIdx.y;
  const int b0 = blockIdx.z * 32;
  const int kslice = K / ksplit, kw = kslice / 4;
  const int kbeg = ks * kslice + wave * kw;

  const int jr0 = j0 + (lane & 31);
  const S* wp = W0;
  int jr = jr0;
  if (jr >= r0) { jr -= r0; wp = W1; if (jr >= r1) { jr -= r1; wp = W2; } }
  const bool wok = jr0 < ntot;
  const S* wrow = wok ? wp + (int64_t)jr * K : W0;
  const int b = b0 + (lane & 31);
  const bool hok = b < B;
  const S* hrow = h + (int64_t)(hok ? b : 0) * K;

  f32x16_t acc = f32x16_t{};
  const int koff = (lane >> 5) * E;
  for (int k = kbeg; k < kbeg + kw; k += KG * 4) {
    uint4 a[4], bw[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int kk = k + u * KG + koff;
      const bool in = kk < kbeg + kw;
      a[u] = (hok && in) ? *(const uint4*)(hrow + kk) : make_uint4(0, 0, 0, 0);
      bw[u] = (wok && in) ? *(const uint4*)(wrow + kk) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) mma32<T>(acc, a[u], bw[u]);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int row = 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
    red[wave][row * 33 + (lane & 31)] = acc[i];
  }
  __syncthreads();
  for (int e = tid; e < 32 * 32; e += 256) {
    const int row = e >> 5, col = e & 31;
    const float v = red[0][row * 33 + col] + red[1][row * 33 + col] + red[2][row * 33 + col] +
                    red[3][row * 33 + col];
    if (b0 + row < B && j0 + col < ntot)
      part[((int64_t)ks * B + b0 + row) * ntot + j0 + col] = v;
  }
}

// One workgroup per sequence: sum the K-split partials, fold the new row into
// the online state, emit the finished entry when (pos+1) % m == 0, and write
// the window row into the ring ([A] Compressor decode branch).
template <class T, int G>
__global__ __launch_bounds__(256) void decode_update_kernel(
    const float* __restrict__ part, int ksplit, int B, int N, int c, int m, int ov, int has_win,
    const float* __restrict__ ape, const int64_t* __restrict__ posv, float* __restrict__ state,
    typename T::S* __restrict__ cache, int64_t max_entries, typename T::S* __restrict__ ring,
    int n_win, int qk_norm, float eps, int r, float theta, EntryMap em) {
  __shared__ float red[4];
  const int b = blockIdx.x;
  const int j = threadIdx.x;  // channel pair (2j, 2j+1)
  const bool live = j < G;
  // the partials and the state do not depend on the position: their loads
  // are issued with the position's
  const int64_t pos = posv[b];
  const int w = (1 + ov) * c;
  const int ns = ov ? 3 : 1;
  float* st = state + (int64_t)b * ns * 3 * c;

  // Sum of the K-slice partials of columns (col, col+1), slices in order.  All
  // columns this thread needs are summed up front so that their loads are in
  // flight together.
  // (Loads are unconditional -- slices past ksplit re-read the last one and
  // add zero -- so that no branch separates them.)
  auto colsum2 = [&](int col) {
    float2 v[kMaxKSplit];
#pragma unroll
    for (int k = 0; k < kMaxKSplit; ++k)
      v[k] = *(const float2*)(part + ((int64_t)min(k, ksplit - 1) * B + b) * N + col);
    float2 acc = v[0];  // ksplit >= 1
#pragma unroll
    for (int k = 1; k < kMaxKSplit; ++k) {
      acc.x += k < ksplit ? v[k].x : 0.f;
      acc.y += k < ksplit ? v[k].y : 0.f;
    }
    return acc;
  };
  const int ca = ov ? c : 0;  // a-series (or the only series) columns
  float2 kva = make_float2(0.f, 0.f), za = kva, kvb = kva, zb = kva, wn = kva;
  if (live) {
    kva = colsum2(ca + 2 * j);
    za = colsum2(w + ca + 2 * j);
    if (ov) {
      kvb = colsum2(2 * j);
      zb = colsum2(w + 2 * j);
    }
    if (has_win) wn = colsum2(2 * w + 2 * j);
  }
  float2 sv[9];  // state rows of channels (2j, 2j+1): 3 per series
#pragma unroll
  for (int i = 0; i < 9; ++i)
    sv[i] = (live && i < 3 * ns) ? *(const float2*)(st + i * c + 2 * j) : make_float2(0.f, 0.f);
  if (pos < 0) return;  // uniform per block: no token for this sequence
  const int rr = (int)(pos % m);
  const bool emit = (rr == m - 1);
  const int64_t blk = pos / m;

  float e0 = 0.f, e1 = 0.f;
  if (live) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int ch = 2 * j + q;
      auto sg = [&](int i) { return q ? sv[i].y : sv[i].x; };
      float mx = sg(0), sm = sg(1), ac = sg(2);
      osm_push(mx, sm, ac, (q ? za.y : za.x) + ape[(int64_t)rr * w + ca + ch], q ? kva.y : kva.x);
      float mb = -INFINITY, sb = 0.f, ab = 0.f;
      if (ov) {
        mb = sg(3); sb = sg(4); ab = sg(5);
        osm_push(mb, sb, ab, (q ? zb.y : zb.x) + ape[(int64_t)rr * w + ch], q ? kvb.y : kvb.x);
      }
      if (emit) {
        float em = mx, es = sm, ea = ac;
        if (ov) osm_merge(em, es, ea, sg(6), sg(7), sg(8));
        const float v = ea / es;
        if (q == 0) e0 = v; else e1 = v;
        // the block is finished: its b-series becomes "previous", the rest resets
        if (ov) { st[6 * c + ch] = mb; st[7 * c + ch] = sb; st[8 * c + ch] = ab; }
        mx = -INFINITY; sm = 0.f; ac = 0.f;
        mb = -INFINITY; sb = 0.f; ab = 0.f;
      }
      st[0 * c + ch] = mx; st[1 * c + ch] = sm; st[2 * c + ch] = ac;
      if (ov) { st[3 * c + ch] = mb; st[4 * c + ch] = sb; st[5 * c + ch] = ab; }
    }
  }
  if (emit) {  // uniform across the block
    row_finish<T, G>(e0, e1, j, c, (int64_t)m * blk, qk_norm, eps, r, theta, red);
    if (live && blk < max_entries) {
      typename T::S* dst = cache + em.row(b, blk, max_entries) * c;
      T::st(dst, 2 * j, e0);
      T::st(dst, 2 * j + 1, e1);
    }
  }
  if (has_win) {
    float v0 = wn.x, v1 = wn.y;
    row_finish<T, G>(v0, v1, j, c, pos, qk_norm, eps, r, theta, red);
    if (live) {
      typename T::S* dst = ring + ((int64_t)b * n_win + pos % n_win) * c;
      T::st(dst, 2 * j, v0);
      T::st(dst, 2 * j + 1, v1);
    }
  }
}

// ===========================================================================
// Host launchers
// ===========================================================================
template <int TM, int TN>
static void gemm_bf16_tiles(const void* A, int64_t lda, int64_t M, int K, const WeightStack& w,
                            const GemmOuts& outs, bool bf16_out, int groups, int64_t a_zoff,
                            int64_t w_zoff, int64_t o_zoff, hipStream_t st) {
  const int N = w.total();
  const int mblocks = (int)((M + TM - 1) / TM), ntiles = (N + TN - 1) / TN;
  const int mgroups = ((mblocks + 7) / 8 + 7) / 8;  // groups of 8 M blocks per die
  const dim3 g((unsigned)(8 * mgroups * 8 * ntiles), (unsigned)groups);
  if (bf16_out)
    proj_gemm_bf16_kernel<uint16_t, TM, TN><<<g, 512, 0, st>>>(
        (const uint16_t*)A, lda, M, K, (const uint16_t*)w.w[0], w.rows[0],
        (const uint16_t*)w.w[1], w.rows[1], (const uint16_t*)w.w[2], w.rows[2], outs, mblocks,
        ntiles, a_zoff, w_zoff, o_zoff);
  else
    proj_gemm_bf16_kernel<float, TM, TN><<<g, 512, 0, st>>>(
        (const uint16_t*)A, lda, M, K, (const uint16_t*)w.w[0], w.rows[0],
        (const uint16_t*)w.w[1], w.rows[1], (const uint16_t*)w.w[2], w.rows[2], outs, mblocks,
        ntiles, a_zoff, w_zoff, o_zoff);
}

// Tile shape: 256x256 when that gives every CU a workgroup (per group of a
// grouped product), else the smaller tiles, which give narrow products (few
// 256-column tiles, a partly empty last one) more workgroups.
hipError_t launch_gemm_bf16(const void* A, int64_t lda, int64_t M, int K, const WeightStack& w,
                            const GemmOuts& outs, bool bf16_out, int groups, int64_t a_zoff,
                            int64_t w_zoff, int64_t o_zoff, hipStream_t st) {
  const int N = w.total();
  if (M == 0 || N == 0 || groups == 0) return hipSuccess;
  const int64_t wg256 = (int64_t)groups * ((M + 255) / 256) * ((N + 255) / 256);
  if (wg256 >= kGemmBigTileMinWorkgroups)
    gemm_bf16_tiles<256, 256>(A, lda, M, K, w, outs, bf16_out, groups, a_zoff, w_zoff, o_zoff, st);
  else
    gemm_bf16_tiles<kGemmSmallTM, 128>(A, lda, M, K, w, outs, bf16_out, groups, a_zoff, w_zoff,
                                       o_zoff, st);
  return hipGetLastError();
}

hipError_t launch_proj_gemm(int dtype, const void* A, int64_t M, int K, const WeightStack& w,
                            float* out, int64_t ldo, hipStream_t st) {
  const int N = w.total();
  dim3 grid((N + 127) / 128, (unsigned)((M + 127) / 128));
  if (dtype == CSA_BF16) {
    GemmOuts o;
    o.p[0] = out;
    o.p[1] = out + w.rows[0];
    o.p[2] = out + w.rows[0] + w.rows[1];
    o.ld[0] = o.ld[1] = o.ld[2] = ldo;
    return launch_gemm_bf16(A, K, M, K, w, o, false, 1, 0, 0, 0, st);
  } else if (N <= kF32KSplitMaxN) {  // by N only: the same kernel for every M
    const dim3 g64((N + 63) / 64, (unsigned)((M + 63) / 64));
    proj_gemm_f32_ksplit_kernel<<<g64, 256, 0, st>>>((const float*)A, M, K, (const float*)w.w[0],
                                                     w.rows[0], (const float*)w.w[1], w.rows[1],
                                                     (const float*)w.w[2], w.rows[2], out, ldo);
  } else {
    proj_gemm_kernel<F32><<<grid, 256, 0, st>>>((const float*)A, M, K, (const float*)w.w[0],
                                                 w.rows[0], (const float*)w.w[1], w.rows[1],
                                                 (const float*)w.w[2], w.rows[2], out, ldo);
  }
  return hipGetLastError();
}

#define CSA_DISPATCH_G(c, ...)                                  \
  switch (c) {                                                  \
    case 32: { constexpr int G = 16; __VA_ARGS__; } break;      \
    case 64: { constexpr int G = 32; __VA_ARGS__; } break;      \
    case 128: { constexpr int G = 64; __VA_ARGS__; } break;     \
    case 256: { constexpr int G = 128; __VA_ARGS__; } break;    \
    case 512: { constexpr int G = 256; __VA_ARGS__; } break;    \
    default: return hipErrorInvalidValue;                       \
  }

hipError_t launch_pool_entries(int dtype, const float* P, int64_t ld, int64_t n, int c, int m,
                               int ov, const float* ape, int qk_norm, float eps, int r,
                               float theta, void* out, int64_t pos0, hipStream_t st, int prev0,
                               EntryMap em) {
  const int64_t ne = n / m;
  if (ne == 0) return hipSuccess;
  CSA_DISPATCH_G(c, {
    if (m >= kPoolSplitM) {  // a choice by m alone: chunks and one-shot calls agree
      if (dtype == CSA_BF16)
        pool_entries_split_kernel<BF16, G><<<(unsigned)ne, 256, 0, st>>>(
            P, ld, ne, c, m, ov, ape, qk_norm, eps, r, theta, (BF16::S*)out, pos0, prev0, em);
      else
        pool_entries_split_kernel<F32, G><<<(unsigned)ne, 256, 0, st>>>(
            P, ld, ne, c, m, ov, ape, qk_norm, eps, r, theta, (float*)out, pos0, prev0, em);
    } else {
      dim3 grid((unsigned)((ne + 256 / G - 1) / (256 / G)));
      if (dtype == CSA_BF16)
        pool_entries_kernel<BF16, G><<<grid, 256, 0, st>>>(P, ld, ne, c, m, ov, ape, qk_norm, eps,
                                                           r, theta, (BF16::S*)out, pos0, prev0, em);
      else
        pool_entries_kernel<F32, G><<<grid, 256, 0, st>>>(P, ld, ne, c, m, ov, ape, qk_norm, eps,
                                                          r, theta, (float*)out, pos0, prev0, em);
    }
  });
  return hipGetLastError();
}

hipError_t launch_window_rows(int dtype, const float* P, int64_t ld, int col, int64_t n, int c,
                              int qk_norm, float eps, int r, float theta, void* out, void* ring,
                              int n_win, int64_t pos0, hipStream_t st) {
  if (n == 0) return hipSuccess;
  CSA_DISPATCH_G(c, {
    dim3 grid((unsigned)((n + 256 / G - 1) / (256 / G)));
    if (dtype == CSA_BF16)
      window_rows_kernel<BF16, G><<<grid, 256, 0, st>>>(P, ld, col, n, c, qk_norm, eps, r, theta,
                                                        (BF16::S*)out, (BF16::S*)ring, n_win, pos0);
    else
      window_rows_kernel<F32, G><<<grid, 256, 0, st>>>(P, ld, col, n, c, qk_norm, eps, r, theta,
                                                       (float*)out, (float*)ring, n_win, pos0);
  });
  return hipGetLastError();
}

hipError_t launch_stash_state(const float* P, int64_t ld, int64_t n, int c, int m, int ov,
                              const float* ape, float* state, hipStream_t st) {
  stash_state_kernel<<<1, 256, 0, st>>>(P, ld, n, c, m, ov, ape, state);
  return hipGetLastError();
}

hipError_t launch_state_init(float* state, int64_t per_seq, int batch, int c, hipStream_t st) {
  const int64_t total = per_seq * batch;
  const unsigned blocks = (unsigned)((total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096);
  state_init_kernel<<<blocks, 256, 0, st>>>(state, per_seq, c, batch);
  return hipGetLastError();
}

int decode_proj_ksplit(int N, int K, int dtype) {
  const int kg4 = (dtype == CSA_BF16 ? 16 : 8) * 4;  // smallest per-wave slice
  const int tiles = (N + 31) / 32;
  // At most kMaxKSplit slices: the update kernel sums the slices of a column in
  // one workgroup per sequence, so more slices would make that sum slower.
  int ks = 1;
  while (tiles * ks < 512 && K % (ks * 2 * kg4) == 0 && ks < kMaxKSplit) ks *= 2;
  return ks;
}

hipError_t launch_decode_proj(int dtype, const void* h, int B, int K, const WeightStack& w,
                              float* part, int ksplit, hipStream_t st) {
  const int N = w.total();
  dim3 grid((N + 31) / 32, ksplit, (B + 31) / 32);
  if (dtype == CSA_BF16) {
    typedef BF16::S S;
    decode_proj_kernel<BF16><<<grid, 256, 0, st>>>((const S*)h, B, K, (const S*)w.w[0], w.rows[0],
                                                    (const S*)w.w[1], w.rows[1], (const S*)w.w[2],
                                                    w.rows[2], part, ksplit);
  } else {
    decode_proj_kernel<F32><<<grid, 256, 0, st>>>((const float*)h, B, K, (const float*)w.w[0],
                                                   w.rows[0], (const float*)w.w[1], w.rows[1],
                                                   (const float*)w.w[2], w.rows[2], part, ksplit);
  }
  return hipGetLastError();
}

hipError_t launch_decode_update(int dtype, const float* part, int ksplit, int B, int N, int c,
                                int m, int ov, int has_win, const float* ape, const int64_t* pos,
                                float* state, void* cache, int64_t max_entries, void* ring,
                                int n_win, int qk_norm, float eps, int r, float theta,
                                hipStream_t st, EntryMap em) {
  CSA_DISPATCH_G(c, {
    const int threads = G < 64 ? 64 : G;
    if (dtype == CSA_BF16)
      decode_update_kernel<BF16, G><<<B, threads, 0, st>>>(
          part, ksplit, B, N, c, m, ov, has_win, ape, pos, state, (BF16::S*)cache, max_entries,
          (BF16::S*)ring, n_win, qk_norm, eps, r, theta, em);
    else
      decode_update_kernel<F32, G><<<B, threads, 0, st>>>(
          part, ksplit, B, N, c, m, ov, has_win, ape, pos, state, (float*)cache, max_entries,
          (float*)ring, n_win, qk_norm, eps, r, theta, em);
  });
  return hipGetLastError();
}

}  // namespace csa
