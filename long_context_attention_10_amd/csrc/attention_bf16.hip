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

typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
#define CSA_LDS __attribute__((address_space(3)))

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

// 16 bytes per lane from global memory straight into LDS (global_load_lds):
// lane l's bytes land at lds_base + 16*l, lds_base wave-uniform (in M0).
// Written as inline asm so that the compiler does not track it -- with the
// builtin it conservatively waits for the load before every LDS read, which
// serialises the gather with the compute.  This kernel enforces completion
// itself (wait_vmem, then a barrier) before a filled buffer is read, and no
// other code in it uses M0.
CSA_DEV void lds_dma16(const void* g, const void* lds_dst) {
  const uint32_t base =
      __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(CSA_LDS const void*)lds_dst);
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(g), "s"(base)
      : "memory");
}

CSA_DEV void wait_vmem() { __builtin_amdgcn_s_waitcnt(0); }

}  // namespace

template <int C, bool SPARSE>
__global__ __launch_bounds__(256, 2) void mqa_prefill_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ win,
    const uint16_t* __restrict__ comp, const int32_t* __restrict__ idx,
    const float* __restrict__ sink, uint16_t* __restrict__ out, int64_t n, int nh, int k, int m,
    int n_win, float scale, int qk_norm, float eps, int r, float theta, int64_t n_entries) {
  typedef Geo<C> G;
  constexpr int NKG = C / 32;   // 32-wide k-groups of the head dim
  constexpr int NCB = C / 16;   // 16-channel output blocks
  __shared__ __align__(16) uint8_t smem[G::BUF];
  __shared__ int valid[2][kT];
  __shared__ int sidx[SPARSE ? kMaxK : 1];
  __shared__ float2 rope_tab[C / 2];  // (cos, sin) of this token's RoPE pairs

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int lc = lane & 15, lg = lane >> 4;

  // XCD-aware order: the 8 dies each take a contiguous range of tokens, so a
  // die's L2 keeps the window rows its consecutive tokens share.
  const int64_t per = (n + 7) >> 3;
  const int64_t t = (int64_t)(blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (t >= n) return;

  const int nwin = (int)min64(n_win, t + 1);
  const int64_t ncomp = SPARSE ? (int64_t)k : min64((t + 1) / m, n_entries);
  const int64_t ncand = nwin + ncomp;
  const int ntiles = (int)((ncand + kT - 1) / kT);
  const int32_t* irow = SPARSE ? idx + t * (int64_t)k : nullptr;
  const uint16_t* qrow = q + t * (int64_t)nh * C;

  // ------------------------ index row and RoPE angles -> LDS; q -> registers
  if (SPARSE)
    for (int j = tid; j < k; j += 256) sidx[j] = irow[j];
  if (tid < r / 2) {  // one angle per RoPE pair, shared by prologue and epilogue
    float cs, sn;
    rope_cs(t, tid, r, theta, &cs, &sn);
    rope_tab[tid] = make_float2(cs, sn);
  }
  // lane (lg, lc) holds Q[head][32g + 8lg .. +8] for g = 0..C/32-1: the B
  // operand of S^T = K Q^T.  Loaded straight from global memory so that the
  // first candidate tile can stream into LDS at the same time.
  const int head = wave * 16 + lc;
  uint4 qraw[NKG];
  {
    const uint16_t* qh = qrow + (int64_t)(head < nh ? head : 0) * C + lg * 8;
#pragma unroll
    for (int g = 0; g < NKG; ++g) qraw[g] = *(const uint4*)(qh + g * 32);
  }
  __syncthreads();  // sidx and rope_tab are visible

  // ------------------------------------------------ candidate tile loader
  auto issue_tile = [&](int ti, int buf) {
    uint8_t* base = smem + buf * G::TILE;
    constexpr int BPW = kT / G::RPI / 4;  // bursts (1 KiB each) per wave
    const uint8_t* src[BPW];
    // resolve every row first, then issue the loads back to back
#pragma unroll
    for (int u = 0; u < BPW; ++u) {
      const int bi = wave + 4 * u;
      const int row = bi * G::RPI + lane / (64 / G::RPI);
      const int64_t j = (int64_t)ti * kT + row;
      const uint16_t* r = win;  // a valid row for masked candidates
      bool ok = false;
      if (j < ncand) {
        if (j < nwin) {
          r = win + (t - nwin + 1 + j) * C;
          ok = true;
        } else {
          const int64_t e = SPARSE ? (int64_t)sidx[j - nwin] : j - nwin;
          if (e >= 0 && e < n_entries) { r = comp + e * C; ok = true; }
        }
      }
      src[u] = (const uint8_t*)r + (lane % (64 / G::RPI)) * 16;
      if ((lane % (64 / G::RPI)) == 0) valid[buf][row] = ok;
    }
#pragma unroll
    for (int u = 0; u < BPW; ++u) lds_dma16(src[u], base + (wave + 4 * u) * G::BURST);
  };

  if (ntiles > 0) issue_tile(0, 0);

  // --------------------------------- q prologue: RMSNorm, RoPE, bf16 regs
  bf16x8_t qf[NKG];
  {
    float ss = 0.f;
#pragma unroll
    for (int g = 0; g < NKG; ++g) {
      float v[8];
      chunk_to_f32<BF16>(qraw[g], v);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += v[e] * v[e];
    }
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
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
            const float2 cs = rope_tab[(ch - (C - r)) >> 1];
            const float x0 = v[e], x1 = v[e + 1];
            v[e] = x0 * cs.x - x1 * cs.y;
            v[e + 1] = x0 * cs.y + x1 * cs.x;
          }
        }
      }
      qf[g] = __builtin_bit_cast(bf16x8_t, f32_to_chunk<BF16>(v));
    }
  }

  // ----------------------------------------------------- softmax state
  constexpr float LOG2E = 1.4426950408889634f;
  const float sl2 = scale * LOG2E;
  float run_m = (head < nh ? sink[head] : 0.f) * LOG2E;  // log2 units
  float run_l = 1.f;

  // O accumulators in two halves of at most 16 blocks: the compiler keeps
  // fully unrolled 16-entry arrays in registers, not 32-entry ones.
  constexpr int NLO = NCB > 16 ? 16 : NCB;
  constexpr int NHI = NCB > 16 ? NCB - 16 : 1;
  f32x4_t o_lo[NLO], o_hi[NHI];
#pragma unroll
  for (int cb = 0; cb < NLO; ++cb) o_lo[cb] = f32x4_t{};
#pragma unroll
  for (int cb = 0; cb < NHI; ++cb) o_hi[cb] = f32x4_t{};

  wait_vmem();  // tile 0 (and q) have landed
  __syncthreads();

  // Candidate slot permutation.  Lane group lg (lanes 16*lg..16*lg+15) holds,
  // after the logits, the 8 tile rows pi(lg, h, i) = 16*(lg/2) + 8*h + 4*(lg%2) + i
  // (h = 0, 1; i = 0..3); those rows are also its PV reduction slots 8*lg+4*h+i.
  // With 1056-byte LDS rows (8 banks apart) both the 16-byte K reads (rows
  // pi(lc/4, b, lc%4) for lanes lc) and the transpose reads (4 consecutive
  // rows per 16-lane group) touch distinct banks.
  auto pi = [](int g, int h, int i) { return 16 * (g >> 1) + 8 * h + 4 * (g & 1) + i; };
  const int koff0 = G::off(pi(lc >> 2, 0, lc & 3)) + lg * 16;
  const int koff1 = G::off(pi(lc >> 2, 1, lc & 3)) + lg * 16;
  const int troff0 = G::off(pi(lg, 0, lc >> 2)) + 8 * (lc & 3);
  const int troff1 = G::off(pi(lg, 1, lc >> 2)) + 8 * (lc & 3);

  for (int ti = 0; ti < ntiles; ++ti) {
    const int buf = ti & 1;
    if (ti + 1 < ntiles) issue_tile(ti + 1, buf ^ 1);
    const uint8_t* kv = smem + buf * G::TILE;

    // S^T = K Q^T for the tile: block b's A rows are K rows pi(lc/4, b, lc%4)
    f32x4_t s[2] = {f32x4_t{}, f32x4_t{}};
#pragma unroll
    for (int g = 0; g < NKG; ++g) {
      const bf16x8_t a0 = *(const bf16x8_t*)(kv + koff0 + g * 64);
      const bf16x8_t a1 = *(const bf16x8_t*)(kv + koff1 + g * 64);
      s[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qf[g], s[0], 0, 0, 0);
      s[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qf[g], s[1], 0, 0, 0);
    }
    // online softmax for head `head` (this lane's column) in log2 units
    float z[8];
    float mx = -INFINITY;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float zz = valid[buf][pi(lg, b, i)] ? s[b][i] * sl2 : -INFINITY;
        z[4 * b + i] = zz;
        mx = fmaxf(mx, zz);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const bool need = mx > run_m + 8.f;
    if (__any(need)) {  // wave-uniform rescale of O
      const float nm = fmaxf(run_m, mx);
      const float alpha = __builtin_amdgcn_exp2f(run_m - nm);
      run_l *= alpha;
      run_m = nm;
#pragma unroll
      for (int cb = 0; cb < NLO; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i) o_lo[cb][i] *= alpha;
      if constexpr (NCB > 16) {
#pragma unroll
        for (int cb = 0; cb < NHI; ++cb)
#pragma unroll
          for (int i = 0; i < 4; ++i) o_hi[cb][i] *= alpha;
      }
    }
    f32x8_t p;
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      p[j] = __builtin_amdgcn_exp2f(z[j] - run_m);
      ps += p[j];
    }
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    run_l += ps;
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
    for (int cb = 0; cb < NLO; ++cb) pv(cb, o_lo[cb]);
    if constexpr (NCB > 16) {
#pragma unroll
      for (int cb = 0; cb < NHI; ++cb) pv(NLO + cb, o_hi[cb]);
    }
    wait_vmem();
    __syncthreads();
  }

  // ------------------------------------------------------------ epilogue
  // O^T lane layout: block cb, element i = O[head][cb*16 + 4*lg + i]
  const float inv = 1.f / run_l;
  uint8_t* ostage = smem;  // [head][C] bf16, padded like q
  auto emit = [&](int cb, const f32x4_t& acc) {
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = acc[i] * inv;
    const int ch0 = cb * 16 + 4 * lg;
    if (r > 0 && ch0 >= C - r) {
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        const float2 cs = rope_tab[(ch0 + i - (C - r)) >> 1];
        const float x0 = v[i], x1 = v[i + 1];
        v[i] = x0 * cs.x + x1 * cs.y;      // rotate by -t
        v[i + 1] = -x0 * cs.y + x1 * cs.x;
      }
    }
    const uint32_t w0 = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
    const uint32_t w1 = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
    *(uint2*)(ostage + G::off(head) + ch0 * 2) = make_uint2(w0, w1);
  };
#pragma unroll
  for (int cb = 0; cb < NLO; ++cb) emit(cb, o_lo[cb]);
  if constexpr (NCB > 16) {
#pragma unroll
    for (int cb = 0; cb < NHI; ++cb) emit(NLO + cb, o_hi[cb]);
  }
  __syncthreads();
  uint16_t* orow = out + t * (int64_t)nh * C;
  const int chunks = nh * C / 8;  // 16-byte chunks of this token's output
  for (int ci = tid; ci < chunks; ci += 256) {
    const int h = ci / (C / 8), cc = ci % (C / 8);
    *(uint4*)(orow + (int64_t)h * C + cc * 8) = *(const uint4*)(ostage + G::off(h) + cc * 16);
  }
}

hipError_t launch_mqa_prefill_bf16(const csa_attn_desc& d, int mode, const void* q, const void* win,
                                   const void* comp, const int32_t* idx, const float* sink,
                                   void* out, hipStream_t st) {
  const unsigned grid = (unsigned)(((d.n + 7) / 8) * 8);
#define CSA_FAST(CC)                                                                          \
  if (d.c == CC) {                                                                           \
    if (mode == ATTN_SPARSE)                                                                 \
      mqa_prefill_bf16_kernel<CC, true><<<grid, 256, 0, st>>>(                               \
          (const uint16_t*)q, (const uint16_t*)win, (const uint16_t*)comp, idx, sink,         \
          (uint16_t*)out, d.n, d.n_heads, d.k, d.m, d.n_win, d.scale, d.qk_norm, d.eps,       \
          d.rope_dims, d.rope_theta, d.n_entries);                                            \
    else                                                                                     \
      mqa_prefill_bf16_kernel<CC, false><<<grid, 256, 0, st>>>(                              \
          (const uint16_t*)q, (const uint16_t*)win, (const uint16_t*)comp, idx, sink,         \
          (uint16_t*)out, d.n, d.n_heads, d.k, d.m, d.n_win, d.scale, d.qk_norm, d.eps,       \
          d.rope_dims, d.rope_theta, d.n_entries);                                            \
    return hipGetLastError();                                                                \
  }
  CSA_FAST(128) CSA_FAST(256) CSA_FAST(512)
#undef CSA_FAST
  return hipErrorInvalidValue;
}

}  // namespace csa
