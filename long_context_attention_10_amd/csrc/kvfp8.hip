// FP8 storage of KV rows ([A] "Q, K, V 映射与位置编码注入" and the Compressor:
// act_quant of kv[..., :-rd] with block size 64; [R] 2.3.4: the KV cache keeps
// the RoPE dims in BF16 and the others in FP8).  The c - r channels without
// RoPE become E4M3 codes with one power-of-two scale per block of 64, the
// smallest 2^e with max |x| <= 448 * 2^e and e >= -117, each x / 2^e rounded
// to the nearest E4M3 value (ties to the even mantissa); the r RoPE channels
// are copied as bf16.  Row layout: see kv8_row_bytes in csa_common.h.
#include "csa_common.h"
#include "csa_launch.h"

namespace csa {

// |x| <= 448 (a scaled value): its E4M3 code, round to nearest, ties to even.
// Below 2^-6 the grid is m * 2^-9 (m = 0..8, where 8 is the smallest normal,
// code 8); above, the 3 kept mantissa bits are rounded on the 20 dropped ones,
// a carry moving into the exponent field.
CSA_DEV uint32_t e4m3_code(float x) {
  const float a = fabsf(x);
  uint32_t mag;
  if (a < 0.015625f) {
    mag = (uint32_t)rintf(a * 512.f);  // exact product; rintf rounds half to even
  } else {
    const uint32_t ua = __float_as_uint(a);
    const uint32_t ex = (ua >> 23) - 127 + 7;  // exponent field, 1..15
    const uint32_t man = ua & 0x7fffffu;
    uint32_t q = man >> 20;
    const uint32_t rem = man & 0xfffffu;
    q += (rem > 0x80000u) || (rem == 0x80000u && (q & 1u));
    mag = (ex << 3) + q;
  }
  return mag ? (mag | ((__float_as_uint(x) >> 24) & 0x80u)) : 0u;
}

// One wave per row of c = 512: lane l holds channels 8l .. 8l+7.
// rows: rows to convert; with posv (decode) wave b converts row
//   ring == 0: b * n + pos[b] / m, when (pos[b] + 1) % m == 0 (the entry the
//              step emitted), through the entry map;
//   ring != 0: b * n + pos[b] % n (the window slot of the new token).
template <class T>
__global__ __launch_bounds__(256) void kv_fp8_quant_kernel(
    const typename T::S* __restrict__ src, int64_t rows, int r, uint8_t* __restrict__ dst,
    const int64_t* __restrict__ posv, int64_t n, int m, int ring, EntryMap em) {
  constexpr int C = 512;
  const int lane = threadIdx.x & 63;
  int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // whole wave
  if (posv) {
    const int64_t p = posv[row];
    if (p < 0) return;
    if (ring) {
      row = row * n + p % n;
    } else {
      if ((p + 1) % m != 0 || p / m >= n) return;
      row = em.row(row, p / m, n);
    }
  }
  const int RB = kv8_row_bytes(C, r);
  const int nf = C - r;  // FP8 channels
  const typename T::S* x = src + row * C + 8 * lane;
  uint8_t* d = dst + row * RB;
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = T::ld(x, i);
  if (8 * lane < nf) {
    float am = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(v[i]));
#pragma unroll
    for (int o = 4; o >= 1; o >>= 1) am = fmaxf(am, __shfl_xor(am, o, 64));  // the 64-block
    int e = 0;
    if (am > 0.f) {
      int k;
      const float f = frexpf(am, &k);  // am = f * 2^k, 0.5 <= f < 1; 448 = 0.875 * 2^9
      e = f <= 0.875f ? k - 9 : k - 8;
    }
    e = e < -117 ? -117 : e;  // smallest grid step 2^(e-9) = 2^-126, an fp32 normal
    const float inv = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e, exact scaling
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w0 |= e4m3_code(v[i] * inv) << (8 * i);
      w1 |= e4m3_code(v[i + 4] * inv) << (8 * i);
    }
    *(uint2*)(d + 8 * lane) = make_uint2(w0, w1);
    if ((lane & 7) == 0) d[nf + 2 * r + lane / 8] = (uint8_t)(e + 127);
  } else {
    // a RoPE channel block: stored as bf16 (a copy when the source is bf16)
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (uint32_t)f32_to_bf16(v[2 * i]) | ((uint32_t)f32_to_bf16(v[2 * i + 1]) << 16);
    *(uint4*)(d + nf + 16 * (lane - nf / 8)) = make_uint4(w[0], w[1], w[2], w[3]);
  }
  if (lane == 0)  // the row's padding bytes, so that whole rows are defined
    for (int b = nf + 2 * r + nf / 64; b < RB; ++b) d[b] = 0;
}

hipError_t launch_kv_fp8_quant(int dtype, const void* src, int64_t rows, int r, uint8_t* dst,
                               const int64_t* pos, int64_t n, int m, int ring, hipStream_t st,
                               EntryMap em) {
  if (rows == 0) return hipSuccess;
  const unsigned g = (unsigned)((rows + 3) / 4);
  if (dtype == CSA_BF16)
    kv_fp8_quant_kernel<BF16><<<g, 256, 0, st>>>((const uint16_t*)src, rows, r, dst, pos, n, m,
                                                 ring, em);
  else
    kv_fp8_quant_kernel<F32><<<g, 256, 0, st>>>((const float*)src, rows, r, dst, pos, n, m, ring,
                                                em);
  return hipGetLastError();
}

}  // namespace csa
