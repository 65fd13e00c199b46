// Device-side building blocks shared by the libcsa kernels (gfx950 only).
//
// Element storage: fp32 as float, bf16 as uint16_t bit patterns.  Matrix-core
// operands are always moved as 16-byte chunks per lane ("uint4"), which hold
// 8 bf16 or 4 fp32 values that are consecutive along the reduction axis.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define CSA_DEV __device__ __forceinline__

namespace csa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
#define CSA_LDS __attribute__((address_space(3)))

// ---------------------------------------------------------------- bf16 <-> f32
CSA_DEV float bf16_to_f32(uint16_t x) { return __uint_as_float(((uint32_t)x) << 16); }

// Round to nearest, ties to even: gfx950's hardware conversion
// (v_cvt_pk_bf16_f32).
CSA_DEV uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

struct F32 {
  typedef float S;  // storage
  static constexpr int kPerChunk = 4;
  CSA_DEV static float ld(const S* p, int64_t i) { return p[i]; }
  CSA_DEV static void st(S* p, int64_t i, float v) { p[i] = v; }
  CSA_DEV static S cvt(float v) { return v; }
  CSA_DEV static float f(S v) { return v; }
};

struct BF16 {
  typedef uint16_t S;
  static constexpr int kPerChunk = 8;
  CSA_DEV static float ld(const S* p, int64_t i) { return bf16_to_f32(p[i]); }
  CSA_DEV static void st(S* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
  CSA_DEV static S cvt(float v) { return f32_to_bf16(v); }
  CSA_DEV static float f(S v) { return bf16_to_f32(v); }
};

// Unpack / pack a 16-byte chunk to/from fp32 values.
template <class T> CSA_DEV void chunk_to_f32(const uint4& c, float* v);
template <> CSA_DEV void chunk_to_f32<F32>(const uint4& c, float* v) {
  v[0] = __uint_as_float(c.x); v[1] = __uint_as_float(c.y);
  v[2] = __uint_as_float(c.z); v[3] = __uint_as_float(c.w);
}
template <> CSA_DEV void chunk_to_f32<BF16>(const uint4& c, float* v) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
template <class T> CSA_DEV uint4 f32_to_chunk(const float* v);
template <> CSA_DEV uint4 f32_to_chunk<F32>(const float* v) {
  return make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                    __float_as_uint(v[3]));
}
typedef __attribute__((__vector_size__(8 * sizeof(float)))) float f32x8_t;
template <> CSA_DEV uint4 f32_to_chunk<BF16>(const float* v) {
  const f32x8_t f = {v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7]};
  return __builtin_bit_cast(uint4, __builtin_convertvector(f, bf16x8_t));
}

// ------------------------------------------------------------ matrix cores
// 16x16 output block.  Lane l supplies A row (l % 16) and B column (l % 16);
// its 16-byte chunk covers reduction indices [g*E, g*E+E) of a 4*E-wide
// k-group, g = l / 16, E = elements per chunk.  acc[i] = D[4*(l/16)+i][l%16].
template <class T> CSA_DEV void mma16(f32x4_t& acc, const uint4& a, const uint4& b);
template <> CSA_DEV void mma16<BF16>(f32x4_t& acc, const uint4& a, const uint4& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
}
template <> CSA_DEV void mma16<F32>(f32x4_t& acc, const uint4& a, const uint4& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
}

// 32x32 output block.  Lane l supplies A row (l % 32), B column (l % 32), its
// chunk covering [g*E, g*E+E) of a 2*E-wide k-group, g = l / 32.
// acc[i] = D[8*(i/4) + 4*(l/32) + (i%4)][l % 32].
template <class T> CSA_DEV void mma32(f32x16_t& acc, const uint4& a, const uint4& b);
template <> CSA_DEV void mma32<BF16>(f32x16_t& acc, const uint4& a, const uint4& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
}
template <> CSA_DEV void mma32<F32>(f32x16_t& acc, const uint4& a, const uint4& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
}

// 32x32 output block of the scaled matrix instruction with E2M1 (FP4) A and
// B.  Lane l supplies A row (l % 32) and B column (l % 32): 32 consecutive
// values of the 64-wide k-group, [32*(l/32), 32*(l/32) + 32), as 16 bytes
// (value 2i in the low nibble of byte i, 2i + 1 in the high one), and that
// block's power-of-two scale as the biased exponent e + 127 in byte 0 of sa /
// sb (each lane scales its own 32 values).  acc layout as mma32.
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8_t;
CSA_DEV void mma32_fp4(f32x16_t& acc, const uint4& a, uint32_t sa, const uint4& b, uint32_t sb) {
  const i32x8_t av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  const i32x8_t bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 4, 4, 0, (int)sa, 0, (int)sb);
}

// ---------------------------------------------------------------- RoPE
// cos/sin of pos * theta^(-2p/r) for pair p.  The angle is formed and reduced
// modulo 2*pi in fp64 so that positions up to 2^20 and beyond keep fp32
// accuracy; the reduced angle is then evaluated in fp32.
CSA_DEV void rope_cs(int64_t pos, int pair, int r, float theta, float* cs, float* sn) {
  const double freq = exp2(-(2.0 * pair / (double)r) * log2((double)theta));
  double a = (double)pos * freq;
  const double two_pi = 6.283185307179586476925286766559;
  a -= two_pi * rint(a / two_pi);
  sincosf((float)a, sn, cs);
}

// ------------------------------------------------------------ reductions
CSA_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
CSA_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Max / sum over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48)
// with the permlane swaps: every lane gets the same, bitwise identical value,
// and no LDS instruction is involved.
CSA_DEV float xlane_max(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
CSA_DEV float xlane_sum(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// v + v[lane ^ 32] (the same value, bitwise, in both lanes of each pair).
CSA_DEV float swap32_add(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

// Two half-wave sums in one swap: lanes 0-31 get a + a[lane + 32], lanes
// 32-63 get b[lane - 32] + b (v_permlane32_swap exchanges the upper half of
// its first operand with the lower half of its second).
CSA_DEV float swap32_pair_add(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Where entry e of sequence b sits in a decode cache: row b * n_entries + e
// of a contiguous [B, n_entries] cache when table is null, else row
// table[b * max_pages + e / page] * page + e % page of a page pool.
struct EntryMap {
  const int32_t* table = nullptr;
  int32_t page = 1;
  int32_t max_pages = 0;
  CSA_DEV int64_t row(int64_t b, int64_t e, int64_t n_entries) const {
    if (!table) return b * n_entries + e;
    const uint32_t u = (uint32_t)e;  // entries per sequence are < 2^31 when paged
    return (int64_t)table[b * max_pages + u / (uint32_t)page] * page + u % (uint32_t)page;
  }
};

// ---------------------------------------------------------------- FP8 KV rows
// A KV row of width c with r RoPE channels stored in FP8 ([A] act_quant of the
// channels without RoPE, block 64; [R] 2.3.4): the c - r E4M3 codes, then the
// r RoPE channels as bf16, then one scale byte e + 127 per 64-code block
// (scale 2^e), padded to a multiple of 16 bytes.
__host__ __device__ constexpr inline int kv8_row_bytes(int c, int r) {
  return ((c - r) + 2 * r + (c - r) / 64 + 15) & ~15;
}

// Order-preserving map fp32 -> uint32 (larger float -> larger key).
CSA_DEV uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// 16 bytes per lane from global memory straight into LDS (global_load_lds):
// lane l's bytes land at lds_base + 16*l, lds_base wave-uniform (in M0).
// Written as inline asm so that the compiler does not track it -- with the
// builtin it conservatively waits for the load before every LDS read, which
// serialises a gather with the compute that overlaps it.  Kernels using it
// enforce completion themselves (wait_vmem, then a barrier) before a filled
// buffer is read, and no other code in them uses M0.
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

// Wait for every outstanding memory operation of the wave.
CSA_DEV void wait_vmem() { __builtin_amdgcn_s_waitcnt(0); }

// Wait until at most N vector-memory operations of the wave are outstanding,
// as a compiler barrier: LDS reads of DMA-filled bytes that follow it in
// program order are not moved above it.  Loads complete in issue order, so
// this waits for all but the N newest.
template <int N>
CSA_DEV void wait_vmem_fence_n() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// s_waitcnt immediate that waits until at most n (< 64) vector-memory
// operations of the wave are outstanding; the other counters are left alone
// (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// max(x, 0) in one integer instruction: a float with the sign bit set is a
// negative int32, so a signed max with 0 zeroes exactly the negatives (and
// -0); fmaxf would first canonicalise x, since matrix-core results are not
// known to be canonical.
CSA_DEV float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

CSA_DEV int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }
CSA_DEV int64_t max64(int64_t a, int64_t b) { return a > b ? a : b; }

}  // namespace csa
