// The layer around the four attention calls: the query path and the grouped
// output projection.
//
// Citation keys: [R] = page "DeepSeek-V4 技术解读报告" (juejin.cn), section
// 2.3.1 eq 13-15 and 18 (low-rank query path shared by the attention and the
// indexer), 2.3.1 (d) (grouped output projection); [A] = page
// "DeepSeek-V4：算法架构" (1zeryu.github.io), the "Q, K, V 映射与位置编码注入"
// excerpt (wq_a -> q_norm -> wq_b), the Indexer's weights_proj, and the
// "输出投影" excerpt (wo_a per group, then wo_b).
//
// All products run on the bf16 projection GEMM (32x32x16 MFMA, LDS ring fed
// by direct global->LDS loads); the latent RMSNorm is one small row kernel.
#include "csa_common.h"
#include "csa_launch.h"

namespace csa {

// Latent RMSNorm of the first product: row r of P (stride ld, a multiple of
// 4) holds h.W_DQ^T in columns [0, dc) and h.W_w^T in [dc, dc + ni).  One wave per row: lane l takes
// float4 groups l, l+64, ...; the mean square is a wave sum.  Writes the
// normalised latent (times g, if given) and w^I, each rounded to bf16 once.
__global__ __launch_bounds__(256) void latent_norm_kernel(const float* __restrict__ P, int64_t n,
                                                          int ld, int dc, int ni,
                                                          const float* __restrict__ g, float eps,
                                                          uint16_t* __restrict__ cq,
                                                          uint16_t* __restrict__ wI) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= n) return;  // whole wave
  const float* row = P + r * ld;
  float ss = 0.f;
  for (int j = 4 * lane; j < dc; j += 256) {
    const float4 v = *(const float4*)(row + j);
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  ss = wave_sum(ss);
  const float inv = rsqrtf(ss / (float)dc + eps);
  uint16_t* crow = cq + r * dc;
  for (int j = 4 * lane; j < dc; j += 256) {
    const float4 v = *(const float4*)(row + j);
    float4 s = make_float4(inv, inv, inv, inv);
    if (g) {
      const float4 gg = *(const float4*)(g + j);
      s = make_float4(inv * gg.x, inv * gg.y, inv * gg.z, inv * gg.w);
    }
    const uint32_t w0 = (uint32_t)f32_to_bf16(v.x * s.x) | ((uint32_t)f32_to_bf16(v.y * s.y) << 16);
    const uint32_t w1 = (uint32_t)f32_to_bf16(v.z * s.z) | ((uint32_t)f32_to_bf16(v.w * s.w) << 16);
    *(uint2*)(crow + j) = make_uint2(w0, w1);
  }
  for (int j = lane; j < ni; j += 64) wI[r * ni + j] = f32_to_bf16(row[dc + j]);
}

static int64_t latent_ld(const csa_query_desc& d) { return (d.d_c + d.n_heads_i + 3) & ~3; }

static size_t latent_bytes(const csa_query_desc& d) {
  return ((size_t)d.n * latent_ld(d) * 4 + 255) & ~(size_t)255;
}

size_t query_proj_ws_bytes(const csa_query_desc& d) {
  return latent_bytes(d) + (size_t)d.n * d.d_c * 2;
}

hipError_t launch_query_proj(const csa_query_desc& d, const void* H, const void* W_DQ,
                             const float* g_q, const void* W_w, const void* W_UQ,
                             const void* W_IUQ, void* q_out, void* qI_out, void* wI_out,
                             void* ws, hipStream_t st) {
  if (d.n == 0) return hipSuccess;
  float* P = (float*)ws;  // [n, latent_ld] fp32
  uint16_t* cq = (uint16_t*)((uint8_t*)ws + latent_bytes(d));  // [n, d_c] bf16
  // 1. h . [W_DQ; W_w]^T -> P (fp32)
  WeightStack w1 = {{W_DQ, W_w, nullptr}, {d.d_c, d.n_heads_i, 0}};
  GemmOuts o1;
  o1.p[0] = P;
  o1.p[1] = P + d.d_c;
  o1.p[2] = P;
  o1.ld[0] = o1.ld[1] = o1.ld[2] = latent_ld(d);
  hipError_t e = launch_gemm_bf16(H, d.d, d.n, d.d, w1, o1, false, 1, 0, 0, 0, st);
  if (e != hipSuccess) return e;
  // 2. latent RMSNorm -> c^Q (bf16), w^I (bf16)
  latent_norm_kernel<<<(unsigned)((d.n + 3) / 4), 256, 0, st>>>(
      P, d.n, (int)latent_ld(d), d.d_c, d.n_heads_i, g_q, d.eps, cq, (uint16_t*)wI_out);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // 3. c^Q . [W_UQ; W_IUQ]^T -> q, q^I (bf16)
  WeightStack w2 = {{W_UQ, W_IUQ, nullptr}, {d.n_heads * d.c, d.n_heads_i * d.c_i, 0}};
  GemmOuts o2;
  o2.p[0] = q_out;
  o2.p[1] = qI_out;
  o2.p[2] = q_out;
  o2.ld[0] = (int64_t)d.n_heads * d.c;
  o2.ld[1] = (int64_t)d.n_heads_i * d.c_i;
  o2.ld[2] = o2.ld[0];
  return launch_gemm_bf16(cq, d.d_c, d.n, d.d_c, w2, o2, true, 1, 0, 0, 0, st);
}

size_t output_proj_ws_bytes(const csa_oproj_desc& d) {
  return (size_t)d.n * d.groups * d.d_g * 2;
}

hipError_t launch_output_proj(const csa_oproj_desc& d, const void* o, const void* wo_a,
                              const void* wo_b, void* out, void* ws, hipStream_t st) {
  if (d.n == 0) return hipSuccess;
  const int64_t width = (int64_t)d.n_heads * d.c;
  const int kg = (int)(width / d.groups);
  uint16_t* mid = (uint16_t*)ws;  // [n, groups * d_g] bf16
  // 1. group j: o[:, j*kg : (j+1)*kg] . wo_a[j]^T -> mid[:, j*d_g : (j+1)*d_g]
  WeightStack w1 = {{wo_a, nullptr, nullptr}, {d.d_g, 0, 0}};
  GemmOuts o1;
  o1.p[0] = o1.p[1] = o1.p[2] = mid;
  o1.ld[0] = o1.ld[1] = o1.ld[2] = (int64_t)d.groups * d.d_g;
  hipError_t e = launch_gemm_bf16(o, width, d.n, kg, w1, o1, true, d.groups, kg,
                                  (int64_t)d.d_g * kg, d.d_g, st);
  if (e != hipSuccess) return e;
  // 2. mid . wo_b^T -> out
  WeightStack w2 = {{wo_b, nullptr, nullptr}, {d.d, 0, 0}};
  GemmOuts o2;
  o2.p[0] = o2.p[1] = o2.p[2] = out;
  o2.ld[0] = o2.ld[1] = o2.ld[2] = d.d;
  return launch_gemm_bf16(mid, (int64_t)d.groups * d.d_g, d.n, d.groups * d.d_g, w2, o2, true, 1,
                          0, 0, 0, st);
}

}  // namespace csa
