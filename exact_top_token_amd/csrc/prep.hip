// Per-query preparation for the scoring kernels: the weighted query sum.
//
// The score uses the identity  w ReLU(x) = w x / 2 + w |x| / 2, so that
//     S(t,s) = 1/2 sum_h w_h |q_h . k_s|  +  1/2 (sum_h w_h q_h) . k_s .
// The first sum costs one fused multiply-add per head (|.| is a free operand
// modifier); the second is a single dot product with the weighted query
// qbar_t = sum_h w_h q_h.  qbar is computed here in float64 and stored as up
// to S terms in the query's MFMA operand type, qbar ~ sum_j sigma_j f_j
// (fp8: each term rescaled to the E4M3 range and taken from the residual of
// the previous ones; bf16: successive bf16 residuals; fp32: one term), so the
// scoring kernels evaluate it as S extra MFMA rows next to the heads.
// Whatever the terms leave out is measured exactly (e = ||qbar - sum_j
// sigma_j f_j||, float64) and enters the certificate's rounding margin.
#include "dosa_device.h"

namespace dosa {

__device__ __forceinline__ float dec_fp8_p(uint32_t x) {
  const uint32_t e = (x >> 3) & 15u, m = x & 7u;
  const float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
  return (x & 0x80u) ? -mag : mag;
}

__device__ __forceinline__ uint32_t enc_fp8_p(float x) {
  const uint32_t s = (x < 0.f) ? 0x80u : 0u;
  const float a = fminf(fabsf(x), 448.f);
  if (a < 0.015625f) return s | (uint32_t)rintf(a * 512.f);
  int e;
  const float f = frexpf(a, &e);
  uint32_t m = (uint32_t)rintf((f * 2.f - 1.f) * 8.f);
  int E = e - 1 + 7;
  if (m == 8) { m = 0; ++E; }
  if (E > 15 || (E == 15 && m == 7)) { E = 15; m = 6; }
  return s | ((uint32_t)E << 3) | m;
}

// One 64-lane wavefront per query; lane i owns elements i, i+64 (d <= 128).
// The query's H x d row and its weights are first staged in LDS with 16-byte
// loads that are all in flight together, so the per-element sums read LDS
// instead of waiting on one global load per head.
template <int C, int H, int D>
__global__ __launch_bounds__(64) void qbar_kernel(const PrepLaunch p) {
  constexpr int QB = (C == C_F32) ? 4 : (C == C_FP8 ? 1 : 2);
  constexpr int QW = queries_per_wave(C, H, D);
  constexpr int S = 16 / QW;                     // weighted-query terms per query
  constexpr int NT = (C == C_F32) ? 1 : (C == C_FP8 ? (S < 4 ? S : 4) : (S < 3 ? S : 3));
  constexpr int PER = (D + 63) / 64;
  constexpr int ROWB = H * D * QB;               // bytes of H head rows (a multiple of 16)
  constexpr int NCH = (ROWB / 16 + 63) / 64;     // 16-byte chunks per lane
  __shared__ __attribute__((aligned(16))) uint8_t qrow[ROWB];
  __shared__ float wrow[H];
  const int q = blockIdx.x;
  const int lane = lane_id();
  if (q >= p.total_q) return;
  const int Hr = p.H;                            // heads stored per query (<= H)
  const int NC = Hr * D * QB / 16;               // 16-byte chunks of the stored row
  {
    const v4i* src = reinterpret_cast<const v4i*>(static_cast<const uint8_t*>(p.q) + (int64_t)q * NC * 16);
    v4i c[NCH];
#pragma unroll
    for (int u = 0; u < NCH; ++u) c[u] = (lane + 64 * u < NC) ? src[lane + 64 * u] : v4i{0, 0, 0, 0};
    const float wv = lane < Hr ? p.w[(int64_t)q * Hr + lane] : 0.f;
#pragma unroll
    for (int u = 0; u < NCH; ++u)
      if (lane + 64 * u < NC) reinterpret_cast<v4i*>(qrow)[lane + 64 * u] = c[u];
    if (lane < H) wrow[lane] = wv;
  }
  __syncthreads();
  const uint8_t* qraw = qrow;
  // lane owns the PER consecutive elements PER*lane .. PER*lane + PER - 1
  // (d = 64: one, d = 128: a pair, decoded together: fp8 by the hardware
  // converter, exact for every finite E4M3 code)
  double r[PER];
#pragma unroll
  for (int v = 0; v < PER; ++v) r[v] = 0.0;
  for (int h = 0; h < Hr; ++h) {
    const double wh = (double)wrow[h];
    float x[PER];
    if constexpr (PER == 2 && C == C_FP8) {
      const uint32_t two = (uint32_t)reinterpret_cast<const uint16_t*>(qraw)[(h * D) / 2 + lane];
      const uint32_t bf = fp8x2_to_bf16x2<false>(two);
      x[0] = __uint_as_float(bf << 16);
      x[1] = __uint_as_float(bf & 0xFFFF0000u);
    } else if constexpr (PER == 2 && C == C_F32) {
      const float2 f = reinterpret_cast<const float2*>(qraw)[(h * D) / 2 + lane];
      x[0] = f.x;
      x[1] = f.y;
    } else if constexpr (PER == 2) {
      const uint32_t bf = reinterpret_cast<const uint32_t*>(qraw)[(h * D) / 2 + lane];
      x[0] = __uint_as_float(bf << 16);
      x[1] = __uint_as_float(bf & 0xFFFF0000u);
    } else {
      const int i = lane;
      if constexpr (C == C_F32) x[0] = reinterpret_cast<const float*>(qraw)[h * D + i];
      else if constexpr (C == C_FP8) x[0] = dec_fp8_p(qraw[h * D + i]);
      else x[0] = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(qraw)[h * D + i] << 16);
    }
#pragma unroll
    for (int v = 0; v < PER; ++v) r[v] = fma(wh, (double)x[v], r[v]);
  }
  uint8_t* rows = static_cast<uint8_t*>(p.rows) + (int64_t)q * S * D * QB;
  float* sig = p.sig + (int64_t)q * S;
  double mag = 0.0;
#pragma unroll 1
  for (int j = 0; j < S; ++j) {
    if (j >= NT) {
      for (int i = lane; i < D * QB; i += 64) rows[j * D * QB + i] = 0;
      if (lane == 0) sig[j] = 0.f;
      continue;
    }
    float sg = 1.f;
    if constexpr (C == C_FP8) {
      double mx = 0.0;
#pragma unroll
      for (int v = 0; v < PER; ++v) mx = fmax(mx, fabs(r[v]));
      for (int off = 32; off > 0; off >>= 1) mx = fmax(mx, __shfl_xor(mx, off, 64));
      sg = (mx > 0.0) ? (float)(mx / 448.0) : 1.f;
      if (!(sg > 0.f)) sg = 1.f;
    }
    double fn = 0.0;
#pragma unroll
    for (int v = 0; v < PER; ++v) {
      const int i = PER * lane + v;
      if (i >= D) continue;
      double dv;
      if constexpr (C == C_FP8) {
        const uint32_t code = enc_fp8_p((float)(r[v] / (double)sg));
        rows[j * D + i] = (uint8_t)code;
        dv = (double)dec_fp8_p(code);
      } else if constexpr (C == C_F32) {
        const float f = (float)r[v];
        reinterpret_cast<float*>(rows)[j * D + i] = f;
        dv = (double)f;
      } else {
        const uint32_t u = __float_as_uint((float)r[v]);
        const uint32_t b = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
        reinterpret_cast<uint16_t*>(rows)[j * D + i] = (uint16_t)b;
        dv = (double)__uint_as_float(b << 16);
      }
      r[v] -= (double)sg * dv;
      fn += dv * dv;
    }
    for (int off = 32; off > 0; off >>= 1) fn += __shfl_xor(fn, off, 64);
    if (lane == 0) sig[j] = sg;
    mag += (double)sg * sqrt(fn);
  }
  double e2 = 0.0;
#pragma unroll
  for (int v = 0; v < PER; ++v) e2 += r[v] * r[v];
  for (int off = 32; off > 0; off >>= 1) e2 += __shfl_xor(e2, off, 64);
  if (p.counts != nullptr)
    for (int r = lane; r < p.n_regions; r += 64) p.counts[(int64_t)r * p.total_q + q] = 0u;
  if (p.tpart != nullptr)
    for (int r = lane; r < p.n_parts; r += 64) p.tpart[(int64_t)q * p.n_parts + r] = 0u;
  if (lane == 0) {
    if (q == 0 && p.flag != nullptr) {
      p.flag[0] = 0;
      p.flag[1] = 0;
    }
    if (p.tshare != nullptr) p.tshare[q] = 0u;
    p.err[(int64_t)q * 2] = (float)(sqrt(e2) * 1.0000005);   // ||qbar - sum sigma f|| (rounded up)
    p.err[(int64_t)q * 2 + 1] = (float)(mag * 1.0000005);    // sum_j sigma_j ||f_j||
  }
}

template <int C, int H, int D>
static hipError_t prep_t(const PrepLaunch& p, hipStream_t s) {
  hipLaunchKernelGGL((qbar_kernel<C, H, D>), dim3(p.total_q), dim3(64), 0, s, p);
  return hipGetLastError();
}

template <int C>
static hipError_t prep_c(int H, int d, const PrepLaunch& p, hipStream_t s) {
#define DOSA_HD(HH, DD) \
  if (HP == HH && d == DD) return prep_t<C, HH, DD>(p, s);
  const int HP = padded_heads(H);
  DOSA_HD(8, 64) DOSA_HD(16, 64) DOSA_HD(32, 64) DOSA_HD(64, 64)
  DOSA_HD(8, 128) DOSA_HD(16, 128) DOSA_HD(32, 128) DOSA_HD(64, 128)
#undef DOSA_HD
  return hipErrorInvalidValue;
}

hipError_t launch_prep(int combo, int H, int d, const PrepLaunch& p, hipStream_t s) {
  if (p.total_q == 0) return hipSuccess;
  switch (combo) {
    case C_F32: return prep_c<C_F32>(H, d, p, s);
    case C_BF16: return prep_c<C_BF16>(H, d, p, s);
    case C_FP8: return prep_c<C_FP8>(H, d, p, s);
    case C_BF16Q_FP8K: return prep_c<C_BF16Q_FP8K>(H, d, p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace dosa
