// The DoSA certificate on gfx950: per-key norms, the per-query plan, the bound
// pass and survivor compaction, and the host-side sequence that ties them to
// the seed and survivor scoring passes.
//
// Certificate (DoSA pages: podcast transcript, Method section -- seed subset
// threshold; upper-bounding omitted positive heads by nonnegative
// projections with a joint residual bound; lower-bounding what negative heads
// subtract by an aggregate over an activation-derived support; a combined
// score bound for candidate refinement; zicq.com summary items 1-3):
//
//   UB(t,s) = sum_{p in P} c_p ReLU(q_p.k_s) + rho'_t ||k_s|| - ReLU(a_t.k_s)  >=  S(t,s)
//
// with proxies P (positive heads of largest w_h||q_h||), nonnegative
// least-squares coefficients alpha_hp of every other positive head on the
// proxies, c_p = w_p + sum_h w_h alpha_hp, residuals r_h, the joint constant
// rho^2 = sum_{h,j} w_h w_j max(0, <r_h, r_j>), the support A (negative heads
// positive on at least a given fraction of sampled seed keys) and
// a = sum_{h in A} |w_h| q_h.  rho' = rho + a rounding margin that keeps
// UB >= S for the fp32 values both kernels compute.  A key is pruned iff
// UB < tau, tau being the K-th largest seed score.
#include <cstring>
#include <type_traits>
#include <vector>

#include "dosa_device.h"

namespace dosa {

// ---------------------------------------------------------------------------
// scalar decoders (exact)
// ---------------------------------------------------------------------------
// E4M3FN code (low byte of x) -> its value, by the hardware converter (to
// bf16, which holds every finite E4M3 value exactly, then a shift)
__device__ __forceinline__ float dec_fp8(uint32_t x) {
  return __uint_as_float(fp8x2_to_bf16x2<false>(x & 0xFFu) << 16);
}
__device__ __forceinline__ float dec_bf16(uint32_t b) { return __uint_as_float(b << 16); }

template <int C>
__device__ __forceinline__ float q_elem(const void* base, int64_t i) {
  if constexpr (C == C_F32) return static_cast<const float*>(base)[i];
  else if constexpr (C == C_FP8) return dec_fp8(static_cast<const uint8_t*>(base)[i]);
  else return dec_bf16(static_cast<const uint16_t*>(base)[i]);
}
template <int C>
__device__ __forceinline__ float k_elem(const void* base, int64_t i) {
  if constexpr (C == C_F32) return static_cast<const float*>(base)[i];
  else if constexpr (C == C_BF16) return dec_bf16(static_cast<const uint16_t*>(base)[i]);
  else return dec_fp8(static_cast<const uint8_t*>(base)[i]);
}

// fp32 -> E4M3FN code, round to nearest (|x| <= 448 assumed).  The plan keeps
// the exact residual of whatever code comes out, so the rounding rule only
// affects tightness.
__device__ __forceinline__ uint32_t enc_fp8(float x) {
  const uint32_t s = (x < 0.f) ? 0x80u : 0u;
  float a = fminf(fabsf(x), 448.f);
  if (a < 0.015625f) {                       // subnormal range: m * 2^-9
    const uint32_t m = (uint32_t)rintf(a * 512.f);
    return s | m;                            // m == 8 is the smallest normal (code 0x08)
  }
  int e;
  const float f = frexpf(a, &e);             // a = f * 2^e, f in [0.5, 1)
  uint32_t m = (uint32_t)rintf((f * 2.f - 1.f) * 8.f);
  int E = e - 1 + 7;
  if (m == 8) { m = 0; ++E; }
  if (E > 15 || (E == 15 && m == 7)) { E = 15; m = 6; }
  return s | ((uint32_t)E << 3) | m;
}
__device__ __forceinline__ uint32_t enc_bf16(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ---------------------------------------------------------------------------
// per-key norms ||k_s|| (dequantised), rounded up
// ---------------------------------------------------------------------------
template <int C>
struct KBytes { static constexpr int value = (C == C_F32) ? 4 : (C == C_BF16 ? 2 : 1); };
template <int C>
struct QBytes { static constexpr int value = (C == C_F32) ? 4 : (C == C_FP8 ? 1 : 2); };

// The 16/BYTES values held in one 16-byte chunk of a row.
template <int BYTES>
__device__ __forceinline__ void dec16(const uint4 v, float* o) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (BYTES == 4) {
      o[j] = __uint_as_float(w[j]);
    } else if constexpr (BYTES == 2) {
      o[2 * j] = dec_bf16(w[j] & 0xFFFFu);
      o[2 * j + 1] = dec_bf16(w[j] >> 16);
    } else {
#pragma unroll
      for (int b = 0; b < 4; ++b) o[4 * j + b] = dec_fp8((w[j] >> (8 * b)) & 0xFFu);
    }
  }
}

// CH = d*bytes/16 lanes per key, one 16-byte chunk each (coalesced rows); the
// partial sums of squares meet by shuffles.  Grid: (key blocks, sequences), so
// a block knows its sequence and every key row costs at most one page-table
// read; blocks past a sequence's end exit.  kNormIter keys per lane group.
constexpr int kNormIter = 4;

template <int C, int D>
__global__ __launch_bounds__(256) void key_norm_kernel(const NormLaunch p) {
  if (p.needed != nullptr && *p.needed == 0) return;   // the plan marked every query hopeless
  constexpr int KBY = KBytes<C>::value;
  constexpr int CH = D * KBY / 16;            // lanes per key
  constexpr int KPB = 256 / CH;               // keys per block and iteration
  constexpr int VPC = 16 / KBY;               // values per chunk
  const int t = threadIdx.x;
  const int sub = t % CH;
#pragma unroll 1
  for (int b = blockIdx.y; b < p.batch; b += gridDim.y) {   // grid.y is capped at 65535
  const int base = p.cu_kv[b];
  const int n = p.cu_kv[b + 1] - base;
  // blocks of KPB * kNormIter keys, strided over grid.x (capped, so that a
  // batch of short and long sequences does not launch a workgroup per block
  // of the longest one for every sequence)
#pragma unroll 1
  for (int bx = blockIdx.x; bx * KPB * kNormIter < n; bx += gridDim.x) {
  const int first = bx * KPB * kNormIter + t / CH;
  uint4 v[kNormIter];
  int64_t rows[kNormIter];
#pragma unroll
  for (int it = 0; it < kNormIter; ++it) {
    const int key = first + it * KPB;
    rows[it] = -1;
    v[it] = make_uint4(0u, 0u, 0u, 0u);
    if (key < n) {
      rows[it] = key_row(p.in, base, b, key);
      v[it] = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(p.in.k) + rows[it] * D * KBY)[sub];
    }
  }
#pragma unroll
  for (int it = 0; it < kNormIter; ++it) {
    float f[VPC];
    dec16<KBY>(v[it], f);
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < VPC; ++j) acc = fmaf(f[j], f[j], acc);
#pragma unroll
    for (int off = CH / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, CH);
    if (sub == 0 && rows[it] >= 0) {
      float nv = sqrtf(acc);
      if constexpr (HasKScale<C>::value) nv *= p.in.k_scale[rows[it]];
      p.norms[(int64_t)base + first + it * KPB] = nv * 1.0000153f;   // covers the fp32 sum/sqrt/scale rounding (<< 2^-16)
    }
  }
  }
  }
}

// ---------------------------------------------------------------------------
// key-block summaries for the block certificate: per block of 64 consecutive
// keys of a sequence (the last one may be short), a centre stored in the key
// storage type (fp8: codes times a per-block scale), the radius of the block
// around that centre, its largest key norm and the centre's norm.  Any centre
// gives a valid bound; this one is the block mean, rounded to the storage
// type, and the radius is measured against the rounded centre itself.
// One wavefront per block: the rows are staged in LDS, lane i averages
// elements i (and i + 64), then lane s measures key s.  Sums are fp32 of
// exactly decoded values; radius and norms are rounded up (2^-16 relative for
// the sums of at most 128 squares and the square root, plus 2^-21 of the
// magnitudes for the fp32 rounding of the dequantised values and differences).
// ---------------------------------------------------------------------------
template <int C, int D>
__global__ __launch_bounds__(64) void key_block_kernel(const NormLaunch p) {
  if (p.needed != nullptr && *p.needed == 0) return;   // the plan marked every query hopeless
  constexpr int KBY = KBytes<C>::value;
  constexpr int ROWB = D * KBY;
  constexpr int RS = ROWB + 16;                        // padded LDS row (bytes)
  constexpr int CPR = ROWB / 16;                       // 16-byte chunks per row
  constexpr int PER = (D + 63) / 64;                   // elements per lane
  __shared__ __attribute__((aligned(16))) uint8_t rows[kKeyBlock * RS];
  __shared__ float ksc[kKeyBlock];
  __shared__ float cen[D];
  const int lane = lane_id();
  auto elem = [&](int s, int i) -> float {             // stored value i of staged key s (undecoded scale)
    const uint8_t* r = rows + s * RS;
    if constexpr (KBY == 4) return reinterpret_cast<const float*>(r)[i];
    else if constexpr (KBY == 2) return dec_bf16((uint32_t)reinterpret_cast<const uint16_t*>(r)[i]);
    else return dec_fp8((uint32_t)r[i]);
  };
#pragma unroll 1
  for (int b = blockIdx.y; b < p.batch; b += gridDim.y) {
    const int n = p.cu_kv[b + 1] - p.cu_kv[b];
    const int k0 = blockIdx.x * kKeyBlock;
    if (k0 >= n) continue;
    const int ns = min(kKeyBlock, n - k0);
    const int64_t blk = (int64_t)p.cu_blk[b] + blockIdx.x;
    // stage the block's rows and scales
    for (int c = lane; c < ns * CPR; c += 64) {
      const int s = c / CPR, part = c % CPR;
      const int64_t row = key_row(p.in, p.cu_kv[b], b, k0 + s);
      *reinterpret_cast<uint4*>(rows + s * RS + 16 * part) =
          reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(p.in.k) + row * ROWB)[part];
    }
    if (lane < ns) ksc[lane] = HasKScale<C>::value ? p.in.k_scale[key_row(p.in, p.cu_kv[b], b, k0 + lane)] : 1.f;
    __syncthreads();
    // mean, rounded to the storage type (fp8: per-block scale = max |mean| / 448)
    float mean[PER];
    float amax = 0.f;
#pragma unroll
    for (int v = 0; v < PER; ++v) {
      const int i = lane + 64 * v;
      float acc = 0.f;
      if (i < D)
        for (int s = 0; s < ns; ++s) acc = fmaf(ksc[s], elem(s, i), acc);
      mean[v] = acc / (float)ns;
      amax = fmaxf(amax, fabsf(mean[v]));
    }
    for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    float sc = 1.f;
    if constexpr (KBY == 1) {
      sc = amax > 0.f ? amax / 448.f : 1.f;
      if (!(sc > 0.f)) sc = 1.f;
    }
    uint8_t* code = p.blk_code + blk * ROWB;
#pragma unroll
    for (int v = 0; v < PER; ++v) {
      const int i = lane + 64 * v;
      if (i >= D) continue;
      float cv;
      if constexpr (KBY == 4) {
        reinterpret_cast<float*>(code)[i] = mean[v];
        cv = mean[v];
      } else if constexpr (KBY == 2) {
        const uint32_t bits = enc_bf16(mean[v]);
        reinterpret_cast<uint16_t*>(code)[i] = (uint16_t)bits;
        cv = dec_bf16(bits);
      } else {
        const uint32_t c8 = enc_fp8(mean[v] / sc);
        code[i] = (uint8_t)c8;
        cv = sc * dec_fp8(c8);
      }
      cen[i] = cv;
    }
    __syncthreads();
    // lane s: distance of key s from the centre, and its norm
    float d2 = 0.f, n2 = 0.f, c2 = 0.f;
    if (lane < ns) {
      const float ks = ksc[lane];
      for (int i = 0; i < D; ++i) {
        const float e = elem(lane, i);
        const float df = ks * e - cen[i];
        d2 = fmaf(df, df, d2);
        n2 = fmaf(e, e, n2);
      }
    }
    for (int i = lane; i < D; i += 64) c2 = fmaf(cen[i], cen[i], c2);
    for (int off = 32; off > 0; off >>= 1) c2 += __shfl_xor(c2, off, 64);
    float dmax = sqrtf(d2), nmax = (lane < ns) ? sqrtf(n2) * ksc[lane] : 0.f;
    for (int off = 32; off > 0; off >>= 1) {
      dmax = fmaxf(dmax, __shfl_xor(dmax, off, 64));
      nmax = fmaxf(nmax, __shfl_xor(nmax, off, 64));
    }
    if (lane == 0) {
      const float cn = sqrtf(c2) * 1.0000153f;
      const float nb = nmax * 1.0000153f;
      float* info = p.blk_info + blk * 4;
      info[0] = sc;
      info[1] = dmax * 1.0000153f + 4.7683716e-7f * (nb + cn);   // + 2^-21 (N + ||c||)
      info[2] = nb;
      info[3] = cn;
    }
    __syncthreads();   // the staged rows are rewritten by the next sequence's block
  }
}

// ---------------------------------------------------------------------------
// per-query plan, one workgroup of 256 threads per query
// ---------------------------------------------------------------------------
// Nonnegative least squares of a head on <= 3 proxies, exhaustive over
// supports (exact): minimise a^T G a - 2 b^T a subject to a >= 0.  Every loop
// is unrolled over compile-time bounds so the small arrays stay in registers.
__device__ __forceinline__ double det3(double m00, double m01, double m02, double m10, double m11, double m12,
                                       double m20, double m21, double m22) {
  return m00 * (m11 * m22 - m12 * m21) - m01 * (m10 * m22 - m12 * m20) + m02 * (m10 * m21 - m11 * m20);
}

__device__ __forceinline__ void nnls3(int p, const double Gp[3][3], const double b[3], double out[3]) {
  double best = 0.0;
  out[0] = out[1] = out[2] = 0.0;
#pragma unroll
  for (int mask = 1; mask < 8; ++mask) {
    if (mask >= (1 << p)) continue;
    const int n = ((mask & 1) ? 1 : 0) + ((mask & 2) ? 1 : 0) + ((mask & 4) ? 1 : 0);
    const int i0 = (mask & 1) ? 0 : ((mask & 2) ? 1 : 2);
    const int i1 = (n < 2) ? i0 : ((mask & 1) ? ((mask & 2) ? 1 : 2) : 2);
    double a0 = 0.0, a1 = 0.0, a2 = 0.0;
    bool ok;
    if (n == 1) {
      const double g = Gp[i0][i0];
      ok = g > 0.0;
      a0 = ok ? b[i0] / g : 0.0;
    } else if (n == 2) {
      const double g00 = Gp[i0][i0], g01 = Gp[i0][i1], g11 = Gp[i1][i1];
      const double det = g00 * g11 - g01 * g01;
      ok = det > 1e-12 * g00 * g11;
      a0 = ok ? (b[i0] * g11 - b[i1] * g01) / det : 0.0;
      a1 = ok ? (b[i1] * g00 - b[i0] * g01) / det : 0.0;
    } else {
      const double det = det3(Gp[0][0], Gp[0][1], Gp[0][2], Gp[1][0], Gp[1][1], Gp[1][2], Gp[2][0], Gp[2][1], Gp[2][2]);
      ok = det > 1e-12 * Gp[0][0] * Gp[1][1] * Gp[2][2];
      if (ok) {
        a0 = det3(b[0], Gp[0][1], Gp[0][2], b[1], Gp[1][1], Gp[1][2], b[2], Gp[2][1], Gp[2][2]) / det;
        a1 = det3(Gp[0][0], b[0], Gp[0][2], Gp[1][0], b[1], Gp[1][2], Gp[2][0], b[2], Gp[2][2]) / det;
        a2 = det3(Gp[0][0], Gp[0][1], b[0], Gp[1][0], Gp[1][1], b[1], Gp[2][0], Gp[2][1], b[2]) / det;
      }
    }
    if (!ok || a0 < 0.0 || a1 < 0.0 || a2 < 0.0) continue;
    // the candidate as a full 3-vector
    double c[3] = {0.0, 0.0, 0.0};
    if (n == 3) { c[0] = a0; c[1] = a1; c[2] = a2; }
    else {
      c[i0] = a0;
      if (n == 2) c[i1] = a1;
    }
    double f = 0.0;
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      f -= 2.0 * b[i] * c[i];
#pragma unroll
      for (int j = 0; j < 3; ++j) f += c[i] * Gp[i][j] * c[j];
    }
    if (f < best) {
      best = f;
      out[0] = c[0]; out[1] = c[1]; out[2] = c[2];
    }
  }
}

constexpr float kSkipFrac = 0.7f;   // sampled survival above which the bound pass is skipped
constexpr int kSampleKeys = 64;     // keys sampled for activations and for the skip test
constexpr float kJointGain = 0.1f;  // sampled extra pruning that pays for the joint constant

// Cross-lane exchanges without the LDS crossbar: DPP moves within a row of
// 16 lanes, readlane across rows.  A row-local DPP move of a value that every
// lane holds (all lanes of the wavefront active).
template <int CTRL, typename T>
__device__ __forceinline__ T dpp_mov(T v) {
  if constexpr (sizeof(T) == 8) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
    return __builtin_bit_cast(T, ((uint64_t)hi << 32) | lo);
  } else {
    return __builtin_bit_cast(T, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
  }
}
template <typename T>
__device__ __forceinline__ T lane_value(T v, int l) {
  if constexpr (sizeof(T) == 8) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
    return __builtin_bit_cast(T, ((uint64_t)hi << 32) | lo);
  } else {
    return __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
  }
}
struct OpAdd { template <typename T> __device__ T operator()(T a, T b) const { return a + b; } };
struct OpMax { template <typename T> __device__ T operator()(T a, T b) const { return a > b ? a : b; } };

// Reduction over the P consecutive lanes that share one head (P = 4, 8, 16,
// 32 or 64): xor 1 and xor 2 by quad permutes, then the mirrored half of 8
// and of 16 lanes, then the rows' values by readlane.  Every lane of a part
// gets the same value (each step combines two equal-shaped partials).
template <int P, typename T, typename Op>
__device__ __forceinline__ T part_reduce(T v, Op op) {
  static_assert(P == 4 || P == 8 || P == 16 || P == 32 || P == 64, "part size");
  v = op(v, dpp_mov<0xB1>(v));                          // quad_perm [1,0,3,2]: lane ^ 1
  v = op(v, dpp_mov<0x4E>(v));                          // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (P >= 8) v = op(v, dpp_mov<0x141>(v));   // row_half_mirror: the other quad of 8
  if constexpr (P >= 16) v = op(v, dpp_mov<0x140>(v));  // row_mirror: the other half of 16
  if constexpr (P >= 32) {
    const T r0 = lane_value(v, 0), r1 = lane_value(v, 16), r2 = lane_value(v, 32), r3 = lane_value(v, 48);
    if constexpr (P == 32) v = (lane_id() < 32) ? op(r0, r1) : op(r2, r3);
    else v = op(op(r0, r1), op(r2, r3));
  }
  return v;
}
template <int P, typename T>
__device__ __forceinline__ T part_sum(T v) { return part_reduce<P>(v, OpAdd{}); }
template <typename T>
__device__ __forceinline__ T wave_sum(T v) { return part_reduce<64>(v, OpAdd{}); }
template <typename T>
__device__ __forceinline__ T wave_max(T v) { return part_reduce<64>(v, OpMax{}); }

// Layout: thread t works on head t / PARTS and owns that head's elements
// part + PARTS*e (e < EL), PARTS = 256 / H; per-head dot products are lane
// partial sums reduced over the PARTS lanes.  Per-head scalars live in lane h
// of wavefront 0 (H <= 64).  Every global load is issued at the start: the
// query, the activation keys (up to 64, evenly spaced back from the query
// inside its seed window) and the skip-test keys (up to 64, evenly spaced
// over the group's bounded range).  Key-by-head and key-by-row products that
// only steer decisions (activation counts, the skip test) run on MFMA in the
// stored operand types; the certificate's own constants are fp64.
template <int C, int H, int D>
__global__ __launch_bounds__(256) void plan_kernel(const PlanLaunch p) {
  using O = Ops<C, D>;
  constexpr int QB = QBytes<C>::value, KBY = KBytes<C>::value;
  constexpr int PARTS = 256 / H, EL = D / PARTS;
  constexpr int QCH = H * D * QB / 16;              // 16-byte chunks of the query
  constexpr int NQV = (QCH + 255) / 256;
  constexpr int CPK = D * KBY / 16;                 // 16-byte chunks of a key row
  constexpr int NKV = (kSampleKeys * CPK + 255) / 256;
  constexpr int KRS = D * KBY + 16;                 // LDS row stride of staged keys (bytes)
  static_assert(H <= 64 && 256 % H == 0 && D % PARTS == 0, "plan layout");
  if (skip_launch(p.mode, p.run_if)) return;
  const GroupInfo gr = p.groups[blockIdx.x];
  const int slot = blockIdx.y;
  if (slot >= gr.nq) return;
  const int qrow = gr.q_row0 + slot;
  const int pos = gr.pos0 + slot;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int hh = t / PARTS, part = t % PARTS;
  const int g = lane >> 4, col = lane & 15;

  constexpr int QS = D + 4;                        // LDS row stride of the query (elements)
  // the query in its stored type (decoded on read: fp8 and bf16 values are
  // exact in fp32), rows of QS elements; a decoded fp32 copy would double or
  // quadruple the kernel's LDS and cost a resident workgroup per CU
  typedef typename std::conditional<QB == 4, float, typename std::conditional<QB == 2, uint16_t, uint8_t>::type>::type qraw_t;
  __shared__ __align__(16) qraw_t qf[H * QS];
  auto qval = [&](int idx) -> float {
    if constexpr (QB == 4) return qf[idx];
    else if constexpr (QB == 2) return dec_bf16((uint32_t)qf[idx]);
    else return dec_fp8((uint32_t)qf[idx]);
  };
  __shared__ __align__(16) uint8_t kraw[kSampleKeys * KRS];   // staged keys, stored type
  __shared__ __align__(16) uint8_t rowl[4 * D * QB];          // the certificate rows
  __shared__ double wd[H], qn2[H], alpha[H][3], gph[3][H];
  __shared__ double avec[D];
  __shared__ float ksc[kSampleKeys];                          // skip-test keys: scale
  __shared__ int prox[3], act[H], inO[H];
  __shared__ double hsum[8];                       // c_0..c_2, rho_sep, rho_lo, sum |w_h| ||q_h||, margin
  __shared__ float cfs[6];                         // row multipliers, rho_lo, rho_sep + margin (scaled)
  __shared__ double red4[4];
  __shared__ float rnorm[4];                       // norms of the 4 stored certificate rows (rounded up)
  __shared__ int np_s, nsurv_s, nsep_s;
  __shared__ float ssc[4][kSampleKeys];             // probe plan: per-wavefront partial scores of the
  __shared__ float sfin[kSampleKeys];               // activation keys, their scores, the estimate
  __shared__ float tau_s;
  __shared__ double pvals[64];                     // proxy choice: w_h ||q_h|| (or -1) per head lane

  // ---- 0. issue the loads
  // Heads stored per query (a multiple of 8, at most H): the head slots past
  // Hr get zero rows and zero weight, so they are neither positive nor
  // negative heads and every sum below skips them.
  const int Hr = p.in.H;
  const int qch = Hr * D * QB / 16;                // 16-byte chunks of the stored query row
  const uint8_t* qrow_raw = static_cast<const uint8_t*>(p.in.q) + (int64_t)qrow * Hr * D * QB;
  uint4 qv[NQV];
#pragma unroll
  for (int j = 0; j < NQV; ++j) {
    const int c = t + 256 * j;
    qv[j] = (c < qch) ? reinterpret_cast<const uint4*>(qrow_raw)[c] : make_uint4(0u, 0u, 0u, 0u);
  }
  typename O::frag qa[O::STEPS];                   // MFMA rows: heads 16*wave + col
  if (wave * 16 + col < Hr) O::load_q(qrow_raw + (wave * 16 + col) * D * QB, g, qa);
  else O::zero(qa);
  const float wv = (t < Hr) ? p.in.w[(int64_t)qrow * Hr + t] : 0.f;
  const bool est = p.tau == nullptr;               // probe plan: the threshold is estimated below
  const float tau_in = est ? -INFINITY : p.tau[qrow];
  const float qscale = HasQScale<C>::value ? p.in.q_scale[qrow] : 1.f;
  const float l_err_f = p.lerr[(int64_t)qrow * 2], l_mag_f = p.lerr[(int64_t)qrow * 2 + 1];
  const bool use_neg = (p.flags & DOSA_NO_NEGATIVE) == 0;
  const int n_last = gr.pos0 + gr.nq;
  const int wlo = max(0, n_last - p.seed_window);
  const int span = pos - wlo + 1;                   // window keys visible to this query
  const int ns = (use_neg || est) ? min(kSampleKeys, max(span, 0)) : 0;
  const int astep = max(1, span / max(ns, 1));
  const int nb = gr.n_bounded;
  // skip-test keys loaded (the sample size once the threshold is known)
  const int nsb_ld = ((p.flags & DOSA_NO_PRUNE) == 0 && (est || tau_in > -INFINITY)) ? min(kSampleKeys, nb) : 0;
  const uint8_t* kbase = static_cast<const uint8_t*>(p.in.k);
  uint4 kav[NKV], ksv[NKV];
#pragma unroll
  for (int j = 0; j < NKV; ++j) {
    const int c = t + 256 * j;
    const int i = c / CPK, sub = c % CPK;
    kav[j] = make_uint4(0u, 0u, 0u, 0u);
    ksv[j] = make_uint4(0u, 0u, 0u, 0u);
    if (i < ns) {
      const int64_t row = key_row(p.in, gr.key_base, gr.seq, pos - i * astep);
      kav[j] = reinterpret_cast<const uint4*>(kbase + row * D * KBY)[sub];
    }
    if (i < nsb_ld) {
      const int64_t row = key_row(p.in, gr.key_base, gr.seq, gr.bound_lo + (int)(((int64_t)i * nb) / nsb_ld));
      ksv[j] = reinterpret_cast<const uint4*>(kbase + row * D * KBY)[sub];
    }
  }
  float kscale = 1.f, kscale_a = 1.f;
  if (t < nsb_ld) {
    const int key = gr.bound_lo + (int)(((int64_t)t * nb) / nsb_ld);
    if constexpr (HasKScale<C>::value) kscale = p.in.k_scale[key_row(p.in, gr.key_base, gr.seq, key)];
  }
  if (est && t < ns) {   // the activation key's scale, for its score
    if constexpr (HasKScale<C>::value) kscale_a = p.in.k_scale[key_row(p.in, gr.key_base, gr.seq, pos - t * astep)];
  }

  // ---- 1. query and activation keys (stored type) to LDS
#pragma unroll
  for (int j = 0; j < NQV; ++j) {
    const int c = t + 256 * j;
    if (c < qch) {
      const int e = c * (16 / QB);                   // first element of the chunk (one row holds it whole)
      uint32_t* dst = reinterpret_cast<uint32_t*>(&qf[(e / D) * QS + e % D]);
      dst[0] = qv[j].x; dst[1] = qv[j].y; dst[2] = qv[j].z; dst[3] = qv[j].w;
    }
  }
  for (int i = t; i < (H - Hr) * D; i += 256) qf[(Hr + i / D) * QS + i % D] = (qraw_t)0;
#pragma unroll
  for (int j = 0; j < NKV; ++j) {
    const int c = t + 256 * j;
    const int i = c / CPK, sub = c % CPK;
    if (i < ns) *reinterpret_cast<uint4*>(kraw + i * KRS + 16 * sub) = kav[j];
  }
  if (t < H) {
    wd[t] = (double)wv;
    act[t] = 0;
  }
  if (t < kSampleKeys) ksc[t] = kscale;
  ssc[wave][lane] = 0.f;
  if (t == 0) tau_s = -INFINITY;
  __syncthreads();

  // ---- 2. activation counts of the negative heads on the window keys
  // (MFMA: rows = heads 16*wave.., columns = 16 keys per tile)
  if (ns > 0 && wave * 16 < H) {
    int cnt[4] = {0, 0, 0, 0};
    for (int tile = 0; tile * 16 < ns; ++tile) {
      const int key = tile * 16 + col;
      typename O::frag B[O::STEPS];
      O::load_k(kraw + key * KRS, g, B);
      v4f c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < O::STEPS; ++st) c = O::mma(qa[st], B[st], c);
#pragma unroll
      for (int i = 0; i < 4; ++i) cnt[i] += (key < ns && c[i] > 0.f) ? 1 : 0;
      if (est) {   // this wavefront's heads' part of the key's score (unscaled)
        float sp = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int h = wave * 16 + 4 * g + i;
          sp = fmaf(h < H ? (float)wd[h] : 0.f, fmaxf(c[i], 0.f), sp);
        }
        sp += __shfl_xor(sp, 16, 64);
        sp += __shfl_xor(sp, 32, 64);
        if (g == 0 && key < ns) ssc[wave][key] = sp;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      cnt[i] = part_sum<16>(cnt[i]);
      const int h = wave * 16 + 4 * g + i;
      if (col == 0 && h < H) act[h] = cnt[i];
    }
  }

  // ---- 3. squared norms, proxies, proxy inner products (fp64 of exact values)
  float qr[EL];
#pragma unroll
  for (int e = 0; e < EL; ++e) qr[e] = qval(hh * QS + part + PARTS * e);
  {
    double s2 = 0.0;
#pragma unroll
    for (int e = 0; e < EL; ++e) s2 = fma((double)qr[e], (double)qr[e], s2);
    s2 = part_sum<PARTS>(s2);
    if (part == 0) qn2[hh] = s2;
  }
  __syncthreads();
  if (est && t < ns) sfin[t] = (ssc[0][t] + ssc[1][t] + ssc[2][t] + ssc[3][t]) * qscale * kscale_a;
  if (wave == 0) {
    // positive heads of largest w_h ||q_h||, lower head index on ties: head
    // h's rank in (value desc, index asc) order, counted over the staged
    // values; the first min(num_proxies, #positive heads) ranks are proxies
    const double v = (lane < H && wd[lane] > 0.0) ? wd[lane] * sqrt(qn2[lane]) : -1.0;
    pvals[lane] = v;
    wave_sync();
    int above = 0;
#pragma unroll 8
    for (int j = 0; j < 64; ++j) {
      const double o = pvals[j];
      above += (o > v || (o == v && j < lane)) ? 1 : 0;
    }
    const int n = min(p.num_proxies, (int)__popcll(ballot(v >= 0.0)));
    if (v >= 0.0 && above < n) prox[above] = lane;
    if (lane == 0) np_s = n;
  }
  __syncthreads();
  const int np = np_s;
  // probe plan: the estimated threshold is the sample's score of rank
  // ceil(ns * topk / n_seed), n_seed the seed keys this query sees; none
  // (nothing to prune) when it sees fewer than topk
  if (est && t < ns) {
    const int64_t n_seed = (int64_t)span + min(p.seed_prefix, wlo);
    if (n_seed >= p.topk) {
      const int r = (int)min<int64_t>(ns, max<int64_t>(1, ((int64_t)ns * p.topk + n_seed - 1) / n_seed));
      const float mine = sfin[t];
      int above = 0;
      for (int j = 0; j < ns; ++j) above += (sfin[j] > mine || (sfin[j] == mine && j < t)) ? 1 : 0;
      if (above == r - 1) tau_s = mine;
    }
  }
  for (int r = 0; r < np; ++r) {
    const int pr = prox[r] * QS + part;
    double dsum = 0.0;
#pragma unroll
    for (int e = 0; e < EL; ++e) dsum = fma((double)qr[e], (double)qval(pr + PARTS * e), dsum);
    dsum = part_sum<PARTS>(dsum);
    if (part == 0) gph[r][hh] = dsum;
  }
  __syncthreads();

  // ---- 4. nonnegative projections of the other positive heads (lane h of
  // wavefront 0), residual norms, and the head sums; in parallel the other
  // wavefronts form the aggregate a = sum_{h in A} |w_h| q_h (fp64, unscaled)
  // and stage the skip-test keys over the activation keys
  if (wave == 0) {
    const int h = lane;
    double cv[3] = {0.0, 0.0, 0.0}, ps = 0.0, pl = 0.0, wq = 0.0;
    if (h < H) {
      bool o = wd[h] > 0.0;
      for (int u = 0; u < np; ++u) o = o && (prox[u] != h);
      double a[3] = {0.0, 0.0, 0.0};
      double Gp[3][3], b[3];
#pragma unroll
      for (int r = 0; r < 3; ++r) {
        b[r] = (r < np) ? gph[r][h] : 0.0;
#pragma unroll
        for (int c = 0; c < 3; ++c) Gp[r][c] = (r < np && c < np) ? gph[r][prox[c]] : 0.0;
      }
      if (o && np > 0) nnls3(np, Gp, b, a);
      alpha[h][0] = a[0]; alpha[h][1] = a[1]; alpha[h][2] = a[2];
      double r2 = qn2[h];
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        r2 -= 2.0 * a[u] * b[u];
#pragma unroll
        for (int v = 0; v < 3; ++v) r2 += a[u] * Gp[u][v] * a[v];
      }
      r2 = fmax(r2, 0.0);
      inO[h] = o ? 1 : 0;
      if (o) {
#pragma unroll
        for (int u = 0; u < 3; ++u) cv[u] = wd[h] * a[u];
        ps = wd[h] * sqrt(r2);
        pl = wd[h] * wd[h] * r2;
      }
      wq = fabs(wd[h]) * sqrt(qn2[h]);
    }
    cv[0] = wave_sum(cv[0]); cv[1] = wave_sum(cv[1]); cv[2] = wave_sum(cv[2]);
    ps = wave_sum(ps); pl = wave_sum(pl); wq = wave_sum(wq);
    if (lane == 0) {
      for (int u = 0; u < 3; ++u) hsum[u] = (u < np) ? wd[prox[u]] + cv[u] : 0.0;
      hsum[3] = ps;                      // separable residual constant (>= the joint one)
      hsum[4] = sqrt(fmax(pl, 0.0));     // diagonal of the joint sum (<= the joint one)
      hsum[5] = wq;
    }
  } else {
    const double need = (double)p.neg_frac * (double)ns;
    for (int i = t - 64; i < D; i += 192) {
      double sacc = 0.0;
      if (use_neg) {
#pragma unroll 8
        for (int h = 0; h < H; ++h) {
          const bool in_a = wd[h] < 0.0 && (ns > 0 ? (double)act[h] >= need : p.neg_frac <= 0.f);
          if (in_a) sacc = fma(-wd[h], (double)qval(h * QS + i), sacc);
        }
      }
      avec[i] = sacc;
    }
  }
  __syncthreads();   // activation keys no longer read
  const float tau = est ? tau_s : tau_in;
  const int nsb = tau > -INFINITY ? nsb_ld : 0;
#pragma unroll
  for (int j = 0; j < NKV; ++j) {
    const int c = t + 256 * j;
    const int i = c / CPK, sub = c % CPK;
    if (i < nsb) *reinterpret_cast<uint4*>(kraw + i * KRS + 16 * sub) = ksv[j];
  }
  if (t == 0) nsurv_s = 0;

  // ---- 5. operand rows (wavefront 0): proxies re-encoded from their exact
  // decoded values (the same values), then terms of the aggregate; written to
  // the workspace and to LDS
  uint8_t* rows = static_cast<uint8_t*>(p.rows) + (int64_t)qrow * 4 * D * QB;
  double sig[4] = {0, 0, 0, 0}, fnorm[4] = {0, 0, 0, 0}, ea = 0.0;
  if (wave == 0) {
    for (int e = lane; e < np * D; e += 64) {
      const int r = e / D, i = e % D;
      const float v = qval(prox[r] * QS + i);
      if constexpr (QB == 1) rowl[r * D + i] = (uint8_t)enc_fp8(v);
      else if constexpr (QB == 4) reinterpret_cast<float*>(rowl)[r * D + i] = v;
      else reinterpret_cast<uint16_t*>(rowl)[r * D + i] = (uint16_t)enc_bf16(v);
    }
    constexpr int PER = (D + 63) / 64;
    double res[PER];
#pragma unroll
    for (int v = 0; v < PER; ++v) res[v] = (lane + 64 * v < D) ? avec[lane + 64 * v] : 0.0;
    for (int r = np; r < 4; ++r) {
      float sg = 1.f;
      if constexpr (QB == 1) {
        double mx = 0.0;
#pragma unroll
        for (int v = 0; v < PER; ++v) mx = fmax(mx, fabs(res[v]));
        mx = wave_max(mx);
        sg = (mx > 0.0) ? (float)(mx / 448.0) : 1.f;
        if (!(sg > 0.f)) sg = 1.f;   // underflow guard
      }
      double fn = 0.0;
#pragma unroll
      for (int v = 0; v < PER; ++v) {
        const int i = lane + 64 * v;
        if (i >= D) continue;
        double dv;
        if constexpr (QB == 1) {
          const uint32_t code = enc_fp8((float)(res[v] / (double)sg));
          rowl[r * D + i] = (uint8_t)code;
          dv = (double)dec_fp8(code);
        } else if constexpr (QB == 4) {
          const float f = (float)res[v];
          reinterpret_cast<float*>(rowl)[r * D + i] = f;
          dv = (double)f;
        } else {
          const uint32_t b = enc_bf16((float)res[v]);
          reinterpret_cast<uint16_t*>(rowl)[r * D + i] = (uint16_t)b;
          dv = (double)dec_bf16(b);
        }
        res[v] -= (double)sg * dv;
        fn += dv * dv;
      }
      fn = wave_sum(fn);
      sig[r] = sg;
      fnorm[r] = sqrt(fn);
    }
    double e2 = 0.0;
#pragma unroll
    for (int v = 0; v < PER; ++v) e2 += res[v] * res[v];
    ea = sqrt(wave_sum(e2));
    if (lane == 0) {
      // Rounding margin: forward error of the fp32 dot products and sums in
      // the score and bound kernels (Higham, dot-product error gamma_n), with
      // u = 2^-22 (4x the fp32 unit roundoff) and n = d + H + 16; rho enters
      // via its separable upper bound.  The score kernels evaluate
      // sum_h w_h ReLU(x_h) as sum_h (w_h/2)|x_h| + qbar.k/2 with qbar held as
      // a few terms; their error and magnitude (unscaled) enter too.
      const double u = 1.0 / 4194304.0;
      const double nn = (double)(D + H + 16);
      const double gam = nn * u / (1.0 - nn * u);
      double cq = 0.0, sf = 0.0;
      for (int r = 0; r < np; ++r) cq += hsum[r] * sqrt(qn2[prox[r]]);
      for (int r = np; r < 4; ++r) sf += sig[r] * fnorm[r];
      const double margin =
          2.0 * gam * (hsum[5] + cq + sf + hsum[3] + 0.5 * (double)l_mag_f) + ea + 0.5 * (double)l_err_f;
      hsum[6] = margin;
      const double qs = (double)qscale;
      for (int r = 0; r < 4; ++r) cfs[r] = (r < np) ? (float)(hsum[r] * qs) : (float)(sig[r] * qs);
      cfs[4] = (float)(hsum[4] * qs);
      cfs[5] = (float)((hsum[3] + margin) * qs);
    }
  }
  __syncthreads();
  for (int c = t; c < 4 * D * QB / 16; c += 256)
    reinterpret_cast<uint4*>(rows)[c] = reinterpret_cast<const uint4*>(rowl)[c];

  // ---- 6. skip test (wavefront 0): the bound pass's arithmetic on the
  // sampled bounded keys, once with rho replaced by its diagonal lower bound
  // (an optimistic certificate) and once with the separable constant (the
  // valid certificate without the joint term).  If at least kSkipFrac of the
  // sample would survive even the optimistic one, the bound pass is not worth
  // running; the joint constant is worked out only where it would prune a
  // clearly larger part of the sample than the separable one.  Skipping
  // either is always correct, so these are cost decisions only.
  if (t == 0) nsep_s = 0;
  if (wave == 1) {
    // Euclidean norm of each stored row (the values the bound pass multiplies),
    // for the key-block bound: fp32 sums of squares of exactly decoded values,
    // rounded up by 2^-16 relative
    for (int r = 0; r < 4; ++r) {
      float acc = 0.f;
      for (int i = lane; i < D; i += 64) {
        float v;
        if constexpr (QB == 1) v = dec_fp8((uint32_t)rowl[r * D + i]);
        else if constexpr (QB == 4) v = reinterpret_cast<const float*>(rowl)[r * D + i];
        else v = dec_bf16((uint32_t)reinterpret_cast<const uint16_t*>(rowl)[r * D + i]);
        acc = fmaf(v, v, acc);
      }
      acc = wave_sum(acc);
      if (lane == 0) rnorm[r] = sqrtf(acc) * 1.0000153f;
    }
  }
  if (wave == 0 && nsb > 0) {
    typename O::frag A[O::STEPS];
    if (col < 4) O::load_q(rowl + col * D * QB, g, A);
    else O::zero(A);
    int n_surv = 0, n_sep = 0;
    for (int tile = 0; tile * 16 < nsb; ++tile) {
      const int i = tile * 16 + col;
      typename O::frag B[O::STEPS];
      O::load_k(kraw + i * KRS, g, B);
      v4f c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < O::STEPS; ++st) c = O::mma(A[st], B[st], c);
      float pz = 0.f, nz = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (r < np) pz += cfs[r] * fmaxf(c[r], 0.f);
        else nz += cfs[r] * c[r];
      }
      const float kn2 = frag_norm2<O>(B);   // the sampled key's norm from its fragments
      const bool ok = g == 0 && i < nsb;
      const float base = ok ? ksc[i] * (pz - fmaxf(nz, 0.f)) : 0.f;
      const float kn = ok ? ksc[i] * norm_up(kn2) : 0.f;
      n_surv += (int)__popcll(__ballot(ok && base + cfs[4] * kn >= tau));
      n_sep += (int)__popcll(__ballot(ok && base + cfs[5] * kn >= tau));
    }
    if (lane == 0) {
      nsurv_s = n_surv;
      nsep_s = n_sep;
    }
  }
  __syncthreads();
  const bool hopeless = nsb == 0 || (float)nsurv_s >= kSkipFrac * (float)nsb;
  const bool joint = !est && !hopeless && (p.flags & DOSA_SEPARABLE_RHO) == 0 &&
                     (nsb < 16 || (float)(nsep_s - nsurv_s) >= fmaxf(2.f, kJointGain * (float)nsb));

  // ---- 7. joint residual constant rho^2 = sum_{h,j in O} w_h w_j max(0, <r_h, r_j>)
  // from the head Gram matrix on fp64 MFMA (16x16x4: lane l feeds row l%16,
  // k l/16 of both operands and holds rows l/16 + 4i of column l%16 of the
  // result; products and sums of the decoded fp8/bf16 values are exact or
  // nearly so in fp64).  Wavefront w takes tiles (bi, bj), bi <= bj, round
  // robin; off-diagonal tiles count twice.
  double rho = hsum[3];
  if (joint) {
    constexpr int NBLK = (H + 15) / 16;
    constexpr int NT = NBLK * (NBLK + 1) / 2;
    double acc = 0.0;
    const int lr = lane & 15, lk = lane >> 4;
    for (int tt = wave; tt < NT; tt += 4) {
      int bi = 0, rem = tt;
      while (rem >= NBLK - bi) { rem -= NBLK - bi; ++bi; }
      const int bj = bi + rem;
      const int ha = 16 * bi + lr, hb = 16 * bj + lr;       // operand rows of this lane
      const int pa = (ha < H ? ha : 0) * QS + lk;
      const int pb = (hb < H ? hb : 0) * QS + lk;
      typedef double v4d __attribute__((ext_vector_type(4)));
      v4d gacc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll 8
      for (int k = 0; k < D / 4; ++k) {
        const double a = (ha < H) ? (double)qval(pa + 4 * k) : 0.0;
        const double b = (hb < H) ? (double)qval(pb + 4 * k) : 0.0;
        gacc = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, gacc, 0, 0, 0);
      }
      const int j = 16 * bj + lr;                          // column of this lane's results
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = 16 * bi + lk + 4 * i;
        if (h < H && j < H && inO[h] && inO[j]) {
          double r = gacc[i];
          for (int u = 0; u < np; ++u) r -= alpha[h][u] * gph[u][j] + alpha[j][u] * gph[u][h];
          for (int u = 0; u < np; ++u)
            for (int v = 0; v < np; ++v) r += alpha[h][u] * alpha[j][v] * gph[u][prox[v]];
          acc += (bi == bj ? 1.0 : 2.0) * wd[h] * wd[j] * fmax(r, 0.0);
        }
      }
    }
    acc = wave_sum(acc);
    if (lane == 0) red4[wave] = acc;
    __syncthreads();
    rho = sqrt(fmax(red4[0] + red4[1] + red4[2] + red4[3], 0.0));
  }

  // ---- 8. coefficients
  if (t == 0) {
    const double qs = (double)qscale;
    const double rho_p = (rho + hsum[6]) * qs;
    float* cf = p.coef + (int64_t)qrow * kCoefStride;
    for (int r = 0; r < 4; ++r) cf[r] = (r < np) ? (float)(hsum[r] * qs) : (float)(sig[r] * qs);
    cf[4] = (float)rho_p * 1.0000005f;
    cf[5] = tau;
    cf[6] = (float)np;
    cf[7] = hopeless ? 1.f : 0.f;
    for (int r = 0; r < 4; ++r) cf[8 + r] = rnorm[r];
    if (!hopeless && p.prunes != nullptr) atomicOr(p.prunes, 1);   // the bound pass has work: key norms are needed
    if (p.ticket != nullptr) {
      // probe: the last planned query decides whether the call runs the
      // certificate pipeline (some probe query can prune: the prunes flag,
      // cleared by the prep kernel, was raised) or dense scoring
      __threadfence();
      if (atomicAdd(p.ticket, 1) == p.decide_nq - 1) {
        __threadfence();
        const bool any = __hip_atomic_load(p.prunes, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
        *p.decide_mode = any ? MODE_PRUNED : MODE_UNPRUNED;
        if (!any && p.stats != nullptr) atomicAdd(&p.stats[10], 1ull);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bound pass: wavefront (group, split) streams a 64-key-aligned share of the
// group's bounded keys; MFMA rows = 4 certificate rows x 4 queries
// ---------------------------------------------------------------------------
template <int C, int D>
__global__ __launch_bounds__(64) void bound_kernel(const BoundLaunch p) {
  using O = Ops<C, D>;
  constexpr int STEPS = O::STEPS;
  constexpr int KBYTES = D * O::KB;
  if (skip_launch(p.mode, p.run_if)) return;
  const int lane = lane_id();
  const int gi = blockIdx.x / p.splits, sp = blockIdx.x % p.splits;
  const GroupInfo gr = p.groups[gi];
  const int col = lane & 15, g = lane >> 4;
  const int lo_all = gr.bound_lo, n_all = gr.n_bounded;
  const int nw = (n_all + 63) / 64;
  const int w0 = (int)((int64_t)nw * sp / p.splits), w1 = (int)((int64_t)nw * (sp + 1) / p.splits);
  const int lo = lo_all + 64 * w0, hi = min(lo_all + 64 * w1, lo_all + n_all);
  unsigned long long* mw = p.masks + (int64_t)gi * p.mask_words;
  // this lane's output rows 4g..4g+3 = the 4 certificate rows of query slot g
  const bool qok = g < gr.nq;
  const int qrow = gr.q_row0 + g;
  float cf[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) cf[i] = qok ? p.coef[(int64_t)qrow * kCoefStride + i] : 0.f;
  const int npx = (int)cf[6];
  const bool hopeless = !qok || cf[7] != 0.f;
  const u64 hm = __ballot(qok && hopeless);
  const u64 okm = __ballot(qok);
  const bool all_hopeless = (hm == okm);
  const u64 nbounded = (u64)max(hi - lo, 0) * (u64)gr.nq;
  if (all_hopeless) {
    // every key survives; compaction reads the plan's flags instead of masks.
    // The group's first split counts the whole group.
    if (p.stats != nullptr && lane == 0 && sp == 0) {
      const u64 all = (u64)n_all * (u64)gr.nq;
      atomicAdd(&p.stats[2], all);
      atomicAdd(&p.stats[3], all);
      if (p.count_skipped) atomicAdd(&p.stats[7], 1ull);
    }
    if (p.debug_ub == nullptr && p.debug_mask == nullptr) return;
  }
  typename O::frag A[STEPS];
  {
    const int ra = lane & 15;
    const int qa = ra >> 2, rr = ra & 3;
    if (qa < gr.nq)
      O::load_q(static_cast<const uint8_t*>(p.rows) + ((int64_t)(gr.q_row0 + qa) * 4 + rr) * D * O::QB, g, A);
    else
      O::zero(A);
  }
  const uint8_t* kbytes = static_cast<const uint8_t*>(p.in.k);
  u64 word = 0, n_surv = 0;
  auto load = [&](int key, typename O::frag* B, float& ks, float& kn) {
    if (key < hi) {
      const int64_t row = key_row(p.in, gr.key_base, gr.seq, key);
      O::load_k(kbytes + row * KBYTES, g, B);
      ks = HasKScale<C>::value ? p.in.k_scale[row] : 1.f;
      kn = p.norms[(int64_t)gr.norm_base + key];
    } else {
      O::zero(B);
      ks = 1.f;
      kn = 0.f;
    }
  };
  auto bound = [&](int kb, const typename O::frag* B, float ks, float kn) {
    const int key = kb + col;
    v4f c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < STEPS; ++s) c = O::mma(A[s], B[s], c);
    float pos = 0.f, neg = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < npx) pos += cf[i] * fmaxf(c[i], 0.f);
      else neg += cf[i] * c[i];
    }
    const float ub = ks * (pos - fmaxf(neg, 0.f)) + cf[4] * kn;
    const bool valid = qok && key < hi;
    const bool surv = valid && (hopeless || ub >= cf[5]);
    if (p.debug_ub != nullptr && valid) p.debug_ub[(int64_t)qrow * p.debug_ld + key] = ub;
    if (p.debug_mask != nullptr && surv)
      atomicOr(&p.debug_mask[(int64_t)qrow * p.debug_mask_ld + (key >> 6)], 1ull << (key & 63));
    if (all_hopeless) return;
    const u64 m = __ballot(surv);
    const uint32_t u = (uint32_t)(m | (m >> 16) | (m >> 32) | (m >> 48)) & 0xFFFFu;
    n_surv += __popcll(m);
    const int bi = (kb - lo_all) >> 4;
    word |= (u64)u << (16 * (bi & 3));
    if ((bi & 3) == 3 || kb + 16 >= hi) {
      if (lane == 0) mw[bi >> 2] = word;
      word = 0;
    }
  };
#pragma unroll 1
  for (int kb = lo; kb < hi; kb += 32) {
    typename O::frag B0[STEPS], B1[STEPS];
    float ks0, kn0, ks1, kn1;
    load(kb + col, B0, ks0, kn0);
    load(kb + 16 + col, B1, ks1, kn1);
    bound(kb, B0, ks0, kn0);
    if (kb + 16 < hi) bound(kb + 16, B1, ks1, kn1);
  }
  if (!all_hopeless && p.stats != nullptr && lane == 0) {
    atomicAdd(&p.stats[2], nbounded);
    atomicAdd(&p.stats[3], n_surv);
    atomicAdd(&p.stats[9], (u64)max(hi - lo, 0));
  }
}

// ---------------------------------------------------------------------------
// bound pass over LDS key tiles: a workgroup takes up to 32 consecutive
// queries of one sequence -- groups_per_wave query groups per wavefront, so
// that each wavefront fills the 4 query slots of its MFMA rows (16 rows = 4
// certificate rows x 4 queries) -- and a 64-key-aligned share of their
// bounded keys.  The groups share the first bounded key; each group's range
// ends where its own seed window starts.  Keys, their scales and norms are
// staged through LDS (double-buffered, register prefetch), so every key is
// read once per workgroup.  Each group gets one 64-bit union-survivor word per
// 64 keys.
// ---------------------------------------------------------------------------
template <int C, int D, int GPW, bool BLOCKS>
__global__ __launch_bounds__(64 * kTileWaves) void bound_tiled_kernel(const BoundLaunch p) {
  using O = Ops<C, D>;
  constexpr int STEPS = O::STEPS;
  constexpr int KBYTES = D * O::KB;
  constexpr int ROW = KBYTES + 16;                   // padded LDS row
  constexpr int CPK = KBYTES / 16;
  constexpr int NCH = (64 * CPK + 64 * kTileWaves - 1) / (64 * kTileWaves);
  __shared__ __attribute__((aligned(16))) uint8_t ktile[2][64 * ROW];
  __shared__ float kinfo[2][2][64];                  // [buffer][scale, norm][key]
  // key-block test (BLOCKS): bit t set if tile t is loaded / if this wavefront bounds it
  __shared__ uint32_t keep[BLOCKS ? kMaxBoundTiles / 32 : 1];
  __shared__ uint32_t keep_w[kTileWaves][BLOCKS ? kMaxBoundTiles / 32 : 1];
  if (skip_launch(p.mode, p.run_if)) return;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x) >> 6;
  const int lane = lane_id();
  const WorkItem it = p.items[blockIdx.x];
  const GroupInfo g0 = p.groups[it.group];
  constexpr int gpw = GPW, qw = 4 / GPW;              // groups per wavefront, query slots per group
  const int gbase = it.group + wave * gpw, gend = it.group + it.pad;
  const bool active = gbase < gend;
  const int col = lane & 15, g = lane >> 4;
  const int lo = it.a0, hi = it.a1;                  // keys [lo, hi), lo - bound_lo a multiple of 64
  // this lane's output rows 4g..4g+3 = the 4 certificate rows of query slot g:
  // query gq of group gj of the wavefront
  const int gj = g / qw, gq = g % qw;
  const bool gok = gbase + gj < gend;
  const GroupInfo gr = p.groups[gok ? gbase + gj : it.group];
  const int ghi = min(hi, gr.bound_lo + gr.n_bounded);   // the group's bounded keys end here
  const bool qok = gok && gq < gr.nq;
  const int qrow = gr.q_row0 + gq;
  float cf[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) cf[i] = qok ? p.coef[(int64_t)qrow * kCoefStride + i] : 0.f;
  const int npx = (int)cf[6];
  const bool hopeless = !qok || cf[7] != 0.f;
  // lanes of this lane's group, and whether every query of it is hopeless
  const u64 gmask = (qw == 4) ? ~0ull : (((1ull << (16 * qw)) - 1ull) << (16 * qw * gj));
  const u64 prunable = __ballot(qok && !hopeless);
  const bool g_hopeless = (prunable & gmask) == 0ull;
  const bool all_hopeless = prunable == 0ull;        // every group of this wavefront
  const bool g_lead = gok && gq == 0 && col == 0;    // one lane per group keeps its books
  if (p.stats != nullptr && g_lead && g_hopeless && it.b0 == 0) {
    const u64 all = (u64)gr.n_bounded * (u64)gr.nq;   // the group's first share counts the whole group
    atomicAdd(&p.stats[2], all);
    atomicAdd(&p.stats[3], all);
    if (p.count_skipped) atomicAdd(&p.stats[7], 1ull);
  }
  // the whole workgroup leaves if no wavefront has work (and no dump is asked for)
  const bool dump = p.debug_ub != nullptr || p.debug_mask != nullptr;
  if (__syncthreads_and(!active || all_hopeless) && !dump) return;
  if (!BLOCKS && p.stats != nullptr && threadIdx.x == 0)
    atomicAdd(&p.stats[9], (u64)max(hi - lo, 0));   // rows this workgroup streams
  typename O::frag A[STEPS];
  {
    const int ra = lane & 15;
    const int qa = ra >> 2, rr = ra & 3;
    const int ga = gbase + qa / qw, ia = qa % qw;
    bool ok = false;
    int64_t arow = 0;
    if (ga < gend) {
      const GroupInfo gg = p.groups[ga];
      ok = ia < gg.nq;
      arow = (int64_t)(gg.q_row0 + ia) * 4 + rr;
    }
    if (ok)
      O::load_q(static_cast<const uint8_t*>(p.rows) + arow * D * O::QB, g, A);
    else
      O::zero(A);
  }
  const uint8_t* kbytes = static_cast<const uint8_t*>(p.in.k);
  const int ntiles = (hi - lo + 63) / 64;
  v4i stage[NCH];
  float st_s = 1.f, st_n = 0.f;
  auto fetch = [&](int t) {
    const int tid = lane_fresh() + 64 * wave;
    const int kb = lo + 64 * t;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int ch = tid + c * 64 * kTileWaves;
      const int slot = ch / CPK, part = ch % CPK;
      const int key = kb + slot;
      if (slot < 64 && key < hi) {
        const int64_t row = key_row(p.in, g0.key_base, g0.seq, key);
        stage[c] = *reinterpret_cast<const v4i*>(kbytes + row * KBYTES + part * 16);
      } else {
        stage[c] = v4i{0, 0, 0, 0};
      }
    }
    if (tid < 64) {
      const int key = kb + tid;
      const bool v = key < hi;
      st_s = (HasKScale<C>::value && v) ? p.in.k_scale[key_row(p.in, g0.key_base, g0.seq, key)] : 1.f;
      st_n = v ? p.norms[(int64_t)g0.norm_base + key] : 0.f;
    }
  };
  auto commit = [&](int bufi) {
    const int tid = lane_fresh() + 64 * wave;
    wait_vmem();
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int ch = tid + c * 64 * kTileWaves;
      const int slot = ch / CPK, part = ch % CPK;
      if (slot < 64) *reinterpret_cast<v4i*>(&ktile[bufi][slot * ROW + part * 16]) = stage[c];
    }
    if (tid < 64) {
      kinfo[bufi][0][tid] = st_s;
      kinfo[bufi][1][tid] = st_n;
    }
  };
  // Row multipliers split by role, zero elsewhere: proxy rows enter as
  // c_p ReLU(x), aggregate rows as sigma_j x (adding the zero terms leaves
  // both sums bit for bit what the role test would give).
  float cpos[4], cneg[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    cpos[i] = (i < npx) ? cf[i] : 0.f;
    cneg[i] = (i < npx) ? 0.f : cf[i];
  }
  // groups of this wavefront that keep books (not hopeless), as lane masks
  u64 keep_lanes = 0;
  for (int j = 0; j < gpw; ++j) {
    const u64 mj = (qw == 4) ? ~0ull : (((1ull << (16 * qw)) - 1ull) << (16 * qw * j));
    if (gbase + j < gend && (prunable & mj) != 0ull) keep_lanes |= mj;
  }
  u64 n_surv = 0;
  const bool work = active && !(all_hopeless && !dump);
  // Key-block test (DoSA pages: the transcript's Conclusion, certificates over
  // key blocks).  Tiles are 64-key blocks when the item starts on a block
  // boundary.  A lane of a query that keeps survivor books vetoes skipping a
  // tile unless the block bound
  //   BUB = sum_p c_p ReLU(s x_p + |r_p| rad) + rho' N - ReLU(s x_a - |a| rad) + margin
  // (x = row . centre on MFMA, s the centre's scale) is below its tau; tiles no
  // lane vetoes are never loaded, and their survivor words are zero.
  const bool blocks_on = BLOCKS && (lo & (kKeyBlock - 1)) == 0 && ntiles <= kMaxBoundTiles;
  float nr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) nr[i] = (BLOCKS && qok) ? p.coef[(int64_t)qrow * kCoefStride + 8 + i] : 0.f;
  // the centre fragment and summary of block column col of chunk c0
  struct BlockFrag {
    typename O::frag B[STEPS];
    v4f inf;
  };
  auto block_load = [&](int c0, BlockFrag& f) {
    const int bt = c0 + col;
    const int64_t blk = (int64_t)g0.blk_base + (lo >> 6) + bt;
    if (bt < ntiles) {
      O::load_k(p.blk_code + blk * KBYTES, g, f.B);
      f.inf = *reinterpret_cast<const v4f*>(p.blk_info + blk * 4);
    } else {
      O::zero(f.B);
      f.inf = v4f{1.f, 0.f, 0.f, 0.f};
    }
  };
  // block bound of this lane's query for block column col of chunk c0 (all lanes take part)
  auto block_bound_of = [&](int c0, const BlockFrag& f, bool& bv) -> float {
    bv = c0 + col < ntiles;
    const v4f inf = f.inf;
    const typename O::frag* B = f.B;
    v4f c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < STEPS; ++s) c = O::mma(A[s], B[s], c);
    const float sc = inf[0], rad = inf[1], nb = inf[2], cn = inf[3];
    float pos = 0.f, neg = 0.f, wsum = 0.f, nrad = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pos += cpos[i] * fmaxf(fmaf(sc, c[i], nr[i] * rad), 0.f);
      neg += cneg[i] * (sc * c[i]);
      nrad += cneg[i] * nr[i];
      wsum += (cpos[i] + cneg[i]) * nr[i];
    }
    neg -= nrad * rad;
    // rounding margin: 2 gamma_n (sum_r cf_r |r| (|c| + rad) + rho' N), n = d + 16, u = 2^-22
    constexpr float gam = (float)((D + 16) * 2.384185791015625e-7 / (1.0 - (D + 16) * 2.384185791015625e-7));
    const float base = pos - fmaxf(neg, 0.f) + cf[4] * nb;
    const float mg = 2.f * gam * (wsum * (cn + rad) + cf[4] * nb);
    return base + mg + 1e-6f * fabsf(base);
  };
  auto block_bound = [&](int c0, bool& bv) -> float {
    BlockFrag f;
    block_load(c0, f);
    return block_bound_of(c0, f, bv);
  };
  if (BLOCKS && blocks_on) {
    const int tid = (int)threadIdx.x;
    for (int i = tid; i < (ntiles + 31) / 32; i += 64 * kTileWaves) keep[i] = 0u;
    for (int i = lane; i < (ntiles + 31) / 32; i += 64) keep_w[wave][i] = 0u;
    __syncthreads();
    if (work) {
      const bool books = ((keep_lanes >> lane) & 1ull) != 0ull;
      // the next chunk's centres load while this chunk's bounds are evaluated
      BlockFrag fcur, fnext;
      block_load(0, fcur);
      for (int c0 = 0; c0 < ntiles; c0 += 16) {
        if (c0 + 16 < ntiles) block_load(c0 + 16, fnext);
        bool bv;
        const float bub = block_bound_of(c0, fcur, bv);
        const bool veto = bv && books && qok && (hopeless || !(bub < cf[5]));
        const u64 m = __ballot(veto);
        const uint32_t u = (uint32_t)(m | (m >> 16) | (m >> 32) | (m >> 48)) & 0xFFFFu;
        if (lane == 0 && u != 0u) {
          atomicOr(&keep[c0 >> 5], u << (c0 & 31));
          keep_w[wave][c0 >> 5] |= u << (c0 & 31);   // only this wavefront writes its row
        }
        if (c0 + 16 < ntiles) fcur = fnext;
      }
    }
    __syncthreads();
    // skipped tiles: zero survivor words for the groups that keep books; with a
    // dump, the block bound as every key's bound (and hopeless queries' bits)
    if (work) {
      for (int c0 = 0; c0 < ntiles; c0 += 16) {
        const uint32_t kw = (keep[c0 >> 5] >> (c0 & 31)) & 0xFFFFu;
        const uint32_t live = (ntiles - c0 >= 16) ? 0xFFFFu : ((1u << (ntiles - c0)) - 1u);
        if ((~kw & live) == 0u) continue;            // every tile of the chunk is loaded
        if (lane == 0) {
          for (int b = 0; b < 16; ++b) {
            if (!((live >> b) & 1u) || ((kw >> b) & 1u)) continue;
            const int kb = lo + 64 * (c0 + b);
            for (int j = 0; j < gpw; ++j) {
              if (gbase + j >= gend) break;
              const u64 mj = (qw == 4) ? ~0ull : (((1ull << (16 * qw)) - 1ull) << (16 * qw * j));
              if ((keep_lanes & mj) == 0ull) continue;
              p.masks[(int64_t)(gbase + j) * p.mask_words + ((kb - g0.bound_lo) >> 6)] = 0ull;
            }
          }
          if (p.stats != nullptr && wave == 0) atomicAdd(&p.stats[11], (u64)__popc(~kw & live));
        }
        if (dump) {
          bool bv;
          const float bub = block_bound(c0, bv);
          const int bt = c0 + col;
          if (bv && qok && !((kw >> col) & 1u)) {
            const int kb = lo + 64 * bt;
            for (int s2 = 0; s2 < 64; ++s2) {
              const int key = kb + s2;
              if (key >= ghi) break;
              if (p.debug_ub != nullptr) p.debug_ub[(int64_t)qrow * p.debug_ld + key] = bub;
              if (p.debug_mask != nullptr && hopeless)
                atomicOr(&p.debug_mask[(int64_t)qrow * p.debug_mask_ld + (key >> 6)], 1ull << (key & 63));
            }
          }
        }
      }
    }
  }
  auto kept = [&](int t) -> bool { return !blocks_on || ((keep[t >> 5] >> (t & 31)) & 1u) != 0u; };
  auto next_kept = [&](int t) -> int {   // first loaded tile at or after t (ntiles if none)
    if constexpr (!BLOCKS) return min(t, ntiles);
    while (t < ntiles && !kept(t)) {
      if (blocks_on && (t & 31) == 0 && keep[t >> 5] == 0u) t += 32;
      else ++t;
    }
    return min(t, ntiles);
  };
  if (BLOCKS && p.stats != nullptr && threadIdx.x == 0) {
    u64 rows = 0;   // key rows this workgroup streams
    for (int t = next_kept(0); t < ntiles; t = next_kept(t + 1)) rows += (u64)min(64, hi - (lo + 64 * t));
    atomicAdd(&p.stats[9], rows);
  }
  drain_memory();   // the certificate rows and coefficients, before the prefetching loop
  // Tile t+1 (the next loaded tile) is loaded while tile t is bounded and
  // written to LDS before the tile's survivor words are stored; the last
  // iteration reloads its own tile into the idle buffer, so no load stays
  // pending across the back edge.
  int t = next_kept(0);
  if (t < ntiles) {
    fetch(t);
    commit(0);
  }
  __syncthreads();
  int bufi = 0;
#pragma unroll 1
  while (t < ntiles) {
    const int tn = next_kept(t + 1);
    fetch(tn < ntiles ? tn : t);
    const int kb = lo + 64 * t;
    // one survivor word per group of the wavefront (wavefront-uniform)
    u64 words[gpw];
#pragma unroll
    for (int j = 0; j < gpw; ++j) words[j] = 0ull;
    // a tile this wavefront's queries all prune by the block bound keeps zero
    // survivor words without per-key bounds (with a dump, every key is bounded)
    const bool mine = !BLOCKS || !blocks_on || dump || ((keep_w[wave][t >> 5] >> (t & 31)) & 1u) != 0u;
    if (work && mine) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int kslot = b * 16 + col;
        const int key = kb + kslot;
        typename O::frag B[STEPS];
        O::load_k(&ktile[bufi][kslot * ROW], g, B);
        v4f c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < STEPS; ++s) c = O::mma(A[s], B[s], c);
        float pos = 0.f, neg = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pos += cpos[i] * fmaxf(c[i], 0.f);
          neg += cneg[i] * c[i];
        }
        const float ub = kinfo[bufi][0][kslot] * (pos - fmaxf(neg, 0.f)) + cf[4] * kinfo[bufi][1][kslot];
        const bool valid = qok && key < ghi;
        if (p.debug_ub != nullptr && valid) p.debug_ub[(int64_t)qrow * p.debug_ld + key] = ub;
        const bool surv = valid && (hopeless || ub >= cf[5]);
        if (p.debug_mask != nullptr && surv)
          atomicOr(&p.debug_mask[(int64_t)qrow * p.debug_mask_ld + (key >> 6)], 1ull << (key & 63));
        const u64 m = __ballot(surv);
        n_surv += __popcll(m & keep_lanes);
        // each group's union over its query slots
#pragma unroll
        for (int j = 0; j < gpw; ++j) {
          u64 u = 0;
#pragma unroll
          for (int q = 0; q < qw; ++q) u |= (m >> (16 * (qw * j + q))) & 0xFFFFull;
          words[j] |= u << (16 * b);
        }
      }
    }
    commit(bufi ^ 1);
    if (work && lane == 0) {
#pragma unroll
      for (int j = 0; j < gpw; ++j) {
        if (gbase + j >= gend) break;
        const u64 mj = (qw == 4) ? ~0ull : (((1ull << (16 * qw)) - 1ull) << (16 * qw * j));
        if ((keep_lanes & mj) == 0ull) continue;
        p.masks[(int64_t)(gbase + j) * p.mask_words + ((kb - g0.bound_lo) >> 6)] = words[j];
      }
    }
    __syncthreads();
    bufi ^= 1;
    t = tn;
  }
  if (work && lane == 0 && p.stats != nullptr) {
    // pairs bounded in this share by the wavefront's groups that were not hopeless
    u64 nbounded = 0;
    for (int j = 0; j < gpw; ++j) {
      if (gbase + j >= gend) break;
      const GroupInfo gg = p.groups[gbase + j];
      if (((prunable >> (16 * qw * j)) & (qw == 4 ? ~0ull : ((1ull << (16 * qw)) - 1ull))) == 0ull) continue;
      nbounded += (u64)max(min(hi, gg.bound_lo + gg.n_bounded) - lo, 0) * (u64)gg.nq;
    }
    atomicAdd(&p.stats[2], nbounded);
    atomicAdd(&p.stats[3], n_surv);
  }
}

// ---------------------------------------------------------------------------
// compaction: one workgroup per tile (up to 8 query groups that bound the same
// key range).  Each group has a survivor bitmask; a group whose every query
// the plan marked hopeless has none and keeps all its bounded keys.  The masks
// become ascending key lists, routed one of two ways:
//   calls with tiles: if scoring the tile's union of survivors U with the
//     LDS-tiled kernel costs less than walking every group's own list U_g
//     (groups * |U| <= kTileGain * sum_g |U_g|: the tiled kernel scores a
//     pair several times faster than the per-group kernel, and its shares
//     are launched longest first; 8 measured faster than 4 and equal to 16
//     on MI355X), the union goes
//     to the list of the tile's first group and every group of the tile is
//     flagged; otherwise each group gets its own list.
//   calls without tiles (one wavefront per group): a tile whose survivors are
//     at least kDenseFrac of its bounded keys is flagged and scored over its
//     whole bounded range; otherwise each group gets its own list.
// Wavefronts expand contiguous runs of mask words, one word per iteration and
// one key per lane, so the list stores are coalesced.
// ---------------------------------------------------------------------------
constexpr float kDenseFrac = 0.4f;
constexpr int kTileGain = 8;

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += (uint32_t)__shfl_xor((int)v, off, 64);
  return v;
}

// keys of mask words [w0, w1) in ascending order at out + base (word wd holds
// keys key0 + 64 wd + bit); called by a whole wavefront
template <class Word>
__device__ __forceinline__ void expand_words(const Word& word, int w0, int w1, int key0, int32_t* out,
                                             uint32_t base) {
  const int lane = lane_id();
  const u64 below = (1ull << lane) - 1ull;
  for (int wb = w0; wb < w1; wb += 64) {
    const u64 mine = (wb + lane < w1) ? word(wb + lane) : 0ull;
    const int n = min(64, w1 - wb);
    for (int j = 0; j < n; ++j) {
      const u64 m = __shfl(mine, j, 64);
      if ((m >> lane) & 1ull) out[base + (uint32_t)__popcll(m & below)] = key0 + 64 * (wb + j) + lane;
      base += (uint32_t)__popcll(m);
    }
  }
}

__global__ __launch_bounds__(512) void compact_kernel(const CompactLaunch p) {
  if (skip_launch(p.mode, p.run_if)) return;
  const int gi0 = p.tiles[(int64_t)blockIdx.x * p.tile_stride].group;
  const GroupInfo head = p.groups[gi0];
  const int tn = head.tile_n;
  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  const int nb = head.n_bounded;                // the same for every group of the tile
  const int nw = (nb + 63) / 64;
  __shared__ uint32_t surv[8], part[8];
  __shared__ int32_t hopeless[8];
  if (threadIdx.x < 8) {
    bool h = true;
    if ((int)threadIdx.x < tn) {
      const GroupInfo g = p.groups[gi0 + threadIdx.x];
      for (int i = 0; i < g.nq; ++i) h = h && p.coef[(int64_t)(g.q_row0 + i) * kCoefStride + 7] != 0.f;
    }
    hopeless[threadIdx.x] = h ? 1 : 0;
  }
  if (wave < tn) {
    const GroupInfo g = p.groups[gi0 + wave];
    const int nr = p.r1 - p.r0;
    for (int e = lane; e < g.nq * nr; e += 64)
      *p.cb.count(g.q_row0 + e / nr, p.r0 + e % nr) = 0u;
  }
  __syncthreads();
  auto word = [&](int g, int wd) -> u64 {
    if (hopeless[g]) {
      const int rem = nb - 64 * wd;
      return rem >= 64 ? ~0ull : ((1ull << rem) - 1ull);
    }
    return p.masks[(int64_t)(gi0 + g) * p.mask_words + wd];
  };
  auto uword = [&](int wd) -> u64 {
    u64 m = 0;
    for (int g = 0; g < tn; ++g) m |= word(g, wd);
    return m;
  };
  // survivors per group, and of the union over each wavefront's run of words
  uint32_t c = 0;
  if (wave < tn) {
    if (hopeless[wave]) c = (lane == 0) ? (uint32_t)nb : 0u;
    else
      for (int wd = lane; wd < nw; wd += 64) c += (uint32_t)__popcll(word(wave, wd));
  }
  c = wave_sum_u32(c);
  const int seg = (nw + 7) / 8;
  const int s0 = min(nw, wave * seg), s1 = min(nw, s0 + seg);
  uint32_t u = 0;
  if (p.allow_union)
    for (int wd = s0 + lane; wd < s1; wd += 64) u += (uint32_t)__popcll(uword(wd));
  u = wave_sum_u32(u);
  if (lane == 0) {
    surv[wave] = (wave < tn) ? c : 0u;
    part[wave] = u;
  }
  __syncthreads();
  uint64_t ts = 0, tu = 0;
  uint32_t ubase = 0;
  for (int i = 0; i < 8; ++i) {
    ts += surv[i];
    tu += part[i];
    if (i < wave) ubase += part[i];
  }
  bool whole;
  if (p.allow_union) whole = p.force_lists == 0 && (uint64_t)tn * tu <= (uint64_t)kTileGain * ts;
  else whole = (float)ts >= kDenseFrac * (float)((uint64_t)nb * (uint64_t)tn);
  // With query tiles the tile's groups share one list area of n_bounded + 16 per
  // group entries: the union list, or the groups' own lists one after the
  // other (that route is taken only when they total less than the union).
  uint32_t start = 0;
  if (!whole && p.allow_union)
    for (int i = 0; i < wave && i < tn; ++i) start += (surv[i] + 15u) & ~15u;
  if (wave < tn && lane == 0) {
    p.group_flags[gi0 + wave] = whole ? 1 : 0;
    p.list_len[gi0 + wave] = (whole && p.allow_union && wave == 0) ? (int32_t)tu : (whole ? 0 : (int32_t)c);
    p.list_start[gi0 + wave] = (int32_t)start;
  }
  if (whole) {
    if (p.allow_union) expand_words(uword, s0, s1, head.bound_lo, p.lists + head.list_off, ubase);
  } else if (wave < tn) {
    const GroupInfo gr = p.groups[gi0 + wave];
    expand_words([&](int wd) { return word(wave, wd); }, 0, nw, gr.bound_lo, p.lists + gr.list_off + start, 0u);
  }
}

__global__ void stats_add_kernel(unsigned long long* st, const dosa_stats add) {
  constexpr int n = (int)(sizeof(dosa_stats) / sizeof(unsigned long long));
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    const unsigned long long* a = reinterpret_cast<const unsigned long long*>(&add);
    for (int i = 0; i < n; ++i)
      if (a[i]) atomicAdd(&st[i], a[i]);
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
// The pruned path's decision after planning its probe tile (the call's last
// query tile, its longest contexts): if the certificate cannot prune a single
// query there, the call scores every key densely instead.  Exactness does not
// depend on it; only which kernels do the work.
hipError_t launch_stats_add(unsigned long long* stats, const unsigned long long* v, hipStream_t s) {
  dosa_stats a;
  static_assert(sizeof(dosa_stats) == 12 * sizeof(unsigned long long), "stats layout");
  memcpy(&a, v, sizeof(a));
  hipLaunchKernelGGL(stats_add_kernel, dim3(1), dim3(64), 0, s, stats, a);
  return hipGetLastError();
}

template <int C, int D>
static hipError_t norms_t(const NormLaunch& p, hipStream_t s) {
  constexpr int per_block = 256 / (D * KBytes<C>::value / 16) * kNormIter;
  const int nb = (int)((p.max_kv + per_block - 1) / per_block);
  if (nb == 0 || p.batch == 0) return hipSuccess;
  const int gy = p.batch < 65535 ? p.batch : 65535;
  const int gcap = 2048 / gy > 1 ? 2048 / gy : 1;
  const int gx = nb < gcap ? nb : gcap;   // about 2048 workgroups, each striding over key blocks
  hipLaunchKernelGGL((key_norm_kernel<C, D>), dim3(gx, gy), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int C>
static hipError_t norms_c(int d, const NormLaunch& p, hipStream_t s) {
  return d == 64 ? norms_t<C, 64>(p, s) : norms_t<C, 128>(p, s);
}

template <int C, int D>
static hipError_t blocks_t(const NormLaunch& p, hipStream_t s) {
  const int nb = (int)((p.max_kv + kKeyBlock - 1) / kKeyBlock);
  if (nb == 0 || p.batch == 0) return hipSuccess;
  hipLaunchKernelGGL((key_block_kernel<C, D>), dim3(nb, p.batch < 65535 ? p.batch : 65535), dim3(64), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_key_blocks(int combo, int d, const NormLaunch& p, hipStream_t s) {
  if (p.total_k == 0 || p.blk_code == nullptr) return hipSuccess;
  switch (combo) {
    case C_F32: return d == 64 ? blocks_t<C_F32, 64>(p, s) : blocks_t<C_F32, 128>(p, s);
    case C_BF16: return d == 64 ? blocks_t<C_BF16, 64>(p, s) : blocks_t<C_BF16, 128>(p, s);
    default: return d == 64 ? blocks_t<C_FP8, 64>(p, s) : blocks_t<C_FP8, 128>(p, s);   // fp8 keys
  }
}

hipError_t launch_key_norms(int combo, int d, const NormLaunch& p, hipStream_t s) {
  if (p.total_k == 0) return hipSuccess;
  switch (combo) {
    case C_F32: return norms_c<C_F32>(d, p, s);
    case C_BF16: return norms_c<C_BF16>(d, p, s);
    default: return norms_c<C_FP8>(d, p, s);   // fp8 keys (both fp8 combos)
  }
}

template <int C, int H, int D>
static hipError_t plan_t(const PlanLaunch& p, hipStream_t s) {
  hipLaunchKernelGGL((plan_kernel<C, H, D>), dim3(p.n_groups, queries_per_wave(C, H, D)), dim3(256), 0, s, p);   // one workgroup per query slot of a group
  return hipGetLastError();
}

template <int C>
static hipError_t plan_c(int H, int d, const PlanLaunch& p, hipStream_t s) {
#define DOSA_HD(HH, DD) \
  if (HP == HH && d == DD) return plan_t<C, HH, DD>(p, s);
  const int HP = padded_heads(H);
  DOSA_HD(8, 64) DOSA_HD(16, 64) DOSA_HD(32, 64) DOSA_HD(64, 64)
  DOSA_HD(8, 128) DOSA_HD(16, 128) DOSA_HD(32, 128) DOSA_HD(64, 128)
#undef DOSA_HD
  return hipErrorInvalidValue;
}

hipError_t launch_plan(int combo, int H, int d, const PlanLaunch& p, hipStream_t s) {
  if (p.n_groups == 0) return hipSuccess;
  switch (combo) {
    case C_F32: return plan_c<C_F32>(H, d, p, s);
    case C_BF16: return plan_c<C_BF16>(H, d, p, s);
    case C_FP8: return plan_c<C_FP8>(H, d, p, s);
    case C_BF16Q_FP8K: return plan_c<C_BF16Q_FP8K>(H, d, p, s);
  }
  return hipErrorInvalidValue;
}

template <int C>
static hipError_t bound_c(int d, const BoundLaunch& p, hipStream_t s) {
  if (p.items != nullptr) {
    if (p.n_items == 0) return hipSuccess;
#define DOSA_BT(DD, G)                                                                                            \
  if (d == DD && p.groups_per_wave == G) {                                                                        \
    if (p.blk_code != nullptr)                                                                                    \
      hipLaunchKernelGGL((bound_tiled_kernel<C, DD, G, true>), dim3(p.n_items), dim3(64 * kTileWaves), 0, s, p);  \
    else                                                                                                          \
      hipLaunchKernelGGL((bound_tiled_kernel<C, DD, G, false>), dim3(p.n_items), dim3(64 * kTileWaves), 0, s, p); \
    return hipGetLastError();                                                                                     \
  }
    DOSA_BT(64, 1) DOSA_BT(64, 2) DOSA_BT(64, 4) DOSA_BT(128, 1) DOSA_BT(128, 2) DOSA_BT(128, 4)
#undef DOSA_BT
    return hipErrorInvalidValue;
  }
  const int nb = p.n_groups * p.splits;
  if (d == 64) hipLaunchKernelGGL((bound_kernel<C, 64>), dim3(nb), dim3(64), 0, s, p);
  else hipLaunchKernelGGL((bound_kernel<C, 128>), dim3(nb), dim3(64), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_bound(int combo, int H, int d, const BoundLaunch& p, hipStream_t s) {
  (void)H;
  if (p.n_groups == 0) return hipSuccess;
  switch (combo) {
    case C_F32: return bound_c<C_F32>(d, p, s);
    case C_BF16: return bound_c<C_BF16>(d, p, s);
    case C_FP8: return bound_c<C_FP8>(d, p, s);
    case C_BF16Q_FP8K: return bound_c<C_BF16Q_FP8K>(d, p, s);
  }
  return hipErrorInvalidValue;
}

// Share lengths of the tiled survivor items as the survivor kernel will cut
// them (0 for shares it skips and for tiles routed to per-group lists), then a
// bitonic sort on (length, ~item) descending: the longest shares first, equal
// lengths in item order.  A tile's shares have equal lengths, so they sort
// next to each other; within each run of 32 sorted items, item j goes to
// launch slot 8 (j mod 4) + j / 4, which puts 4 neighbours on slots of one
// residue mod 8.  Workgroups go to the 8 XCDs round robin by launch index, so
// a tile's shares then share one L2 for its query fragments (1% faster
// survivor scoring on MI355X).
__global__ __launch_bounds__(1024) void order_kernel(const OrderLaunch p) {
  __shared__ u64 key[kMaxOrderItems];
  if (skip_launch(p.mode, p.run_if)) return;
  const int n = p.n_items;
  int N = 1;
  while (N < n) N <<= 1;
  for (int i = threadIdx.x; i < N; i += blockDim.x) {
    uint32_t len = 0;
    if (i < n) {
      const WorkItem it = p.items[i];
      bool all = true;
      for (int g = 0; g < it.pad; ++g) all = all && (p.tile_flags[it.group + g] != 0);
      if (all) {
        const int L = p.list_len[it.group];
        const int nsh = min(it.a1, max(1, (L + kUnionMinShare - 1) / kUnionMinShare));
        if (it.a0 < nsh)
          len = (uint32_t)((int64_t)L * (it.a0 + 1) / nsh - (int64_t)L * it.a0 / nsh);
      }
    }
    key[i] = (i < n) ? (((u64)len << 32) | (u64)(0xFFFFFFFFu - (uint32_t)i)) : 0ull;
  }
  __syncthreads();
  for (int size = 2; size <= N; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < (N >> 1); i += blockDim.x) {
        const int lo = 2 * stride * (i / stride) + (i % stride);
        const int hi = lo + stride;
        const bool desc = (lo & size) == 0;
        const u64 a = key[lo], b = key[hi];
        if (desc ? (a < b) : (a > b)) { key[lo] = b; key[hi] = a; }
      }
      __syncthreads();
    }
  }
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int c0 = i & ~31, j = i & 31;
    const int dst = (c0 + 32 <= n) ? c0 + (j & 3) * 8 + (j >> 2) : i;
    p.order[dst] = (int32_t)(0xFFFFFFFFu - (uint32_t)key[i]);
  }
}

hipError_t launch_order(const OrderLaunch& p, hipStream_t s) {
  if (p.n_items <= 0 || p.n_items > kMaxOrderItems) return hipErrorInvalidValue;
  hipLaunchKernelGGL(order_kernel, dim3(1), dim3(1024), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_compact(const CompactLaunch& p, hipStream_t s) {
  if (p.n_tiles == 0) return hipSuccess;
  hipLaunchKernelGGL(compact_kernel, dim3(p.n_tiles), dim3(512), 0, s, p);
  return hipGetLastError();
}

}  // namespace dosa
