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
#include <vector>

#include "dosa_device.h"

namespace dosa {

// ---------------------------------------------------------------------------
// scalar decoders (exact)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float dec_fp8(uint32_t x) {
  const uint32_t e = (x >> 3) & 15u, m = x & 7u;
  const float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
  return (x & 0x80u) ? -mag : mag;
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
// per-key norms ||k_s|| (dequantised), rounded up; per-sequence minimum
// ---------------------------------------------------------------------------
__global__ void fill_f32(float* p, int n, float v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// 16 lanes per key (coalesced row reads), 16 keys per pass of a 256-thread
// block, kNormKeys consecutive logical keys per block.  The per-sequence
// minimum is kept per lane group and flushed with one atomic per sequence
// change.
constexpr int kNormKeys = 1024;

template <int C, int D>
__global__ __launch_bounds__(256) void key_norm_kernel(const NormLaunch p) {
  constexpr int PER = D / 16;   // elements per lane
  const int t = threadIdx.x;
  const int grp = t >> 4, l16 = t & 15;
  const int64_t k0 = (int64_t)blockIdx.x * kNormKeys;
  const int64_t k1 = min<int64_t>(k0 + kNormKeys, p.total_k);
  int cur_seq = -1;
  float cur_min = INFINITY;
  int b = 0;
  {
    int lo = 0, hi = p.batch;   // last b with cu_kv[b] <= k0
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (p.cu_kv[mid] <= k0) lo = mid; else hi = mid;
    }
    b = lo;
  }
  for (int64_t i = k0 + grp; i < k1; i += 16) {
    while (b + 1 < p.batch && p.cu_kv[b + 1] <= i) ++b;
    const int key = (int)(i - p.cu_kv[b]);
    const int64_t row = key_row(p.in, p.cu_kv[b], b, key);
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const float v = k_elem<C>(p.in.k, row * D + l16 * PER + e);
      acc = fmaf(v, v, acc);
    }
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 16);
    float n = sqrtf(acc);
    if constexpr (HasKScale<C>::value) n *= p.in.k_scale[row];
    n *= 1.0000153f;                           // covers the fp32 sum/sqrt/scale rounding (<< 2^-16)
    if (l16 == 0) p.norms[i] = n;
    if (b != cur_seq) {
      if (cur_seq >= 0 && l16 == 0)
        atomicMin(reinterpret_cast<unsigned int*>(p.norm_min) + cur_seq, __float_as_uint(cur_min));
      cur_seq = b;
      cur_min = INFINITY;
    }
    cur_min = fminf(cur_min, n * 0.9999695f);
  }
  if (cur_seq >= 0 && l16 == 0)
    atomicMin(reinterpret_cast<unsigned int*>(p.norm_min) + cur_seq, __float_as_uint(cur_min));
}

// ---------------------------------------------------------------------------
// per-query plan, one workgroup of 256 threads per query
// ---------------------------------------------------------------------------
__device__ __forceinline__ double block_sum(double v, double* red) {
  const int t = threadIdx.x;
  red[t] = v;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (t < s) red[t] += red[t + s];
    __syncthreads();
  }
  const double r = red[0];
  __syncthreads();
  return r;
}
__device__ __forceinline__ double block_max(double v, double* red) {
  const int t = threadIdx.x;
  red[t] = v;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (t < s) red[t] = fmax(red[t], red[t + s]);
    __syncthreads();
  }
  const double r = red[0];
  __syncthreads();
  return r;
}

// Nonnegative least squares of a head on <= 3 proxies, exhaustive over
// supports (exact): minimise a^T G a - 2 b^T a subject to a >= 0.
__device__ void nnls3(int p, const double Gp[3][3], const double b[3], double out[3]) {
  double best = 0.0;
  out[0] = out[1] = out[2] = 0.0;
  for (int mask = 1; mask < (1 << p); ++mask) {
    int idx[3], n = 0;
    for (int i = 0; i < p; ++i)
      if (mask & (1 << i)) idx[n++] = i;
    double a[3] = {0, 0, 0};
    bool ok = true;
    if (n == 1) {
      const double g = Gp[idx[0]][idx[0]];
      ok = g > 0.0;
      if (ok) a[0] = b[idx[0]] / g;
    } else if (n == 2) {
      const double g00 = Gp[idx[0]][idx[0]], g01 = Gp[idx[0]][idx[1]], g11 = Gp[idx[1]][idx[1]];
      const double det = g00 * g11 - g01 * g01;
      ok = det > 1e-12 * g00 * g11;
      if (ok) {
        a[0] = (b[idx[0]] * g11 - b[idx[1]] * g01) / det;
        a[1] = (b[idx[1]] * g00 - b[idx[0]] * g01) / det;
      }
    } else {
      double M[3][3];
      for (int r = 0; r < 3; ++r)
        for (int c = 0; c < 3; ++c) M[r][c] = Gp[idx[r]][idx[c]];
      const double det = M[0][0] * (M[1][1] * M[2][2] - M[1][2] * M[2][1]) -
                         M[0][1] * (M[1][0] * M[2][2] - M[1][2] * M[2][0]) +
                         M[0][2] * (M[1][0] * M[2][1] - M[1][1] * M[2][0]);
      ok = det > 1e-12 * M[0][0] * M[1][1] * M[2][2];
      if (ok) {
        for (int c = 0; c < 3; ++c) {
          double Mc[3][3];
          for (int r = 0; r < 3; ++r)
            for (int cc = 0; cc < 3; ++cc) Mc[r][cc] = (cc == c) ? b[idx[r]] : M[r][cc];
          a[c] = (Mc[0][0] * (Mc[1][1] * Mc[2][2] - Mc[1][2] * Mc[2][1]) -
                  Mc[0][1] * (Mc[1][0] * Mc[2][2] - Mc[1][2] * Mc[2][0]) +
                  Mc[0][2] * (Mc[1][0] * Mc[2][1] - Mc[1][1] * Mc[2][0])) / det;
        }
      }
    }
    if (!ok) continue;
    bool feas = true;
    for (int i = 0; i < n; ++i) feas = feas && (a[i] >= 0.0);
    if (!feas) continue;
    double f = 0.0;
    for (int i = 0; i < n; ++i) {
      f -= 2.0 * b[idx[i]] * a[i];
      for (int j = 0; j < n; ++j) f += a[i] * Gp[idx[i]][idx[j]] * a[j];
    }
    if (f < best) {
      best = f;
      out[0] = out[1] = out[2] = 0.0;
      for (int i = 0; i < n; ++i) out[idx[i]] = a[i];
    }
  }
}

constexpr float kSkipFrac = 0.7f;   // sampled survival above which the bound pass is skipped

template <int C, int H, int D>
__global__ __launch_bounds__(256) void plan_kernel(const PlanLaunch p) {
  constexpr int QB = (C == C_F32) ? 4 : (C == C_FP8 ? 1 : 2);
  const GroupInfo gr = p.groups[blockIdx.x];
  const int slot = blockIdx.y;
  if (slot >= gr.nq) return;
  const int qrow = gr.q_row0 + slot;
  const int pos = gr.pos0 + slot;
  const int t = threadIdx.x;

  __shared__ float qf[H][D + 1];     // decoded, unscaled (exact in fp32)
  constexpr int SCR = (H * H > 32 * D) ? H * H : 32 * D;   // doubles
  __shared__ double scratch[SCR];    // sampled seed keys, later the head Gram matrix
  double (*G)[H] = reinterpret_cast<double (*)[H]>(scratch);
  __shared__ double wd[H];
  __shared__ double qn2[H];          // ||q_h||^2
  __shared__ double gph[3][H];       // <q_p, q_h> for the proxies
  __shared__ double alpha[H][3];
  __shared__ double rn2[H];          // ||r_h||^2
  __shared__ int prox[3];
  __shared__ int np_s;
  __shared__ int act[H];
  __shared__ double red[256];
  __shared__ double cvec[3];
  __shared__ double avec[D];
  __shared__ double res[D];

  const void* qbase = p.in.q;
  const int64_t qoff = (int64_t)qrow * H * D;
  for (int e = t; e < H * D; e += 256) qf[e / D][e % D] = q_elem<C>(qbase, qoff + e);
  for (int h = t; h < H; h += 256) {
    wd[h] = (double)p.in.w[(int64_t)qrow * H + h];
    act[h] = 0;
  }
  __syncthreads();
  for (int h = t; h < H; h += 256) {
    double s2 = 0.0;
    for (int i = 0; i < D; ++i) s2 += (double)qf[h][i] * (double)qf[h][i];
    qn2[h] = s2;
  }
  __syncthreads();
  // proxies: positive heads of largest w_h ||q_h|| (lower head index on ties)
  if (t == 0) {
    int n = 0;
    for (int r = 0; r < p.num_proxies; ++r) {
      int best = -1;
      double bv = -1.0;
      for (int h = 0; h < H; ++h) {
        if (!(wd[h] > 0.0)) continue;
        bool used = false;
        for (int u = 0; u < n; ++u) used = used || (prox[u] == h);
        if (used) continue;
        const double v = wd[h] * sqrt(qn2[h]);
        if (v > bv) { bv = v; best = h; }
      }
      if (best < 0) break;
      prox[n++] = best;
    }
    np_s = n;
  }
  __syncthreads();
  const int np = np_s;
  for (int e = t; e < np * H; e += 256) {
    const int r = e / H, h = e % H;
    double s2 = 0.0;
    for (int i = 0; i < D; ++i) s2 += (double)qf[prox[r]][i] * (double)qf[h][i];
    gph[r][h] = s2;
  }
  __syncthreads();
  auto in_O = [&](int h) {
    if (!(wd[h] > 0.0)) return false;
    for (int u = 0; u < np; ++u)
      if (prox[u] == h) return false;
    return true;
  };
  // nonnegative projections of the other positive heads; residual norms
  for (int h = t; h < H; h += 256) {
    double a[3] = {0, 0, 0};
    double Gp[3][3], b[3];
    for (int r = 0; r < 3; ++r) {
      b[r] = (r < np) ? gph[r][h] : 0.0;
      for (int c = 0; c < 3; ++c) Gp[r][c] = (r < np && c < np) ? gph[r][prox[c]] : 0.0;
    }
    if (in_O(h) && np > 0) nnls3(np, Gp, b, a);
    alpha[h][0] = a[0]; alpha[h][1] = a[1]; alpha[h][2] = a[2];
    double r2 = qn2[h];
    for (int u = 0; u < np; ++u) r2 -= 2.0 * a[u] * b[u];
    for (int u = 0; u < np; ++u)
      for (int v = 0; v < np; ++v) r2 += a[u] * Gp[u][v] * a[v];
    rn2[h] = fmax(r2, 0.0);
  }
  __syncthreads();
  // c_p = w_p + sum_{h in O} w_h alpha_hp
  for (int u = 0; u < np; ++u) {
    double v = 0.0;
    for (int h = t; h < H; h += 256)
      if (in_O(h)) v += wd[h] * alpha[h][u];
    v = block_sum(v, red);
    if (t == 0) cvec[u] = wd[prox[u]] + v;
  }
  // separable residual constant (an upper bound of the joint one) and the
  // diagonal of the joint sum (a lower bound of it)
  double ps = 0.0, pl = 0.0;
  for (int h = t; h < H; h += 256)
    if (in_O(h)) {
      ps += wd[h] * sqrt(rn2[h]);
      pl += wd[h] * wd[h] * rn2[h];
    }
  const double rho_sep = block_sum(ps, red);
  const double rho_lo = sqrt(fmax(block_sum(pl, red), 0.0));
  // activation statistics of the negative heads on up to 64 keys sampled
  // from the seed window (staged in LDS)
  const int n_last = gr.pos0 + gr.nq;
  const int wlo = max(0, n_last - p.seed_window);
  const int span = pos - wlo + 1;
  const int ns = min(64, max(span, 0));
  const bool use_neg = (p.flags & DOSA_NO_NEGATIVE) == 0;
  float* kf = reinterpret_cast<float*>(scratch);   // [64][D]
  if (use_neg && ns > 0) {
    const int step = max(1, span / ns);
    for (int e = t; e < ns * D; e += 256) {
      const int i = e / D, c = e % D;
      const int key = pos - i * step;
      const int64_t row = key_row(p.in, gr.key_base, gr.seq, key);
      kf[i * D + c] = k_elem<C>(p.in.k, row * D + c);
    }
    __syncthreads();
    const int h = t & (H - 1);
    const int part_id = t / H;
    const int nparts = 256 / H;
    if (wd[h] < 0.0) {
      int c = 0;
      for (int i = part_id; i < ns; i += nparts) {
        float sacc = 0.f;
        for (int e = 0; e < D; ++e) sacc = fmaf(qf[h][e], kf[i * D + e], sacc);
        c += (sacc > 0.f) ? 1 : 0;
      }
      atomicAdd(&act[h], c);
    }
  }
  __syncthreads();
  // aggregate a = sum_{h in A} |w_h| q_h, in fp64, unscaled units
  const double need = (double)p.neg_frac * (double)ns;
  for (int i = t; i < D; i += 256) {
    double sacc = 0.0;
    if (use_neg)
      for (int h = 0; h < H; ++h)
        if (wd[h] < 0.0 && (ns > 0 ? (double)act[h] >= need : p.neg_frac <= 0.f)) sacc += -wd[h] * (double)qf[h][i];
    avec[i] = sacc;
    res[i] = sacc;
  }
  __syncthreads();
  // operand rows: proxies verbatim, then terms of the aggregate
  uint8_t* rows = static_cast<uint8_t*>(p.rows) + (int64_t)qrow * 4 * D * QB;
  const uint8_t* qraw = static_cast<const uint8_t*>(p.in.q) + (int64_t)qrow * H * D * QB;
  for (int e = t; e < np * D * QB; e += 256) {
    const int r = e / (D * QB), o = e % (D * QB);
    rows[r * D * QB + o] = qraw[(int64_t)prox[r] * D * QB + o];
  }
  double sig[4] = {0, 0, 0, 0};
  double fnorm[4] = {0, 0, 0, 0};
  for (int r = np; r < 4; ++r) {
    float sg = 1.f;
    if constexpr (C == C_FP8) {
      double mx = 0.0;
      for (int i = t; i < D; i += 256) mx = fmax(mx, fabs(res[i]));
      mx = block_max(mx, red);
      sg = (mx > 0.0) ? (float)(mx / 448.0) : 1.f;
      if (!(sg > 0.f)) sg = 1.f;   // underflow guard
    }
    double fn = 0.0;
    for (int i = t; i < D; i += 256) {
      const double v = res[i];
      double dv;
      if constexpr (C == C_FP8) {
        const uint32_t code = enc_fp8((float)(v / (double)sg));
        rows[r * D + i] = (uint8_t)code;
        dv = (double)dec_fp8(code);
      } else if constexpr (C == C_F32) {
        const float f = (float)v;
        reinterpret_cast<float*>(rows)[r * D + i] = f;
        dv = (double)f;
      } else {
        const uint32_t b = enc_bf16((float)v);
        reinterpret_cast<uint16_t*>(rows)[r * D + i] = (uint16_t)b;
        dv = (double)dec_bf16(b);
      }
      res[i] = v - (double)sg * dv;
      fn += dv * dv;
    }
    fn = block_sum(fn, red);
    sig[r] = sg;
    fnorm[r] = sqrt(fn);
  }
  double ea = 0.0;
  for (int i = t; i < D; i += 256) ea += res[i] * res[i];
  ea = sqrt(block_sum(ea, red));
  double an = 0.0;
  for (int i = t; i < D; i += 256) an += avec[i] * avec[i];
  an = sqrt(block_sum(an, red));
  double wq = 0.0;
  for (int h = t; h < H; h += 256) wq += fabs(wd[h]) * sqrt(qn2[h]);
  wq = block_sum(wq, red);
  const double qs = HasQScale<C>::value ? (double)p.in.q_scale[qrow] : 1.0;
  // rounding margin: forward error of the fp32 dot products and sums in the
  // score and bound kernels (Higham, dot-product error gamma_n), with
  // u = 2^-22 (4x the fp32 unit roundoff) and n = d + H + 16; rho enters via
  // its separable upper bound.  The score kernels evaluate
  // sum_h w_h ReLU(x_h) as sum_h (w_h/2)|x_h| + qbar.k/2 with qbar held as a
  // few terms; their error and magnitude (unscaled) enter as well.
  const double u = 1.0 / 4194304.0;
  const double nn = (double)(D + H + 16);
  const double gam = nn * u / (1.0 - nn * u);
  double cq = 0.0, sf = 0.0;
  for (int r = 0; r < np; ++r) cq += cvec[r] * sqrt(qn2[prox[r]]);
  for (int r = np; r < 4; ++r) sf += sig[r] * fnorm[r];
  const double l_err = (double)p.lerr[(int64_t)qrow * 2], l_mag = (double)p.lerr[(int64_t)qrow * 2 + 1];
  const double margin = 2.0 * gam * (wq + cq + sf + rho_sep + 0.5 * l_mag) + ea + 0.5 * l_err;
  const float tau = p.tau[qrow];
  // Whether the bound pass is worth running for this query.  Skipping it
  // (every key survives) is always correct, so this is a cost decision: with
  // an optimistic certificate (rho replaced by its diagonal lower bound),
  // evaluate up to 64 keys sampled evenly from the bounded range; if at least
  // kSkipFrac of them would still survive, the query is scored densely.
  __shared__ int n_surv_s;
  if (t == 0) n_surv_s = 0;
  const int nb = gr.n_bounded;
  const int nsb = min(64, nb);
  bool skip = !(tau > -INFINITY) || (p.flags & DOSA_NO_PRUNE) || nsb == 0;
  if (!skip) {
    __syncthreads();
    for (int e = t; e < nsb * D; e += 256) {
      const int i = e / D, c = e % D;
      const int key = gr.bound_lo + (int)(((int64_t)i * nb) / nsb);
      const int64_t row = key_row(p.in, gr.key_base, gr.seq, key);
      kf[i * D + c] = k_elem<C>(p.in.k, row * D + c);
    }
    __syncthreads();
    if (t < nsb) {
      const int key = gr.bound_lo + (int)(((int64_t)t * nb) / nsb);
      const int64_t row = key_row(p.in, gr.key_base, gr.seq, key);
      const double ks = HasKScale<C>::value ? (double)p.in.k_scale[row] : 1.0;
      double ub = 0.0, ad = 0.0, kn2 = 0.0;
      for (int r = 0; r < np; ++r) {
        double xd = 0.0;
        for (int e = 0; e < D; ++e) xd += (double)qf[prox[r]][e] * (double)kf[t * D + e];
        ub += cvec[r] * fmax(xd, 0.0);
      }
      for (int e = 0; e < D; ++e) {
        ad += avec[e] * (double)kf[t * D + e];
        kn2 += (double)kf[t * D + e] * (double)kf[t * D + e];
      }
      ub = (ub - fmax(ad, 0.0) + rho_lo * sqrt(kn2)) * qs * ks;
      if (ub >= (double)tau) atomicAdd(&n_surv_s, 1);
    }
    __syncthreads();
    skip = (float)n_surv_s >= kSkipFrac * (float)nsb;
  }
  const bool hopeless = skip;
  double rho = rho_sep;
  const bool separable = (p.flags & DOSA_SEPARABLE_RHO) != 0;
  if (!hopeless && !separable) {
    // joint constant: rho^2 = sum_{h,j in O} w_h w_j max(0, <r_h, r_j>) from the head Gram matrix
    __syncthreads();
    for (int pr = t; pr < H * H; pr += 256) {
      const int h = pr / H, j = pr % H;
      if (j < h || !in_O(h) || !in_O(j)) continue;
      double s2 = 0.0;
      for (int i = 0; i < D; ++i) s2 += (double)qf[h][i] * (double)qf[j][i];
      G[h][j] = s2;
      G[j][h] = s2;
    }
    __syncthreads();
    double part = 0.0;
    for (int pr = t; pr < H * H; pr += 256) {
      const int h = pr / H, j = pr % H;
      if (!in_O(h) || !in_O(j)) continue;
      double r = G[h][j];
      for (int uu = 0; uu < np; ++uu) r -= alpha[h][uu] * gph[uu][j] + alpha[j][uu] * gph[uu][h];
      for (int uu = 0; uu < np; ++uu)
        for (int vv = 0; vv < np; ++vv) r += alpha[h][uu] * alpha[j][vv] * gph[uu][prox[vv]];
      part += wd[h] * wd[j] * fmax(r, 0.0);
    }
    rho = sqrt(fmax(block_sum(part, red), 0.0));
  }
  if (t == 0) {
    const double rho_p = (rho + margin) * qs;
    float* cf = p.coef + (int64_t)qrow * 8;
    for (int r = 0; r < 4; ++r) cf[r] = (r < np) ? (float)(cvec[r] * qs) : (float)(sig[r] * qs);
    cf[4] = (float)rho_p * 1.0000005f;
    cf[5] = tau;
    cf[6] = (float)np;
    cf[7] = hopeless ? 1.f : 0.f;
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
  for (int i = 0; i < 8; ++i) cf[i] = qok ? p.coef[(int64_t)qrow * 8 + i] : 0.f;
  const int npx = (int)cf[6];
  const bool hopeless = !qok || cf[7] != 0.f;
  const u64 hm = __ballot(qok && hopeless);
  const u64 okm = __ballot(qok);
  const bool all_hopeless = (hm == okm);
  const u64 nbounded = (u64)max(hi - lo, 0) * (u64)gr.nq;
  if (all_hopeless) {
    for (int wd = w0 + lane; wd < w1; wd += 64) {
      const int rem = n_all - wd * 64;
      mw[wd] = rem >= 64 ? ~0ull : ((1ull << rem) - 1ull);
    }
    if (p.stats != nullptr && lane == 0) {
      atomicAdd(&p.stats[2], nbounded);
      atomicAdd(&p.stats[3], nbounded);
      if (sp == 0) atomicAdd(&p.stats[7], 1ull);
    }
    if (p.debug_ub == nullptr) return;
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
  }
}

// ---------------------------------------------------------------------------
// compaction: one workgroup per tile, one wavefront per query group.  Each
// wavefront counts its group's union survivors (popcounts of the bitmask);
// if the tile's survivors are at least kDenseFrac of its bounded keys, the
// tile is flagged for the tiled kernel, which walks the bounded range
// directly.  Otherwise each wavefront turns its bitmask into an ascending key
// list: per-lane popcounts, a wavefront prefix sum for the write offsets,
// then each lane expands its word.
// ---------------------------------------------------------------------------
constexpr float kDenseFrac = 0.4f;

__global__ __launch_bounds__(512) void compact_kernel(const CompactLaunch p) {
  const int gi0 = blockIdx.x;
  const GroupInfo head = p.groups[gi0];
  if (head.tile_first != gi0) return;          // one workgroup per tile
  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  __shared__ uint32_t surv[8];
  __shared__ uint32_t bounded[8];
  const bool active = wave < head.tile_n;
  const int gi = gi0 + (active ? wave : 0);
  const GroupInfo gr = p.groups[gi];
  const int nw = active ? (gr.n_bounded + 63) / 64 : 0;
  const unsigned long long* mw = p.masks + (int64_t)gi * p.mask_words;
  uint32_t c = 0;
  for (int wd = lane; wd < nw; wd += 64) c += __popcll(mw[wd]);
  for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off, 64);
  if (lane == 0) {
    surv[wave] = active ? c : 0u;
    bounded[wave] = active ? (uint32_t)gr.n_bounded : 0u;
  }
  __syncthreads();
  uint64_t ts = 0, tb = 0;
  for (int i = 0; i < 8; ++i) {
    ts += surv[i];
    tb += bounded[i];
  }
  const bool dense = (float)ts >= kDenseFrac * (float)tb;
  if (!active) return;
  if (lane == 0) p.group_flags[gi] = dense ? 1 : 0;
  if (dense) {
    if (lane == 0) p.list_len[gi] = 0;
    return;
  }
  int32_t* out = p.lists + gr.list_off;
  uint32_t base = 0;
  for (int w0 = 0; w0 < nw; w0 += 64) {
    const int wd = w0 + lane;
    u64 m = (wd < nw) ? mw[wd] : 0ull;
    const uint32_t cnt = __popcll(m);
    uint32_t incl = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t v = __shfl_up(incl, off, 64);
      if (lane >= off) incl += v;
    }
    uint32_t at = base + incl - cnt;
    const int k0 = gr.bound_lo + 64 * wd;
    while (m) {
      const int b = __ffsll((long long)m) - 1;
      out[at++] = k0 + b;
      m &= m - 1ull;
    }
    base += __shfl(incl, 63, 64);
  }
  if (lane == 0) p.list_len[gi] = (int32_t)base;
}

__global__ void stats_add_kernel(unsigned long long* st, const dosa_stats add) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    const unsigned long long* a = reinterpret_cast<const unsigned long long*>(&add);
    for (int i = 0; i < 8; ++i)
      if (a[i]) atomicAdd(&st[i], a[i]);
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_stats_add(unsigned long long* stats, const unsigned long long* v, hipStream_t s) {
  dosa_stats a;
  static_assert(sizeof(dosa_stats) == 8 * sizeof(unsigned long long), "stats layout");
  memcpy(&a, v, sizeof(a));
  hipLaunchKernelGGL(stats_add_kernel, dim3(1), dim3(64), 0, s, stats, a);
  return hipGetLastError();
}

template <int C>
static hipError_t norms_c(int d, const NormLaunch& p, hipStream_t s) {
  const int nb = (int)((p.total_k + kNormKeys - 1) / kNormKeys);
  if (d == 64) hipLaunchKernelGGL((key_norm_kernel<C, 64>), dim3(nb), dim3(256), 0, s, p);
  else hipLaunchKernelGGL((key_norm_kernel<C, 128>), dim3(nb), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_key_norms(int combo, int d, const NormLaunch& p, hipStream_t s) {
  hipLaunchKernelGGL(fill_f32, dim3((p.batch + 255) / 256), dim3(256), 0, s, p.norm_min, p.batch, INFINITY);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.total_k == 0) return e;
  switch (combo) {
    case C_F32: return norms_c<C_F32>(d, p, s);
    case C_BF16: return norms_c<C_BF16>(d, p, s);
    default: return norms_c<C_FP8>(d, p, s);   // fp8 keys (both fp8 combos)
  }
}

template <int C, int H, int D>
static hipError_t plan_t(const PlanLaunch& p, hipStream_t s) {
  hipLaunchKernelGGL((plan_kernel<C, H, D>), dim3(p.n_groups, 4), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int C>
static hipError_t plan_c(int H, int d, const PlanLaunch& p, hipStream_t s) {
#define DOSA_HD(HH, DD) \
  if (H == HH && d == DD) return plan_t<C, HH, DD>(p, s);
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

hipError_t launch_compact(const CompactLaunch& p, hipStream_t s) {
  if (p.n_groups == 0) return hipSuccess;
  hipLaunchKernelGGL(compact_kernel, dim3(p.n_groups), dim3(512), 0, s, p);
  return hipGetLastError();
}

}  // namespace dosa
