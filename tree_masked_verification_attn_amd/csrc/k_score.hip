// Per-token scores of sampled tokens from the unprocessed logits, one pass over each row.
//
// PreSTO, Appendix D.3 (the patched sampler): for the sampled token x of a row the forward pass
// returns log q_tau(x) from the processed logits (temperature tau: q_tau = softmax(l / tau)), the
// base-model log p0(x) from the unprocessed copy (p0 = softmax(l)), and the full-vocabulary
// entropy of p0 in natural log, H = -sum p0 log p0 -- the per-token inputs of the log-acceptance
// (PreSTO Section 3.2, Example 3).  Progressive Tree Drafting, Section 3.2: under greedy decoding
// a node's verification token is its highest-probability prediction (here: the argmax of the
// logits, smallest id among equal maxima), also returned.
//
// One 512-thread workgroup per row (persistent over rows).  Each step of 32 KB is read with the
// next step's loads in flight; a thread keeps, against its running maximum m (log2 units):
//   s1 = sum 2^(t), s2 = sum 2^(t) * t, st = sum 2^(t / tau),    t = (l - m) log2e,
// rescaled when m rises (once per step, from the step's maximum), so that
//   log S1 = ln2 (m + log2 s1),  sum p0 (l - M) = ln2 s2 / s1,  H = log S1 - that,
// and each thread notes the unit of its first largest logit (per-unit maxima, compared only in steps
// whose maximum beats its best), re-reading that one unit at the end of the row for the position.
// When 1 / tau is a whole number up to 8 (PreSTO's tau = 1 / alpha), 2^(t / tau) = (2^t)^(1 / tau)
// by squaring (a kernel compiled per exponent).  The units of a partial last step past the row's
// end are set to -inf, so the element loops carry no bounds checks.
#include "tav_internal.h"

namespace tav {
namespace {

constexpr int kScoreThreads = 512;
constexpr int kScoreUnits = 4;                       // sixteen-byte units per thread and step
constexpr int kScoreStep = kScoreThreads * kScoreUnits;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename LT>
__device__ inline float elem(const uint4& u, int e);
template <>
__device__ inline float elem<uint16_t>(const uint4& u, int e) {
  const uint32_t w = (e >> 1) == 0 ? u.x : (e >> 1) == 1 ? u.y : (e >> 1) == 2 ? u.z : u.w;
  return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
}
template <>
__device__ inline float elem<float>(const uint4& u, int e) {
  return __uint_as_float(e == 0 ? u.x : e == 1 ? u.y : e == 2 ? u.z : u.w);
}

// x^K for a whole K in 1..8, by squaring (compile-time K)
template <int K>
__device__ inline float ipow(float x) {
  const float x2 = x * x, x4 = x2 * x2;
  if constexpr (K == 1) return x;
  else if constexpr (K == 2) return x2;
  else if constexpr (K == 3) return x2 * x;
  else if constexpr (K == 4) return x4;
  else if constexpr (K == 5) return x4 * x;
  else if constexpr (K == 6) return x4 * x2;
  else if constexpr (K == 7) return x4 * x2 * x;
  else return x4 * x4;
}

// 2^(t / tau): by squaring when 1 / tau is the whole number KP, else a second exponential
template <int KP>
__device__ inline float pow_tau(float x, float t, float inv_tau) {
  if constexpr (KP > 0) return ipow<KP>(x);
  else return __builtin_amdgcn_exp2f(t * inv_tau);
}

// The units of a partial last step past the row's end: set to -inf (no mass, never the maximum),
// so the arithmetic needs no per-element bounds checks.
template <typename LT>
__device__ inline uint4 neg_inf_unit();
template <>
__device__ inline uint4 neg_inf_unit<uint16_t>() { return make_uint4(0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u); }
template <>
__device__ inline uint4 neg_inf_unit<float>() { return make_uint4(0xFF800000u, 0xFF800000u, 0xFF800000u, 0xFF800000u); }

template <typename LT, int KP>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(ScoreArgs a) {
  constexpr int EPU = 16 / sizeof(LT);
  __shared__ double red[kScoreThreads / 64][4];
  __shared__ float bred[kScoreThreads / 64];
  __shared__ int ired[kScoreThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int V = a.V, nunits = V / EPU;
  const int nsteps = (nunits + kScoreStep - 1) / kScoreStep;
  const float inv_tau = 1.f / a.tau;
  for (int row = blockIdx.x; row < a.N; row += gridDim.x) {
    const LT* lr = (const LT*)a.logits + (size_t)row * V;
    auto load = [&](uint4 (&r)[kScoreUnits], int s) __attribute__((always_inline)) {
#pragma unroll
      for (int k = 0; k < kScoreUnits; ++k) {
        const int u = s * kScoreStep + k * kScoreThreads + tid;
        r[k] = *(const uint4*)(lr + (size_t)(u < nunits ? u : 0) * EPU);
      }
    };
    uint4 cur[kScoreUnits];
    load(cur, 0);
    float m = -INFINITY, s1 = 0.f, s2 = 0.f, st = 0.f;   // m in log2 units
    float best = -INFINITY;
    int bu = -1;   // the unit holding this thread's first largest logit
    for (int s = 0; s < nsteps; ++s) {
      uint4 nxt[kScoreUnits];
      if (s + 1 < nsteps) load(nxt, s + 1);
      if ((s + 1) * kScoreStep > nunits) {   // the partial last step
#pragma unroll
        for (int k = 0; k < kScoreUnits; ++k)
          if (s * kScoreStep + k * kScoreThreads + tid >= nunits) cur[k] = neg_inf_unit<LT>();
      }
      float um[kScoreUnits];
#pragma unroll
      for (int k = 0; k < kScoreUnits; ++k) {
        um[k] = elem<LT>(cur[k], 0);
#pragma unroll
        for (int e = 1; e < EPU; ++e) um[k] = fmaxf(um[k], elem<LT>(cur[k], e));
      }
      float mx = um[0];
#pragma unroll
      for (int k = 1; k < kScoreUnits; ++k) mx = fmaxf(mx, um[k]);
      if (mx > best) {   // a new best: its first unit (positions rise with (step, unit) in a thread)
        best = mx;
        int kk = kScoreUnits - 1;
#pragma unroll
        for (int k = kScoreUnits - 2; k >= 0; --k) kk = um[k] == mx ? k : kk;
        bu = s * kScoreStep + kk * kScoreThreads + tid;
      }
      const float m2 = mx * kLog2e;
      if (m2 > m) {   // rescale the running sums to the new maximum
        if (m != -INFINITY) {
          const float d = m - m2;   // < 0
          const float f = __builtin_amdgcn_exp2f(d);
          s2 = f * (s2 + s1 * d);
          s1 *= f;
          st *= pow_tau<KP>(f, d, inv_tau);
        }
        m = m2;
      }
      if (m != -INFINITY) {
#pragma unroll
        for (int k = 0; k < kScoreUnits; ++k) {
#pragma unroll
          for (int e = 0; e < EPU; ++e) {
            // t <= 0 (a NaN logit makes s1 NaN, which is reported); a -inf logit gives 2^t = 0,
            // and its t is clamped in the product so that 0 * -inf does not appear
            const float t = fmaf(elem<LT>(cur[k], e), kLog2e, -m);
            const float x = __builtin_amdgcn_exp2f(t);
            s1 += x;
            s2 = fmaf(x, fmaxf(t, -1.0e30f), s2);
            st += pow_tau<KP>(x, t, inv_tau);
          }
        }
      }
      if (s + 1 < nsteps) {
#pragma unroll
        for (int k = 0; k < kScoreUnits; ++k) cur[k] = nxt[k];
      }
    }
    // the position of this thread's best inside its unit (one re-read of that unit, from the cache;
    // issued now, used after the sums' reductions)
    uint4 bunit = make_uint4(0u, 0u, 0u, 0u);
    if (bu >= 0) bunit = *(const uint4*)(lr + (size_t)bu * EPU);
    // the block's maximum, then every thread's sums moved to it and added in fp64
    float wm = m;
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) wm = fmaxf(wm, __shfl_xor(wm, d));
    if (lane == 0) bred[wave] = wm;
    __syncthreads();
    float M2 = -INFINITY;
#pragma unroll
    for (int w = 0; w < kScoreThreads / 64; ++w) M2 = fmaxf(M2, bred[w]);
    double d1 = 0.0, d2 = 0.0, dt = 0.0;
    if (m != -INFINITY) {
      const double d = (double)m - (double)M2;   // <= 0
      const double f = exp2(d);
      d1 = f * (double)s1;
      d2 = f * ((double)s2 + (double)s1 * d);
      dt = exp2(d * (double)inv_tau) * (double)st;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      d1 += __shfl_xor(d1, o);
      d2 += __shfl_xor(d2, o);
      dt += __shfl_xor(dt, o);
    }
    int bi = -1;
    if (bu >= 0) {
      int ee = EPU - 1;
#pragma unroll
      for (int e = EPU - 2; e >= 0; --e) ee = elem<LT>(bunit, e) == best ? e : ee;
      bi = bu * EPU + ee;
    }
    float wb = best;
    int wi = bi;
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) {
      const float ob = __shfl_xor(wb, d);
      const int oi = __shfl_xor(wi, d);
      if (ob > wb || (ob == wb && (unsigned)oi < (unsigned)wi)) {
        wb = ob;
        wi = oi;
      }
    }
    if (lane == 0) {
      red[wave][0] = d1;
      red[wave][1] = d2;
      red[wave][2] = dt;
      red[wave][3] = (double)wb;
      ired[wave] = wi;
    }
    __syncthreads();
    if (tid == 0) {
      double S1 = 0.0, S2 = 0.0, ST = 0.0;
      float bb = -INFINITY;
      int A = -1;
      for (int w = 0; w < kScoreThreads / 64; ++w) {
        S1 += red[w][0];
        S2 += red[w][1];
        ST += red[w][2];
        const float ob = (float)red[w][3];
        const int oi = ired[w];
        if (ob > bb || (ob == bb && (unsigned)oi < (unsigned)A)) {
          bb = ob;
          A = oi;
        }
      }
      uint32_t err = 0;
      const double Mn = (double)M2 * (double)kLn2;          // max l (natural units)
      const double lnS1 = log(S1);                          // log sum exp(l - M)
      if (!(S1 >= 1.0 && S1 < INFINITY) || !(ST > 0.0 && ST < INFINITY) || M2 == -INFINITY)
        err |= TAV_DEV_NONFINITE_LOGITS;
      float lp0 = NAN, lq = NAN;
      if (a.token) {
        const int tok = a.token[row];
        if (tok < 0 || tok >= V) {
          err |= TAV_DEV_BAD_TOKEN;
        } else {
          const double x = (double)(sizeof(LT) == 2
                                        ? __uint_as_float(((uint32_t)((const uint16_t*)lr)[tok]) << 16)
                                        : ((const float*)lr)[tok]);
          lp0 = (float)(x - Mn - lnS1);
          lq = (float)((x - Mn) * (double)inv_tau - log(ST));
        }
      }
      if (err) {
        lp0 = lq = NAN;
        atomicOr(a.status, err);
      }
      if (a.lp0) a.lp0[row] = lp0;
      if (a.lq) a.lq[row] = lq;
      if (a.ent) a.ent[row] = err ? NAN : (float)(lnS1 - (S2 / S1) * (double)kLn2);
      if (a.argmax) a.argmax[row] = M2 == -INFINITY ? -1 : A;
    }
    __syncthreads();   // red / bred reused by the next row
  }
}

template <typename LT, int KP>
hipError_t launch_score_k(const ScoreArgs& a, int num_cus, hipStream_t s) {
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, score_kernel<LT, KP>, kScoreThreads, 0);
  if (e != hipSuccess) return e;
  if (per_cu < 1) per_cu = 1;
  const int grid = a.N < per_cu * num_cus ? a.N : per_cu * num_cus;
  score_kernel<LT, KP><<<grid, kScoreThreads, 0, s>>>(a);
  return hipGetLastError();
}

template <typename LT>
hipError_t launch_score_t(const ScoreArgs& a, int num_cus, hipStream_t s) {
  switch (a.kpow) {
    case 1: return launch_score_k<LT, 1>(a, num_cus, s);
    case 2: return launch_score_k<LT, 2>(a, num_cus, s);
    case 3: return launch_score_k<LT, 3>(a, num_cus, s);
    case 4: return launch_score_k<LT, 4>(a, num_cus, s);
    case 5: return launch_score_k<LT, 5>(a, num_cus, s);
    case 6: return launch_score_k<LT, 6>(a, num_cus, s);
    case 7: return launch_score_k<LT, 7>(a, num_cus, s);
    case 8: return launch_score_k<LT, 8>(a, num_cus, s);
    default: return launch_score_k<LT, 0>(a, num_cus, s);
  }
}

}  // namespace

hipError_t launch_score(const ScoreArgs& a, bool bf16, int num_cus, hipStream_t s) {
  if (a.N == 0) return hipSuccess;
  return bf16 ? launch_score_t<uint16_t>(a, num_cus, s) : launch_score_t<float>(a, num_cus, s);
}

}  // namespace tav
