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
// and the argmax is located only in steps whose maximum beats the best so far.  When 1 / tau is
// a whole number up to 8 (PreSTO's tau = 1 / alpha), 2^(t / tau) = (2^t)^(1 / tau) by squaring.
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

// x^k for a whole k in 1..8 (k = 0: unused)
__device__ inline float ipow(float x, int k) {
  const float x2 = x * x, x4 = x2 * x2;
  float r = (k & 1) ? x : 1.f;
  if (k & 2) r *= x2;
  if (k & 4) r *= x4;
  if (k & 8) r *= x4 * x4;
  return r;
}

template <typename LT>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(ScoreArgs a) {
  constexpr int EPU = 16 / sizeof(LT);
  __shared__ double red[kScoreThreads / 64][4];
  __shared__ float bred[kScoreThreads / 64];
  __shared__ int ired[kScoreThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int V = a.V, nunits = V / EPU;
  const int nsteps = (nunits + kScoreStep - 1) / kScoreStep;
  const float inv_tau = 1.f / a.tau;
  const int kpow = a.kpow;                      // 1 / tau when it is a whole number in 1..8, else 0
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
    int bi = -1;
    for (int s = 0; s < nsteps; ++s) {
      uint4 nxt[kScoreUnits];
      if (s + 1 < nsteps) load(nxt, s + 1);
      float mx = -INFINITY;
#pragma unroll
      for (int k = 0; k < kScoreUnits; ++k)
        if (s * kScoreStep + k * kScoreThreads + tid < nunits) {
#pragma unroll
          for (int e = 0; e < EPU; ++e) mx = fmaxf(mx, elem<LT>(cur[k], e));
        }
      if (mx > best) {   // the step holds a new best: its first position (positions rise in a thread)
        best = mx;
        bool found = false;
#pragma unroll
        for (int k = 0; k < kScoreUnits; ++k) {
          const int u = s * kScoreStep + k * kScoreThreads + tid;
#pragma unroll
          for (int e = 0; e < EPU; ++e)
            if (!found && u < nunits && elem<LT>(cur[k], e) == mx) {
              bi = u * EPU + e;
              found = true;
            }
        }
      }
      const float m2 = mx * kLog2e;
      if (m2 > m) {   // rescale the running sums to the new maximum
        if (m != -INFINITY) {
          const float d = m - m2;   // < 0
          const float f = __builtin_amdgcn_exp2f(d);
          s2 = f * (s2 + s1 * d);
          s1 *= f;
          st *= kpow ? ipow(f, kpow) : __builtin_amdgcn_exp2f(d * inv_tau);
        }
        m = m2;
      }
      if (m != -INFINITY) {
#pragma unroll
        for (int k = 0; k < kScoreUnits; ++k)
          if (s * kScoreStep + k * kScoreThreads + tid < nunits) {
#pragma unroll
            for (int e = 0; e < EPU; ++e) {
              // t <= 0 (a NaN logit makes s1 NaN, which is reported); a -inf logit gives 2^t = 0,
              // and its t is clamped in the product so that 0 * -inf does not appear
              const float t = fmaf(elem<LT>(cur[k], e), kLog2e, -m);
              const float x = __builtin_amdgcn_exp2f(t);
              s1 += x;
              s2 = fmaf(x, fmaxf(t, -1.0e30f), s2);
              st += kpow ? ipow(x, kpow) : __builtin_amdgcn_exp2f(t * inv_tau);
            }
          }
      }
      if (s + 1 < nsteps) {
#pragma unroll
        for (int k = 0; k < kScoreUnits; ++k) cur[k] = nxt[k];
      }
    }
    // the block's maximum, then every thread's sums moved to it and added in fp64
    float wm = m;
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) wm = fmaxf(wm, __shfl_xor(wm, d));
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
      bred[wave] = wm;
      ired[wave] = wi;
      red[wave][3] = (double)wb;
    }
    __syncthreads();
    float M2 = -INFINITY;
#pragma unroll
    for (int w = 0; w < kScoreThreads / 64; ++w) M2 = fmaxf(M2, bred[w]);
    float bb = -INFINITY;
    int A = -1;
#pragma unroll
    for (int w = 0; w < kScoreThreads / 64; ++w) {
      const float ob = (float)red[w][3];
      const int oi = ired[w];
      if (ob > bb || (ob == bb && (unsigned)oi < (unsigned)A)) {
        bb = ob;
        A = oi;
      }
    }
    __syncthreads();   // red is reused below
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
    if (lane == 0) {
      red[wave][0] = d1;
      red[wave][1] = d2;
      red[wave][2] = dt;
    }
    __syncthreads();
    if (tid == 0) {
      double S1 = 0.0, S2 = 0.0, ST = 0.0;
      for (int w = 0; w < kScoreThreads / 64; ++w) {
        S1 += red[w][0];
        S2 += red[w][1];
        ST += red[w][2];
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

template <typename LT>
hipError_t launch_score_t(const ScoreArgs& a, int num_cus, hipStream_t s) {
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, score_kernel<LT>, kScoreThreads, 0);
  if (e != hipSuccess) return e;
  if (per_cu < 1) per_cu = 1;
  const int grid = a.N < per_cu * num_cus ? a.N : per_cu * num_cus;
  score_kernel<LT><<<grid, kScoreThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_score(const ScoreArgs& a, bool bf16, int num_cus, hipStream_t s) {
  if (a.N == 0) return hipSuccess;
  return bf16 ? launch_score_t<uint16_t>(a, num_cus, s) : launch_score_t<float>(a, num_cus, s);
}

}  // namespace tav
