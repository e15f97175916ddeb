// Verification of the scored trees.
//
// RheoSampling, Section 3.3 Algorithm 1 (RheoVerification), applied layer by
// layer from the root: a sampled candidate u_s is accepted with probability
// min(1, p(u_s) / q~(u_s)); on rejection the residual r = norm(max(0, p - q~))
// replaces p; the remaining candidates are tested one by one against r, each
// rejection zeroing that token and renormalising; if all are rejected the
// output token is drawn from r.  Without a sampled candidate r = p, which is
// the sequential rejection of Progressive Tree Drafting (Section 3.2, Appendix
// E / F).  p = softmax(logits / T) (RheoSampling Section 5.4).
//
// vocab_kernel (one 1024-thread workgroup per node) reads the node's logits
// row once into registers (bf16: 19 x 16 bytes per thread covers 155648
// tokens) and its draft row once, and produces M = max l/T, S = sum exp(l/T-M),
// Z = sum (p - q~)+ and the token the final draw would give if the walk ended
// at this node.  Sums run per lane in fp32 and across lanes in fp64.
// walk_kernel (one wave per sequence) then takes the accept/reject decisions
// in fp64 from these statistics and point reads of the logits / draft rows.
#include "tav_internal.h"

namespace tav {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWaves = kVocabThreads / 64;

template <typename LT>
__device__ inline float to_f(LT x);
template <>
__device__ inline float to_f<uint16_t>(uint16_t x) { return __uint_as_float(((uint32_t)x) << 16); }
template <>
__device__ inline float to_f<float>(float x) { return x; }

// Element e (compile-time after unrolling) of a 16-byte unit of logits.
template <typename LT>
__device__ inline float unit_elem(const uint4& u, int e);
template <>
__device__ inline float unit_elem<uint16_t>(const uint4& u, int e) {
  const uint32_t w = (e >> 1) == 0 ? u.x : (e >> 1) == 1 ? u.y : (e >> 1) == 2 ? u.z : u.w;
  return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
}
template <>
__device__ inline float unit_elem<float>(const uint4& u, int e) {
  return __uint_as_float(e == 0 ? u.x : e == 1 ? u.y : e == 2 ? u.z : u.w);
}

template <typename LT>
__device__ inline float logit_at(const void* logits, size_t idx) {
  return to_f<LT>(((const LT*)logits)[idx]);
}

__device__ inline double wave_sum_d(double x) {
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) x += __shfl_xor(x, d);
  return x;
}
__device__ inline float wave_sum_f(float x) {
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) x += __shfl_xor(x, d);
  return x;
}
__device__ inline float wave_max_f(float x) {
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) x = fmaxf(x, __shfl_xor(x, d));
  return x;
}

template <typename LT>
__global__ __launch_bounds__(kVocabThreads) void vocab_kernel(VocabArgs a) {
  constexpr int EPU = 16 / sizeof(LT);  // logits per 16-byte unit
  constexpr int SLOTS = kVocabSlots;
  constexpr int CHUNK = 64 * EPU;       // elements of one (slot, wave) chunk
  __shared__ float red_f[kWaves];
  __shared__ double red_d[kWaves];
  __shared__ float csum[SLOTS * kWaves];
  __shared__ int det_tok[kMaxChildren];
  __shared__ int n_det, has_sampled, n_kids;
  __shared__ int pick_chunk;
  __shared__ float pick_rem;
  __shared__ int pick_token;

  const int v = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int V = a.V;
  int lo = 0, hi = a.B;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (a.node_offsets[mid] <= v) lo = mid; else hi = mid;
  }
  const int b = lo;
  const int s0 = a.node_offsets[b];
  const int n = a.node_offsets[b + 1] - s0;
  const int local = v - s0;
  if (tid == 0) { n_det = 0; has_sampled = 0; n_kids = 0; pick_chunk = -1; pick_token = -1; }
  __syncthreads();
  // children of this node: their tokens (deterministic ones are zeroed in the final draw)
  for (int j = tid + 1; j < n; j += kVocabThreads) {
    if (a.parent[s0 + j] == local) {
      atomicAdd(&n_kids, 1);
      if (a.sampled[s0 + j]) {
        atomicAdd(&has_sampled, 1);
      } else {
        const int k = atomicAdd(&n_det, 1);
        if (k < kMaxChildren) det_tok[k] = a.token[s0 + j];
      }
    }
  }
  __syncthreads();
  const int ndet = min(n_det, kMaxChildren);
  if (tid == 0 && n_kids > kMaxChildren) atomicOr(a.status, (uint32_t)TAV_DEV_TOO_MANY_CHILDREN);
  const int dr = a.draft_row[v];
  const bool use_draft = has_sampled > 0 && dr >= 0 && dr < a.R;
  const float Tb = a.temperature[b];
  if (!(Tb > 0.f && Tb < INFINITY)) {
    if (tid == 0) atomicOr(a.status, (uint32_t)TAV_DEV_BAD_TEMPERATURE);
  }
  const float invT = 1.f / Tb;

  // ---- pass 1: the whole row into registers, max of l/T ----
  const LT* row = (const LT*)a.logits + (size_t)v * V;
  uint4 r[SLOTS];
  float mx = -INFINITY;
  int bad = 0;
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) {
    const int e0 = (i * kVocabThreads + tid) * EPU;
    r[i] = e0 < V ? *(const uint4*)(row + e0) : make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) {
    const int e0 = (i * kVocabThreads + tid) * EPU;
    if (e0 < V) {
#pragma unroll
      for (int e = 0; e < EPU; ++e) {
        const float z = unit_elem<LT>(r[i], e) * invT;
        bad |= (z != z) | (z == INFINITY);
        mx = fmaxf(mx, z);
      }
    }
  }
  if (__syncthreads_or(bad) && tid == 0) atomicOr(a.status, (uint32_t)TAV_DEV_NONFINITE_LOGITS);
  mx = wave_max_f(mx);
  if (lane == 0) red_f[wave] = mx;
  __syncthreads();
  float M = red_f[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) M = fmaxf(M, red_f[w]);
  if (M == -INFINITY) {  // every logit is -inf: the row has no mass
    if (tid == 0) atomicOr(a.status, (uint32_t)TAV_DEV_NONFINITE_LOGITS);
    M = 0.f;
  }
  const float Ml2 = M * kLog2e;

  double sl = 0.0;
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) {
    const int e0 = (i * kVocabThreads + tid) * EPU;
    if (e0 < V) {
      float su = 0.f;
#pragma unroll
      for (int e = 0; e < EPU; ++e) su += __builtin_amdgcn_exp2f(unit_elem<LT>(r[i], e) * invT * kLog2e - Ml2);
      sl += (double)su;
    }
  }
  sl = wave_sum_d(sl);
  if (lane == 0) red_d[wave] = sl;
  __syncthreads();
  double S = 0.0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) S += red_d[w];
  const float invS = (float)(1.0 / S);
  __syncthreads();

  // ---- pass 2: final-draw weights w = (p - q~)+ or p, chunk sums, Z ----
  const float* drow = use_draft ? a.draft + (size_t)dr * V : nullptr;
  double zl = 0.0;
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) {
    const int e0 = (i * kVocabThreads + tid) * EPU;
    float ws = 0.f;
    if (e0 < V) {
      float q[EPU];
      if (use_draft) {
#pragma unroll
        for (int h = 0; h < EPU / 4; ++h) {
          const float4 t = *(const float4*)(drow + e0 + 4 * h);
          q[4 * h + 0] = t.x; q[4 * h + 1] = t.y; q[4 * h + 2] = t.z; q[4 * h + 3] = t.w;
        }
      }
#pragma unroll
      for (int e = 0; e < EPU; ++e) {
        const float p = __builtin_amdgcn_exp2f(unit_elem<LT>(r[i], e) * invT * kLog2e - Ml2) * invS;
        ws += use_draft ? fmaxf(0.f, p - q[e]) : p;
      }
    }
    zl += (double)ws;
    ws = wave_sum_f(ws);
    if (lane == 0) csum[i * kWaves + wave] = ws;
  }
  zl = wave_sum_d(zl);
  if (lane == 0) red_d[wave] = zl;
  __syncthreads();
  double Zt = 0.0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) Zt += red_d[w];
  const float Z = use_draft ? (float)Zt : 0.f;

  // remove the deterministic children's tokens from the chunk sums
  auto weight_at = [&](int tok) -> float {
    const float z = logit_at<LT>(a.logits, (size_t)v * V + tok) * invT;
    const float p = __builtin_amdgcn_exp2f(z * kLog2e - Ml2) * invS;
    return use_draft ? fmaxf(0.f, p - drow[tok]) : p;
  };
  if (tid < ndet) {
    const int tok = det_tok[tid];
    if (tok >= 0 && tok < V) {
      const int unit = tok / EPU;
      atomicAdd(&csum[(unit / kVocabThreads) * kWaves + (unit % kVocabThreads) / 64], -weight_at(tok));
    }
  }
  __syncthreads();
  if (tid == 0) {
    double W = 0.0;
    for (int c = 0; c < SLOTS * kWaves; ++c) W += (double)fmaxf(csum[c], 0.f);
    if (W > 0.0) {
      const double target = (double)a.uniforms[(size_t)v * 2 + 1] * W;
      double cum = 0.0;
      int c = 0, last = -1;
      for (; c < SLOTS * kWaves; ++c) {
        const double cs = (double)fmaxf(csum[c], 0.f);
        if (cs > 0.0) last = c;
        if (cum + cs > target && cs > 0.0) break;
        cum += cs;
      }
      if (c == SLOTS * kWaves) {  // rounding put the target past the total: last chunk with mass
        c = last;
        cum -= (double)fmaxf(csum[c], 0.f);
      }
      pick_chunk = c;
      pick_rem = (float)(target - cum);
    }
  }
  __syncthreads();
  const int pc = pick_chunk;
  if (pc >= 0 && wave == pc % kWaves) {
    const int slot = pc / kWaves;
    // this wave holds the chunk's logits in registers slot `slot`
    float wv[EPU];
    float lsum = 0.f;
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
      if (i == slot) {
        const int e0 = (i * kVocabThreads + tid) * EPU;
#pragma unroll
        for (int e = 0; e < EPU; ++e) {
          float w = 0.f;
          if (e0 + e < V) {
            const float p = __builtin_amdgcn_exp2f(unit_elem<LT>(r[i], e) * invT * kLog2e - Ml2) * invS;
            w = use_draft ? fmaxf(0.f, p - drow[e0 + e]) : p;
            for (int k = 0; k < ndet; ++k)
              if (det_tok[k] == e0 + e) w = 0.f;
          }
          wv[e] = w;
          lsum += w;
        }
      }
    }
    // inclusive scan of the lanes' sums
    float incl = lsum;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const float y = __shfl_up(incl, d, 64);
      if (lane >= d) incl += y;
    }
    const float rem = pick_rem;
    const unsigned long long hit = __ballot(incl > rem && lsum > 0.f);
    int chosen_lane;
    if (hit) {
      chosen_lane = __ffsll((long long)hit) - 1;
    } else {  // rounding: the last lane holding mass
      const unsigned long long has = __ballot(lsum > 0.f);
      chosen_lane = has ? 63 - __clzll((long long)has) : -1;
    }
    if (lane == chosen_lane) {
      float cum = incl - lsum;
      int tok = -1, lastpos = -1;
      const int e0 = (slot * kVocabThreads + tid) * EPU;
#pragma unroll
      for (int e = 0; e < EPU; ++e) {
        if (wv[e] > 0.f) lastpos = e0 + e;
        cum += wv[e];
        if (tok < 0 && wv[e] > 0.f && cum > rem) tok = e0 + e;
      }
      pick_token = tok >= 0 ? tok : lastpos;
    }
  }
  __syncthreads();
  if (tid == 0) {
    a.stats[(size_t)v * 3 + 0] = M;
    a.stats[(size_t)v * 3 + 1] = (float)S;
    a.stats[(size_t)v * 3 + 2] = Z;
    a.term_token[v] = pick_token;
  }
}

// One wave per sequence: the layer-by-layer walk (decisions in fp64).
__global__ __launch_bounds__(64) void walk_kernel(WalkArgs a) {
  __shared__ int kids[kMaxChildren];
  __shared__ int nk_s;
  const int b = blockIdx.x, lane = threadIdx.x;
  const int s0 = a.node_offsets[b];
  const int n = a.node_offsets[b + 1] - s0;
  const int V = a.V;
  const double T = (double)a.temperature[b];
  const float invT = 1.f / a.temperature[b];
  for (int j = lane; j < n; j += 64) a.node_status[s0 + j] = 0;
  for (int j = lane; j < a.max_path; j += 64) a.path[(size_t)b * a.max_path + j] = -1;
  __syncthreads();
  uint32_t err = 0;
  int plen = 1, v = 0, bonus = -1;
  if (lane == 0) {
    a.node_status[s0] = 1;
    if (a.max_path > 0) a.path[(size_t)b * a.max_path] = 0;
    else err |= TAV_DEV_PATH_OVERFLOW;
  }
  (void)T;
  for (int iter = 0; iter < n && !err; ++iter) {
    // children of v in ascending id
    if (lane == 0) nk_s = 0;
    __syncthreads();
    for (int base = 1; base < n; base += 64) {
      const int j = base + lane;
      const bool is_kid = j < n && a.parent[s0 + j] == v;
      const unsigned long long m = __ballot(is_kid);
      const int before = __popcll(m & ((1ull << lane) - 1ull));
      const int cnt = __popcll(m);
      const int at = nk_s;
      if (is_kid && at + before < kMaxChildren) kids[at + before] = j;
      __syncthreads();
      if (lane == 0) nk_s = at + cnt;
      __syncthreads();
    }
    const int nk_all = nk_s;
    if (nk_all > kMaxChildren) { err |= TAV_DEV_TOO_MANY_CHILDREN; break; }
    const int nk = nk_all;
    int next = -1;
    if (lane == 0) {
      const size_t lrow = (size_t)(s0 + v) * V;
      const double Mv = (double)a.stats[(size_t)(s0 + v) * 3 + 0];
      const double Sv = (double)a.stats[(size_t)(s0 + v) * 3 + 1];
      const double Zv = (double)a.stats[(size_t)(s0 + v) * 3 + 2];
      auto p_at = [&](int tok) -> double {
        const float l = a.logits_bf16 ? logit_at<uint16_t>(a.logits, lrow + tok)
                                      : logit_at<float>(a.logits, lrow + tok);
        return exp((double)(l * invT) - Mv) / Sv;
      };
      int s = -1, nsamp = 0;
      for (int k = 0; k < nk; ++k) {
        const int c = kids[k];
        const int tok = a.token[s0 + c];
        if (tok < 0 || tok >= V) err |= TAV_DEV_BAD_TOKEN;
        if (a.sampled[s0 + c]) { s = c; ++nsamp; }
        for (int k2 = 0; k2 < k; ++k2)
          if (a.token[s0 + kids[k2]] == tok) err |= TAV_DEV_DUP_SIBLING_TOKEN;
      }
      if (nsamp > 1) err |= TAV_DEV_MULTI_SAMPLED;
      const int dr = a.draft_row[s0 + v];
      const float* q = nullptr;
      if (s >= 0) {
        if (dr < 0 || dr >= a.R) err |= TAV_DEV_NO_DRAFT;
        else q = a.draft + (size_t)dr * V;
      }
      if (!err) {
        bool resid = false;
        if (s >= 0) {
          const int ts = a.token[s0 + s];
          const double qs = (double)q[ts];
          if (!(qs > 0.0)) {
            err |= TAV_DEV_ZERO_DRAFT_MASS;
          } else {
            const double ratio = fmin(1.0, p_at(ts) / qs);
            if ((double)a.uniforms[(size_t)(s0 + s) * 2] <= ratio) {
              next = s;
            } else {
              a.node_status[s0 + s] = 2;
              resid = true;
            }
          }
        }
        if (!err && next < 0) {
          double rej = 0.0;
          for (int k = 0; k < nk && next < 0; ++k) {
            const int c = kids[k];
            if (c == s) continue;
            const int tok = a.token[s0 + c];
            const double p = p_at(tok);
            const double r0 = resid ? (Zv > 0.0 ? fmax(0.0, p - (double)q[tok]) / Zv : 0.0) : p;
            const double rem = 1.0 - rej;
            const double rc = rem > 0.0 ? r0 / rem : 0.0;
            if ((double)a.uniforms[(size_t)(s0 + c) * 2] <= rc) {
              next = c;
            } else {
              a.node_status[s0 + c] = 2;
              rej += r0;
            }
          }
        }
        if (!err && next >= 0) {
          a.node_status[s0 + next] = 1;
          if (plen >= a.max_path) err |= TAV_DEV_PATH_OVERFLOW;
          else a.path[(size_t)b * a.max_path + plen] = next;
          ++plen;
        } else if (!err) {
          bonus = a.term_token[s0 + v];
          if (bonus < 0) err |= TAV_DEV_EMPTY_RESIDUAL;
        }
      }
    }
    next = __shfl(next, 0);
    err = __shfl(err, 0);
    if (next < 0) break;
    v = next;
  }
  if (lane == 0) {
    if (err) atomicOr(a.status, err);
    a.path_len[b] = err ? 0 : min(plen, a.max_path);
    a.bonus[b] = err ? -1 : bonus;
  }
}

}  // namespace

hipError_t launch_vocab(const VocabArgs& a, bool bf16_logits, hipStream_t s) {
  if (a.N == 0) return hipSuccess;
  if (bf16_logits) vocab_kernel<uint16_t><<<a.N, kVocabThreads, 0, s>>>(a);
  else vocab_kernel<float><<<a.N, kVocabThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_walk(const WalkArgs& a, hipStream_t s) {
  walk_kernel<<<a.B, 64, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace tav
