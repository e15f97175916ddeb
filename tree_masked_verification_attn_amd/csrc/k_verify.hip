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

__device__ inline void dma16(const void* gsrc, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}
template <int N>
__device__ inline void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

constexpr int kDraftStages = 4;

template <typename LT>
__global__ __launch_bounds__(kVocabThreads) void vocab_kernel(VocabArgs a) {
  constexpr int EPU = 16 / sizeof(LT);  // logits per 16-byte unit (8 bf16 / 4 f32)
  constexpr int DPS = EPU / 4;          // 16-byte draft loads per thread and slot
  constexpr int SLOTS = kVocabSlots;
  constexpr int NCH = SLOTS * kWaves;   // chunks of 64 * EPU consecutive tokens
  constexpr int STAGE = kVocabThreads * EPU * 4;
  __shared__ __attribute__((aligned(1024))) uint8_t dstage[kDraftStages][STAGE];
  __shared__ float red_f[kWaves];
  __shared__ double red_d[kWaves];
  __shared__ float csum[NCH];
  __shared__ int kid_id[kMaxChildren];
  __shared__ int kid_tok[kMaxChildren];
  __shared__ uint8_t kid_smp[kMaxChildren];
  __shared__ int n_kids, n_samp, bad_s;
  __shared__ int pick_chunk;
  __shared__ float pick_rem;
  __shared__ int pick_token;

  const int v = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  if (tid == 0) { n_kids = 0; n_samp = 0; bad_s = 0; pick_chunk = -1; pick_token = -1; }
  __syncthreads();
  // children of this node (and a check of the parent array at the same time)
  uint32_t err = 0;
  for (int j = tid; j < n; j += kVocabThreads) {
    const int pj = a.parent[s0 + j];
    if (j == 0 ? pj != -1 : (pj < 0 || pj >= j)) err |= TAV_DEV_BAD_PARENT;
    if (j > 0 && pj == local) {
      const int k = atomicAdd(&n_kids, 1);
      const uint8_t sj = a.sampled[s0 + j];
      if (k < kMaxChildren) { kid_id[k] = j; kid_tok[k] = a.token[s0 + j]; kid_smp[k] = sj; }
      if (sj) atomicAdd(&n_samp, 1);
    }
  }
  __syncthreads();
  const int nk = min(n_kids, kMaxChildren);
  if (tid == 0) {
    if (n_kids > kMaxChildren) err |= TAV_DEV_TOO_MANY_CHILDREN;
    if (n_samp > 1) err |= TAV_DEV_MULTI_SAMPLED;
  }
  if (tid < nk) {
    const int tk = kid_tok[tid];
    if (tk < 0 || tk >= V) err |= TAV_DEV_BAD_TOKEN;
    for (int k = 0; k < tid; ++k)
      if (kid_tok[k] == tk) err |= TAV_DEV_DUP_SIBLING_TOKEN;
  }
  const int dr = a.draft_row[v];
  const bool has_sampled = n_samp > 0;
  if (tid == 0 && has_sampled && (dr < 0 || dr >= a.R)) err |= TAV_DEV_NO_DRAFT;
  const bool use_draft = has_sampled && dr >= 0 && dr < a.R;
  const float Tb = a.temperature[b];
  if (tid == 0 && !(Tb > 0.f && Tb < INFINITY)) err |= TAV_DEV_BAD_TEMPERATURE;
  const float invT = 1.f / Tb;

  // ---- the logits row into registers (19 x 16 bytes per thread), draft DMA started ----
  const LT* row = (const LT*)a.logits + (size_t)v * V;
  uint4 r[SLOTS];
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) {
    const int e0 = (i * kVocabThreads + tid) * EPU;
    r[i] = *(const uint4*)(row + (e0 < V ? e0 : 0));
  }
  const float* drow = a.draft + (size_t)(use_draft ? dr : 0) * V;
  // draft slot i of this thread: elements e0 .. e0+EPU-1, copied to stage i % kDraftStages
  // at [j][wave][lane] (16 bytes each); every lane issues every copy (addresses clamped
  // inside the row) so the per-wave count of outstanding copies is exact
  auto issue_draft = [&](int i) {
    const int e0 = (i * kVocabThreads + tid) * EPU;
    const float* src = drow + (e0 < V ? e0 : 0);
#pragma unroll
    for (int j = 0; j < DPS; ++j)
      dma16(src + 4 * j, dstage[i % kDraftStages] + (j * kWaves + wave) * 1024);
  };
  if (use_draft) {
#pragma unroll
    for (int i = 0; i < kDraftStages - 1; ++i) issue_draft(i);
  }

  // ---- pass 1: M = max l/T, S = sum exp(l/T - M) ----
  float mx = -INFINITY;
  int nonfinite = 0;
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) {
    const int e0 = (i * kVocabThreads + tid) * EPU;
    if (e0 < V) {
#pragma unroll
      for (int e = 0; e < EPU; ++e) {
        const float z = unit_elem<LT>(r[i], e) * invT;
        nonfinite |= (z != z) | (z == INFINITY);
        mx = fmaxf(mx, z);
      }
    }
  }
  if (nonfinite) err |= TAV_DEV_NONFINITE_LOGITS;
  mx = wave_max_f(mx);
  if (lane == 0) red_f[wave] = mx;
  __syncthreads();
  float M = red_f[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) M = fmaxf(M, red_f[w]);
  if (M == -INFINITY) {  // every logit is -inf: the row has no mass
    err |= TAV_DEV_NONFINITE_LOGITS;
    M = 0.f;
  }
  const float Ml2 = M * kLog2e;
  const float invTl2 = invT * kLog2e;
  double sl = 0.0;
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) {
    const int e0 = (i * kVocabThreads + tid) * EPU;
    if (e0 < V) {
      float su = 0.f;
#pragma unroll
      for (int e = 0; e < EPU; ++e) su += __builtin_amdgcn_exp2f(unit_elem<LT>(r[i], e) * invTl2 - Ml2);
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

  // ---- pass 2: final-draw weights w = (p - q~)+ or p, per-chunk sums, Z ----
  double zl = 0.0;
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) {
    float q[EPU];
    if (use_draft) {
      const int after = (SLOTS - 1 - i) < (kDraftStages - 2) ? (SLOTS - 1 - i) : (kDraftStages - 2);
      if (after >= 2) wait_vm<2 * DPS>();
      else if (after == 1) wait_vm<DPS>();
      else wait_vm<0>();
#pragma unroll
      for (int j = 0; j < DPS; ++j) {
        const float4 t = *(const float4*)(dstage[i % kDraftStages] + (j * kWaves + wave) * 1024 + lane * 16);
        q[4 * j + 0] = t.x; q[4 * j + 1] = t.y; q[4 * j + 2] = t.z; q[4 * j + 3] = t.w;
      }
      if (i + kDraftStages - 1 < SLOTS) issue_draft(i + kDraftStages - 1);
    }
    const int e0 = (i * kVocabThreads + tid) * EPU;
    float ws = 0.f;
    if (e0 < V) {
#pragma unroll
      for (int e = 0; e < EPU; ++e) {
        const float p = __builtin_amdgcn_exp2f(unit_elem<LT>(r[i], e) * invTl2 - Ml2) * invS;
        ws += use_draft ? fmaxf(0.f, p - q[e]) : p;
      }
    }
    zl += (double)ws;
    ws = wave_sum_f(ws);
    if (lane == 0) csum[i * kWaves + wave] = ws;
  }
  zl = wave_sum_d(zl);
  __syncthreads();
  if (lane == 0) red_d[wave] = zl;

  // the children's own point values for the walk, and their removal from the final draw
  auto weight_of = [&](float p, int tok) -> float { return use_draft ? fmaxf(0.f, p - drow[tok]) : p; };
  if (tid < nk) {
    const int tok = kid_tok[tid];
    const int c = kid_id[tid];
    if (tok >= 0 && tok < V) {
      const float z = logit_at<LT>(a.logits, (size_t)v * V + tok);
      a.child_p[s0 + c] = exp((double)(z * invT) - (double)M) / S;
      a.child_q[s0 + c] = use_draft ? drow[tok] : 0.f;
      if (!kid_smp[tid]) {
        const float p = __builtin_amdgcn_exp2f(z * invTl2 - Ml2) * invS;
        const int unit = tok / EPU;
        atomicAdd(&csum[(unit / kVocabThreads) * kWaves + (unit % kVocabThreads) / 64], -weight_of(p, tok));
      }
    }
  }
  __syncthreads();
  double Zt = 0.0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) Zt += red_d[w];
  const float Z = use_draft ? (float)Zt : 0.f;

  // locate the chunk of the final draw: wave 0 scans the NCH chunk sums
  if (wave == 0) {
    constexpr int PER = (NCH + 63) / 64;
    double part = 0.0;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int c = lane * PER + k;
      if (c < NCH) part += (double)fmaxf(csum[c], 0.f);
    }
    double incl = part;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const double y = __shfl_up(incl, d, 64);
      if (lane >= d) incl += y;
    }
    const double W = __shfl(incl, 63);
    if (W > 0.0) {
      const double target = (double)a.uniforms[(size_t)v * 2 + 1] * W;
      const unsigned long long hit = __ballot(incl > target && part > 0.0);
      int L0;
      if (hit) L0 = __ffsll((long long)hit) - 1;
      else {
        const unsigned long long has = __ballot(part > 0.0);
        L0 = 63 - __clzll((long long)has);
      }
      if (lane == L0) {
        double cum = incl - part;
        int cfound = -1, clast = -1;
        for (int k = 0; k < PER; ++k) {
          const int c = lane * PER + k;
          if (c >= NCH) break;
          const double cs = (double)fmaxf(csum[c], 0.f);
          if (cs > 0.0) {
            clast = c;
            if (cfound < 0 && cum + cs > target) { cfound = c; break; }
          }
          cum += cs;
        }
        if (cfound < 0) {  // rounding put the target past the total: last chunk with mass
          cfound = clast;
          cum -= (double)fmaxf(csum[clast], 0.f);
        }
        pick_chunk = cfound;
        pick_rem = (float)(target - cum);
      }
    }
  }
  __syncthreads();
  const int pc = pick_chunk;
  if (pc >= 0 && wave == pc % kWaves) {
    const int slot = pc / kWaves;
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
            const float p = __builtin_amdgcn_exp2f(unit_elem<LT>(r[i], e) * invTl2 - Ml2) * invS;
            w = weight_of(p, e0 + e);
            for (int k = 0; k < nk; ++k)
              if (kid_tok[k] == e0 + e && !kid_smp[k]) w = 0.f;
          }
          wv[e] = w;
          lsum += w;
        }
      }
    }
    float incl = lsum;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const float y = __shfl_up(incl, d, 64);
      if (lane >= d) incl += y;
    }
    const float rem = pick_rem;
    const unsigned long long hit = __ballot(incl > rem && lsum > 0.f);
    int chosen;
    if (hit) chosen = __ffsll((long long)hit) - 1;
    else {
      const unsigned long long has = __ballot(lsum > 0.f);
      chosen = has ? 63 - __clzll((long long)has) : -1;
    }
    if (lane == chosen) {
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
  if (err) atomicOr(&bad_s, (int)err);
  __syncthreads();
  if (tid == 0) {
    a.stats[(size_t)v * 3 + 0] = M;
    a.stats[(size_t)v * 3 + 1] = (float)S;
    a.stats[(size_t)v * 3 + 2] = Z;
    a.term_token[v] = pick_token;
    if (bad_s) atomicOr(a.status, (uint32_t)bad_s);
  }
}

constexpr int kWalkLds = 2048;  // nodes whose walk data fit in LDS

// One wave per sequence: the layer-by-layer walk, decisions in fp64 from the values the
// vocabulary kernel left: p(token) and q~(token) of every child, Z and the final draw of
// every node.  Sequences of up to 2048 nodes are staged in LDS first.
__global__ __launch_bounds__(64) void walk_kernel(WalkArgs a) {
  __shared__ int par_s[kWalkLds];
  __shared__ uint8_t smp_s[kWalkLds];
  __shared__ int kids[kMaxChildren];
  const int b = blockIdx.x, lane = threadIdx.x;
  const int s0 = a.node_offsets[b];
  const int n = a.node_offsets[b + 1] - s0;
  const bool staged = n <= kWalkLds;
  for (int j = lane; j < n; j += 64) {
    a.node_status[s0 + j] = 0;
    if (staged) { par_s[j] = a.parent[s0 + j]; smp_s[j] = a.sampled[s0 + j]; }
  }
  for (int j = lane; j < a.max_path; j += 64) a.path[(size_t)b * a.max_path + j] = -1;
  __syncthreads();
  uint32_t err = 0;
  int plen = 1, v = 0, bonus = -1;
  if (lane == 0) {
    a.node_status[s0] = 1;
    a.path[(size_t)b * a.max_path] = 0;
  }
  for (int iter = 0; iter < n; ++iter) {
    // children of v in ascending id (sampled child found on the way)
    int nk = 0, s = -1;
    for (int base = 1; base < n; base += 64) {
      const int j = base + lane;
      const int pj = j < n ? (staged ? par_s[j] : a.parent[s0 + j]) : -2;
      const bool is_kid = pj == v;
      const unsigned long long m = __ballot(is_kid);
      if (is_kid) {
        const int at = nk + __popcll(m & ((1ull << lane) - 1ull));
        if (at < kMaxChildren) kids[at] = j;
        if (staged ? smp_s[j] : a.sampled[s0 + j]) s = j;
      }
      nk += __popcll(m);
    }
    __syncthreads();
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) s = max(s, __shfl_xor(s, d));
    if (nk > kMaxChildren) { err |= TAV_DEV_TOO_MANY_CHILDREN; break; }
    int next = -1;
    if (lane == 0) {
      bool resid = false;
      const double Zv = (double)a.stats[(size_t)(s0 + v) * 3 + 2];
      if (s >= 0) {
        const double qs = (double)a.child_q[s0 + s];
        if (!(qs > 0.0)) {
          err |= TAV_DEV_ZERO_DRAFT_MASS;
        } else {
          const double ratio = fmin(1.0, a.child_p[s0 + s] / qs);
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
          const double p = a.child_p[s0 + c];
          const double r0 = resid ? (Zv > 0.0 ? fmax(0.0, p - (double)a.child_q[s0 + c]) / Zv : 0.0) : p;
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
    next = __shfl(next, 0);
    err = __shfl(err, 0);
    __syncthreads();
    if (next < 0 || err) break;
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
