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
// The vocabulary work of every node (M, S, Z, p and q~ at the children's tokens,
// the would-be final draw) is done by the kernels of vocab_worker.h: streaming
// workers (512-thread workgroups taking nodes from a queue), then the pick of
// every node (one wave each).  walk_kernel
// (one wave per sequence) then takes the accept/reject decisions in fp64 from
// these values.
#include "tav_internal.h"
#include "vocab_worker.h"

namespace tav {
namespace {

// Streaming workers that take nodes from the device queue until none is left (as many workgroups
// per compute unit as fit).  Shape: threads, sixteen-byte units per thread and step, KB of a dense
// draft node's logits row kept in LDS for its second pass, waves per SIMD the registers allow.
#ifndef TAV_VW_THREADS
#define TAV_VW_THREADS 512
#endif
#ifndef TAV_VW_UNITS
#define TAV_VW_UNITS 8
#endif
#ifndef TAV_VW_CACHE_KB
#define TAV_VW_CACHE_KB 128
#endif
#ifndef TAV_VW_WAVES_PER_EU
#define TAV_VW_WAVES_PER_EU 2
#endif
using WorkerCfg = vw::Cfg<TAV_VW_THREADS, TAV_VW_UNITS, TAV_VW_CACHE_KB>;
template <typename LT>
__global__ __launch_bounds__(TAV_VW_THREADS) __attribute__((amdgpu_waves_per_eu(TAV_VW_WAVES_PER_EU)))
void vocab_worker_kernel(VocabArgs a) {
  __shared__ vw::Lds<WorkerCfg> L;
  vw::vocab_stream<LT, WorkerCfg>(a, L);
}

// The pick of every node: one wave per node, kPickWaves nodes per workgroup.
constexpr int kPickWaves = 4;
template <typename LT>
__global__ __launch_bounds__(64 * kPickWaves) void pick_kernel(VocabArgs a) {
  __shared__ vw::PickLds P[kPickWaves];
  const int wave = threadIdx.x >> 6;
  const int v = blockIdx.x * kPickWaves + wave;
  if (v >= a.N) return;
  vw::pick_node<LT>(a, P[wave], v);
}

constexpr int kWalkLds = 1024;  // nodes whose walk data fit in LDS

// One wave per sequence: the layer-by-layer walk, decisions in fp64 from the values the
// vocabulary kernels left: p(token) and q~(token) of every child, Z and the final draw of
// every node.  For sequences of up to kWalkLds nodes these values, the parents and the
// sampled flags are first staged in LDS (one round of loads).
__global__ __launch_bounds__(64) void walk_kernel(WalkArgs a) {
  __shared__ int par_s[kWalkLds];
  __shared__ uint8_t smp_s[kWalkLds];
  __shared__ double cp_s[kWalkLds];
  __shared__ float cq_s[kWalkLds];
  __shared__ float u_s[kWalkLds];
  __shared__ float z_s[kWalkLds];
  __shared__ int tt_s[kWalkLds];
  __shared__ int kids[kMaxChildren];
  const int b = blockIdx.x, lane = threadIdx.x;
  const int s0 = a.node_offsets[b];
  const int n = a.node_offsets[b + 1] - s0;
  // a sequence with an error found by an earlier kernel of the call: sentinel outputs (its error
  // bits also go into the status word here: a call whose start was folded into the prelude reports
  // the preparation's errors in seq_err only)
  const uint32_t serr = a.seq_err[b];
  if (serr != 0u || (a.status[0] & TAV_DEV_PLAN_MISMATCH) != 0u) {
    if (lane == 0 && serr) atomicOr(a.status, serr);
    for (int j = lane; j < n; j += 64) a.node_status[s0 + j] = 0;
    for (int j = lane; j < a.max_path; j += 64) a.path[(size_t)b * a.max_path + j] = -1;
    if (lane == 0) {
      a.path_len[b] = 0;
      a.bonus[b] = -1;
    }
    return;
  }
  const bool staged = n <= kWalkLds;
  for (int j = lane; j < n; j += 64) {
    a.node_status[s0 + j] = 0;
    if (staged) {
      par_s[j] = a.parent[s0 + j];
      smp_s[j] = a.sampled[s0 + j];
      cp_s[j] = a.child_p[s0 + j];
      cq_s[j] = a.child_q[s0 + j];
      u_s[j] = a.uniforms[(size_t)(s0 + j) * 2];
      z_s[j] = a.stats[(size_t)(s0 + j) * 3 + 2];
      tt_s[j] = a.term_token[s0 + j];
    }
  }
  for (int j = lane; j < a.max_path; j += 64) a.path[(size_t)b * a.max_path + j] = -1;
  auto parent_of = [&](int j) { return staged ? par_s[j] : a.parent[s0 + j]; };
  auto sampled_of = [&](int j) { return staged ? (int)smp_s[j] : (int)a.sampled[s0 + j]; };
  auto p_of = [&](int j) { return staged ? cp_s[j] : a.child_p[s0 + j]; };
  auto q_of = [&](int j) { return (double)(staged ? cq_s[j] : a.child_q[s0 + j]); };
  auto u_of = [&](int j) { return (double)(staged ? u_s[j] : a.uniforms[(size_t)(s0 + j) * 2]); };
  __syncthreads();
  uint32_t err = 0;
  int plen = 1, v = 0, bonus = -1;
  // temperature 0: greedy decoding (Progressive Tree Drafting, Section 3.2) -- the child whose
  // token is the node's verification token (p = 1 there, 0 elsewhere) is accepted, the children
  // passed over before it (sampled child first, then ascending id) are rejected
  const bool greedy = a.temperature[b] == 0.f;
  if (lane == 0) {
    a.node_status[s0] = 1;
    a.path[(size_t)b * a.max_path] = 0;
  }
  for (int iter = 0; iter < n; ++iter) {
    // children of v in ascending id (sampled child found on the way)
    int nk = 0, s = -1;
    for (int base = 1; base < n; base += 64) {
      const int j = base + lane;
      const int pj = j < n ? parent_of(j) : -2;
      const bool is_kid = pj == v;
      const unsigned long long m = __ballot(is_kid);
      if (is_kid) {
        const int at = nk + __popcll(m & ((1ull << lane) - 1ull));
        if (at < kMaxChildren) kids[at] = j;
        if (sampled_of(j)) s = j;
      }
      nk += __popcll(m);
    }
    __syncthreads();
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) s = max(s, __shfl_xor(s, d));
    if (nk > kMaxChildren) { err |= TAV_DEV_TOO_MANY_CHILDREN; break; }
    int next = -1;
    if (lane == 0 && greedy) {
      if (s >= 0) {
        if (p_of(s) == 1.0) next = s;
        else a.node_status[s0 + s] = 2;
      }
      for (int k = 0; k < nk && next < 0; ++k) {
        const int c = kids[k];
        if (c == s) continue;
        if (p_of(c) == 1.0) next = c;
        else a.node_status[s0 + c] = 2;
      }
      if (next >= 0) {
        a.node_status[s0 + next] = 1;
        if (plen >= a.max_path) err |= TAV_DEV_PATH_OVERFLOW;
        else a.path[(size_t)b * a.max_path + plen] = next;
        ++plen;
      } else {
        bonus = staged ? tt_s[v] : a.term_token[s0 + v];
        if (bonus < 0) err |= TAV_DEV_EMPTY_RESIDUAL;
      }
    } else if (lane == 0) {
      bool resid = false;
      const double Zv = (double)(staged ? z_s[v] : a.stats[(size_t)(s0 + v) * 3 + 2]);
      // the tests u <= min(1, p / q~) and u <= r / (1 - rejected mass) are taken as products
      // (u q~ <= p, u (1 - rejected) <= r): the same decisions up to the last bits of the ratios, with
      // no fp64 division on the walk's serial path (one reciprocal of Z per residual node)
      if (s >= 0) {
        const double qs = q_of(s);
        if (!(qs > 0.0)) {
          err |= TAV_DEV_ZERO_DRAFT_MASS;
        } else if (u_of(s) * qs <= p_of(s)) {
          next = s;
        } else {
          a.node_status[s0 + s] = 2;
          resid = true;
        }
      }
      if (!err && next < 0) {
        const double invZ = resid && Zv > 0.0 ? 1.0 / Zv : 0.0;
        double rej = 0.0;
        for (int k = 0; k < nk && next < 0; ++k) {
          const int c = kids[k];
          if (c == s) continue;
          const double p = p_of(c);
          const double r0 = resid ? fmax(0.0, p - q_of(c)) * invZ : p;
          const double rem = 1.0 - rej;
          const double uc = u_of(c);
          if (rem > 0.0 ? uc * rem <= r0 : uc <= 0.0) {
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
        bonus = staged ? tt_s[v] : a.term_token[s0 + v];
        if (bonus < 0) err |= TAV_DEV_EMPTY_RESIDUAL;
      }
    }
    next = __shfl(next, 0);
    err = __shfl(err, 0);
    __syncthreads();
    if (next < 0 || err) break;
    v = next;
  }
  __syncthreads();
  if (err) {   // an error found by the walk itself: the same sentinel outputs
    for (int j = lane; j < n; j += 64) a.node_status[s0 + j] = 0;
    for (int j = lane; j < a.max_path; j += 64) a.path[(size_t)b * a.max_path + j] = -1;
  }
  if (lane == 0) {
    if (err) atomicOr(a.status, err);
    a.path_len[b] = err ? 0 : min(plen, a.max_path);
    a.bonus[b] = err ? -1 : bonus;
  }
}

template <typename LT>
hipError_t launch_vocab_t(const VocabArgs& a, int num_cus, hipStream_t s) {
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, vocab_worker_kernel<LT>,
                                                              WorkerCfg::kThreads, 0);
  if (e != hipSuccess) return e;
  if (per_cu < 1) per_cu = 1;
  const int grid = a.N < per_cu * num_cus ? a.N : per_cu * num_cus;
  vocab_worker_kernel<LT><<<grid, WorkerCfg::kThreads, 0, s>>>(a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  pick_kernel<LT><<<(a.N + kPickWaves - 1) / kPickWaves, 64 * kPickWaves, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_vocab(const VocabArgs& a, bool bf16_logits, int num_cus, hipStream_t s) {
  if (a.N == 0) return hipSuccess;
  return bf16_logits ? launch_vocab_t<uint16_t>(a, num_cus, s) : launch_vocab_t<float>(a, num_cus, s);
}

hipError_t launch_walk(const WalkArgs& a, hipStream_t s) {
  walk_kernel<<<a.B, 64, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace tav
