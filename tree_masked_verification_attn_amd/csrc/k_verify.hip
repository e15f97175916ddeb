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
// every node (one wave each), which also takes the node's accept/reject step in
// fp64 (a step depends on the node's own values only).  walk_kernel (one
// workgroup per sequence) follows the accepted children from the root.
#include "tav_internal.h"
#include "vocab_worker.h"
#include "attn_merge.h"

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

constexpr int kWalkThreads = 256;
constexpr int kWalkLds = 1024;   // nodes whose steps are staged in LDS
constexpr int kPathLds = 256;    // path entries kept in LDS
constexpr int kWalkPre = 4;      // nodes per thread whose parent and mark are loaded before the chase

// The walk of sequence b (one 256-thread workgroup): from the root, each node's accepted child (the
// steps the pick took for every node) until a node accepts none; the path's last node gives the
// bonus token (its final draw).  Statuses: 1 on the path, 2 for a child rejected by its parent's step
// where that parent lies on the path, else 0.  A sequence with an error found by an earlier kernel
// of the call, or by the walk, gets the sentinel outputs (statuses 0, path -1, path_len 0, bonus -1).
__device__ void walk_sequence(const WalkArgs& a, int b) {
  __shared__ StepRec st_s[kWalkLds];
  __shared__ int path_s[kPathLds];
  __shared__ int res[4];   // sentinel flag, path length, bonus, error bits
  const int tid = threadIdx.x;
  const int s0 = a.node_offsets[b];
  const int n = a.node_offsets[b + 1] - s0;
  int32_t* path = a.path + (size_t)b * a.max_path;
  if (tid == 0) {
    // errors of the sequence found earlier in the call (their bits also go into the status word
    // here: a call whose start was folded into the prelude reports the preparation's errors in
    // seq_err only); read by one thread so that the whole workgroup takes the same branch
    const uint32_t serr = a.seq_err[b];
    if (serr) atomicOr(a.status, serr);
    res[0] = serr != 0u || (a.status[0] & TAV_DEV_PLAN_MISMATCH) != 0u;
  }
  for (int j = tid; j < n && j < kWalkLds; j += kWalkThreads) st_s[j] = a.step[s0 + j];
  int pj[kWalkPre];
  uint8_t mj[kWalkPre];
#pragma unroll
  for (int i = 0; i < kWalkPre; ++i) {
    const int j = tid + i * kWalkThreads;
    pj[i] = j < n ? a.parent[s0 + j] : -1;
    mj[i] = j < n ? a.node_status[s0 + j] : 0;
  }
  __syncthreads();
  if (tid == 0 && !res[0]) {
    int v = 0, plen = 1, bonus = -1;
    uint32_t err = 0;
    path_s[0] = 0;
    // one step of the chase; false when the path ends.  The steps of nodes below kWalkLds come from
    // LDS, the others from memory, in two loops (ids ascend along the path), so that each load has
    // one address space; path entries past kPathLds go straight to memory, the others are written
    // out by the whole workgroup after the chase.
    auto follow = [&](const StepRec& r) -> bool {
      if (r.err) { err = r.err; return false; }
      if (r.next < 0) { bonus = r.bonus; return false; }
      if (r.next <= v || r.next >= n) { err = TAV_DEV_BAD_PARENT; return false; }   // (children follow parents)
      if (plen >= a.max_path) { err = TAV_DEV_PATH_OVERFLOW; return false; }
      if (plen < kPathLds) path_s[plen] = r.next;
      else path[plen] = r.next;
      ++plen;
      v = r.next;
      return true;
    };
    bool more = true;
    while (more && v < kWalkLds && v < n) more = follow(st_s[v]);
    while (more && v < n) more = follow(a.step[s0 + v]);
    if (err) atomicOr(a.status, err);
    res[0] = err != 0u;
    res[1] = plen;
    res[2] = bonus;
  }
  __syncthreads();
  if (res[0]) {
    for (int j = tid; j < n; j += kWalkThreads) a.node_status[s0 + j] = 0;
    for (int j = tid; j < a.max_path; j += kWalkThreads) path[j] = -1;
    if (tid == 0) {
      a.path_len[b] = 0;
      a.bonus[b] = -1;
    }
    return;
  }
  const int plen = res[1];
  const int nl = plen < kPathLds ? plen : kPathLds;   // path entries in LDS
  for (int j = tid; j < nl; j += kWalkThreads) path[j] = path_s[j];
  // node x is on the path iff it is one of its (ascending) entries: the first kPathLds in LDS, the
  // rest in memory (written by thread 0 before the barrier above)
  auto on_path = [&](int x) -> bool {
    if (x <= path_s[nl - 1]) {
      int lo = 0, hi = nl;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (path_s[mid] < x) lo = mid + 1; else hi = mid;
      }
      return path_s[lo] == x;
    }
    int lo = nl, hi = plen;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (path[mid] < x) lo = mid + 1; else hi = mid;
    }
    return lo < plen && path[lo] == x;
  };
  auto status_of = [&](int j, int pr, uint8_t mk) -> uint8_t {
    return on_path(j) ? 1 : (j > 0 && mk == 2 && on_path(pr)) ? 2 : 0;
  };
#pragma unroll
  for (int i = 0; i < kWalkPre; ++i) {
    const int j = tid + i * kWalkThreads;
    if (j < n) a.node_status[s0 + j] = status_of(j, pj[i], mj[i]);
  }
  for (int j = tid + kWalkPre * kWalkThreads; j < n; j += kWalkThreads)
    a.node_status[s0 + j] = status_of(j, a.parent[s0 + j], a.node_status[s0 + j]);
  for (int j = plen + tid; j < a.max_path; j += kWalkThreads) path[j] = -1;
  if (tid == 0) {
    a.path_len[b] = plen;
    a.bonus[b] = res[2];
  }
}

// Workgroups [0, B) walk the sequences; the next nm workgroups merge the cut bf16 attention row
// blocks (merge_kernel's work, laid out by merge_grid) and the next ns write sentinel rows of
// sequences with attention errors (one sequence each; bf16 or, with f32, float32 outputs): work
// that runs beside the walks instead of in a launch of its own.
__global__ __launch_bounds__(kWalkThreads) __attribute__((amdgpu_waves_per_eu(8))) void walk_kernel(WalkArgs w, AttnArgs a, int D, int log2G, int nm,
                                                            int by_boundary, int ns, int f32) {
  const int blk = blockIdx.x;
  if (blk < w.B) {
    walk_sequence(w, blk);
    return;
  }
  const int m = blk - w.B;
  if (m < nm) {
    merge_block<__bf16>(a, D, log2G, m, by_boundary != 0);
  } else if (m - nm < ns) {
    if (f32) sentinel_rows<float>(a, D, m - nm);
    else sentinel_rows<__bf16>(a, D, m - nm);
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

hipError_t launch_walk(const WalkArgs& w, const Plan* plan, const AttnArgs* attn, bool f32_sentinels,
                       hipStream_t s) {
  const MergeGrid mg = attn ? merge_grid(plan->total_rb, plan->W) : MergeGrid{0, false};
  const int nm = attn && !f32_sentinels ? mg.units * plan->Hkv * (kRowsPerWG / kMergeRows) : 0;
  const int ns = attn ? plan->B : 0;
  const int D = attn ? plan->D : 0, log2G = attn ? plan->log2G : 0;
  walk_kernel<<<w.B + nm + ns, kWalkThreads, 0, s>>>(w, attn ? *attn : AttnArgs{}, D, log2G, nm,
                                                    mg.by_boundary ? 1 : 0, ns, f32_sentinels ? 1 : 0);
  return hipGetLastError();
}

}  // namespace tav
