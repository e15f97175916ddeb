// PreSTO log-acceptance and the MH walk over the prefetched subtree.
//
// PreSTO, Section 3.2 and Example 3 / Equation 6: for the request of an
// acceptance child with cut c, proposal y keeps the parent state x up to c and
// replaces tokens c+1..T, and
//   log A(y, x) = min{0, sum_{t>c} [lq_x(t) - lq_y(t)] + alpha sum_{t>c} [lp0_y(t) - lp0_x(t)]}.
// A rejection child keeps its parent's state, so x's token t comes from the
// deepest accepted request above the node whose cut is below t (Condition 1
// keeps cuts non-increasing along accepted edges), else from the root state.
// Step (3) / Appendix B.3 Example 5: from the root, go to the acceptance child
// iff u <= A, else to the rejection child; stop at a leaf, at a deferred
// request, or after max_transitions transitions.
#include "tav_internal.h"

namespace tav {
namespace {

constexpr int kMaxChain = 1024;  // accepted requests above one node

__global__ __launch_bounds__(256) void presto_logA_kernel(PrestoArgs a) {
  __shared__ int node_s, bad_s, nchain;
  __shared__ int chain_req[kMaxChain];
  __shared__ double red[4];
  const int i = blockIdx.x, tid = threadIdx.x;
  if (tid == 0) { node_s = -1; bad_s = 0; nchain = 0; }
  __syncthreads();
  for (int v = tid; v < a.M; v += blockDim.x) {
    if (a.pf_is_accept[v] && a.pf_request[v] == i) {
      if (atomicCAS(&node_s, -1, v) != -1) bad_s = 1;
    }
  }
  __syncthreads();
  const int node = node_s;
  if (node > 0 && (a.pf_parent[node] < 0 || a.pf_parent[node] >= node)) bad_s = 1;
  __syncthreads();
  const int c = a.cut[i];
  const int off_i = a.suffix_off[i];
  if (node <= 0 || bad_s || c < 0 || c >= a.T || a.suffix_off[i + 1] - off_i != a.T - c) {
    if (tid == 0) {
      atomicOr(a.status, (uint32_t)TAV_DEV_PRESTO_BAD_TREE);
      a.log_accept[i] = NAN;
      a.log_accept64[i] = NAN;
    }
    return;
  }
  if (tid == 0) {  // accepted requests above the parent state, deepest first
    int x = a.pf_parent[node], k = 0, guard = 0;
    while (x > 0 && guard < a.M) {
      const int r = a.pf_request[x];
      if (a.pf_is_accept[x] && r >= 0) {
        if (r >= a.R || a.cut[r] < 0 || a.cut[r] >= a.T ||
            a.suffix_off[r + 1] - a.suffix_off[r] != a.T - a.cut[r])
          bad_s = 1;
        else if (k < kMaxChain)
          chain_req[k] = r;
        ++k;
      }
      if (a.pf_parent[x] >= x || a.pf_parent[x] < 0) { bad_s = 1; break; }
      x = a.pf_parent[x];
      ++guard;
    }
    if (k > kMaxChain || guard >= a.M) bad_s = 1;
    nchain = k < kMaxChain ? k : kMaxChain;
  }
  __syncthreads();
  if (bad_s) {
    if (tid == 0) atomicOr(a.status, (uint32_t)TAV_DEV_PRESTO_BAD_TREE);
    return;
  }
  const int nc = nchain;
  double acc = 0.0;
  for (int t = c + 1 + tid; t <= a.T; t += blockDim.x) {
    double lqx = (double)a.root_lq[t - 1], lpx = (double)a.root_lp0[t - 1];
    for (int k = 0; k < nc; ++k) {
      const int r = chain_req[k];
      const int cr = a.cut[r];
      if (cr < t) {
        const int idx = a.suffix_off[r] + (t - cr - 1);
        lqx = (double)a.lq[idx];
        lpx = (double)a.lp0[idx];
        break;
      }
    }
    const int iy = off_i + (t - c - 1);
    acc += (lqx - (double)a.lq[iy]) + a.alpha * ((double)a.lp0[iy] - lpx);
  }
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) acc += __shfl_xor(acc, d);
  if ((tid & 63) == 0) red[tid >> 6] = acc;
  __syncthreads();
  if (tid == 0) {
    const double s = red[0] + red[1] + red[2] + red[3];
    const double la = s < 0.0 ? s : 0.0;
    a.log_accept64[i] = la;
    a.log_accept[i] = (float)la;
  }
}

__global__ __launch_bounds__(64) void presto_walk_kernel(PrestoArgs a) {
  const int lane = threadIdx.x;
  for (int j = lane; j < a.M; j += 64) a.pf_path[j] = -1;
  __syncthreads();
  int v = 0, k = 0;
  uint32_t err = 0;
  if (lane == 0) a.pf_path[0] = 0;
  while (k < a.max_transitions && k + 1 < a.M) {
    int acc_c = -1, rej_c = -1;
    for (int base = 1; base < a.M; base += 64) {
      const int j = base + lane;
      const bool kid = j < a.M && a.pf_parent[j] == v;
      const unsigned long long m = __ballot(kid && a.pf_is_accept[j]);
      const unsigned long long r = __ballot(kid && !a.pf_is_accept[j]);
      if (m && acc_c < 0) acc_c = base + __ffsll((long long)m) - 1;
      if (r && rej_c < 0) rej_c = base + __ffsll((long long)r) - 1;
    }
    if (acc_c < 0 || rej_c < 0) break;      // leaf of the prefetched subtree
    const int req = a.pf_request[acc_c];
    if (req < 0) break;                      // proposal deferred to a later batch
    if (req >= a.R) { err |= TAV_DEV_PRESTO_BAD_TREE; break; }
    const double A = exp(a.log_accept64[req]);
    v = ((double)a.u[v] <= A) ? acc_c : rej_c;
    ++k;
    if (lane == 0) a.pf_path[k] = v;
  }
  if (lane == 0) {
    a.pf_path_len[0] = k + 1;
    if (err) atomicOr(a.status, err);
  }
}

}  // namespace

hipError_t launch_presto(const PrestoArgs& a, hipStream_t s) {
  if (a.R > 0) presto_logA_kernel<<<a.R, 256, 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  presto_walk_kernel<<<1, 64, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace tav
