// Host-side construction of PreSTO's prefetching tree: which suffix requests go into one batch.
//
// PreSTO, Section 3.2 step (1): node v of the prefetching tree holds an MH state with cut c_v (the
// root: the current state, cut T).  Expanding v creates an acceptance child v+ carrying a new
// suffix-resampling request with cut c+ drawn uniformly from {0..T-1}, and a rejection child v-
// that keeps v's state and cut.  Condition 1: v+'s request can go into this batch iff c+ <= c_v.
//   BFS rule: breadth-first from the root; a feasible acceptance child joins the batch and is
//   queued, an infeasible one is deferred (created, not queued); the rejection child is always
//   queued; stop at N_pf requests or an empty queue.
//   Predictive rule (Appendix C.1-C.4): among the candidate nodes I_max (depth < K', Condition 1
//   at the acceptance child, every strict ancestor likewise), choose an ancestor-closed set I of at
//   most N_pf nodes maximising sum_{v in I} R^(v) (Equation 17), with reaching weights
//   R^(v0) = 1, R^(v+-) = R^(v) h^(v+-) (Equation 11) and h^(v+) = (1 + P^(accept) -
//   P^(reject)) / 2 (Equation 14) from a three-class logistic regression on the cut fraction.
//   The pages solve it by the dynamic program of Equation 19.  Here it is solved best-first: every
//   h^ lies in (0, 1), so R^ never rises from a node to its child, the N_pf candidates with the
//   largest R^ form an ancestor-closed set, and no other set of N_pf candidates has a larger sum --
//   the same optimum as Equation 19 in O(N_pf log N_pf) instead of a recursion over the whole
//   binary tree below the root.
// After scoring, tav_prefetch_reach gives the epsilon-rounded branch probabilities (Equation 10),
// the reaching weights and the expected number of completed transitions (Lemma 1, Equation 12).
//
// Nodes are named by heap index (root 1, acceptance child 2h, rejection child 2h + 1) and listed
// in ascending heap index; the cut of the acceptance child with heap index h is drawn from the
// SplitMix64 generator (Steele, Lea and Flood) keyed by (seed, h).
#include <math.h>

#include <algorithm>
#include <deque>
#include <queue>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "tav_internal.h"

namespace tav {
namespace {

constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ull;

uint64_t splitmix64(uint64_t x) {
  uint64_t z = x + kGolden;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

int depth_of(uint64_t h) { return 63 - __builtin_clzll(h); }

struct Cuts {
  uint64_t seed;
  int T;
  // acceptance child h: floor(U T) with U the top 53 bits of the generator over 2^53 (exact
  // integer arithmetic); rejection child: its parent's cut; root: T
  int operator()(uint64_t h) const {
    while (h > 1 && (h & 1)) h >>= 1;
    if (h == 1) return T;
    const uint64_t z = splitmix64(seed + h * kGolden);
    return (int)(((unsigned __int128)(z >> 11) * (unsigned)T) >> 53);
  }
};

double predicted_h(const float* w, int cut_plus, int T) {
  const double f = (double)cut_plus / (double)T;
  double z[3], m = -INFINITY;
  for (int k = 0; k < 3; ++k) {
    z[k] = (double)w[2 * k] + (double)w[2 * k + 1] * f;
    m = std::max(m, z[k]);
  }
  double e[3], s = 0.0;
  for (int k = 0; k < 3; ++k) s += (e[k] = exp(z[k] - m));
  return 0.5 * (1.0 + e[1] / s - e[0] / s);   // classes: certain reject, certain accept, uncertain
}

void write_tree(const std::vector<uint64_t>& nodes_in, const std::unordered_set<uint64_t>& requests,
                const Cuts& cut, tav_prefetch_out* out) {
  std::vector<uint64_t> nodes = nodes_in;
  std::sort(nodes.begin(), nodes.end());
  std::unordered_map<uint64_t, int> pos;
  for (size_t i = 0; i < nodes.size(); ++i) pos[nodes[i]] = (int)i;
  int nreq = 0;
  for (size_t i = 0; i < nodes.size(); ++i) {
    const uint64_t h = nodes[i];
    out->parent[i] = h == 1 ? -1 : pos[h >> 1];
    out->is_accept[i] = (h > 1 && (h & 1) == 0) ? 1 : 0;
    out->cut[i] = cut(h);
    out->request[i] = -1;
    if (requests.count(h)) {
      out->request[i] = nreq;
      if (out->request_cut) out->request_cut[nreq] = cut(h);
      ++nreq;
    }
    if (out->heap) out->heap[i] = (int64_t)h;
  }
  out->num_nodes = (int)nodes.size();
  out->num_requests = nreq;
}

}  // namespace
}  // namespace tav

using namespace tav;

extern "C" tav_status tav_prefetch_build(const tav_prefetch_params* p, tav_prefetch_out* out) {
  if (!p || !out || !out->parent || !out->is_accept || !out->request || !out->cut)
    return tav_host_fail(TAV_ERR_NULL_POINTER, "prefetch params / output arrays are NULL");
  if (p->T < 1 || p->budget < 1 || p->budget > 62 || p->depth_cap < 1)
    return tav_host_fail(TAV_ERR_BAD_SHAPE, "prefetch: T >= 1, budget in [1, 62] and depth_cap >= 1 (got %d, %d, %d)",
                         p->T, p->budget, p->depth_cap);
  if (p->rule != TAV_PREFETCH_BFS && p->rule != TAV_PREFETCH_PREDICTIVE)
    return tav_host_fail(TAV_ERR_INVALID_ARGUMENT, "prefetch rule must be TAV_PREFETCH_BFS or TAV_PREFETCH_PREDICTIVE");
  for (int k = 0; k < 6; ++k)
    if (!isfinite(p->class_w[k])) return tav_host_fail(TAV_ERR_INVALID_ARGUMENT, "class weights must be finite");
  if (out->capacity < 2 * p->budget + 1)
    return tav_host_fail(TAV_ERR_BAD_SHAPE, "capacity %d < 2 * budget + 1", out->capacity);
  const Cuts cut{p->seed, p->T};
  const int T = p->T, K = std::min(p->depth_cap, 62);
  auto expandable = [&](uint64_t h) { return depth_of(h) < K && cut(2 * h) <= cut(h); };
  std::vector<uint64_t> nodes{1};
  std::unordered_set<uint64_t> requests;
  double fhat = 0.0;
  if (p->rule == TAV_PREFETCH_BFS) {
    std::deque<uint64_t> queue{1};
    std::unordered_map<uint64_t, double> reach{{1, 1.0}};   // R^ of nodes reachable in this batch
    while (!queue.empty() && (int)requests.size() < p->budget) {
      const uint64_t v = queue.front();
      queue.pop_front();
      if (depth_of(v) >= K) continue;
      if ((int)nodes.size() + 2 > out->capacity)
        return tav_host_fail(TAV_ERR_BAD_SHAPE, "prefetch tree exceeds capacity %d", out->capacity);
      const uint64_t a = 2 * v, r = 2 * v + 1;
      nodes.push_back(a);
      nodes.push_back(r);
      if (cut(a) <= cut(v)) {
        requests.insert(a);
        queue.push_back(a);
        auto it = reach.find(v);
        if (it != reach.end()) {   // v expanded with its request, reachable: a transition there
          fhat += it->second;
          const double hp = predicted_h(p->class_w, cut(a), T);
          reach[a] = it->second * hp;
          reach[r] = it->second * (1.0 - hp);
        }
      }
      queue.push_back(r);
    }
  } else {
    // best-first over the candidates by R^ (ties: shallower, then smaller heap index)
    struct Item {
      double R;
      uint64_t h;
      bool operator<(const Item& o) const {
        if (R != o.R) return R < o.R;
        const int d = depth_of(h), od = depth_of(o.h);
        if (d != od) return d > od;
        return h > o.h;
      }
    };
    std::priority_queue<Item> heap;
    heap.push({1.0, 1});
    int chosen = 0;
    while (!heap.empty() && chosen < p->budget) {
      const Item it = heap.top();
      heap.pop();
      if (!expandable(it.h)) continue;   // not a candidate (its strict ancestors are selected)
      ++chosen;
      fhat += it.R;
      const uint64_t a = 2 * it.h, r = 2 * it.h + 1;
      nodes.push_back(a);
      nodes.push_back(r);
      requests.insert(a);
      const double hp = predicted_h(p->class_w, cut(a), T);
      heap.push({it.R * hp, a});
      heap.push({it.R * (1.0 - hp), r});
    }
  }
  write_tree(nodes, requests, cut, out);
  out->predicted_transitions = fhat;
  return tav_host_ok();
}

extern "C" tav_status tav_prefetch_reach(int32_t num_nodes, const int32_t* parent, const uint8_t* is_accept,
                                         const int32_t* request, int32_t num_requests, const float* log_accept,
                                         float eps, double* reach, double* expected_transitions) {
  if (!parent || !is_accept || !request || !log_accept || !expected_transitions)
    return tav_host_fail(TAV_ERR_NULL_POINTER, "prefetch reach: an array is NULL");
  if (num_nodes < 1 || num_requests < 0) return tav_host_fail(TAV_ERR_BAD_SHAPE, "prefetch reach: sizes");
  if (!(eps >= 0.f && eps < 0.5f)) return tav_host_fail(TAV_ERR_INVALID_ARGUMENT, "eps must be in [0, 1/2)");
  if (parent[0] != -1) return tav_host_fail(TAV_ERR_BAD_SHAPE, "node 0 must be the root");
  std::vector<int> acc(num_nodes, -1);
  for (int v = 1; v < num_nodes; ++v) {
    if (parent[v] < 0 || parent[v] >= v) return tav_host_fail(TAV_ERR_BAD_SHAPE, "parent[%d] must be an earlier node", v);
    if (is_accept[v]) acc[parent[v]] = v;
    if (request[v] >= num_requests) return tav_host_fail(TAV_ERR_BAD_SHAPE, "request[%d] out of range", v);
  }
  // h(v+; eps) of Equation 10, R of Equation 11, F = sum of R over the expanded nodes (Equation 12)
  std::vector<double> R(num_nodes, 0.0);
  R[0] = 1.0;
  double F = 0.0;
  for (int v = 0; v < num_nodes; ++v) {
    if (v > 0) {
      const int pv = parent[v], a = acc[pv];
      if (a >= 0 && request[a] >= 0) {
        const double A = exp((double)log_accept[request[a]]);
        const double h = A <= eps ? 0.0 : (A >= 1.0 - eps ? 1.0 : A);
        R[v] = R[pv] * (is_accept[v] ? h : 1.0 - h);
      }
    }
    if (acc[v] >= 0 && request[acc[v]] >= 0) F += R[v];
    if (reach) reach[v] = R[v];
  }
  *expected_transitions = F;
  return tav_host_ok();
}
