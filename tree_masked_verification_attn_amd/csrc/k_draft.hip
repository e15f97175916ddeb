// Draft-tree construction on the GPU: expand-then-rerank with RheoSampling's hybrid pool and
// global pruning, producing the parent array, tokens, sampled flags and sparse draft rows that the
// scoring pass consumes.
//
// RheoSampling, Section 2.1 (EAGLE's dynamic tree): at each depth the drafter runs on the selected
// parents; each parent gets a candidate pool; a candidate's path score is the product of the proxy
// probabilities on its root path; the highest-scoring candidates of a depth are the next depth's
// parents; after D depths the tree is pruned to R nodes by score.  Section 3.2 and Appendix C.1: a
// hybrid pool takes the top-m lead tokens (proxy q), one token Y drawn from the tail off the leads
// (proxy min{q(x_m), z}, z = 1 - sum of the leads' q; q(x_1) + eps when m = 0), then the highest
// remaining tokens as fills; the draft logits are truncated to their top entries before the
// softmax (the sparse draft); global pruning breaks score ties by depth, then left to right.
//
// Per depth, one 1024-thread workgroup per (sequence, parent): the row's S largest logits are
// found from the bf16 bit patterns -- a lower bound L from the threads' own maxima (the S-th
// largest of them), the pairs (key, id) with key >= L gathered in LDS, a two-pass radix select
// there (over the whole row again if they do not fit); tokens at the threshold value go to the
// smaller ids, sorted by (logit, id); q = softmax over the support in fp64, the tail of softmax(z / T) for the
// sampled token (inverse CDF in token-id order), the pool, the children's scores, and for a hybrid
// parent its draft row (support ids ascending, q~).  One workgroup per sequence then ranks the
// depth's candidates for the next parents (rank = number of candidates ahead: deterministic, no
// sort), and at the end keeps the R best of all candidates: a byte-wise radix select on the
// scores' fp64 bit patterns, candidates tied at the threshold ranked by (depth, id).
#include "tav_internal.h"

namespace tav {
namespace {

constexpr int kDraftThreads = 256;    // frontier ranking
constexpr int kExpandThreads = 1024;  // one logits row per workgroup
constexpr int kNearCap = 4096;        // near-top (key, id) pairs kept in LDS for the collection
constexpr int kEqCap = 2048;   // tokens at the threshold logit held for the smallest-id choice

__device__ inline uint32_t bf16_key(uint32_t b) { return b ^ ((b & 0x8000u) ? 0xFFFFu : 0x8000u); }
// Calls f(key, token) for every element of a bf16 row of nunits * 8 entries, each thread keeping
// four 16-byte loads in flight (one workgroup streams a whole row, so latency hiding is per thread).
template <class F>
__device__ inline void scan_row(const uint16_t* row, int nunits, F&& f) {
  constexpr int kUnroll = 4;
  for (int u0 = threadIdx.x; u0 < nunits; u0 += kUnroll * kExpandThreads) {
    uint4 x[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      const int u = u0 + k * kExpandThreads;
      if (u < nunits) x[k] = *(const uint4*)(row + (size_t)u * 8);
    }
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      const int u = u0 + k * kExpandThreads;
      if (u >= nunits) break;
      const uint32_t w4[4] = {x[k].x, x[k].y, x[k].z, x[k].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) f((w4[e >> 1] >> (16 * (e & 1))) & 0xFFFFu, u * 8 + e);
    }
  }
}

// Number of threads of the (kExpandThreads-wide) block with pred set; every thread gets it.
__device__ inline int block_count(bool pred, int* lds) {
  const int c = __popcll(__ballot(pred));
  if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = c;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int w = 0; w < kExpandThreads / 64; ++w) t += lds[w];
  __syncthreads();
  return t;
}

// Slot of this lane in a wave-aggregated append to *counter (one LDS atomic per wave), or -1
// when take is false.
__device__ inline int wave_append(bool take, int* counter) {
  const unsigned long long m = __ballot(take);
  if (m == 0) return -1;
  const int lane = __lane_id();
  const int leader = __ffsll((long long)__ballot(1)) - 1;
  int base = 0;
  if (lane == leader) base = atomicAdd(counter, __popcll(m));
  base = __shfl(base, leader);
  return take ? base + __popcll(m & ((1ull << lane) - 1)) : -1;
}

__device__ inline float key_value(uint32_t k) {
  const uint32_t b = (k & 0x8000u) ? (k ^ 0x8000u) : (k ^ 0xFFFFu);
  return __uint_as_float(b << 16);
}

__global__ __launch_bounds__(kExpandThreads) void draft_expand_kernel(DraftArgs a, int d, const uint16_t* logits,
                                                                      const float* uniforms) {
  __shared__ int hist[256];
  __shared__ int red[kExpandThreads / 64];
  __shared__ int n_sel, n_eq, n_near;
  __shared__ uint32_t sel_key[kMaxDraftSupport];
  __shared__ int sel_id[kMaxDraftSupport];
  __shared__ int eq_id[kEqCap];
  __shared__ uint32_t near_key[kNearCap];
  __shared__ int near_id[kNearCap];
  __shared__ uint32_t s_key[kMaxDraftSupport];   // the support by (logit desc, id asc)
  __shared__ int s_id[kMaxDraftSupport];
  __shared__ int id_rank[kMaxDraftSupport];      // position of each support entry in token-id order
  __shared__ double qd[kMaxDraftSupport], qt[kMaxDraftSupport];
  __shared__ int bad;
  const int b = blockIdx.x / a.Kd, j = blockIdx.x % a.Kd, tid = threadIdx.x;
  const int S = a.S, V = a.V, nunits = V / 8;
  const size_t cb = (size_t)b * a.C;   // this sequence's candidates
  int* cand_parent = a.cand_parent + cb;
  int* cand_token = a.cand_token + cb;
  double* cand_score = a.cand_score + cb;
  uint8_t* cand_sampled = a.cand_sampled + cb;
  uint8_t* cand_depth = a.cand_depth + cb;
  int pid;
  if (d == 1) {
    pid = 0;
    if (tid == 0) {   // the root
      cand_parent[0] = -1;
      cand_token[0] = -1;
      cand_score[0] = 1.0;
      cand_sampled[0] = 0;
      cand_depth[0] = 0;
    }
  } else {
    pid = a.frontier[(size_t)b * a.K + j];
    if (pid < 0) return;
  }
  const uint16_t* row = logits + ((size_t)b * a.Kd + j) * V;
  if (tid == 0) { n_sel = 0; n_eq = 0; n_near = 0; bad = 0; }
  for (int i = tid; i < 256; i += kExpandThreads) hist[i] = 0;
  __syncthreads();
  // ---- pass 1: each thread's largest key (non-finite logits are errors)
  int nonfin = 0;
  uint32_t kmax = 0;
  scan_row(row, nunits, [&](uint32_t bits, int) {
    nonfin |= (bits & 0x7F80u) == 0x7F80u;
    kmax = max(kmax, bf16_key(bits));
  });
  if (nonfin) atomicOr(&bad, (int)TAV_DEV_NONFINITE_LOGITS);
  // L = the S-th largest of the threads' maxima (binary search on the 16-bit key with ballot
  // counts): at least S elements are >= L, so the support lies among the keys >= L -- for rows
  // without heavy ties only a little more than S of them
  uint32_t lo = 0, hi = 0xFFFFu;
  while (lo < hi) {
    const uint32_t mid = (lo + hi + 1) >> 1;
    const int c = block_count(kmax >= mid, red);
    if (c >= S) lo = mid; else hi = mid - 1;
  }
  const uint32_t L = lo;
  // ---- pass 2: the (key, id) pairs at or above L into LDS
  scan_row(row, nunits, [&](uint32_t bits, int id) {
    const uint32_t k = bf16_key(bits);
    const int at = wave_append(k >= L, &n_near);
    if (at >= 0 && at < kNearCap) { near_key[at] = k; near_id[at] = id; }
  });
  __syncthreads();
  const int nn = n_near;
  const bool in_lds = nn <= kNearCap;
  // ---- the threshold: radix select (high byte, then low byte) over the LDS pairs, or over the
  // whole row when they did not fit
  auto radix_pass = [&](auto&& each) {
    if (in_lds) {
      for (int i = tid; i < nn; i += kExpandThreads) each(near_key[i]);
    } else {
      scan_row(row, nunits, [&](uint32_t bits, int) { each(bf16_key(bits)); });
    }
  };
  int above = 0;
  radix_pass([&](uint32_t k) { atomicAdd(&hist[k >> 8], 1); });
  __syncthreads();
  int b1 = 0;
  {
    int cum = 0;
    for (int h = 255; h >= 0; --h) {
      if (cum + hist[h] >= S) { b1 = h; above = cum; break; }
      cum += hist[h];
    }
  }
  __syncthreads();
  for (int i = tid; i < 256; i += kExpandThreads) hist[i] = 0;
  __syncthreads();
  radix_pass([&](uint32_t k) {
    if ((k >> 8) == (uint32_t)b1) atomicAdd(&hist[k & 0xFF], 1);
  });
  __syncthreads();
  int b2 = 0;
  {
    int cum = above;
    for (int h = 255; h >= 0; --h) {
      if (cum + hist[h] >= S) { b2 = h; above = cum; break; }
      cum += hist[h];
    }
  }
  const uint32_t thr = ((uint32_t)b1 << 8) | (uint32_t)b2;
  const int need_eq = S - above;   // >= 1
  // ---- collection: keys above the threshold, and the tokens at it
  auto collect = [&](uint32_t k, int id) {
    if (k > thr) {
      const int at = atomicAdd(&n_sel, 1);
      if (at < kMaxDraftSupport) { sel_key[at] = k; sel_id[at] = id; }
    } else if (k == thr) {
      const int at = atomicAdd(&n_eq, 1);
      if (at < kEqCap) eq_id[at] = id;
    }
  };
  if (in_lds) {
    for (int i = tid; i < nn; i += kExpandThreads) collect(near_key[i], near_id[i]);
  } else {
    scan_row(row, nunits, [&](uint32_t bits, int id) { collect(bf16_key(bits), id); });
  }
  __syncthreads();
  if (n_eq > kEqCap) {
    if (tid == 0) atomicOr(&bad, (int)TAV_DEV_DRAFT_TIES);
    __syncthreads();
  }
  const int neq = min(n_eq, kEqCap);
  // the need_eq smallest ids among the tokens at the threshold: rank of each by id
  for (int i = tid; i < neq; i += kExpandThreads) {
    const int id = eq_id[i];
    int r = 0;
    for (int k = 0; k < neq; ++k) r += eq_id[k] < id;
    if (r < need_eq && above + r < kMaxDraftSupport) { sel_key[above + r] = thr; sel_id[above + r] = id; }
  }
  __syncthreads();
  // the support by (key desc, id asc) and its token-id order
  for (int i = tid; i < S; i += kExpandThreads) {
    const uint32_t k = sel_key[i];
    const int id = sel_id[i];
    int r = 0, ri = 0;
    for (int t = 0; t < S; ++t) {
      const uint32_t kt = sel_key[t];
      const int it = sel_id[t];
      r += kt > k || (kt == k && it < id);
      ri += it < id;
    }
    s_key[r] = k;
    s_id[r] = id;
    id_rank[r] = ri;
  }
  __syncthreads();
  const int err = bad;
  const bool hyb = a.hybrid == TAV_DRAFT_HYBRID_ALL || (a.hybrid == TAV_DRAFT_HYBRID_FIRST && j == 0);
  const int slots = a.slots, m = a.m;
  const int cbase = a.base[d] + j * slots;   // ids of this parent's candidates
  // ---- wave 0: q over the support (fp64), the pool, the children
  if (tid < 64) {
    const int lane = tid;
    const double zmax = (double)key_value(s_key[0]);
    const double invT = 1.0 / (double)a.temperature;
    double s1 = 0.0, st = 0.0;
    for (int i = lane; i < S; i += 64) {
      const double z = (double)key_value(s_key[i]) - zmax;
      const double e1 = exp(z), et = exp(z * invT);
      qd[i] = e1;
      qt[i] = et;
      s1 += e1;
      st += i >= m || !hyb ? et : 0.0;
    }
    for (int o = 32; o > 0; o >>= 1) {
      s1 += __shfl_xor(s1, o);
      st += __shfl_xor(st, o);
    }
    for (int i = lane; i < S; i += 64) {
      qd[i] /= s1;
      qt[i] = (hyb && i < m) ? 0.0 : qt[i] / st;   // the tail off the leads (hybrid pools)
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    const double pscore = cand_score[pid];
    if (hyb) {
      // the sampled token: inverse CDF in token-id order over the tail
      __shared__ double tail_by_id[kMaxDraftSupport];
      __shared__ int sorted_of_id[kMaxDraftSupport];
      for (int i = lane; i < S; i += 64) {
        tail_by_id[id_rank[i]] = qt[i];
        sorted_of_id[id_rank[i]] = i;
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
      // lane l holds id positions 2l, 2l+1 (S <= 128): inclusive prefix sums in fp64
      const double a0 = 2 * lane < S ? tail_by_id[2 * lane] : 0.0;
      const double a1 = 2 * lane + 1 < S ? tail_by_id[2 * lane + 1] : 0.0;
      double inc = a0 + a1;
      for (int o = 1; o < 64; o <<= 1) {
        const double y = __shfl_up(inc, o, 64);
        if (lane >= o) inc += y;
      }
      const double before = inc - (a0 + a1);
      const double u = (double)uniforms[(size_t)b * a.Kd + j];
      const double c0 = before + a0, c1 = inc;
      int pos = -1;
      if (2 * lane < S && a0 > 0.0 && c0 > u && before <= u) pos = 2 * lane;
      else if (2 * lane + 1 < S && a1 > 0.0 && c1 > u && c0 <= u) pos = 2 * lane + 1;
      unsigned long long hit = __ballot(pos >= 0);
      int ypos;
      if (hit) {
        ypos = __shfl(pos, __ffsll((long long)hit) - 1);
      } else {   // u at or past the rounded total: the last token with mass
        int lastp = -1;
        if (2 * lane + 1 < S && a1 > 0.0) lastp = 2 * lane + 1;
        else if (2 * lane < S && a0 > 0.0) lastp = 2 * lane;
        const unsigned long long has = __ballot(lastp >= 0);
        ypos = has ? __shfl(lastp, 63 - __clzll((long long)has)) : 0;
      }
      const int ys = sorted_of_id[ypos];   // the sampled entry in the logit order
      if (lane == 0) {
        const double zres = [&] { double t = 1.0; for (int i = 0; i < m; ++i) t -= qd[i]; return t; }();
        const double proxy_y = m > 0 ? fmin(qd[m - 1], zres) : qd[0] + (double)a.eps;
        int slot = 0, fi = m;
        for (; slot < slots; ++slot) {
          int src;
          double proxy;
          uint8_t smp = 0;
          if (slot < m) { src = slot; proxy = qd[slot]; }
          else if (slot == m) { src = ys; proxy = proxy_y; smp = 1; }
          else {
            if (fi == ys) ++fi;
            src = fi++;
            proxy = qd[src];
          }
          const int c = cbase + slot;
          cand_parent[c] = pid;
          cand_token[c] = s_id[src];
          cand_score[c] = pscore * proxy;
          cand_sampled[c] = smp;
          cand_depth[c] = (uint8_t)d;
        }
      }
      // the parent's draft row: support ids ascending, q~ there
      int32_t* ridx = a.row_idx + (cb + pid) * S;
      float* rval = a.row_val + (cb + pid) * S;
      for (int i = lane; i < S; i += 64) {
        ridx[id_rank[i]] = s_id[i];
        rval[id_rank[i]] = (float)qt[i];
      }
    } else if (lane == 0) {
      for (int slot = 0; slot < slots; ++slot) {
        const int c = cbase + slot;
        cand_parent[c] = pid;
        cand_token[c] = s_id[slot];
        cand_score[c] = pscore * qd[slot];
        cand_sampled[c] = 0;
        cand_depth[c] = (uint8_t)d;
      }
    }
    if (lane == 0 && err) {
      atomicOr(a.status, (uint32_t)err);
      atomicOr(a.seq_err + b, (uint32_t)err);
    }
  }
}

// The next parents: the K best of depth d's candidates by (score desc, id asc); one block per
// sequence (rank of each candidate = the number ahead of it).
__global__ __launch_bounds__(kDraftThreads) void draft_frontier_kernel(DraftArgs a, int d, int32_t* frontier_out) {
  __shared__ double sc[kMaxDraftCandidates];
  const int b = blockIdx.x, tid = threadIdx.x;
  const size_t cb = (size_t)b * a.C;
  const int c0 = a.base[d], n = a.base[d + 1] - c0;
  const int kn = a.kcount[d + 1];   // parents of depth d + 1 (0 after the last depth)
  for (int i = tid; i < a.K; i += kDraftThreads) {
    a.frontier[(size_t)b * a.K + i] = -1;
    if (frontier_out) frontier_out[(size_t)b * a.K + i] = -1;
  }
  for (int i = tid; i < n; i += kDraftThreads) sc[i] = a.cand_score[cb + c0 + i];
  __syncthreads();
  for (int i = tid; i < n; i += kDraftThreads) {
    const double s = sc[i];
    int r = 0;
#pragma unroll 8
    for (int t = 0; t < n; ++t) {
      const double st = sc[t];
      r += st > s || (st == s && t < i);
    }
    if (r < kn) {
      a.frontier[(size_t)b * a.K + r] = c0 + i;
      if (frontier_out) frontier_out[(size_t)b * a.K + r] = c0 + i;
    }
  }
}

// Global prune to R nodes by (score desc, depth asc, id asc); nodes renumbered by (depth, id),
// which is ascending id; outputs per sequence b at rows b * (R + 1) ... (b + 1) * (R + 1) - 1.
__global__ __launch_bounds__(kExpandThreads) void draft_prune_kernel(DraftArgs a, DraftOut o) {
  __shared__ uint8_t kept[kMaxDraftCandidates];
  __shared__ int new_id[kMaxDraftCandidates];
  __shared__ uint64_t key[kMaxDraftCandidates];
  __shared__ uint8_t dp[kMaxDraftCandidates];
  __shared__ int row_cand[kMaxDraftCandidates];   // also the candidates tied at the threshold
  __shared__ int hist[256];
  __shared__ int red[16];
  __shared__ int n_rows, n_tie, sel_digit, sel_above;
  const int b = blockIdx.x, tid = threadIdx.x;
  const size_t cb = (size_t)b * a.C;
  const int C = a.base[a.D + 1], R = a.R;
  // the scores are products of probabilities (>= 0): their fp64 bit patterns order as integers
  for (int c = tid; c < C; c += kExpandThreads) {
    key[c] = (uint64_t)__double_as_longlong(a.cand_score[cb + c]);
    dp[c] = a.cand_depth[cb + c];
    kept[c] = 1;
  }
  if (tid == 0) n_tie = 0;
  __syncthreads();
  const int Rk = min(R, C - 1);   // non-root candidates kept
  if (Rk < C - 1) {
    // the Rk-th largest key among candidates 1..C-1: radix select, one byte per pass from the top
    uint64_t prefix = 0;
    int above = 0;
    for (int shift = 56; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += kExpandThreads) hist[i] = 0;
      __syncthreads();
      for (int c = 1 + tid; c < C; c += kExpandThreads) {
        const uint64_t k = key[c];
        if (shift == 56 || ((k ^ prefix) >> (shift + 8)) == 0) atomicAdd(&hist[(k >> shift) & 0xFF], 1);
      }
      __syncthreads();
      // bins from the top (waves 0-3, one bin per lane): inclusive scan; the bin where the count
      // reaches Rk is the next byte
      int v = 0, inc = 0;
      if (tid < 256) {
        v = hist[255 - tid];
        inc = v;
        const int lane = tid & 63;
        for (int o2 = 1; o2 < 64; o2 <<= 1) {
          const int y = __shfl_up(inc, o2, 64);
          if (lane >= o2) inc += y;
        }
        if (lane == 63) red[tid >> 6] = inc;
      }
      __syncthreads();
      if (tid < 256) {
        for (int w = 0; w < (tid >> 6); ++w) inc += red[w];
        if (above + inc >= Rk && above + inc - v < Rk) { sel_digit = 255 - tid; sel_above = above + inc - v; }
      }
      __syncthreads();
      prefix |= (uint64_t)sel_digit << shift;
      above = sel_above;
    }
    // candidates tied at the threshold: the first Rk - above by (depth asc, id asc)
    for (int c = 1 + tid; c < C; c += kExpandThreads) {
      const uint64_t k = key[c];
      kept[c] = k > prefix;
      if (k == prefix) row_cand[atomicAdd(&n_tie, 1)] = c;
    }
    __syncthreads();
    const int nt = n_tie, need = Rk - above;
    for (int i = tid; i < nt; i += kExpandThreads) {
      const int c = row_cand[i], dc = dp[c];
      int r = 0;
      for (int t = 0; t < nt; ++t) {
        const int ct = row_cand[t], dt = dp[ct];
        r += dt < dc || (dt == dc && ct < c);
      }
      kept[c] = r < need;
    }
  }
  __syncthreads();
  // ids of the kept nodes in ascending candidate id (the root first): exclusive block scan of
  // the kept flags, two candidates per thread
  {
    const int c0 = 2 * tid;
    const int k0 = c0 < C ? kept[c0] : 0, k1 = c0 + 1 < C ? kept[c0 + 1] : 0;
    int inc = k0 + k1;
    const int lane = tid & 63, wv = tid >> 6;
    for (int o2 = 1; o2 < 64; o2 <<= 1) {
      const int y = __shfl_up(inc, o2, 64);
      if (lane >= o2) inc += y;
    }
    if (lane == 63) red[wv] = inc;
    __syncthreads();
    int before = inc - (k0 + k1);
    int total = 0;
    for (int w = 0; w < 16; ++w) {
      before += w < wv ? red[w] : 0;
      total += red[w];
    }
    if (c0 < C) new_id[c0] = k0 ? before : -1;
    if (c0 + 1 < C) new_id[c0 + 1] = k1 ? before + k0 : -1;
    if (tid == 0) n_rows = 0;
    __syncthreads();
    if (tid == 0) red[0] = total;
  }
  const size_t ob = (size_t)b * (R + 1);
  uint32_t err = 0;
  for (int c = tid; c < C; c += kExpandThreads) {
    const int v = new_id[c];
    if (v < 0) continue;
    const int p = a.cand_parent[cb + c];
    const int pv = c == 0 ? -1 : new_id[p];
    if (c > 0 && pv < 0) err |= TAV_DEV_BAD_PARENT;   // not ancestor-closed (cannot happen)
    o.parent[ob + v] = pv;
    o.token[ob + v] = c == 0 ? -1 : a.cand_token[cb + c];
    const uint8_t smp = c == 0 ? 0 : a.cand_sampled[cb + c];
    o.sampled[ob + v] = smp;
    if (o.cand_id) o.cand_id[ob + v] = c;
    // a kept sampled node: its parent's draft row goes to the parent's output row (a pool has
    // at most one sampled slot, so each parent is listed once)
    if (smp && pv >= 0) row_cand[atomicAdd(&n_rows, 1)] = p;
  }
  __syncthreads();
  for (int c = tid; c < C; c += kExpandThreads) {
    const int v = new_id[c];
    if (v >= 0) o.draft_row[ob + v] = -1;
  }
  __syncthreads();
  const int nr = n_rows;
  for (int r = tid; r < nr; r += kExpandThreads) {
    const int v = new_id[row_cand[r]];
    o.draft_row[ob + v] = (int)(ob + v);
  }
  for (int e = tid; e < nr * a.S; e += kExpandThreads) {
    const int r = e / a.S, i = e - r * a.S;
    const int c = row_cand[r];
    const int v = new_id[c];
    o.draft_idx[(ob + v) * a.S + i] = a.row_idx[(cb + c) * a.S + i];
    o.draft_val[(ob + v) * a.S + i] = a.row_val[(cb + c) * a.S + i];
  }
  if (red[0] != R + 1) err |= TAV_DEV_PLAN_MISMATCH;
  if (err) {
    atomicOr(a.status, err);
    atomicOr(a.seq_err + b, err);
  }
}

}  // namespace

hipError_t launch_draft_expand(const DraftArgs& a, int d, const uint16_t* logits, const float* uniforms,
                               int32_t* frontier_out, hipStream_t s) {
  draft_expand_kernel<<<a.B * a.Kd, kExpandThreads, 0, s>>>(a, d, logits, uniforms);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  draft_frontier_kernel<<<a.B, kDraftThreads, 0, s>>>(a, d, frontier_out);
  return hipGetLastError();
}

hipError_t launch_draft_prune(const DraftArgs& a, const DraftOut& o, hipStream_t s) {
  draft_prune_kernel<<<a.B, kExpandThreads, 0, s>>>(a, o);
  return hipGetLastError();
}

}  // namespace tav
