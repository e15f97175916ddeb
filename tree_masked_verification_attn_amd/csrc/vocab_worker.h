// Per-node vocabulary work of the verification: a streaming kernel (one workgroup per node,
// taking nodes from a queue) and a pick kernel (one wave per node).
//
// RheoSampling, Section 3.3 Algorithm 1 (RheoVerification): the target distribution at
// node v is p = softmax(l / T) (temperature only in sampling and verification, Section
// 5.4); when v has a sampled child Y drawn from q~ (the draft row of v), Y is tested with
// min(1, p(Y) / q~(Y)) and a rejection replaces p by the residual r = norm(max(0, p - q~));
// the other children are tested against r (or p) one by one, each rejection zeroing its
// token; if the walk ends at v the output token is drawn from what is left.  Without a
// sampled child this is the sequential rejection of Progressive Tree Drafting (Section
// 3.2, Appendix E / F).
//
// For node v the streaming kernel computes, with the logits row streamed from HBM once:
//   M = max l / T, S = sum exp(l / T - M)                (the normaliser of p),
//   Z = sum (p - q~)+ when v has a dense draft row        (the normaliser of r),
//   the weight of every chunk of 512 (bf16) or 256 (f32) tokens under p, or under (p - q~)+,
// and leaves them in the workspace; the pick kernel then takes, for every node at once, p and q~
// at each child's token (the walk's tests) and the token the final draw at v would give (inverse
// CDF in token order with u[v][1], deterministic children's tokens removed).
// Pass 1 streams the row in steps of 64 KB (512 threads x 8 sixteen-byte units, the next step's
// loads in flight while the current one is summed): each wave keeps the largest raw logit m of
// its part of the step as a reference and writes sum exp2(l log2e / T - ref(m)) of every chunk of
// 64 units (one unit per lane) to LDS.  M and S follow from these pieces in fp64.  Pass 2 (nodes
// with a sampled child and a dense draft row) streams the draft row with the logits row again
// (the row's first 128 KB kept in LDS, the rest mostly from the cache) and replaces the chunk
// weights with those of (p - q~)+.  Greedy rows (T = 0) take one pass for the argmax.  The pick:
// point values of the children, the deterministic children's weights taken out of their chunks,
// an fp64 scan over the chunks for u * W, and one chunk re-read.  With sparse draft rows (at most
// 128 support tokens per row, RheoSampling Section 3.2) there is no pass 2: the pick takes the
// support's min(p, q~) out of the chunk weights of p and sums Z over the support.  Nodes are taken
// from a device queue, in the order of an index list (nodes with a dense draft row first, so that
// the long items do not come last); a worker never waits for another workgroup, and claims its
// next node while it streams the current one (after a greedy row, whose pass leaves the LDS cache
// unused, it also copies the next node's first step into that cache).
#pragma once

#include <type_traits>

#include "tav_internal.h"

namespace tav {
namespace vw {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kCwBatch = 8;   // chunk weights per lane loaded together by the pick
constexpr int kNoffLds = 256;   // sequence offsets a worker keeps in LDS (more sequences: read from memory)

// A worker of NT threads reading NU sixteen-byte units per thread and step.  A chunk is 64 units,
// one per lane of a wave, so chunk k * waves + w of a step is unit k of every lane of wave w.
template <int NT, int NU, int CACHE_KB>
struct Cfg {
  static constexpr int kThreads = NT;
  static constexpr int kWaves = NT / 64;
  static constexpr int kUnits = NU;
  static constexpr int kStepUnits = NT * NU;
  static constexpr int kChunksPerStep = kStepUnits / 64;
  static constexpr int kMaxSteps = kMaxChunks / kChunksPerStep;   // rows of up to kMaxChunks chunks
  static constexpr int kMaxPieces = kMaxSteps * kWaves;           // (step, wave) references
  // the first steps of a logits row kept in LDS for the second pass (nodes with a draft row)
  static constexpr int kCacheSteps = (CACHE_KB * 1024) / (kStepUnits * 16);
  static constexpr int kCacheUnits = kCacheSteps > 0 ? kCacheSteps * kStepUnits : 1;
  static_assert((NU == 2 || NU % 4 == 0) && NU <= 64 && NT % 64 == 0, "worker shape");
};

template <class C>
struct Lds {
  float cw[kMaxChunks];                      // chunk weights
  float part[C::kWaves][C::kUnits * 64];     // per-wave transpose of unit sums into chunk sums
  float ref_m[C::kMaxPieces];                // largest raw logit of each (step, wave) piece
  double ref_s[C::kMaxPieces];               // sum exp2(l log2e / T - ref) of each piece
  double red_d[C::kWaves];
  float g_best[C::kWaves];                   // greedy rows: each wave's largest logit ...
  int g_idx[C::kWaves];                      // ... and its smallest token id
  int item, cnt, ns, err, next;
  int noff[kNoffLds];                        // node_offsets[0..B] when B < kNoffLds
  uint4 lc[C::kCacheUnits];                  // dense draft rows: the logits row's first kCacheSteps
                                             // steps (each thread its own units)
};

// The pick's LDS, one per wave.
struct PickLds {
  float cw[kMaxChunks];
  int kid_id[kMaxChildren];                  // children of the node (sequence-local ids, ascending) ...
  int kid_tok[kMaxChildren];                 // ... their tokens
  float kid_w[kMaxChildren];                 // ... their weights in the final draw's chunks
  double kid_p[kMaxChildren];                // ... p (fp64) and q~ at their tokens under this node's
  float kid_q[kMaxChildren];                 // distributions, their acceptance uniforms
  float kid_u[kMaxChildren];
  uint8_t kid_smp[kMaxChildren];             // ... and sampled flags
  int sp_idx[kMaxDraftSupport];              // sparse draft row: support (ascending ids), q~ there
  float sp_val[kMaxDraftSupport];            // and the part of each token's p taken out of its
  float sp_take[kMaxDraftSupport];           // chunk (min(p, q~))
  uint32_t zm[64];                           // final draw: each lane's positions holding a deterministic child
};

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
__device__ inline float logit_at(const void* logits, size_t idx);
template <>
__device__ inline float logit_at<uint16_t>(const void* logits, size_t idx) {
  return __uint_as_float(((uint32_t)((const uint16_t*)logits)[idx]) << 16);
}
template <>
__device__ inline float logit_at<float>(const void* logits, size_t idx) {
  return ((const float*)logits)[idx];
}

// Cross-lane moves for wave reductions, register to register: DPP row operations within rows of 16
// lanes (quad permutations, the 8- and 16-lane mirrors) and the lane swaps between rows.  Applied in
// the order 1, 2, 3, 4, 5, 6 each combines groups of 2, 4, 8, 16, 32, 64 lanes; every lane of a
// group ends with the same value.
constexpr int kDppXor1 = 0xB1;       // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;       // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;
template <int STAGE>
__device__ inline uint32_t lane_move(uint32_t x) {
  if constexpr (STAGE == 1) return __builtin_amdgcn_update_dpp(0, x, kDppXor1, 0xF, 0xF, false);
  else if constexpr (STAGE == 2) return __builtin_amdgcn_update_dpp(0, x, kDppXor2, 0xF, 0xF, false);
  else if constexpr (STAGE == 3) return __builtin_amdgcn_update_dpp(0, x, kDppHalfMirror, 0xF, 0xF, false);
  else if constexpr (STAGE == 4) return __builtin_amdgcn_update_dpp(0, x, kDppMirror, 0xF, 0xF, false);
  else if constexpr (STAGE == 5) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);   // the other row of 32
    return (threadIdx.x & 16) ? r[0] : r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);   // the other half
    return (threadIdx.x & 32) ? r[0] : r[1];
  }
}
template <int STAGE>
__device__ inline float lane_move_f(float x) { return __uint_as_float(lane_move<STAGE>(__float_as_uint(x))); }
template <int STAGE>
__device__ inline double lane_move_d(double x) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(x);
  const uint32_t lo = lane_move<STAGE>((uint32_t)b), hi = lane_move<STAGE>((uint32_t)(b >> 32));
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

__device__ inline double wave_sum_d(double x) {
  x += lane_move_d<1>(x);
  x += lane_move_d<2>(x);
  x += lane_move_d<3>(x);
  x += lane_move_d<4>(x);
  x += lane_move_d<5>(x);
  x += lane_move_d<6>(x);
  return x;
}
__device__ inline float wave_max_f(float x) {
  x = fmaxf(x, lane_move_f<1>(x));
  x = fmaxf(x, lane_move_f<2>(x));
  x = fmaxf(x, lane_move_f<3>(x));
  x = fmaxf(x, lane_move_f<4>(x));
  x = fmaxf(x, lane_move_f<5>(x));
  x = fmaxf(x, lane_move_f<6>(x));
  return x;
}
__device__ inline void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Prefix sums over the 64 lanes of a wave without LDS round trips: inside each row of 16 lanes by
// DPP row shifts (a lane whose source lies outside its row adds 0), then the rows' totals read with
// readlane and added to the later rows.  A fixed order of additions (the same on every run).  Every
// lane of the wave must be active.
template <int CTRL>
__device__ inline uint32_t dpp0(uint32_t x) { return __builtin_amdgcn_update_dpp(0u, x, CTRL, 0xF, 0xF, false); }
constexpr int kDppRowShr = 0x110;    // row_shr:n = kDppRowShr + n
constexpr int kDppWaveShr1 = 0x138;  // wave_shr:1 (lane i takes lane i - 1, lane 0 takes 0)
template <int CTRL>
__device__ inline double dpp0_d(double x) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(x);
  const uint32_t lo = dpp0<CTRL>((uint32_t)b), hi = dpp0<CTRL>((uint32_t)(b >> 32));
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}
__device__ inline double readlane_d(double x, int l) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(x);
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)b, l);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}
__device__ inline float readlane_f(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
__device__ inline double wave_scan_d(double x) {   // inclusive
  x += dpp0_d<kDppRowShr + 1>(x);
  x += dpp0_d<kDppRowShr + 2>(x);
  x += dpp0_d<kDppRowShr + 4>(x);
  x += dpp0_d<kDppRowShr + 8>(x);
  const double t0 = readlane_d(x, 15), t1 = readlane_d(x, 31), t2 = readlane_d(x, 47);
  const double t01 = t0 + t1;
  const int row = (threadIdx.x & 63) >> 4;
  return x + (row == 0 ? 0.0 : row == 1 ? t0 : row == 2 ? t01 : t01 + t2);
}
__device__ inline float wave_scan_f(float x) {   // inclusive
  x += __uint_as_float(dpp0<kDppRowShr + 1>(__float_as_uint(x)));
  x += __uint_as_float(dpp0<kDppRowShr + 2>(__float_as_uint(x)));
  x += __uint_as_float(dpp0<kDppRowShr + 4>(__float_as_uint(x)));
  x += __uint_as_float(dpp0<kDppRowShr + 8>(__float_as_uint(x)));
  const float t0 = readlane_f(x, 15), t1 = readlane_f(x, 31), t2 = readlane_f(x, 47);
  const float t01 = t0 + t1;
  const int row = (threadIdx.x & 63) >> 4;
  return x + (row == 0 ? 0.f : row == 1 ? t0 : row == 2 ? t01 : t01 + t2);
}
__device__ inline uint32_t wave_or(uint32_t x) {
  x |= lane_move<1>(x);
  x |= lane_move<2>(x);
  x |= lane_move<3>(x);
  x |= lane_move<4>(x);
  x |= lane_move<5>(x);
  x |= lane_move<6>(x);
  return x;
}

// log2-domain reference of a piece maximum (a piece of -inf logits uses 0; its sum is 0).
__device__ inline float ref_l2(float m_raw, float invT) {
  return (m_raw == -INFINITY ? 0.f : m_raw * invT) * kLog2e;
}

// Sums x[k] over the 64 lanes of the wave for each k (chunk k * waves + wave of the step),
// through the wave's LDS transpose buffer; returns chunk (lane / (64 / NU))'s total in every lane
// of each group of 64 / NU lanes.
template <int NU>
__device__ inline float wave_chunk_totals(const float (&x)[NU], float* part, int lane) {
  constexpr int TPC = 64 / NU;   // lanes per chunk, each summing NU values
#pragma unroll
  for (int k = 0; k < NU; ++k) part[k * 64 + lane] = x[k];
  wave_sync();
  const float* src = part + (lane / TPC) * 64 + (lane % TPC) * NU;
  float t = 0.f;
  if constexpr (NU % 4 == 0) {
#pragma unroll
    for (int i = 0; i < NU; i += 4) {
      const float4 a4 = *(const float4*)(src + i);
      t += (a4.x + a4.y) + (a4.z + a4.w);
    }
  } else {
#pragma unroll
    for (int i = 0; i < NU; i += 2) {
      const float2 a2 = *(const float2*)(src + i);
      t += a2.x + a2.y;
    }
  }
  // the TPC lanes of each chunk (aligned groups of 8, 16 or 32)
  if constexpr (TPC >= 2) t += lane_move_f<1>(t);
  if constexpr (TPC >= 4) t += lane_move_f<2>(t);
  if constexpr (TPC >= 8) t += lane_move_f<3>(t);
  if constexpr (TPC >= 16) t += lane_move_f<4>(t);
  if constexpr (TPC >= 32) t += lane_move_f<5>(t);
  wave_sync();   // the buffer is reused by the next step
  return t;
}

template <typename LT, class C>
__device__ inline void load_step(uint4 (&r)[C::kUnits], const LT* row, int step, int tid, int nunits) {
  constexpr int EPU = 16 / sizeof(LT);
#pragma unroll
  for (int k = 0; k < C::kUnits; ++k) {
    const int u = step * C::kStepUnits + k * C::kThreads + tid;
    r[k] = *(const uint4*)(row + (size_t)(u < nunits ? u : 0) * EPU);
  }
}

__device__ inline void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// The first step of a row copied from memory straight into the LDS cache, in the cache's layout
// (unit k * NT + tid of the step for thread tid), holding no register while in flight: lane i of wave w
// copies units k * NT + 64 w + i.  Issued through inline assembly, so that the compiler does not wait for
// the copies before unrelated LDS accesses; every later load of the wave completes after them (the
// counter is in order), so once a later load has been waited for, the cache holds the step.
template <typename LT, class C>
__device__ inline void dma_first_step(const LT* row, int nunits, uint32_t lc_addr, int tid) {
  constexpr int EPU = 16 / sizeof(LT);
  const int wave = tid >> 6;
#pragma unroll
  for (int k = 0; k < C::kUnits; ++k) {
    const int u = k * C::kThreads + tid;
    const LT* src = row + (size_t)(u < nunits ? u : 0) * EPU;
    const uint32_t dst = lc_addr + (uint32_t)((k * C::kThreads + wave * 64) * 16);
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, off"
        :: "v"(src), "s"(__builtin_amdgcn_readfirstlane(dst)) : "memory", "m0");
  }
}

// (value, token id) pairs: the larger value wins, equal values go to the smaller id.
__device__ inline void better_of(float& best, int& bi, float ob, int oi) {
  if (ob > best || (ob == best && (unsigned)oi < (unsigned)bi)) {
    best = ob;
    bi = oi;
  }
}

// Greedy decoding (temperature 0; Progressive Tree Drafting, Section 3.2): the node's verification
// token is its highest-probability prediction, the argmax of the logits (smallest id among equal
// maxima).  One pass over the row (the first step's loads already in flight in cur) with no
// exponentials; the walk accepts the child carrying that token.
template <typename LT, class C>
__device__ void greedy_stream(const VocabArgs& a, Lds<C>& L, int v, int b, int s0, int n, uint4 (&cur)[C::kUnits],
                              const LT* row, int nunits, int nsteps) {
  constexpr int kThreads = C::kThreads, kUnits = C::kUnits, kStepUnits = C::kStepUnits;
  constexpr int EPU = 16 / sizeof(LT);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float best = -INFINITY;
  int bu = -1;   // the unit holding this thread's first largest logit
  bool bad = false;
  for (int s = 0; s < nsteps; ++s) {
    uint4 nxt[kUnits];
    if (s + 1 < nsteps) load_step<LT, C>(nxt, row, s + 1, tid, nunits);
    // per-unit maxima (NaN ignored by the max, caught by the unordered compare; +inf caught below)
    float um[kUnits];
#pragma unroll
    for (int k = 0; k < kUnits; ++k) {
      const int u = s * kStepUnits + k * kThreads + tid;
      um[k] = -INFINITY;
      if (u < nunits) {
#pragma unroll
        for (int e = 0; e < EPU; ++e) {
          const float x = unit_elem<LT>(cur[k], e);
          bad |= x != x;
          um[k] = fmaxf(um[k], x);
        }
      }
    }
    float mx = um[0];
#pragma unroll
    for (int k = 1; k < kUnits; ++k) mx = fmaxf(mx, um[k]);
    if (mx > best) {   // a new best: its first unit (positions rise with (step, unit) in a thread)
      best = mx;
      int kk = kUnits - 1;
#pragma unroll
      for (int k = kUnits - 2; k >= 0; --k) kk = um[k] == mx ? k : kk;
      bu = s * kStepUnits + kk * kThreads + tid;
    }
    if (s + 1 < nsteps) {
#pragma unroll
      for (int k = 0; k < kUnits; ++k) cur[k] = nxt[k];
    }
  }
  wait_vm0();   // (nothing else is in flight: the copies of the next node's first step, for one-step rows)
  bad |= best == INFINITY;
  // the position inside the best unit (one re-read of that unit, from the cache)
  int bi = -1;
  if (bu >= 0) {
    const uint4 bunit = *(const uint4*)(row + (size_t)bu * EPU);
    int ee = EPU - 1;
#pragma unroll
    for (int e = EPU - 2; e >= 0; --e) ee = unit_elem<LT>(bunit, e) == best ? e : ee;
    bi = bu * EPU + ee;
  }
#define TAV_GREEDY_STAGE(S)                                                                  \
  better_of(best, bi, lane_move_f<S>(best), (int)lane_move<S>((uint32_t)bi));
  TAV_GREEDY_STAGE(1) TAV_GREEDY_STAGE(2) TAV_GREEDY_STAGE(3) TAV_GREEDY_STAGE(4) TAV_GREEDY_STAGE(5)
  TAV_GREEDY_STAGE(6)
#undef TAV_GREEDY_STAGE
  const bool any_bad = __ballot(bad) != 0ull;
  if (lane == 0) {
    L.g_best[wave] = best;
    L.g_idx[wave] = bi;
    if (any_bad) atomicOr(&L.err, (int)TAV_DEV_NONFINITE_LOGITS);
  }
  __syncthreads();
  if (tid == 0) {
    float M = -INFINITY;
    int A = -1;
#pragma unroll
    for (int w = 0; w < C::kWaves; ++w) better_of(M, A, L.g_best[w], L.g_idx[w]);
    NodeRec r;
    r.S = 1.0;
    r.Z = 0.0;
    r.M = M;
    r.A = A;
    r.b = b;
    r.err = (uint32_t)L.err;
    r.flags = kRecGreedy;
    r.s0 = s0;
    r.n = n;
    r.T = 0.f;   // (greedy rows: temperature 0)
    a.rec[v] = r;
  }
}

// The streaming part of node v: its sequence, whether it has a sampled child, then pass 1 (and
// pass 2), the chunk weights and the node's record into the workspace.  Thread 0 claims the next
// queue slot into qn (read back after the node).
template <typename LT, class C>
__device__ void stream_node(const VocabArgs& a, Lds<C>& L, int v, int& qn, bool& pre_lds) {
  constexpr int kThreads = C::kThreads, kWaves = C::kWaves, kUnits = C::kUnits;
  constexpr int kStepUnits = C::kStepUnits, kChunksPerStep = C::kChunksPerStep;
  constexpr int TPC = 64 / kUnits;   // lanes per chunk total
  constexpr int EPU = 16 / sizeof(LT);
  constexpr int QPU = EPU / 4;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int V = a.V, nunits = V / EPU, nch = a.nch;
  const int nsteps = (nunits + kStepUnits - 1) / kStepUnits;
  const LT* row = (const LT*)a.logits + (size_t)v * V;
  // the first step: from the LDS cache when the previous node of this worker copied it there (its
  // loads were waited for long ago), else its loads go out before anything else; then the claim of the
  // next node and its id
  uint4 cur[kUnits];
  if (pre_lds) {
#pragma unroll
    for (int k = 0; k < kUnits; ++k) cur[k] = L.lc[k * kThreads + tid];
  } else {
    load_step<LT, C>(cur, row, 0, tid, nunits);
  }
  pre_lds = false;
  int nv = -1;
  if (tid == 0) {
    qn = atomicAdd(a.queue, 1);
    nv = qn < a.N ? a.order[qn] : -1;
  }
  // sequence of v: the number of sequence ends node_offsets[1..B] that are <= v (from the worker's LDS
  // copy when the batch has at most kNoffLds sequences)
  const bool noff_lds = a.B < kNoffLds;
  if (tid == 0) { L.cnt = 0; L.ns = 0; L.err = 0; }
  __syncthreads();
  {
    int c = 0;
    if (noff_lds) {
      for (int t = tid + 1; t <= a.B; t += kThreads) c += L.noff[t] <= v;
    } else {
      for (int t = tid + 1; t <= a.B; t += kThreads) c += a.node_offsets[t] <= v;
    }
    if (c) atomicAdd(&L.cnt, c);
  }
  __syncthreads();
  const int b = L.cnt < a.B ? L.cnt : a.B - 1;
  const int s0 = noff_lds ? L.noff[b] : a.node_offsets[b];
  const int n = (noff_lds ? L.noff[b + 1] : a.node_offsets[b + 1]) - s0;
  const float Tb = a.temperature[b];
  const float invT = 1.f / Tb;
  const float invTl2 = invT * kLog2e;
  const int dr = a.draft_row[v];
  const bool dr_ok = dr >= 0 && dr < a.R;
  // whether v has a sampled child (the pick checks the children in full)
  {
    int ns = 0;
    for (int c = tid + 1; c < n; c += kThreads) {
      const int pc = a.parent[s0 + c];
      const uint8_t sm = a.sampled[s0 + c];
      ns += pc == v - s0 && sm != 0;
    }
    if (ns) atomicAdd(&L.ns, ns);
  }
  if (tid == 0) L.next = nv;
  __syncthreads();
  // a greedy row leaves the LDS cache unused and its pass (no exponentials) keeps too few bytes in flight:
  // the next node's first step is copied into the cache while this node streams
  const int next_v = __builtin_amdgcn_readfirstlane(L.next);
  const bool dense_draft = L.ns > 0 && dr_ok && a.K == 0 && Tb != 0.f;
  if (Tb == 0.f && next_v >= 0) {
    const uint32_t lc_addr = (uint32_t)(size_t)(__attribute__((address_space(3))) uint4*)&L.lc[0];
    dma_first_step<LT, C>((const LT*)a.logits + (size_t)next_v * V, nunits, lc_addr, tid);
    pre_lds = true;
  }
  if (Tb == 0.f) {   // greedy decoding: the verification token is the argmax
    greedy_stream<LT, C>(a, L, v, b, s0, n, cur, row, nunits, nsteps);
    return;
  }
  // ---- pass 1: per-piece references and sums, chunk weights relative to their piece
  float* part = L.part[wave];
  for (int s = 0; s < nsteps; ++s) {
    uint4 nxt[kUnits];
    if (s + 1 < nsteps) load_step<LT, C>(nxt, row, s + 1, tid, nunits);
    const int ub = s * kStepUnits + tid;
    float mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < kUnits; ++k)
      if (ub + k * kThreads < nunits) {
#pragma unroll
        for (int e = 0; e < EPU; ++e) mx = fmaxf(mx, unit_elem<LT>(cur[k], e));
      }
    mx = wave_max_f(mx);
    const float r2 = ref_l2(mx, invT);
    // a NaN or +inf logit makes the sum NaN, which is reported by the pick
    float su[kUnits];
#pragma unroll
    for (int k = 0; k < kUnits; ++k) {
      su[k] = 0.f;
      if (ub + k * kThreads < nunits) {
#pragma unroll
        for (int e = 0; e < EPU; ++e) su[k] += __builtin_amdgcn_exp2f(unit_elem<LT>(cur[k], e) * invTl2 - r2);
      }
    }
    if (dense_draft && s < C::kCacheSteps) {
      // kept for the second pass, which reads them back in the same thread
#pragma unroll
      for (int k = 0; k < kUnits; ++k) L.lc[s * kStepUnits + k * kThreads + tid] = cur[k];
    }
    const float ct = wave_chunk_totals(su, part, lane);
    const int c = s * kChunksPerStep + (lane / TPC) * kWaves + wave;
    if ((lane % TPC) == 0 && c < nch) L.cw[c] = ct;
    // the piece's sum in fp64: its chunk totals (each already in all TPC lanes of its group) added
    // across the groups
    double sd = (double)ct;
    if constexpr (TPC <= 1) sd += lane_move_d<1>(sd);
    if constexpr (TPC <= 2) sd += lane_move_d<2>(sd);
    if constexpr (TPC <= 4) sd += lane_move_d<3>(sd);
    if constexpr (TPC <= 8) sd += lane_move_d<4>(sd);
    if constexpr (TPC <= 16) sd += lane_move_d<5>(sd);
    if constexpr (TPC <= 32) sd += lane_move_d<6>(sd);
    if (lane == 0) {
      L.ref_m[s * kWaves + wave] = mx;
      L.ref_s[s * kWaves + wave] = sd;
    }
    if (s + 1 < nsteps) {
#pragma unroll
      for (int k = 0; k < kUnits; ++k) cur[k] = nxt[k];
    }
  }
  __syncthreads();
  // ---- M and S from the pieces (every wave computes the same values)
  const int npieces = nsteps * kWaves;
  float ml = -INFINITY;
  for (int i = lane; i < npieces; i += 64) ml = fmaxf(ml, L.ref_m[i]);
  const float Mraw = wave_max_f(ml);
  const bool no_mass = Mraw == -INFINITY;
  const float M = no_mass ? 0.f : Mraw * invT;
  const float Ml2 = M * kLog2e;
  double sc = 0.0;
  for (int i = lane; i < npieces; i += 64) {
    const double si = L.ref_s[i];
    if (si != 0.0) sc += si * exp2((double)ref_l2(L.ref_m[i], invT) - (double)Ml2);
  }
  const double S = wave_sum_d(sc);
  const float invS = (float)(1.0 / S);
  double Zt = 0.0;
  if (dense_draft) {
    // ---- pass 2: chunk weights of (p - q~)+ and their total Z.  Each step is taken in two
    // halves of kUnits / 2 units per thread, one half computed while the other's loads fly.  The
    // steps in reverse (the last steps of pass 1 are the likeliest still to be in the cache): first
    // those read from memory, then those in the LDS cache, in two loops, so that every load has
    // one known address space (a load through a pointer chosen between LDS and memory is a flat
    // load, which makes every use wait for all loads in flight).
    constexpr int HU = kUnits / 2;
    const float* drow = a.draft + (size_t)dr * V;
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const __attribute__((address_space(3))) u32x4* lc3 = (const __attribute__((address_space(3))) u32x4*)&L.lc[0];
    const __attribute__((address_space(1))) u32x4* row1 = (const __attribute__((address_space(1))) u32x4*)row;
    auto load_half = [&](uint4 (&r)[HU], float4 (&q)[HU][QPU], int s, int h, auto cached)
        __attribute__((always_inline)) {
#pragma unroll
      for (int k = 0; k < HU; ++k) {
        const int u = s * kStepUnits + (h * HU + k) * kThreads + tid;
        const int uc = u < nunits ? u : 0;
        u32x4 x;
        if constexpr (decltype(cached)::value) x = lc3[u];
        else x = row1[uc];
        r[k] = make_uint4(x[0], x[1], x[2], x[3]);
#pragma unroll
        for (int i = 0; i < QPU; ++i) q[k][i] = *(const float4*)(drow + (size_t)uc * EPU + 4 * i);
      }
    };
    float wu[kUnits];
    auto compute_half = [&](const uint4 (&r)[HU], const float4 (&q)[HU][QPU], int s, int h)
        __attribute__((always_inline)) {
#pragma unroll
      for (int k = 0; k < HU; ++k) {
        float w = 0.f;
        if (s * kStepUnits + (h * HU + k) * kThreads + tid < nunits) {
#pragma unroll
          for (int e = 0; e < EPU; ++e) {
            const float4 q4 = q[k][e / 4];
            const float qe = (e & 3) == 0 ? q4.x : (e & 3) == 1 ? q4.y : (e & 3) == 2 ? q4.z : q4.w;
            const float p = __builtin_amdgcn_exp2f(unit_elem<LT>(r[k], e) * invTl2 - Ml2) * invS;
            w += fmaxf(0.f, p - qe);
          }
        }
        wu[h * HU + k] = w;
      }
    };
    double zl = 0.0;
    auto finish = [&](int s) __attribute__((always_inline)) {
#pragma unroll
      for (int k = 0; k < kUnits; ++k) zl += (double)wu[k];
      const float ct = wave_chunk_totals(wu, part, lane);
      const int c = s * kChunksPerStep + (lane / TPC) * kWaves + wave;
      if ((lane % TPC) == 0 && c < nch) L.cw[c] = ct;
    };
    constexpr std::true_type kFromLds{};
    constexpr std::false_type kFromMemory{};
    const int sc = nsteps < C::kCacheSteps ? nsteps : C::kCacheSteps;   // steps [0, sc) are in the cache
    uint4 ra[HU], rb[HU];
    float4 qa[HU][QPU], qb[HU][QPU];
    int s = nsteps - 1;
    if (s >= sc) {
      load_half(ra, qa, s, 0, kFromMemory);
      for (; s >= sc; --s) {
        load_half(rb, qb, s, 1, kFromMemory);
        compute_half(ra, qa, s, 0);
        if (s - 1 >= sc) load_half(ra, qa, s - 1, 0, kFromMemory);
        else if (s > 0) load_half(ra, qa, s - 1, 0, kFromLds);
        compute_half(rb, qb, s, 1);
        finish(s);
      }
    } else {
      load_half(ra, qa, s, 0, kFromLds);
    }
    for (; s >= 0; --s) {
      load_half(rb, qb, s, 1, kFromLds);
      compute_half(ra, qa, s, 0);
      if (s > 0) load_half(ra, qa, s - 1, 0, kFromLds);
      compute_half(rb, qb, s, 1);
      finish(s);
    }
    zl = wave_sum_d(zl);
    if (lane == 0) L.red_d[wave] = zl;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kWaves; ++w) Zt += L.red_d[w];
  } else {
    // chunk weights relative to their piece -> p
    for (int c = tid; c < nch; c += kThreads) {
      const int piece = (c / kChunksPerStep) * kWaves + (c % kWaves);
      L.cw[c] *= __builtin_amdgcn_exp2f(ref_l2(L.ref_m[piece], invT) - Ml2) * invS;
    }
    __syncthreads();
  }
  float* cwo = a.cw + (size_t)v * nch;
  for (int c = tid; c < nch; c += kThreads) cwo[c] = L.cw[c];
  if (tid == 0) {
    NodeRec r;
    r.S = S;
    r.Z = Zt;
    r.M = M;
    r.A = -1;
    r.b = b;
    r.err = (uint32_t)L.err;
    r.flags = (dense_draft ? kRecResidual : 0) | (no_mass ? kRecNoMass : 0);
    r.s0 = s0;
    r.n = n;
    r.T = Tb;
    a.rec[v] = r;
  }
}

// Takes nodes from the device queue (in the order of order[]: nodes with a dense draft row first)
// until none is left.  Called by every thread of a workgroup of C::kThreads threads; L is the
// workgroup's LDS.
template <typename LT, class C>
__device__ void vocab_stream(const VocabArgs& a, Lds<C>& L) {
  if (threadIdx.x == 0) {
    const int i = atomicAdd(a.queue, 1);
    L.item = i < a.N ? a.order[i] : -1;
  }
  for (int t = threadIdx.x; t <= a.B && t < kNoffLds; t += C::kThreads) L.noff[t] = a.node_offsets[t];
  __syncthreads();
  bool pre_lds = false;   // the first step of the worker's next node is in the LDS cache
  for (;;) {
    const int v = L.item;
    if (v < 0) return;
    int qn = 0;
    stream_node<LT, C>(a, L, v, qn, pre_lds);   // (every thread has read L.item before its first barrier)
    if (threadIdx.x == 0) L.item = L.next;
    __syncthreads();   // LDS reused by the next node
  }
}

// The verification step at one node, on one wave, in fp64 from its children's values in P (children
// in ascending id): RheoSampling Section 3.3 Algorithm 1 for one layer -- the sampled child is
// accepted when u q~ <= p (the test u <= min(1, p / q~) without the division); after its rejection
// the residual r = (p - q~)+ / Z replaces p; the other children are tested in turn, child c accepted
// when u_c (1 - rejected mass) <= r(c), the rejected mass being the sum of r over the children
// tested before c.  At temperature 0 (greedy decoding, Progressive Tree Drafting Section 3.2) the
// child whose token is the argmax (p = 1) is accepted and the children tested before it are
// rejected.  A node's step depends on its own values only, so every node's step is taken here and
// the walk follows the accepted children from the root.  The tests of all children are taken at
// once (the rejected mass before each child as a prefix sum over the wave); the first child that
// passes is the accepted one.  Returns its index in the list (-1: none, the final draw at this node
// ends the path) and the sampled child's index in ks; errors that count only if the walk reaches
// this node go to derr.  Wave-uniform results.
__device__ inline int node_step(const PickLds& P, int nk, bool greedy, double Zv, int& ks, uint32_t& derr) {
  const int lane = threadIdx.x & 63;
  ks = -1;   // the sampled child (the last one if several: an error reported by the pick)
  for (int base = 0; base < nk; base += 64) {
    const int k = base + lane;
    const unsigned long long m = __ballot(k < nk && P.kid_smp[k]);
    if (m) ks = base + 63 - __clzll((long long)m);
  }
  if (greedy) {
    if (ks >= 0 && P.kid_p[ks] == 1.0) return ks;
    for (int base = 0; base < nk; base += 64) {
      const int k = base + lane;
      const unsigned long long m = __ballot(k < nk && k != ks && P.kid_p[k] == 1.0);
      if (m) return base + __ffsll((long long)m) - 1;
    }
    return -1;
  }
  bool resid = false;
  if (ks >= 0) {
    const double qs = (double)P.kid_q[ks];
    if (!(qs > 0.0)) {
      derr |= TAV_DEV_ZERO_DRAFT_MASS;
      return -1;
    }
    if ((double)P.kid_u[ks] * qs <= P.kid_p[ks]) return ks;
    resid = true;
  }
  const double invZ = resid && Zv > 0.0 ? 1.0 / Zv : 0.0;
  double carry = 0.0;   // mass of the children of earlier groups of 64
  for (int base = 0; base < nk; base += 64) {
    const int k = base + lane;
    const bool tested = k < nk && k != ks;
    const double p = tested ? P.kid_p[k] : 0.0;
    const double r0 = !tested ? 0.0 : resid ? fmax(0.0, p - (double)P.kid_q[k]) * invZ : p;
    const double incl = wave_scan_d(r0);
    const double before = dpp0_d<kDppWaveShr1>(incl);
    const double rem = 1.0 - (carry + before);
    const double uc = tested ? (double)P.kid_u[k] : 0.0;
    const unsigned long long m = __ballot(tested && (rem > 0.0 ? uc * rem <= r0 : uc <= 0.0));
    if (m) return base + __ffsll((long long)m) - 1;
    carry += readlane_d(incl, 63);
  }
  return -1;
}

// The step's outputs: the rejection marks of the children (node_status: 2 for the children tested
// and rejected, kept by the walk where this node lies on the path) and the node's record (accepted
// child nx, or the final draw `bonus`, an empty residual being an error when the path ends here).
__device__ inline void store_step(const VocabArgs& a, const PickLds& P, int v, int s0, int nk, int nx, int ks,
                                  uint32_t derr, int bonus) {
  const int lane = threadIdx.x & 63;
  if (nx < 0 && !derr && bonus < 0) derr |= TAV_DEV_EMPTY_RESIDUAL;
  // tested: the sampled child first, then the others in order up to the accepted one
  const bool sampled_taken = ks >= 0 && nx == ks;
  for (int k = lane; k < nk; k += 64)
    a.node_status[s0 + P.kid_id[k]] = !sampled_taken && (k == ks || nx < 0 || k < nx) ? 2 : 0;
  if (lane == 0) a.step[v] = StepRec{nx >= 0 ? P.kid_id[nx] : -1, bonus, derr, 0};
}

// Everything the walk needs of node v, on one wave (P: the wave's LDS), from the streaming kernel's
// record and chunk weights.
template <typename LT>
__device__ void pick_node(const VocabArgs& a, PickLds& P, int v) {
  constexpr int EPU = 16 / sizeof(LT);
  constexpr int CT = 64 * EPU;   // tokens per chunk
  const int lane = threadIdx.x & 63;
  const int V = a.V, nch = a.nch;
  // Round one of loads: everything that depends on v alone -- the record, the draft row index, the
  // final draw's uniform, the chunk weights, the node's own parent and a window of the kWin * 64
  // nodes after v (parent, token, sampled flag, acceptance uniform), among which its children lie
  // when its sequence ends inside the window (children come after their parent).
  constexpr int kWin = 2;
  const NodeRec rec = a.rec[v];
  const int dr = a.draft_row[v];
  const float uf = a.uniforms[(size_t)v * 2 + 1];
  const int own_parent = a.parent[v];
  int w_par[kWin], w_tok[kWin];
  uint8_t w_smp[kWin];
  float w_u[kWin];
#pragma unroll
  for (int i = 0; i < kWin; ++i) {
    const int c = v + 1 + 64 * i + lane;
    const int cc = c < a.N ? c : v;
    w_par[i] = a.parent[cc];
    w_tok[i] = a.token[cc];
    w_smp[i] = a.sampled[cc];
    w_u[i] = a.uniforms[(size_t)cc * 2];
  }
  float cwr[kCwBatch];   // this lane's chunk weights c = lane + 64 j (rows of up to 64 * kCwBatch chunks)
  const bool stoch = !(rec.flags & kRecGreedy);
  const float* cwi = a.cw + (size_t)v * nch;
#pragma unroll
  for (int j = 0; j < kCwBatch; ++j) {
    const int c = lane + 64 * j;
    cwr[j] = stoch && c < nch ? cwi[c] : 0.f;
  }
  const int b = rec.b, s0 = rec.s0, n = rec.n;
  const int lv = v - s0;   // v's id in its sequence
  const float Tb = rec.T;
  const float invT = 1.f / Tb;
  const float invTl2 = invT * kLog2e;
  const bool dr_ok = dr >= 0 && dr < a.R;
  uint32_t err = rec.err;
  // every node checks its own parent (a bad one reaches the sequence's error word from that node)
  if (lv == 0 ? own_parent != -1 : (own_parent < 0 || own_parent >= lv)) err |= TAV_DEV_BAD_PARENT;
  if (stoch) {
#pragma unroll
    for (int j = 0; j < kCwBatch; ++j)
      if (lane + 64 * j < nch) P.cw[lane + 64 * j] = cwr[j];
    for (int c = lane + 64 * kCwBatch; c < nch; c += 64) P.cw[c] = cwi[c];   // (longer rows)
  }
  // children of v in ascending id (a compaction with fixed order, so that everything computed from
  // the list is the same on every run): from the window, then from the rest of the sequence
  int nk = 0, ns = 0;
  auto take = [&](int c, bool in_seq, int pc, int tk, uint8_t sm, float u) __attribute__((always_inline)) {
    const bool kid = in_seq && pc == lv;
    const bool smp = kid && sm != 0;
    const unsigned long long m = __ballot(kid);
    if (kid) {
      const int k = nk + __popcll(m & ((1ull << lane) - 1ull));
      if (k < kMaxChildren) {
        P.kid_id[k] = c - s0;
        P.kid_tok[k] = tk;
        P.kid_smp[k] = smp;
        P.kid_u[k] = u;
      }
    }
    nk += __popcll(m);
    ns += __popcll(__ballot(smp));
  };
#pragma unroll
  for (int i = 0; i < kWin; ++i) {
    const int c = v + 1 + 64 * i + lane;
    take(c, c < s0 + n, w_par[i], w_tok[i], w_smp[i], w_u[i]);
  }
  for (int base = v + 1 + 64 * kWin; base < s0 + n; base += 64) {
    const int c = base + lane;
    const bool in_seq = c < s0 + n;
    const int cc = in_seq ? c : v;
    take(c, in_seq, a.parent[cc], a.token[cc], a.sampled[cc], a.uniforms[(size_t)cc * 2]);
  }
  if (!(Tb >= 0.f && Tb < INFINITY)) err |= TAV_DEV_BAD_TEMPERATURE;
  if (nk > kMaxChildren) err |= TAV_DEV_TOO_MANY_CHILDREN;
  nk = nk < kMaxChildren ? nk : kMaxChildren;
  wave_sync();
  if (rec.flags & kRecGreedy) {
    const float M = rec.M;
    const int A = rec.A;
    if (M == -INFINITY) err |= TAV_DEV_NONFINITE_LOGITS;   // no finite logit: no prediction
    for (int k = lane; k < nk; k += 64) {
      const int tk = P.kid_tok[k];
      if (tk < 0 || tk >= V) err |= TAV_DEV_BAD_TOKEN;
      for (int k2 = 0; k2 < k; ++k2)
        if (P.kid_tok[k2] == tk) err |= TAV_DEV_DUP_SIBLING_TOKEN;
      P.kid_p[k] = tk == A ? 1.0 : 0.0;
    }
    err = wave_or(err);
    if (lane == 0) {
      a.stats[(size_t)v * 3 + 0] = M;
      a.stats[(size_t)v * 3 + 1] = 1.f;
      a.stats[(size_t)v * 3 + 2] = 0.f;
      a.term_token[v] = M == -INFINITY ? -1 : A;
      if (err) {
        atomicOr(a.status, err);
        atomicOr(a.seq_err + b, err);
      }
    }
    wave_sync();
    int ks = -1;
    uint32_t derr = 0;
    const int nx = node_step(P, nk, true, 0.0, ks, derr);
    store_step(a, P, v, s0, nk, nx, ks, derr, M == -INFINITY ? -1 : A);
    return;
  }
  const float M = rec.M;
  const float Ml2 = M * kLog2e;
  const double S = rec.S;
  const float invS = (float)(1.0 / S);
  const bool no_mass = (rec.flags & kRecNoMass) != 0;
  const bool use_draft = ns > 0 && dr_ok;
  const bool sparse = a.K > 0;
  double Zt = rec.Z;
  if (ns > 1) err |= TAV_DEV_MULTI_SAMPLED;
  if (ns > 0 && !dr_ok) err |= TAV_DEV_NO_DRAFT;
  if (no_mass || !(S > 0.0 && S < INFINITY)) err |= TAV_DEV_NONFINITE_LOGITS;
  if (((rec.flags & kRecResidual) != 0) != (use_draft && !sparse)) err |= TAV_DEV_PLAN_MISMATCH;
  // sparse draft row (RheoSampling Section 3.2: support of at most 128 tokens, q~ = 0 elsewhere):
  // outside the support (p - q~)+ = p, so the chunk weights of p only lose min(p, q~) at the
  // support tokens, and Z = sum (p - q~)+ = sum over the support of (q~ - p)+ (the two sides of
  // the residual-mass identity, RheoSampling Appendix C Eq. 10) -- no second pass over the row.
  const int K = a.K;
  auto sp_q = [&](int tok) -> float {   // q~ at tok (binary search of the ascending support)
    int lo = 0, hi = K;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (P.sp_idx[mid] < tok) lo = mid + 1; else hi = mid;
    }
    return lo < K && P.sp_idx[lo] == tok ? P.sp_val[lo] : 0.f;
  };
  wave_sync();
  if (use_draft && sparse) {
    const int32_t* didx = a.draft_idx + (size_t)dr * K;
    const float* dval = a.draft_val + (size_t)dr * K;
    const LT* lrow = (const LT*)a.logits + (size_t)v * V;
    double zl = 0.0;
    for (int j = lane; j < K; j += 64) {
      const int tk = didx[j];
      const float qj = dval[j];
      const int prev = j > 0 ? didx[j - 1] : -1;
      const bool ok = tk >= 0 && tk < V && tk > prev && qj >= 0.f && qj < INFINITY;
      float take = 0.f;
      if (ok) {
        const float p = __builtin_amdgcn_exp2f(logit_at<LT>(lrow, tk) * invTl2 - Ml2) * invS;
        take = fminf(p, qj);
        zl += (double)fmaxf(qj - p, 0.f);
      } else {
        err |= TAV_DEV_BAD_DRAFT;
      }
      P.sp_idx[j] = ok ? tk : -1;
      P.sp_val[j] = ok ? qj : 0.f;
      P.sp_take[j] = take;
    }
    Zt = wave_sum_d(zl);
    wave_sync();
    // each chunk's support tokens are consecutive entries; the last entry of a chunk's run sums the
    // run in order and takes it out of the chunk (one lane per chunk, a fixed order of additions)
    for (int j = lane; j < K; j += 64) {
      const int tk = P.sp_idx[j];
      if (tk < 0) continue;
      const int c = tk / CT;
      const int nx = j + 1 < K ? P.sp_idx[j + 1] : -1;
      if (nx >= 0 && nx / CT == c) continue;
      int j0 = j;
      while (j0 > 0 && P.sp_idx[j0 - 1] >= 0 && P.sp_idx[j0 - 1] / CT == c) --j0;
      float t = 0.f;
      for (int i = j0; i <= j; ++i) t += P.sp_take[i];
      P.cw[c] -= t;
    }
    wave_sync();
  }
  // children: point values for the walk; deterministic children leave the final draw.  Children
  // 0..63 are also held one per lane (token; -1 for a sampled child or one whose token is out of
  // range, which leave the final draw untouched) and read back with readlane, without LDS round
  // trips; children past 64 (up to kMaxChildren) come from LDS.
  int det_r = -1;
  float kw_r = 0.f;
  for (int k = lane; k < nk; k += 64) {
    const int tk = P.kid_tok[k];
    const bool tok_ok = tk >= 0 && tk < V;
    // the point loads go out first (token 0 stands in for a bad token), the checks run under them
    const int tkc = tok_ok ? tk : 0;
    const float z = logit_at<LT>(a.logits, (size_t)v * V + tkc);
    const float qd = use_draft && !sparse ? a.draft[(size_t)dr * V + tkc] : 0.f;
    if (!tok_ok) err |= TAV_DEV_BAD_TOKEN;
    if (k < 64) {
      for (int k2 = 0; k2 < min(nk, 64); ++k2)
        if (k2 < k && __builtin_amdgcn_readlane(tk, k2) == tk) err |= TAV_DEV_DUP_SIBLING_TOKEN;
    } else {
      for (int k2 = 0; k2 < k; ++k2)
        if (P.kid_tok[k2] == tk) err |= TAV_DEV_DUP_SIBLING_TOKEN;
    }
    P.kid_p[k] = 0.0;
    P.kid_q[k] = 0.f;
    if (tok_ok) {
      const float qz = !use_draft ? 0.f : sparse ? sp_q(tk) : qd;
      P.kid_p[k] = exp((double)(z * invT) - (double)M) / S;
      P.kid_q[k] = use_draft ? qz : 0.f;
      const float p = __builtin_amdgcn_exp2f(z * invTl2 - Ml2) * invS;
      const float kw = use_draft ? fmaxf(0.f, p - qz) : p;
      P.kid_w[k] = kw;
      if (k < 64) {
        det_r = P.kid_smp[k] ? -1 : tk;
        kw_r = kw;
      }
    }
  }
  wave_sync();
  auto det_tok = [&](int k) -> int {   // token of deterministic child k, or -1
    if (k < 64) return __builtin_amdgcn_readlane(det_r, k);
    const int tk = P.kid_tok[k];
    return !P.kid_smp[k] && tk >= 0 && tk < V ? tk : -1;
  };
  // the deterministic children's weights taken out of their chunks in a fixed order (two runs give the
  // same chunk weights bit for bit): with up to 64 children the last child of each chunk sums the
  // weights of that chunk's children in child order and takes the sum out (one lane per chunk, all
  // chunks at once); more children go one at a time on one lane
  if (nk <= 64) {
    const int myc = lane < nk && det_r >= 0 ? det_r / CT : -1;
    bool last = myc >= 0;
    float sum = 0.f;
    for (int k = 0; k < nk; ++k) {
      const int tk = __builtin_amdgcn_readlane(det_r, k);
      const float wk = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(kw_r), k));
      const bool same = tk >= 0 && tk / CT == myc;
      if (same && k <= lane) sum += wk;
      if (same && k > lane) last = false;
    }
    if (last) P.cw[myc] -= sum;
  } else {
    for (int k = 0; k < nk; ++k) {
      const int tk = det_tok(k);
      const float kw = k < 64 ? __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(kw_r), k)) : P.kid_w[k];
      if (lane == 0 && tk >= 0) P.cw[tk / CT] -= kw;
    }
  }
  wave_sync();
  // fp64 scan over chunks: lane l owns chunks [l * per, (l + 1) * per)
  const int per = (nch + 63) / 64;
  double pm = 0.0;
  for (int k = 0; k < per; ++k) {
    const int c = lane * per + k;
    if (c < nch) pm += (double)fmaxf(P.cw[c], 0.f);
  }
  const double incl = wave_scan_d(pm);
  const double W = readlane_d(incl, 63);
  const double target = (double)uf * W;
  int tok = -1;
  // this node's verification step (Z as the node's statistics report it, in float)
  const float Zf = use_draft ? (float)Zt : 0.f;
  int nx = -2, ks = -1;
  uint32_t derr = 0;
  auto take_step = [&]() __attribute__((always_inline)) { nx = node_step(P, nk, false, (double)Zf, ks, derr); };
  if (W > 0.0) {
    const unsigned long long hit = __ballot(pm > 0.0 && incl > target);
    const unsigned long long has = __ballot(pm > 0.0);
    const int owner = hit ? __ffsll((long long)hit) - 1 : 63 - __clzll((long long)has);
    int pc = -1;
    double rem = 0.0;
    if (lane == owner) {
      double cum = incl - pm, cum_l = 0.0;
      int cl = -1;
      for (int k = 0; k < per; ++k) {
        const int c = lane * per + k;
        if (c >= nch) break;
        const double cs = (double)fmaxf(P.cw[c], 0.f);
        if (cs > 0.0) {
          cl = c; cum_l = cum;
          if (pc < 0 && cum + cs > target) { pc = c; break; }
        }
        cum += cs;
      }
      if (pc < 0) { pc = cl; cum = cum_l; }   // rounding past the total: last chunk with mass
      rem = target - cum;
    }
    pc = __builtin_amdgcn_readlane(pc, owner);
    rem = readlane_d(rem, owner);
    // the final draw inside the chosen chunk
    const int e0 = pc * CT + lane * EPU;
    const bool in = e0 < V;
    const uint4 ru = *(const uint4*)((const LT*)a.logits + (size_t)v * V + (in ? e0 : 0));
    float qv[EPU];
    if (use_draft && sparse) {
      // the support entries inside the chosen chunk (a run of the ascending support)
      int lo = 0, hi = K;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (P.sp_idx[mid] < pc * CT) lo = mid + 1; else hi = mid;
      }
#pragma unroll
      for (int e = 0; e < EPU; ++e) {
        qv[e] = 0.f;
        for (int j = lo; j < K && P.sp_idx[j] >= 0 && P.sp_idx[j] < (pc + 1) * CT; ++j)
          if (P.sp_idx[j] == e0 + e) qv[e] = P.sp_val[j];
      }
    } else if (use_draft) {
#pragma unroll
      for (int i = 0; i < EPU / 4; ++i) {
        const float4 t = *(const float4*)(a.draft + (size_t)dr * V + (in ? e0 : 0) + 4 * i);
        qv[4 * i + 0] = t.x; qv[4 * i + 1] = t.y; qv[4 * i + 2] = t.z; qv[4 * i + 3] = t.w;
      }
    }
    take_step();   // (while the chunk's loads are in flight)
    // positions of this lane's tokens that are deterministic children: each child in the chosen chunk
    // sets its bit in its owner lane's word (an OR, the same whatever the order)
    P.zm[lane] = 0u;
    wave_sync();
    for (int k = lane; k < nk; k += 64) {
      const int d = (k < 64 ? det_r : det_tok(k)) - pc * CT;   // (child k < 64 is this lane's)
      if ((unsigned)d < (unsigned)CT) atomicOr(&P.zm[d / EPU], 1u << (d % EPU));
    }
    wave_sync();
    const uint32_t zmask = P.zm[lane];
    float w[EPU];
    float lsum = 0.f;
#pragma unroll
    for (int e = 0; e < EPU; ++e) {
      float x = 0.f;
      if (in) {
        const float p = __builtin_amdgcn_exp2f(unit_elem<LT>(ru, e) * invTl2 - Ml2) * invS;
        x = use_draft ? fmaxf(0.f, p - qv[e]) : p;
        if ((zmask >> e) & 1u) x = 0.f;
      }
      w[e] = x;
      lsum += x;
    }
    const float inc = wave_scan_f(lsum);
    const float remf = (float)rem;
    const unsigned long long hit2 = __ballot(inc > remf && lsum > 0.f);
    const unsigned long long has2 = __ballot(lsum > 0.f);
    const int chosen = hit2 ? __ffsll((long long)hit2) - 1 : (has2 ? 63 - __clzll((long long)has2) : -1);
    int mine = -1;
    if (lane == chosen) {
      float cum = inc - lsum;
      int lastpos = -1;
#pragma unroll
      for (int e = 0; e < EPU; ++e) {
        if (w[e] > 0.f) lastpos = e0 + e;
        cum += w[e];
        if (mine < 0 && w[e] > 0.f && cum > remf) mine = e0 + e;
      }
      if (mine < 0) mine = lastpos;
    }
    tok = chosen >= 0 ? __builtin_amdgcn_readlane(mine, chosen) : -1;
  }
  // status bits of any lane
  err = wave_or(err);
  if (nx == -2) take_step();   // (no final draw: W = 0)
  if (lane == 0) {
    a.stats[(size_t)v * 3 + 0] = M;
    a.stats[(size_t)v * 3 + 1] = (float)S;
    a.stats[(size_t)v * 3 + 2] = Zf;
    a.term_token[v] = tok;
    if (err) {
      atomicOr(a.status, err);
      atomicOr(a.seq_err + b, err);
    }
  }
  store_step(a, P, v, s0, nk, nx, ks, derr, tok);
}

}  // namespace vw
}  // namespace tav
