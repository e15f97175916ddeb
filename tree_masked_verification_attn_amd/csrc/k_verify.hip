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
// The vocabulary work is three streaming kernels over fixed slices of each row
// (256 threads x 8 sixteen-byte units): vocab_stats_kernel reads every logits
// row once (slice maxima, exp sums and chunk sums); vocab_residual_kernel reads
// the draft row (and the logits row again) only for nodes with a sampled child
// and replaces the chunk sums with those of (p - q~)+; vocab_pick_kernel (one
// workgroup per node) combines the slices into M = max l/T, S = sum exp(l/T-M)
// and Z = sum (p - q~)+, records p and q~ of each child's token, and finds the
// token the final draw would give if the walk ended at the node (fp64 scan over
// chunks, then one chunk re-read).  Sums run per lane in fp32 and across lanes
// in fp64.  walk_kernel (one wave per sequence) then takes the accept/reject
// decisions in fp64 from these values.
#include "tav_internal.h"

namespace tav {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

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

constexpr int kSW = kSliceThreads / 64;           // waves of a slice workgroup
constexpr int kChunksPerSlice = kSliceUnits * kSW;  // chunks of 64 units per slice
constexpr int kResUnits = kSliceUnits / 2;          // units per thread of a residual item
constexpr int kChunksPerHalf = kResUnits * kSW;

// Per-node record written by workgroup (node, slice 0) of the stats kernel.
enum RecField {
  kRecSeq = 0, kRecS0, kRecN, kRecKids, kRecSampled, kRecInvT, kRecErr, kRecSmpMask,
  kRecKidId = 8,                      // kRecKidsMax child ids (local) ...
  kRecKidTok = 8 + kRecKidsMax,       // ... and their tokens
};
static_assert(kRecKidTok + kRecKidsMax <= kRecWords, "record layout");

__device__ inline void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Sequence of node v: the number of sequence ends node_offsets[1..B] that are <= v, counted by
// the whole workgroup with one read per thread.
__device__ int block_seq_of(const int32_t* node_offsets, int B, int v, int* cnt_s) {
  if (threadIdx.x == 0) *cnt_s = 0;
  __syncthreads();
  int c = 0;
  for (int t = threadIdx.x + 1; t <= B; t += blockDim.x) c += node_offsets[t] <= v;
  if (c) atomicAdd(cnt_s, c);
  __syncthreads();
  const int b = *cnt_s;
  return b < B ? b : B - 1;   // v < N = node_offsets[B] already gives b < B
}

// log2-domain reference of a slice maximum (a slice of -inf logits uses 0; its sum is 0).
__device__ inline float ref_l2(float m_raw, float invT) {
  return (m_raw == -INFINITY ? 0.f : m_raw * invT) * kLog2e;
}

// Row statistics from the slice maxima and sums: M = max l / T and S = sum exp(l/T - M).
struct RowStats {
  float M, Ml2, invS;
  double S;
  bool no_mass;
};
__device__ inline RowStats finish_stats(float Mraw, double S_at_Mraw, float invT) {
  RowStats r;
  r.no_mass = Mraw == -INFINITY;
  r.M = r.no_mass ? 0.f : Mraw * invT;
  r.Ml2 = r.M * kLog2e;
  r.S = S_at_Mraw;
  r.invS = (float)(1.0 / S_at_Mraw);
  return r;
}
// Workgroup version: slice values staged in LDS, every thread gets the same values.
__device__ RowStats row_stats_block(const float* sl_m, const double* sl_s, int nsl, float invT,
                                    float* m_s, double* s_s) {
  for (int j = threadIdx.x; j < nsl; j += blockDim.x) { m_s[j] = sl_m[j]; s_s[j] = sl_s[j]; }
  __syncthreads();
  float Mraw = -INFINITY;
  for (int j = 0; j < nsl; ++j) Mraw = fmaxf(Mraw, m_s[j]);
  const float Ml2 = (Mraw == -INFINITY ? 0.f : Mraw * invT) * kLog2e;
  double S = 0.0;
  for (int j = 0; j < nsl; ++j) {
    const double sj = s_s[j];
    if (sj != 0.0) S += sj * exp2((double)ref_l2(m_s[j], invT) - (double)Ml2);
  }
  return finish_stats(Mraw, S, invT);
}

// Sums each unit's per-lane values over the 64 lanes of its wave (one chunk per unit and
// wave), transposed through LDS: 64 / UN threads per chunk, UN values each.  Returns the
// chunk total in the first thread of each group; chunk index (tid * UN) / 64.
template <int UN>
__device__ inline float chunk_totals(const float (&x)[UN], float* part) {
  constexpr int TPC = 64 / UN;   // threads per chunk
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int k = 0; k < UN; ++k) part[(k * kSW + wave) * 64 + lane] = x[k];
  __syncthreads();
  const float* src = part + (tid / TPC) * 64 + (tid % TPC) * UN;
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < UN; i += 4) {
    const float4 a4 = *(const float4*)(src + i);
    t += (a4.x + a4.y) + (a4.z + a4.w);
  }
#pragma unroll
  for (int d = 1; d < TPC; d <<= 1) t += __shfl_xor(t, d);
  return t;
}

// Slice statistics of every (node, slice): one 256-thread workgroup reads kSliceUnits 16-byte
// units per thread of the node's logits row and writes the slice's largest raw logit m, the
// sum s = sum exp2(l * log2e / T - ref_l2(m)) (fp32 per lane and chunk, fp64 across chunks)
// and the same sum over each chunk of 64 units (the weights of the final draw when the node
// has no sampled child).  Workgroup (node, 0) also writes the node's record (sequence, 1/T,
// children, checks of the parent array and temperature) and lists the node when it has a
// sampled child and a draft row.
template <typename LT>
__global__ __launch_bounds__(kSliceThreads) void vocab_stats_kernel(VocabArgs a) {
  constexpr int EPU = 16 / sizeof(LT);
  constexpr int U = kSliceUnits;
  __shared__ __attribute__((aligned(16))) float part[U * kSliceThreads];
  __shared__ float red_f[kSW];
  __shared__ double red_d[kSW];
  __shared__ int cnt_s, kc_s, ks_s, err_s, smask_s;
  __shared__ int kid_i[kRecKidsMax], kid_t[kRecKidsMax];
  const int v = blockIdx.x / a.nsl, j = blockIdx.x % a.nsl;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nunits = a.V / EPU;
  const LT* row = (const LT*)a.logits + (size_t)v * a.V;
  const int u0 = j * (U * kSliceThreads) + tid;
  uint4 r[U];
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const int u = u0 + k * kSliceThreads;
    r[k] = *(const uint4*)(row + (size_t)(u < nunits ? u : 0) * EPU);
  }
  const int b = block_seq_of(a.node_offsets, a.B, v, &cnt_s);
  const float Tb = a.temperature[b];
  const float invT = 1.f / Tb;
  if (j == 0) {   // the node's record
    const int s0 = a.node_offsets[b];
    const int n = a.node_offsets[b + 1] - s0;
    if (tid == 0) { kc_s = 0; ks_s = 0; err_s = 0; smask_s = 0; }
    __syncthreads();
    uint32_t err = 0;
    for (int c = tid; c < n; c += kSliceThreads) {
      const int pc = a.parent[s0 + c];
      if (c == 0 ? pc != -1 : (pc < 0 || pc >= c)) err |= TAV_DEV_BAD_PARENT;
      if (c > 0 && pc == v - s0) {
        const int k = atomicAdd(&kc_s, 1);
        const bool smp = a.sampled[s0 + c] != 0;
        if (smp) atomicAdd(&ks_s, 1);
        if (k < kRecKidsMax) {
          kid_i[k] = c;
          kid_t[k] = a.token[s0 + c];
          if (smp) atomicOr(&smask_s, 1 << k);
        }
      }
    }
    if (tid == 0 && !(Tb > 0.f && Tb < INFINITY)) err |= TAV_DEV_BAD_TEMPERATURE;
    if (err) atomicOr(&err_s, (int)err);
    __syncthreads();
    int32_t* rec = a.rec + (size_t)v * kRecWords;
    const int nk = kc_s < kRecKidsMax ? kc_s : kRecKidsMax;
    if (tid < kRecKidsMax) {
      rec[kRecKidId + tid] = tid < nk ? kid_i[tid] : -1;
      rec[kRecKidTok + tid] = tid < nk ? kid_t[tid] : -1;
    }
    if (tid == 0) {
      rec[kRecSeq] = b; rec[kRecS0] = s0; rec[kRecN] = n; rec[kRecKids] = kc_s;
      rec[kRecSampled] = ks_s; rec[kRecInvT] = __float_as_int(invT); rec[kRecErr] = err_s;
      rec[kRecSmpMask] = smask_s;
      const int dr = a.draft_row[v];
      if (ks_s > 0 && dr >= 0 && dr < a.R) a.dlist[atomicAdd(a.dcount, 1)] = v;
    }
  }
  // largest raw logit (max l / T = (max l) / T for T > 0)
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < U; ++k) {
    if (u0 + k * kSliceThreads < nunits) {
#pragma unroll
      for (int e = 0; e < EPU; ++e) mx = fmaxf(mx, unit_elem<LT>(r[k], e));
    }
  }
  mx = wave_max_f(mx);
  if (lane == 0) red_f[wave] = mx;
  __syncthreads();
  float m = red_f[0];
#pragma unroll
  for (int w = 1; w < kSW; ++w) m = fmaxf(m, red_f[w]);
  const float invTl2 = invT * kLog2e;
  const float r2 = ref_l2(m, invT);
  // a NaN or +inf logit makes the sum NaN; the pick kernel reports it
  float su[U];
  double sl = 0.0;
#pragma unroll
  for (int k = 0; k < U; ++k) {
    su[k] = 0.f;
    if (u0 + k * kSliceThreads < nunits) {
#pragma unroll
      for (int e = 0; e < EPU; ++e) su[k] += __builtin_amdgcn_exp2f(unit_elem<LT>(r[k], e) * invTl2 - r2);
    }
    sl += (double)su[k];
  }
  const float ct = chunk_totals<U>(su, part);
  const int c = j * kChunksPerSlice + (tid * U) / 64;
  if ((tid % (64 / U)) == 0 && c < a.nch) a.ch_w[(size_t)v * a.nch + c] = ct;
  sl = wave_sum_d(sl);
  if (lane == 0) red_d[wave] = sl;
  __syncthreads();
  if (tid == 0) {
    double s = 0.0;
#pragma unroll
    for (int w = 0; w < kSW; ++w) s += red_d[w];
    a.sl_m[(size_t)v * a.nsl + j] = m;
    a.sl_s[(size_t)v * a.nsl + j] = s;
  }
}

// Residual weights (p - q~)+ of the listed rows (nodes with a sampled child): p from the row
// statistics, q~ from the node's draft row.  Overwrites the row's chunk sums with those of
// (p - q~)+ and writes each half slice's sum of (p - q~)+ (fp32 per lane, fp64 across lanes).
// A grid-stride loop over (listed row, half slice), rows taken from the end of the list
// (the most recently read logits rows first); the list length is read on the device.
template <typename LT>
__global__ __launch_bounds__(kSliceThreads) void vocab_residual_kernel(VocabArgs a) {
  constexpr int EPU = 16 / sizeof(LT);
  constexpr int U = kResUnits;
  __shared__ __attribute__((aligned(16))) float part[U * kSliceThreads];
  __shared__ double red_d[kSW];
  __shared__ float m_s[kMaxSlices];
  __shared__ double s_s[kMaxSlices];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nunits = a.V / EPU;
  const int nh = 2 * a.nsl;
  const int cnt = *a.dcount;
  for (int item = blockIdx.x; item < cnt * nh; item += gridDim.x) {
    const int v = a.dlist[cnt - 1 - item / nh], h = item % nh;
    const LT* row = (const LT*)a.logits + (size_t)v * a.V;
    const float* drow = a.draft + (size_t)a.draft_row[v] * a.V;
    const int u0 = h * (U * kSliceThreads) + tid;
    uint4 r[U];
    float4 q[U][EPU / 4];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int u = u0 + k * kSliceThreads;
      const size_t e0 = (size_t)(u < nunits ? u : 0) * EPU;
      r[k] = *(const uint4*)(row + e0);
#pragma unroll
      for (int i = 0; i < EPU / 4; ++i) q[k][i] = *(const float4*)(drow + e0 + 4 * i);
    }
    const float invT = __int_as_float(a.rec[(size_t)v * kRecWords + kRecInvT]);
    const RowStats st = row_stats_block(a.sl_m + (size_t)v * a.nsl, a.sl_s + (size_t)v * a.nsl, a.nsl,
                                        invT, m_s, s_s);
    const float invTl2 = invT * kLog2e;
    float wu[U];
    double zl = 0.0;
#pragma unroll
    for (int k = 0; k < U; ++k) {
      wu[k] = 0.f;
      if (u0 + k * kSliceThreads < nunits) {
#pragma unroll
        for (int e = 0; e < EPU; ++e) {
          const float4 q4 = q[k][e / 4];
          const float qe = (e & 3) == 0 ? q4.x : (e & 3) == 1 ? q4.y : (e & 3) == 2 ? q4.z : q4.w;
          const float p = __builtin_amdgcn_exp2f(unit_elem<LT>(r[k], e) * invTl2 - st.Ml2) * st.invS;
          wu[k] += fmaxf(0.f, p - qe);
        }
      }
      zl += (double)wu[k];
    }
    const float ct = chunk_totals<U>(wu, part);
    const int c = h * kChunksPerHalf + (tid * U) / 64;
    if ((tid % (64 / U)) == 0 && c < a.nch) a.ch_w[(size_t)v * a.nch + c] = ct;
    zl = wave_sum_d(zl);
    if (lane == 0) red_d[wave] = zl;
    __syncthreads();
    if (tid == 0) {
      double z = 0.0;
#pragma unroll
      for (int w = 0; w < kSW; ++w) z += red_d[w];
      a.sl_z[(size_t)v * nh + h] = z;
    }
    __syncthreads();   // LDS reused by the next item
  }
}

// Per node, one wave: the children's point values p(token) / q~(token) for the walk, the row
// statistics (M, S, Z), the checks, and the token the final draw would give if the walk ended
// here: chunk weights (scaled to p, or the residual weights) less the deterministic children's
// own weights, an fp64 scan over chunks for u * W, then one chunk re-read and scanned.
template <typename LT>
__global__ __launch_bounds__(kSliceThreads) void vocab_pick_kernel(VocabArgs a) {
  constexpr int EPU = 16 / sizeof(LT);
  constexpr int CT = 64 * EPU;   // tokens per chunk
  __shared__ float cw_all[kSW][kMaxChunks];
  __shared__ int kid_id_all[kSW][kMaxChildren];
  __shared__ int kid_tok_all[kSW][kMaxChildren];
  __shared__ uint8_t kid_smp_all[kSW][kMaxChildren];
  __shared__ int cnt_all[kSW][2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int v = blockIdx.x * kSW + wave;
  if (v >= a.N) return;   // the wave's node; no workgroup barrier is used below
  float* cw = cw_all[wave];
  int* kid_id = kid_id_all[wave];
  int* kid_tok = kid_tok_all[wave];
  uint8_t* kid_smp = kid_smp_all[wave];
  const int V = a.V, nch = a.nch, nsl = a.nsl;
  // ---- everything indexed by the node alone ----
  const int32_t* rec = a.rec + (size_t)v * kRecWords;
  const int rv = lane < kRecWords ? rec[lane] : 0;
  const int dr = a.draft_row[v];
  float ml = -INFINITY;
  double sl = 0.0, zl = 0.0;
  for (int j = lane; j < nsl; j += 64) {
    ml = a.sl_m[(size_t)v * nsl + j];   // (lane's last slice; nsl <= 64 keeps one per lane)
    sl = a.sl_s[(size_t)v * nsl + j];
    zl += a.sl_z[(size_t)v * 2 * nsl + 2 * j] + a.sl_z[(size_t)v * 2 * nsl + 2 * j + 1];
  }
  for (int c0 = 0; c0 < nch; c0 += 8 * 64) {   // eight loads in flight per lane
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = c0 + i * 64 + lane;
      x[i] = c < nch ? a.ch_w[(size_t)v * nch + c] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = c0 + i * 64 + lane;
      if (c < nch) cw[c] = x[i];
    }
  }
  const int s0 = __shfl(rv, kRecS0), nkids = __shfl(rv, kRecKids), nsamp = __shfl(rv, kRecSampled);
  const float invT = __int_as_float(__shfl(rv, kRecInvT));
  uint32_t err = (uint32_t)__shfl(rv, kRecErr);
  const int smask = __shfl(rv, kRecSmpMask);
  const float invTl2 = invT * kLog2e;
  // row statistics (nsl <= 64: one slice per lane)
  const float Mraw = wave_max_f(ml);
  const float Ml2r = (Mraw == -INFINITY ? 0.f : Mraw * invT) * kLog2e;
  const double sc = (sl != 0.0) ? sl * exp2((double)ref_l2(ml, invT) - (double)Ml2r) : 0.0;
  const RowStats st = finish_stats(Mraw, wave_sum_d(sc), invT);
  const double Zt = wave_sum_d(zl);
  const bool dr_ok = dr >= 0 && dr < a.R;
  const bool use_draft = nsamp > 0 && dr_ok;
  if (nkids > kMaxChildren) err |= TAV_DEV_TOO_MANY_CHILDREN;
  if (nsamp > 1) err |= TAV_DEV_MULTI_SAMPLED;
  if (nsamp > 0 && !dr_ok) err |= TAV_DEV_NO_DRAFT;
  if (st.no_mass || !(st.S > 0.0 && st.S < INFINITY)) err |= TAV_DEV_NONFINITE_LOGITS;
  // children: from the record, or (more than it holds) a scan of the parent array
  int nk;
  if (nkids <= kRecKidsMax) {
    nk = nkids;
    const int kid_i = __shfl(rv, kRecKidId + (lane < kRecKidsMax ? lane : 0));
    const int kid_t = __shfl(rv, kRecKidTok + (lane < kRecKidsMax ? lane : 0));
    if (lane < nk) { kid_id[lane] = kid_i; kid_tok[lane] = kid_t; kid_smp[lane] = (smask >> lane) & 1; }
  } else {
    const int n = __shfl(rv, kRecN);
    nk = 0;
    for (int base = 1; base < n; base += 64) {
      const int c = base + lane;
      const bool is_kid = c < n && a.parent[s0 + c] == v - s0;
      const unsigned long long m = __ballot(is_kid);
      if (is_kid) {
        const int at = nk + __popcll(m & ((1ull << lane) - 1ull));
        if (at < kMaxChildren) { kid_id[at] = c; kid_tok[at] = a.token[s0 + c]; kid_smp[at] = a.sampled[s0 + c]; }
      }
      nk += __popcll(m);
    }
    nk = nk < kMaxChildren ? nk : kMaxChildren;
  }
  wave_sync();
  // non-draft rows: chunk sums relative to their slice -> p
  if (!use_draft) {
    for (int c = lane; c < nch; c += 64) {
      const int jj = c / kChunksPerSlice;
      const float mj = __shfl(ml, jj);
      cw[c] = cw[c] * __builtin_amdgcn_exp2f(ref_l2(mj, invT) - st.Ml2) * st.invS;
    }
  }
  wave_sync();
  // children: point values for the walk; deterministic children leave the final draw
  for (int k = lane; k < nk; k += 64) {
    const int tk = kid_tok[k];
    if (tk < 0 || tk >= V) err |= TAV_DEV_BAD_TOKEN;
    for (int k2 = 0; k2 < k; ++k2)
      if (kid_tok[k2] == tk) err |= TAV_DEV_DUP_SIBLING_TOKEN;
    if (tk >= 0 && tk < V) {
      const float z = logit_at<LT>(a.logits, (size_t)v * V + tk);
      const float qz = dr_ok ? a.draft[(size_t)dr * V + tk] : 0.f;
      const int cid = s0 + kid_id[k];
      a.child_p[cid] = exp((double)(z * invT) - (double)st.M) / st.S;
      a.child_q[cid] = use_draft ? qz : 0.f;
      if (!kid_smp[k]) {
        const float p = __builtin_amdgcn_exp2f(z * invTl2 - st.Ml2) * st.invS;
        atomicAdd(&cw[tk / CT], -(use_draft ? fmaxf(0.f, p - qz) : p));
      }
    }
  }
  wave_sync();
  // fp64 scan over chunks: lane l owns chunks [l * per, (l + 1) * per)
  const int per = (nch + 63) / 64;
  double part = 0.0;
  for (int k = 0; k < per; ++k) {
    const int c = lane * per + k;
    if (c < nch) part += (double)fmaxf(cw[c], 0.f);
  }
  double incl = part;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const double y = __shfl_up(incl, d, 64);
    if (lane >= d) incl += y;
  }
  const double W = __shfl(incl, 63);
  const double target = (double)a.uniforms[(size_t)v * 2 + 1] * W;
  int tok = -1;
  if (W > 0.0) {
    const unsigned long long hit = __ballot(part > 0.0 && incl > target);
    const unsigned long long has = __ballot(part > 0.0);
    const int owner = hit ? __ffsll((long long)hit) - 1 : 63 - __clzll((long long)has);
    int pc = -1;
    double rem = 0.0;
    if (lane == owner) {
      double cum = incl - part, cum_l = 0.0;
      int cl = -1;
      for (int k = 0; k < per; ++k) {
        const int c = lane * per + k;
        if (c >= nch) break;
        const double cs = (double)fmaxf(cw[c], 0.f);
        if (cs > 0.0) {
          cl = c; cum_l = cum;
          if (pc < 0 && cum + cs > target) { pc = c; break; }
        }
        cum += cs;
      }
      if (pc < 0) { pc = cl; cum = cum_l; }   // rounding past the total: last chunk with mass
      rem = target - cum;
    }
    pc = __shfl(pc, owner);
    rem = __shfl(rem, owner);
    // the final draw inside the chosen chunk
    const int e0 = pc * CT + lane * EPU;
    const bool in = e0 < V;
    const uint4 ru = *(const uint4*)((const LT*)a.logits + (size_t)v * V + (in ? e0 : 0));
    float qv[EPU];
    if (use_draft) {
#pragma unroll
      for (int i = 0; i < EPU / 4; ++i) {
        const float4 t = *(const float4*)(a.draft + (size_t)dr * V + (in ? e0 : 0) + 4 * i);
        qv[4 * i + 0] = t.x; qv[4 * i + 1] = t.y; qv[4 * i + 2] = t.z; qv[4 * i + 3] = t.w;
      }
    }
    float w[EPU];
    float lsum = 0.f;
#pragma unroll
    for (int e = 0; e < EPU; ++e) {
      float x = 0.f;
      if (in) {
        const float p = __builtin_amdgcn_exp2f(unit_elem<LT>(ru, e) * invTl2 - st.Ml2) * st.invS;
        x = use_draft ? fmaxf(0.f, p - qv[e]) : p;
        for (int k = 0; k < nk; ++k)
          if (kid_tok[k] == e0 + e && !kid_smp[k]) x = 0.f;
      }
      w[e] = x;
      lsum += x;
    }
    float inc = lsum;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const float y = __shfl_up(inc, d, 64);
      if (lane >= d) inc += y;
    }
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
    tok = chosen >= 0 ? __shfl(mine, chosen) : -1;
  }
  // status bits of any lane
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) err |= (uint32_t)__shfl_xor((int)err, d);
  if (lane == 0) {
    a.stats[(size_t)v * 3 + 0] = st.M;
    a.stats[(size_t)v * 3 + 1] = (float)st.S;
    a.stats[(size_t)v * 3 + 2] = use_draft ? (float)Zt : 0.f;
    a.term_token[v] = tok;
    if (err) atomicOr(a.status, err);
  }
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
    if (lane == 0) {
      bool resid = false;
      const double Zv = (double)(staged ? z_s[v] : a.stats[(size_t)(s0 + v) * 3 + 2]);
      if (s >= 0) {
        const double qs = q_of(s);
        if (!(qs > 0.0)) {
          err |= TAV_DEV_ZERO_DRAFT_MASS;
        } else {
          const double ratio = fmin(1.0, p_of(s) / qs);
          if (u_of(s) <= ratio) {
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
          const double p = p_of(c);
          const double r0 = resid ? (Zv > 0.0 ? fmax(0.0, p - q_of(c)) / Zv : 0.0) : p;
          const double rem = 1.0 - rej;
          const double rc = rem > 0.0 ? r0 / rem : 0.0;
          if (u_of(c) <= rc) {
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
  if (lane == 0) {
    if (err) atomicOr(a.status, err);
    a.path_len[b] = err ? 0 : min(plen, a.max_path);
    a.bonus[b] = err ? -1 : bonus;
  }
}

template <typename LT>
void launch_vocab_t(const VocabArgs& a, int num_cus, hipStream_t s) {
  static int per_cu = 0;   // resident residual workgroups per CU
  if (per_cu == 0 &&
      (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, vocab_residual_kernel<LT>, kSliceThreads, 0) !=
           hipSuccess || per_cu < 1))
    per_cu = 1;
  const int g1 = a.N * a.nsl;
  const int g2 = 2 * g1 < per_cu * num_cus ? 2 * g1 : per_cu * num_cus;
  vocab_stats_kernel<LT><<<g1, kSliceThreads, 0, s>>>(a);
  vocab_residual_kernel<LT><<<g2, kSliceThreads, 0, s>>>(a);
  vocab_pick_kernel<LT><<<ceil_div(a.N, kSW), kSliceThreads, 0, s>>>(a);
}

}  // namespace

hipError_t launch_vocab(const VocabArgs& a, bool bf16_logits, int num_cus, hipStream_t s) {
  if (a.N == 0) return hipSuccess;
  if (bf16_logits) launch_vocab_t<uint16_t>(a, num_cus, s);
  else launch_vocab_t<float>(a, num_cus, s);
  return hipGetLastError();
}

hipError_t launch_walk(const WalkArgs& a, hipStream_t s) {
  walk_kernel<<<a.B, 64, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace tav
