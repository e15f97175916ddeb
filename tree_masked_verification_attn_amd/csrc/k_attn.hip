// Tree-masked attention over a paged prefix plus each node's ancestors.
//
// Every tree node attends to its sequence's cached prefix and to pi(v), the
// node itself and its ancestors (Progressive Tree Drafting, Section 3.1 "Tree
// Construction" and Section 3.2 "Candidate Verification"; RheoSampling scores
// its pruned draft tree in one target forward, Section 2.1; PreSTO's suffix
// requests share the cached prefix x_{0:c}, Section 3.2 and Appendix B.3
// Example 4).  Scores are scale * <q, k>, softmax over the visible keys.
//
// bf16 path (gfx950 MFMA): one workgroup = one work item = (row block, KV
// head, range of 64-key tiles).  A row block holds up to 256 query rows (nodes
// x the G query heads sharing the KV head), so every KV tile is read from HBM
// once and used by all rows.  Each of the 8 waves owns 32 rows and computes
//   S^T = K Q^T   (v_mfma_f32_32x32x16_bf16, keys x rows), online softmax per
//   row in registers (each lane holds one row's scores, so P^T feeds the next
//   MFMA directly), and O^T += V^T P^T.
// K tiles are staged in LDS row-major, V tiles transposed, double-buffered with
// the next tile's global loads issued before the current tile's math.
#include "tav_internal.h"

namespace tav {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

union Bf16Pack8 {
  bf16x8_t v;
  uint2 h[2];
  uint4 u;
  __bf16 e[8];
};

template <int D, int LOG2G>
__global__ __launch_bounds__(512) void attn_bf16_kernel(AttnArgs a) {
  constexpr int G = 1 << LOG2G;
  constexpr int NB = kRowsPerWG >> LOG2G;        // nodes per row block
  constexpr int KS = D / 16;                     // k-steps of S^T = K Q^T
  constexpr int DB = D / 32;                     // 32-wide output blocks of O^T
  constexpr int CH = D / 8;                      // 16-byte chunks per key row
  constexpr int LOADS = (kTileKeys * CH) / 512;  // chunks per thread per operand and tile
  constexpr int KSTR = D + 8;                    // K tile row stride (elements), bank-spread
  constexpr int VSTR = kTileKeys + 4;            // V^T tile row stride (elements)
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kTileKeys * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][D * VSTR];

  if (a.status[0] & TAV_DEV_PLAN_MISMATCH) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h32 = lane >> 5, l32 = lane & 31;
  const int item = blockIdx.x, g = blockIdx.y;

  int lo = 0, hi = a.total_rb;  // row block of this item: largest r with item_off[r] <= item
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (a.item_off[mid] <= item) lo = mid; else hi = mid;
  }
  const int rbi = lo;
  const int i0 = a.item_off[rbi];
  const int nsplit = a.item_off[rbi + 1] - i0;
  const int split = item - i0;
  const int b = a.rb_seq[rbi];
  if (b < 0 || b >= a.B || split < 0 || split >= nsplit) return;
  const int rb = rbi - a.seq_rb_off[b];
  const int s0 = a.node_offsets[b];
  const int n = a.node_offsets[b + 1] - s0;
  const int L = a.prefix_len[b];
  const int node0 = rb * NB;
  const int nodes_here = min(NB, n - node0);
  const int tail_n = min(n, node0 + NB);
  const int Tp = (L + kTileKeys - 1) / kTileKeys;
  const int Ttot = Tp + (tail_n + kTileKeys - 1) / kTileKeys;
  const int t_begin = split * a.tiles_per_split;
  const int t_end = min(Ttot, t_begin + a.tiles_per_split);
  const bool chain = a.is_chain[b] != 0;
  if (!chain && n > kMaxTreeNodes) return;  // rejected by tree preparation
  const int Hq = a.Hq, Hkv = a.Hkv, bs = a.block_size;

  const int row = wave * 32 + l32;
  const int rnode = node0 + (row >> LOG2G);     // sequence-local node of this lane's row
  const bool rvalid = (row >> LOG2G) < nodes_here;
  const int rhead = g * G + (row & (G - 1));

  const uint16_t* qp = (const uint16_t*)a.q;
  bf16x8_t qreg[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    Bf16Pack8 t;
    t.u = make_uint4(0u, 0u, 0u, 0u);
    if (rvalid)
      t.u = *(const uint4*)(qp + ((size_t)(s0 + rnode) * Hq + rhead) * D + ks * 16 + h32 * 8);
    qreg[ks] = t.v;
  }

  const uint16_t* kc = (const uint16_t*)a.k_cache;
  const uint16_t* vc = (const uint16_t*)a.v_cache;
  const uint16_t* kn = (const uint16_t*)a.k_node;
  const uint16_t* vn = (const uint16_t*)a.v_node;
  uint4 kr[LOADS], vr[LOADS];

  auto gload = [&](int t) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int c = tid + i * 512;
      const int key = c / CH, dc = c % CH;
      bool valid;
      size_t off = 0;
      const uint16_t* ks_ = kc;
      const uint16_t* vs_ = vc;
      if (t < Tp) {
        const int k = t * kTileKeys + key;
        valid = k < L;
        if (valid) {
          const int blk = a.block_table[(size_t)b * a.max_blocks + k / bs];
          if ((unsigned)blk >= (unsigned)a.num_blocks) {
            atomicOr(a.status, (uint32_t)TAV_DEV_BAD_BLOCK);
            valid = false;
          } else {
            off = (((size_t)blk * Hkv + g) * bs + (k % bs)) * D + dc * 8;
          }
        }
      } else {
        const int j = (t - Tp) * kTileKeys + key;
        valid = j < tail_n;
        off = ((size_t)(s0 + j) * Hkv + g) * D + dc * 8;
        ks_ = kn;
        vs_ = vn;
      }
      kr[i] = valid ? *(const uint4*)(ks_ + off) : make_uint4(0u, 0u, 0u, 0u);
      vr[i] = valid ? *(const uint4*)(vs_ + off) : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int c = tid + i * 512;
      const int key = c / CH, dc = c % CH;
      *(uint4*)&Ks[buf][key * KSTR + dc * 8] = kr[i];
      const uint16_t* ve = (const uint16_t*)&vr[i];
#pragma unroll
      for (int e = 0; e < 8; ++e) Vt[buf][(dc * 8 + e) * VSTR + key] = ve[e];
    }
  };

  const float sl2 = a.scale * kLog2e;
  float m_run = -INFINITY, l_run = 0.f;
  f32x16_t acc[DB];
#pragma unroll
  for (int mb = 0; mb < DB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[mb][r] = 0.f;

  if (t_begin < t_end) {
    gload(t_begin);
    lstore(0);
  }
  __syncthreads();
  for (int t = t_begin; t < t_end; ++t) {
    const int buf = (t - t_begin) & 1;
    const bool more = t + 1 < t_end;
    if (more) gload(t + 1);

    f32x16_t sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8_t ka = *(const bf16x8_t*)&Ks[buf][(kb * 32 + l32) * KSTR + ks * 16 + h32 * 8];
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[ks], sacc[kb], 0, 0, 0);
      }
    }

    // scale, mask, running max (this lane's row; its partner lane l ^ 32 holds the other keys)
    const bool is_prefix = t < Tp;
    const int tt = t - Tp;
    uint64_t mw = 0;
    if (!is_prefix && !chain && rvalid) mw = a.mask[(size_t)(s0 + rnode) * kMaskWords + tt];
    const bool full_prefix = is_prefix && (t + 1) * kTileKeys <= L;
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kin = kb * 32 + (r >> 2) * 8 + h32 * 4 + (r & 3);
        float s = sacc[kb][r] * sl2;
        if (!full_prefix) {
          bool vis;
          if (is_prefix) {
            vis = t * kTileKeys + kin < L;
          } else {
            const int j = tt * kTileKeys + kin;
            vis = j < tail_n && (chain ? j <= rnode : ((mw >> (j & 63)) & 1ull) != 0ull);
          }
          s = vis ? s : -INFINITY;
        }
        sacc[kb][r] = s;
        mx = fmaxf(mx, s);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;

    Bf16Pack8 pb[4];
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(sacc[kb][r] - m_use);
        psum += p;
        pb[kb * 2 + (r >> 3)].e[r & 7] = (__bf16)p;
      }
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int mb = 0; mb < DB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][r] *= alpha;

    // O^T += V^T P^T; the lane's k-slots are keys {h*4..h*4+3, 8+h*4..8+h*4+3} of each
    // 16-key step, matching where the S^T layout left this lane's probabilities.
#pragma unroll
    for (int mb = 0; mb < DB; ++mb) {
#pragma unroll
      for (int k2 = 0; k2 < 4; ++k2) {
        const uint16_t* vrow = &Vt[buf][(mb * 32 + l32) * VSTR + k2 * 16 + h32 * 4];
        Bf16Pack8 va;
        va.h[0] = *(const uint2*)vrow;
        va.h[1] = *(const uint2*)(vrow + 8);
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va.v, pb[k2].v, acc[mb], 0, 0, 0);
      }
    }

    if (more) lstore(buf ^ 1);
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv_l = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse_nat = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  if (nsplit == 1) {
    if (!rvalid) return;
    uint16_t* op = (uint16_t*)a.out + ((size_t)(s0 + rnode) * Hq + rhead) * D;
#pragma unroll
    for (int mb = 0; mb < DB; ++mb) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        union { __bf16 e[4]; uint2 u; } o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o.e[e] = (__bf16)(acc[mb][rq * 4 + e] * inv_l);
        *(uint2*)(op + mb * 32 + rq * 8 + h32 * 4) = o.u;
      }
    }
    if (h32 == 0 && a.lse) a.lse[(size_t)(s0 + rnode) * Hq + rhead] = lse_nat;
  } else {
    float* po = a.part_o + (((size_t)item * Hkv + g) * kRowsPerWG + row) * D;
#pragma unroll
    for (int mb = 0; mb < DB; ++mb)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq)
        *(float4*)(po + mb * 32 + rq * 8 + h32 * 4) =
            make_float4(acc[mb][rq * 4 + 0] * inv_l, acc[mb][rq * 4 + 1] * inv_l,
                        acc[mb][rq * 4 + 2] * inv_l, acc[mb][rq * 4 + 3] * inv_l);
    if (h32 == 0) a.part_lse[((size_t)item * Hkv + g) * kRowsPerWG + row] = lse_nat;
  }
}

// Online-softmax merge of the split partials: out = sum_s exp(lse_s - LSE) O_s.
template <typename OutT>
__global__ __launch_bounds__(256) void merge_kernel(AttnArgs a, int D, int log2G) {
  const int rbi = blockIdx.x, g = blockIdx.y;
  const int i0 = a.item_off[rbi];
  const int ns = a.item_off[rbi + 1] - i0;
  if (ns <= 1) return;
  const int b = a.rb_seq[rbi];
  if (b < 0 || b >= a.B) return;
  const int NB = kRowsPerWG >> log2G;
  const int G = 1 << log2G;
  const int rb = rbi - a.seq_rb_off[b];
  const int s0 = a.node_offsets[b];
  const int n = a.node_offsets[b + 1] - s0;
  const int node0 = rb * NB;
  const int nodes_here = min(NB, n - node0);
  const int DQ = D / 4;
  for (int task = threadIdx.x; task < kRowsPerWG * DQ; task += blockDim.x) {
    const int row = task / DQ, dq = task % DQ;
    if ((row >> log2G) >= nodes_here) continue;
    const int node = s0 + node0 + (row >> log2G);
    const int head = g * G + (row & (G - 1));
    float M = -INFINITY;
    for (int s = 0; s < ns; ++s)
      M = fmaxf(M, a.part_lse[((size_t)(i0 + s) * a.Hkv + g) * kRowsPerWG + row]);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float den = 0.f;
    for (int s = 0; s < ns; ++s) {
      const size_t base = ((size_t)(i0 + s) * a.Hkv + g) * kRowsPerWG + row;
      const float ls = a.part_lse[base];
      if (ls == -INFINITY) continue;
      const float w = __expf(ls - M);
      const float4 o = *(const float4*)(a.part_o + base * D + dq * 4);
      den += w;
      acc.x += w * o.x; acc.y += w * o.y; acc.z += w * o.z; acc.w += w * o.w;
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    OutT* op = (OutT*)a.out + ((size_t)node * a.Hq + head) * D + dq * 4;
    op[0] = (OutT)(acc.x * inv);
    op[1] = (OutT)(acc.y * inv);
    op[2] = (OutT)(acc.z * inv);
    op[3] = (OutT)(acc.w * inv);
    if (dq == 0 && a.lse) a.lse[(size_t)node * a.Hq + head] = den > 0.f ? M + __logf(den) : -INFINITY;
  }
}

__device__ inline float wave_max(float x) {
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) x = fmaxf(x, __shfl_xor(x, d));
  return x;
}
__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) x += __shfl_xor(x, d);
  return x;
}

// float32 path: one wave per (node, query head); lanes take 64 keys at a time.
template <int D>
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnArgs a) {
  constexpr int DPL = D / 64;  // output elements per lane
  __shared__ float qs[D];
  __shared__ float ps[64];
  if (a.status[0] & TAV_DEV_PLAN_MISMATCH) return;
  const int v = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const int G = a.Hq / a.Hkv, g = h / G;
  int lo = 0, hi = a.B;  // sequence of node v
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (a.node_offsets[mid] <= v) lo = mid; else hi = mid;
  }
  const int b = lo;
  const int s0 = a.node_offsets[b];
  const int local = v - s0;
  const int L = a.prefix_len[b];
  const bool chain = a.is_chain[b] != 0;
  if (!chain && a.node_offsets[b + 1] - s0 > kMaxTreeNodes) return;  // rejected by tree preparation
  uint64_t mw[kMaskWords] = {0ull, 0ull, 0ull, 0ull};
  if (!chain) {
#pragma unroll
    for (int w = 0; w < kMaskWords; ++w) mw[w] = a.mask[(size_t)v * kMaskWords + w];
  }
  const float* q = (const float*)a.q;
  const float* kc = (const float*)a.k_cache;
  const float* vc = (const float*)a.v_cache;
  const float* kn = (const float*)a.k_node;
  const float* vn = (const float*)a.v_node;
  for (int d = lane; d < D; d += 64) qs[d] = q[((size_t)v * a.Hq + h) * D + d];
  __syncthreads();
  auto row_ptr = [&](int k, bool key, bool* ok) -> const float* {
    if (k < L) {
      const int blk = a.block_table[(size_t)b * a.max_blocks + k / a.block_size];
      if ((unsigned)blk >= (unsigned)a.num_blocks) {
        atomicOr(a.status, (uint32_t)TAV_DEV_BAD_BLOCK);
        *ok = false;
        return nullptr;
      }
      const size_t off = (((size_t)blk * a.Hkv + g) * a.block_size + (k % a.block_size)) * D;
      return (key ? kc : vc) + off;
    }
    const int j = k - L;
    *ok = chain || ((mw[j >> 6] >> (j & 63)) & 1ull);
    return (key ? kn : vn) + ((size_t)(s0 + j) * a.Hkv + g) * D;
  };
  float m = -INFINITY, l = 0.f;
  float o[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) o[i] = 0.f;
  const int total = L + local + 1;  // prefix rows, then tree nodes 0..local
  for (int base = 0; base < total; base += 64) {
    const int k = base + lane;
    float s = -INFINITY;
    if (k < total) {
      bool ok = true;
      const float* kp = row_ptr(k, true, &ok);
      if (ok) {
        float dot = 0.f;
        for (int d = 0; d < D; ++d) dot = fmaf(qs[d], kp[d], dot);
        s = dot * a.scale;
      }
    }
    const float mx = wave_max(s);
    const float m_new = fmaxf(m, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = expf(m - m_use);
    const float p = s == -INFINITY ? 0.f : expf(s - m_use);
    l = l * alpha + wave_sum(p);
    m = m_new;
#pragma unroll
    for (int i = 0; i < DPL; ++i) o[i] *= alpha;
    ps[lane] = p;
    __syncthreads();
    const int cnt = min(64, total - base);
    for (int jj = 0; jj < cnt; ++jj) {
      const float pj = ps[jj];
      if (pj == 0.f) continue;
      bool ok = true;
      const float* vp = row_ptr(base + jj, false, &ok);
      if (!ok) continue;
#pragma unroll
      for (int i = 0; i < DPL; ++i) o[i] = fmaf(pj, vp[lane + 64 * i], o[i]);
    }
    __syncthreads();
  }
  float* op = (float*)a.out + ((size_t)v * a.Hq + h) * D;
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int i = 0; i < DPL; ++i) op[lane + 64 * i] = o[i] * inv;
  if (lane == 0 && a.lse) a.lse[(size_t)v * a.Hq + h] = l > 0.f ? m + logf(l) : -INFINITY;
}

template <int D>
hipError_t launch_bf16_d(const Plan& p, const AttnArgs& a, hipStream_t s) {
  dim3 grid(p.total_items, p.Hkv);
  switch (p.log2G) {
    case 0: attn_bf16_kernel<D, 0><<<grid, 512, 0, s>>>(a); break;
    case 1: attn_bf16_kernel<D, 1><<<grid, 512, 0, s>>>(a); break;
    case 2: attn_bf16_kernel<D, 2><<<grid, 512, 0, s>>>(a); break;
    case 3: attn_bf16_kernel<D, 3><<<grid, 512, 0, s>>>(a); break;
    case 4: attn_bf16_kernel<D, 4><<<grid, 512, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const Plan& p, const AttnArgs& a, hipStream_t s) {
  if (p.total_items == 0) return hipSuccess;
  return p.D == 128 ? launch_bf16_d<128>(p, a, s) : launch_bf16_d<64>(p, a, s);
}

hipError_t launch_attn_f32(const Plan& p, const AttnArgs& a, hipStream_t s) {
  dim3 grid(p.N, p.Hq);
  if (p.D == 128) attn_f32_kernel<128><<<grid, 64, 0, s>>>(a);
  else attn_f32_kernel<64><<<grid, 64, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_merge(const Plan& p, const AttnArgs& a, bool bf16_out, hipStream_t s) {
  if (!p.any_split) return hipSuccess;
  dim3 grid(p.total_rb, p.Hkv);
  if (bf16_out) merge_kernel<__bf16><<<grid, 256, 0, s>>>(a, p.D, p.log2G);
  else merge_kernel<float><<<grid, 256, 0, s>>>(a, p.D, p.log2G);
  return hipGetLastError();
}

}  // namespace tav
