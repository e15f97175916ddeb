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
// Prefix tiles reach LDS by global->LDS copies through a ring of four stages
// (three tiles in flight), one barrier per tile; block-table entries are read
// through the scalar cache so they do not drain the copy counter.  K tiles are
// row-major with an XOR swizzle, V tiles d-major in a layout whose operand
// reads are free of bank conflicts.  The softmax scale is folded into one FMA
// per score in the exponent.
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

// Direct global -> LDS copy of 16 bytes per lane; the LDS destination is wave-uniform and
// lane i's bytes land at lds + 16 * i.  Issued through inline assembly: the compiler then
// does not treat every later LDS read as possibly aliasing the copy (which makes it wait for
// all copies in flight before each read, so the copies of later tiles never overlap the
// math).  The copies are ordered explicitly instead: wait_vm on the copy count of each tile,
// a barrier, and compiler-only memory barriers around both.  M0 holds the LDS address; the
// compiler keeps no value of its own in M0 in this kernel.
__device__ inline void dma16(const void* gsrc, void* lds_wave_base) {
  const uint32_t lds_off = (uint32_t)(size_t)(__attribute__((address_space(3))) char*)lds_wave_base;
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :: "v"(gsrc), "s"(__builtin_amdgcn_readfirstlane(lds_off)) : "memory");
}

// s_waitcnt on outstanding vector-memory operations only (lgkm / exp counters untouched).
template <int N>
__device__ inline void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Row of MFMA output m (within a 32-row block) -> key of the tile: bits 2 and 3 of
// each 16-group swapped, so a lane's 8 probabilities of one 16-key group are 8
// consecutive keys and the V^T operand is one 16-byte read.
__device__ inline int sigma(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

constexpr int kStages = 4;          // key tiles in LDS (3 in flight while one is computed)
constexpr float kRescaleSlack = 8.f;  // keep a stale max while the tile max exceeds it by <= 2^8

// Stored 16-byte position of chunk c of key row k in a K tile (bank spreading
// for the MFMA operand reads: rows are 256 B for D = 128 and 128 B for D = 64).
template <int D>
__device__ inline int kpos(int c, int key) {
  return D == 128 ? (c ^ (key & 15)) : (c ^ ((key >> 1) & 7));
}

// Byte offset of (key kk of a 16-key sub-block, d) inside the sub-block's V^T region: groups of
// 32 d rows, each [key half (2)][32 d][8 keys], so the MFMA operand reads (16 lanes = 16
// consecutive d rows of one key half) cover 256 contiguous bytes.
__device__ inline int vt_off(int d, int kk) {
  return (d >> 5) * 1024 + (kk >> 3) * 512 + (d & 31) * 16 + (kk & 7) * 2;
}

typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;

template <int D, int LOG2G>
__global__ __launch_bounds__(512) void attn_bf16_kernel(AttnArgs a) {
  constexpr int G = 1 << LOG2G;
  constexpr int KS = D / 16;               // k-steps of S^T = K Q^T
  constexpr int DB = D / 32;               // 32-wide d blocks of O^T
  constexpr int CH = D / 8;                // 16-byte chunks per key row
  constexpr int NB = kRowsPerWG >> LOG2G;  // nodes per row block
  constexpr int TILE_BYTES = kTileKeys * D * 2;
  constexpr int SUB_BYTES = D * 32;                     // one 16-key sub-block of V^T
  constexpr int KEYS_PER_DMA = 1024 / (D * 2);          // key rows per 1 KB wave load
  constexpr int DMA_PER_OPERAND = TILE_BYTES / 1024 / 8;  // per wave and tile, for K and for V
  constexpr int DMA_PER_TILE = 2 * DMA_PER_OPERAND;
  // LDS: per stage a K tile [64 keys][D] (16-byte chunk c of key k stored at kpos(c, k)) and
  // a V^T tile [4 sub-blocks of 16 keys] laid out by vt_off.
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kStages][2 * TILE_BYTES];

  if (a.status[0] & TAV_DEV_PLAN_MISMATCH) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  // block-table entries are read through the scalar cache: they do not count against the
  // vector-memory counter that paces the tile copies
  const const_i32_ptr btab = (const_i32_ptr)(a.block_table + (size_t)b * a.max_blocks);

  // this lane's query row
  const int row = wave * 32 + l32;
  const int rnode = node0 + (row >> LOG2G);
  const bool rvalid = (row >> LOG2G) < nodes_here;
  const int rhead = g * G + (row & (G - 1));
  bf16x8_t qreg[KS];
  {
    const uint16_t* qp = (const uint16_t*)a.q +
                         ((size_t)(s0 + (rvalid ? rnode : 0)) * Hq + rhead) * D + h32 * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      Bf16Pack8 t;
      t.u = *(const uint4*)(qp + ks * 16);
      if (!rvalid) t.u = make_uint4(0u, 0u, 0u, 0u);
      qreg[ks] = t.v;
    }
  }

  const uint16_t* kc = (const uint16_t*)a.k_cache;
  const uint16_t* vc = (const uint16_t*)a.v_cache;
  const int first_blk = L > 0 ? btab[0] : 0;

  // DMA of prefix tile t into stage st.  Wave w copies key rows 8w..8w+7 of the K tile and
  // d rows (w%2)*D/2 .. of sub-block w/2 of the V^T tile (lanes 0-31 keys 0-7, lanes 32-63
  // keys 8-15 of 32 d rows per copy); every address stays inside a valid block (rows past
  // the prefix read the first block and are masked).
  const int lbs = __builtin_ctz(bs);   // block sizes are powers of two
  // per-lane element offsets of the copies inside a 16-key sub-block (the same for every tile)
  int k_lane[DMA_PER_OPERAND], v_lane[DMA_PER_OPERAND];
#pragma unroll
  for (int i = 0; i < DMA_PER_OPERAND; ++i) {
    const int kt = wave * 8 + i * KEYS_PER_DMA + lane / CH;   // key of the tile
    k_lane[i] = (kt - (wave >> 1) * 16) * D + kpos<D>(lane % CH, kt) * 8;
    const int d = (wave & 1) * (D / 2) + i * 32 + l32;
    v_lane[i] = d * bs + h32 * 8;
  }
  auto issue_prefix = [&](int t, int st) {
    uint8_t* kbase = lds[st];
    uint8_t* vbase = lds[st] + TILE_BYTES;
    const int sb = wave >> 1;
    const int r0 = t * kTileKeys + sb * 16;              // first key row of the sub-block
    int blk = r0 < L ? btab[r0 >> lbs] : first_blk;
    if ((unsigned)blk >= (unsigned)a.num_blocks) {
      if (lane == 0) atomicOr(a.status, (uint32_t)TAV_DEV_BAD_BLOCK);
      blk = 0;
    }
    const int slot0 = r0 & (bs - 1);
    const uint16_t* ksrc = kc + (((size_t)blk * Hkv + g) * bs + slot0) * D;
    const uint16_t* vsrc = vc + ((size_t)blk * Hkv + g) * D * bs + slot0;
#pragma unroll
    for (int i = 0; i < DMA_PER_OPERAND; ++i) {
      dma16(ksrc + k_lane[i], kbase + (wave * 8 + i * KEYS_PER_DMA) * (D * 2));
      dma16(vsrc + v_lane[i], vbase + sb * SUB_BYTES + (((wave & 1) * (D / 2) + i * 32) >> 5) * 1024);
    }
  };

  float m_run = -INFINITY, l_run = 0.f;  // running max (log2 units) and sum of this lane's row
  f32x16_t acc[DB];
#pragma unroll
  for (int mb = 0; mb < DB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[mb][r] = 0.f;
  const float c2 = a.scale * kLog2e;      // score -> log2 units

  // raw scores S^T = K Q^T of the tile in stage st; element r of block kb of this lane is
  // key kb*32 + (r/8)*16 + h32*8 + r%8 of the tile, query row `row`
  auto s_tile = [&](int st, f32x16_t (&sacc)[2]) {
    const uint8_t* kbase = lds[st];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int key = kb * 32 + sigma(l32);
        const bf16x8_t ka = *(const bf16x8_t*)(kbase + key * (D * 2) + kpos<D>(ks * 2 + h32, key) * 16);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[ks], sacc[kb], 0, 0, 0);
      }
    }
  };

  // masking of a tile's scores: kind 1 = the last, partial prefix tile, kind 2 = a tree-tail tile
  auto mask_tile = [&](int t, int kind, f32x16_t (&sacc)[2]) {
    uint64_t mw = 0;
    if (kind == 2 && !chain && rvalid) mw = a.mask[(size_t)(s0 + rnode) * kMaskWords + (t - Tp)];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kin = kb * 32 + (r >> 3) * 16 + h32 * 8 + (r & 7);
        bool vis;
        if (kind == 1) {
          vis = t * kTileKeys + kin < L;
        } else {
          const int j = (t - Tp) * kTileKeys + kin;
          vis = j < tail_n && (chain ? j <= rnode : ((mw >> (j & 63)) & 1ull) != 0ull);
        }
        sacc[kb][r] = vis ? sacc[kb][r] : -INFINITY;
      }
    }
  };

  // online softmax of one tile: P (bf16, this lane's 32 keys as 4 MFMA operands), the new
  // running max / sum, and whether the accumulator needs rescaling by *alpha.  The running
  // max is kept until some row's tile max exceeds it by 2^8 (a wave-uniform decision).
  auto softmax_tile = [&](f32x16_t (&sacc)[2], bf16x8_t (&pb)[4], float& alpha) -> bool {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * c2;
    const bool need = __ballot(mx > m_run + kRescaleSlack) != 0ull;
    const float m_new = need ? fmaxf(m_run, mx) : m_run;
    alpha = fast_exp2(m_run - (m_new == -INFINITY ? 0.f : m_new));
    m_run = m_new;
    const float mu = m_new == -INFINITY ? 0.f : m_new;
    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(fmaf(sacc[kb][r], c2, -mu));
        ps += p;
        pb[kb * 2 + (r >> 3)][r & 7] = (__bf16)p;
      }
    }
    l_run = l_run * alpha + ps;
    return need;
  };

  // O^T += V^T P^T over the four 16-key sub-blocks of the tile in stage st
  auto pv_tile = [&](int st, const bf16x8_t (&pb)[4]) {
    const uint8_t* vbase = lds[st] + TILE_BYTES;
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2) {
#pragma unroll
      for (int mb = 0; mb < DB; ++mb) {
        const bf16x8_t va = *(const bf16x8_t*)(vbase + k2 * SUB_BYTES + mb * 1024 + h32 * 512 + l32 * 16);
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[k2], acc[mb], 0, 0, 0);
      }
    }
  };
  auto rescale = [&](float alpha) {
#pragma unroll
    for (int mb = 0; mb < DB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][r] *= alpha;
  };

  // ---- prefix tiles: DMA ring of kStages tiles (kStages - 1 in flight), one barrier per
  // tile; per tile: scores, softmax, P V ----
  const int p_end = min(t_end, Tp);
  if (t_begin < p_end) {
    int issued = t_begin;
    for (; issued < min(p_end, t_begin + kStages - 1); ++issued) issue_prefix(issued, (issued - t_begin) % kStages);
    for (int t = t_begin; t < p_end; ++t) {
      const int after = issued - 1 - t;       // tiles issued after t, still in flight
      asm volatile("" ::: "memory");          // no LDS access moves across the wait and barrier
      if (after >= 2) wait_vm<2 * DMA_PER_TILE>();
      else if (after == 1) wait_vm<DMA_PER_TILE>();
      else wait_vm<0>();
      __builtin_amdgcn_s_barrier();           // tile t landed for every wave; tile t-1's stage is free
      asm volatile("" ::: "memory");
      if (issued < p_end) {
        issue_prefix(issued, (issued - t_begin) % kStages);
        ++issued;
      }
      const int st = (t - t_begin) % kStages;
      f32x16_t sacc[2];
      if ((t + 1) * kTileKeys > L) {
        // last, partial prefix tile: zero V^T of keys >= L so 0 * stale data never reaches O
        uint8_t* vbase = lds[st] + TILE_BYTES;
        for (int e = tid; e < 4 * D * 16; e += 512) {
          const int sbk = e / (D * 16), d = (e / 16) % D, kk = e % 16;
          if (t * kTileKeys + sbk * 16 + kk >= L) *(uint16_t*)(vbase + sbk * SUB_BYTES + vt_off(d, kk)) = 0;
        }
        __syncthreads();
        s_tile(st, sacc);
        mask_tile(t, 1, sacc);
      } else {
        s_tile(st, sacc);
      }
      bf16x8_t pb[4];
      float alpha;
      if (softmax_tile(sacc, pb, alpha)) rescale(alpha);
      pv_tile(st, pb);
    }
    __syncthreads();
  }

  // ---- tree-tail tiles (the sequence's own nodes), staged through registers ----
  const uint16_t* kn = (const uint16_t*)a.k_node;
  const uint16_t* vn = (const uint16_t*)a.v_node;
  for (int t = max(t_begin, Tp); t < t_end; ++t) {
    uint8_t* kbase = lds[0];
    uint8_t* vbase = lds[0] + TILE_BYTES;
#pragma unroll
    for (int i = 0; i < (kTileKeys * CH) / 512; ++i) {
      const int c = tid + i * 512;                // 64 keys x CH chunks of 8 d
      const int key = c / CH, ch = c % CH;
      const int j = (t - Tp) * kTileKeys + key;
      const bool valid = j < tail_n;
      const size_t off = ((size_t)(s0 + (valid ? j : 0)) * Hkv + g) * D + ch * 8;
      uint4 kv = *(const uint4*)(kn + off);
      uint4 vv = *(const uint4*)(vn + off);
      if (!valid) kv = vv = make_uint4(0u, 0u, 0u, 0u);
      *(uint4*)(kbase + key * (D * 2) + kpos<D>(ch, key) * 16) = kv;
      const uint32_t w4[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *(uint16_t*)(vbase + (key >> 4) * SUB_BYTES + vt_off(ch * 8 + e, key & 15)) =
            (uint16_t)(w4[e >> 1] >> (16 * (e & 1)));
    }
    __syncthreads();
    f32x16_t sacc[2];
    s_tile(0, sacc);
    mask_tile(t, 2, sacc);
    bf16x8_t pb[4];
    float alpha;
    if (softmax_tile(sacc, pb, alpha)) rescale(alpha);
    pv_tile(0, pb);
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
// One block per (row block, KV head, group of 16 rows); a thread owns 4 outputs.
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
  for (int task = threadIdx.x; task < 16 * DQ; task += blockDim.x) {
    const int row = blockIdx.z * 16 + task / DQ, dq = task % DQ;
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
  // pointer to element 0 of key k's key (or value) vector and the stride between its elements
  auto row_ptr = [&](int k, bool key, bool* ok, int* stride) -> const float* {
    *stride = 1;
    if (k < L) {
      const int blk = a.block_table[(size_t)b * a.max_blocks + k / a.block_size];
      if ((unsigned)blk >= (unsigned)a.num_blocks) {
        atomicOr(a.status, (uint32_t)TAV_DEV_BAD_BLOCK);
        *ok = false;
        return nullptr;
      }
      const int slot = k % a.block_size;
      if (key) return kc + (((size_t)blk * a.Hkv + g) * a.block_size + slot) * D;
      *stride = a.block_size;                    // values: [block, head, d, slot]
      return vc + ((size_t)blk * a.Hkv + g) * D * a.block_size + slot;
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
      int st1;
      const float* kp = row_ptr(k, true, &ok, &st1);
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
      int vst;
      const float* vp = row_ptr(base + jj, false, &ok, &vst);
      if (!ok) continue;
#pragma unroll
      for (int i = 0; i < DPL; ++i) o[i] = fmaf(pj, vp[(size_t)(lane + 64 * i) * vst], o[i]);
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
  dim3 grid(p.total_rb, p.Hkv, kRowsPerWG / 16);
  if (bf16_out) merge_kernel<__bf16><<<grid, 256, 0, s>>>(a, p.D, p.log2G);
  else merge_kernel<float><<<grid, 256, 0, s>>>(a, p.D, p.log2G);
  return hipGetLastError();
}

}  // namespace tav
