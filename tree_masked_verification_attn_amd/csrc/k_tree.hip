// Tree preparation, the attention work plan and the packing of the tree nodes' keys / values.
//
// Visibility follows Progressive Tree Drafting, Section 3.1 ("Tree
// Construction"): pi(v) = {v} U pi(P(v)), and a node's position is fixed by
// |pi(v)|; behind a cached prefix of L rows, position = L + depth(v).
//
// For bf16 attention the three jobs run as one launch (prelude_kernel): blocks
// [0, B) prepare one sequence each, block B computes the work plan, and the
// remaining blocks pack one (node block, KV head) each.  None of them reads
// another's output; the attention kernel that follows reads all three.  In the
// whole scoring pass the start of the call (status word, workers' counter,
// per-sequence error words) is folded into the same launch.
#include "tav_internal.h"

#include <algorithm>

namespace tav {
namespace {

constexpr int kPrepThreads = 256;
constexpr int kPlanLds = 2048;   // sequences / row blocks whose plan arrays are staged in LDS

// The LDS of each job.  A launch that runs several jobs in different blocks overlays them (one union),
// so that it holds only the largest and more of its blocks fit on a compute unit.
struct PrepLds {
  int par[kMaxTreeNodes];
};
struct PlanLds {
  int scan[16];
  int off[kPlanLds], tile[kPlanLds], wt[kPlanLds];
};
template <int D>
struct PackLds {
  alignas(16) uint16_t vs[64][D + 8];   // values of up to 64 / block_size heads, [head, slot][d]
  int scan[16];
  int seq, base;
};
struct OrderLds {
  int scan[16];
};


// Inclusive scan of one int per lane over the wave without LDS round trips: DPP row shifts inside each
// row of 16 lanes (a lane whose source lies outside its row adds 0), then the rows' totals read with
// readlane and added to the later rows.  Every lane of the wave must be active.
template <int CTRL>
__device__ inline int dpp_shr(int x) { return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false); }
__device__ inline int wave_inclusive_scan(int x) {
  x += dpp_shr<0x111>(x);   // row_shr:1
  x += dpp_shr<0x112>(x);   // row_shr:2
  x += dpp_shr<0x114>(x);   // row_shr:4
  x += dpp_shr<0x118>(x);   // row_shr:8
  const int t0 = __builtin_amdgcn_readlane(x, 15), t1 = __builtin_amdgcn_readlane(x, 31);
  const int t2 = __builtin_amdgcn_readlane(x, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return x + (row == 0 ? 0 : row == 1 ? t0 : row == 2 ? t0 + t1 : t0 + t1 + t2);
}

// Exclusive scan of one int per thread over the block; also returns the total.  Called by every thread.
__device__ int block_exclusive_scan(int v, int* lds, int* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int x = wave_inclusive_scan(v);
  if (lane == 63) lds[wid] = x;
  __syncthreads();
  int before = 0, tot = 0;
  for (int w = 0; w < nw; ++w) {
    const int t = lds[w];
    before += w < wid ? t : 0;
    tot += t;
  }
  *total = tot;
  __syncthreads();   // (lds is reused by the next scan)
  return before + x - v;
}

struct PrepArgs {
  const int32_t* node_offsets;
  const int32_t* prefix_len;
  const int32_t* parent;
  uint8_t* chain_ws;
  uint64_t* mask_ws;
  int32_t* depth_out;
  int32_t* pos_out;
  uint64_t* mask_out;
  uint8_t* chain_out;
  uint32_t* status;
  uint32_t* seq_err;
  int fused_start;   // the call's start is folded into the prelude: errors go to seq_err[b] only
};

// Sequence b: validate parents, detect a chain, and build depth, position and the 256-bit
// ancestor masks of a non-chain tree.  With fused_start the block first clears seq_err[b] (no start
// kernel ran) and reports its errors there only: another block of the same launch clears the status
// word, and the call's last kernel folds the sequences' error words into it.
__device__ void prep_sequence(const PrepArgs& a, int b, PrepLds& S) {
  int* par_s = S.par;
  const int s0 = a.node_offsets[b];
  const int n = a.node_offsets[b + 1] - s0;
  const int L = a.prefix_len[b];
  if (a.fused_start && threadIdx.x == 0) a.seq_err[b] = 0u;
  int bad = 0, not_chain = 0;
  for (int v = threadIdx.x; v < n; v += blockDim.x) {
    int p = a.parent[s0 + v];
    if (v == 0 ? p != -1 : (p < 0 || p >= v)) bad = 1;
    if (v > 0 && p != v - 1) not_chain = 1;
  }
  bad = __syncthreads_or(bad);
  not_chain = __syncthreads_or(not_chain);
  if (bad) {
    if (threadIdx.x == 0) {
      if (!a.fused_start) atomicOr(a.status, (uint32_t)TAV_DEV_BAD_PARENT);
      atomicOr(a.seq_err + b, (uint32_t)TAV_DEV_BAD_PARENT);
      a.chain_ws[b] = 0;
    }
    return;
  }
  if (threadIdx.x == 0) {
    a.chain_ws[b] = not_chain ? 0 : 1;
    if (a.chain_out) a.chain_out[b] = not_chain ? 0 : 1;
  }
  if (!not_chain) {
    for (int v = threadIdx.x; v < n; v += blockDim.x) {
      if (a.depth_out) a.depth_out[s0 + v] = v;
      if (a.pos_out) a.pos_out[s0 + v] = L + v;
      if (a.mask_out) {
#pragma unroll
        for (int w = 0; w < kMaskWords; ++w) a.mask_out[(size_t)(s0 + v) * kMaskWords + w] = 0ull;
      }
    }
    return;
  }
  if (n > kMaxTreeNodes) {
    if (threadIdx.x == 0) {
      if (!a.fused_start) atomicOr(a.status, (uint32_t)TAV_DEV_TREE_TOO_LARGE);
      atomicOr(a.seq_err + b, (uint32_t)TAV_DEV_TREE_TOO_LARGE);
    }
    return;
  }
  for (int v = threadIdx.x; v < n; v += blockDim.x) par_s[v] = a.parent[s0 + v];
  __syncthreads();
  for (int v = threadIdx.x; v < n; v += blockDim.x) {
    uint64_t w[kMaskWords] = {0ull, 0ull, 0ull, 0ull};
    int x = v, d = 0;
    // walk to the root; parents were validated to be earlier nodes, so this ends
    for (int step = 0; step < kMaxTreeNodes; ++step) {
      w[x >> 6] |= 1ull << (x & 63);
      if (x == 0) break;
      x = par_s[x];
      ++d;
    }
#pragma unroll
    for (int k = 0; k < kMaskWords; ++k) {
      a.mask_ws[(size_t)(s0 + v) * kMaskWords + k] = w[k];
      if (a.mask_out) a.mask_out[(size_t)(s0 + v) * kMaskWords + k] = w[k];
    }
    if (a.depth_out) a.depth_out[s0 + v] = d;
    if (a.pos_out) a.pos_out[s0 + v] = L + d;
  }
}

struct PlanArgs {
  int B, NB, bs, total_rb_host, tiles_host, tail_blocks_host, C, W;
  int fused_start;   // the plan block clears the status word and the workers' counter first
};

// The attention work plan (one block): seq_rb_off[B+1] (row blocks per sequence), rb_seq,
// rb_tile[total_rb+1] (first key tile of each row block, per KV head), tail_blk[B+1] (first
// packed node block of each sequence), each workgroup's share wg_tile / wg_rb, and the record
// of each row block, identical to the host plan; a disagreement with the host's totals sets
// TAV_DEV_PLAN_MISMATCH.  The row-block offsets and tiles are staged in LDS when they fit (SMALL), and
// so are the workgroups' first tiles (SMALL_W); the choice is made at compile time, so that every
// access has one address space (an access through a pointer to either is a flat access, which waits
// for all memory operations in flight).
template <bool SMALL, bool SMALL_W>
__device__ void plan_block_t(const PlanArgs& p, const AttnArgs& a, PlanLds& S) {
  int* scan_s = S.scan;
  int* off_s = S.off;
  int* tile_s = S.tile;
  int* wt_s = S.wt;
  const int B = p.B, NB = p.NB, bs = p.bs, C = p.C, W = p.W;
  const int32_t* node_offsets = a.node_offsets;
  const int32_t* prefix_len = a.prefix_len;
  int32_t* seq_rb_off = const_cast<int32_t*>(a.seq_rb_off);
  int32_t* rb_seq = const_cast<int32_t*>(a.rb_seq);
  int32_t* rb_tile = const_cast<int32_t*>(a.rb_tile);
  int32_t* tail_blk = const_cast<int32_t*>(a.tail_blk);
  int32_t* wg_rb = const_cast<int32_t*>(a.wg_rb);
  int32_t* wg_tile = const_cast<int32_t*>(a.wg_tile);
  int32_t* rb_meta = const_cast<int32_t*>(a.rb_meta);
  if (p.fused_start && threadIdx.x == 0) {   // (only this block writes the status word in this launch)
    a.status[0] = 0u;
    a.status[kCounterWord] = 0u;
  }
  int* off = SMALL ? off_s : seq_rb_off;   // working copies (LDS or the outputs themselves)
  int* tile = SMALL ? tile_s : rb_tile;
  int carry = 0, bcarry = 0;
  for (int base = 0; base < B; base += blockDim.x) {
    const int b = base + threadIdx.x;
    int cnt = 0, nblk = 0;
    if (b < B) {
      const int n = node_offsets[b + 1] - node_offsets[b];
      cnt = (n + NB - 1) / NB;
      nblk = (n + bs - 1) / bs;
    }
    int tot, btot;
    const int ex = block_exclusive_scan(cnt, scan_s, &tot);
    const int bex = block_exclusive_scan(nblk, scan_s, &btot);
    if (b < B) {
      off[b] = carry + ex;
      tail_blk[b] = bcarry + bex;
    }
    carry += tot;
    bcarry += btot;
  }
  if (threadIdx.x == 0) {
    off[B] = carry;
    tail_blk[B] = bcarry;
  }
  const int total_rb = carry;
  if (total_rb != p.total_rb_host || bcarry != p.tail_blocks_host) {
    if (threadIdx.x == 0) atomicOr(a.status, (uint32_t)TAV_DEV_PLAN_MISMATCH);
    return;
  }
  __syncthreads();
  int tcarry = 0;
  for (int base = 0; base < total_rb; base += blockDim.x) {
    const int r = base + threadIdx.x;
    int cnt = 0;
    if (r < total_rb) {
      int lo = 0, hi = B;  // largest b with off[b] <= r
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (off[mid] <= r) lo = mid; else hi = mid;
      }
      const int b = lo;
      const int n = node_offsets[b + 1] - node_offsets[b];
      cnt = rb_tiles(prefix_len[b], n, r - off[b], NB);
      rb_seq[r] = b;
    }
    int tot;
    const int ex = block_exclusive_scan(cnt, scan_s, &tot);
    if (r < total_rb) tile[r] = tcarry + ex;
    tcarry += tot;
  }
  if (threadIdx.x == 0) {
    tile[total_rb] = tcarry;
    if (tcarry != p.tiles_host) atomicOr(a.status, (uint32_t)TAV_DEV_PLAN_MISMATCH);
  }
  if (tcarry != p.tiles_host) return;
  __syncthreads();
  if constexpr (SMALL) {
    for (int b = threadIdx.x; b <= B; b += blockDim.x) seq_rb_off[b] = off[b];
    for (int r = threadIdx.x; r <= total_rb; r += blockDim.x) rb_tile[r] = tile[r];
  }
  // each attention workgroup's first key tile (its share of the weighted tile axis: tile t of
  // row block r at t + kRbCost * r) and the row block holding it
  for (int w = threadIdx.x; w <= W; w += blockDim.x) {
    const int x = w * C;   // weighted position of the share's start
    int lo = 0, hi = total_rb;  // largest r with tile[r] + kRbCost * r <= x
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (tile[mid] + kRbCost * mid <= x) lo = mid; else hi = mid;
    }
    // a share starting inside a row block's fixed-cost gap starts at the next row block
    const int j = w == W ? tcarry : min(tile[lo] + (x - tile[lo] - kRbCost * lo), tile[lo + 1]);
    wg_tile[w] = j;
    if constexpr (SMALL_W) wt_s[w] = j;
    if (w < W) {
      int r = lo;   // the row block holding tile j (an empty share keeps any valid index)
      if (j >= tile[lo + 1] && lo + 1 < total_rb) r = lo + 1;
      wg_rb[w] = r;
    }
  }
  // the attention kernel's record of each row block (the chain flag is read by the attention
  // kernel itself from the preparation's output), with the workgroups holding its first and last
  // tiles for the merge: the largest w with wg_tile[w] <= tile (never an empty share)
  __syncthreads();
  const int* wt = SMALL_W ? wt_s : wg_tile;
  auto owner = [&](int t) {
    int lo = 0, hi = W;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (wt[mid] <= t) lo = mid; else hi = mid;
    }
    return lo;
  };
  for (int r = threadIdx.x; r < total_rb; r += blockDim.x) {
    int lo = 0, hi = B;  // the row block's sequence: largest b with off[b] <= r
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (off[mid] <= r) lo = mid; else hi = mid;
    }
    const int b = lo;
    const int s0 = node_offsets[b];
    const int n = node_offsets[b + 1] - s0;
    const int node0 = (r - off[b]) * NB;
    int32_t* m = rb_meta + (size_t)r * kMetaWords;
    m[kMetaTile0] = tile[r];
    m[kMetaTileEnd] = tile[r + 1];
    m[kMetaS0] = s0;
    m[kMetaN] = n;
    m[kMetaL] = prefix_len[b];
    m[kMetaNode0] = node0;
    m[kMetaTailN] = min(n, node0 + NB);
    m[kMetaFlags] = n <= kMaxTreeNodes ? 2 : 0;
    m[kMetaSeq] = b;
    m[kMetaWf] = owner(tile[r]);
    m[kMetaWl] = owner(tile[r + 1] - 1);
  }
}

__device__ void plan_block(const PlanArgs& p, const AttnArgs& a, PlanLds& S) {
  const bool small = p.B + 1 <= kPlanLds && p.total_rb_host + 1 <= kPlanLds;
  const bool small_w = p.W + 1 <= kPlanLds;
  if (small) {
    if (small_w) plan_block_t<true, true>(p, a, S);
    else plan_block_t<true, false>(p, a, S);
  } else {
    if (small_w) plan_block_t<false, true>(p, a, S);
    else plan_block_t<false, false>(p, a, S);
  }
}

// Copies the keys and values of block_size consecutive tree nodes of one sequence (packed node
// block tb, KV heads [ga, gb)) into the paged cache's layout (keys [block, head, slot, d], values
// [block, head, d, slot]), zero-padded past the sequence's last node, so tree-tail tiles take the
// same copy path as prefix tiles.  The block's node rows ([node, head, d]) are one range of memory
// and so is each destination; keys keep their 16-byte pieces, values are transposed through LDS,
// 64 / block_size heads at a time.  The sequence of block tb is found from the node counts.  Runs on
// kPrepThreads threads.
template <int D>
__device__ void pack_block(const AttnArgs& a, int tb, int ga, int gb, PackLds<D>& S) {
  constexpr int CH = D / 8;     // 16-byte pieces of a row
  const int bs = a.block_size, Hkv = a.Hkv, B = a.B;
  // sequence b with tail offset off(b) <= tb < off(b) + ceil(n_b / bs)
  if (threadIdx.x == 0) S.seq = -1;
  int carry = 0;
  for (int base = 0; base < B; base += blockDim.x) {
    const int b = base + threadIdx.x;
    const int nblk = b < B ? (a.node_offsets[b + 1] - a.node_offsets[b] + bs - 1) / bs : 0;
    int tot;
    const int ex = block_exclusive_scan(nblk, S.scan, &tot);   // (its barriers order S.seq)
    if (b < B && tb >= carry + ex && tb < carry + ex + nblk) {
      S.seq = b;
      S.base = carry + ex;
    }
    carry += tot;
    __syncthreads();
    if (S.seq >= 0) break;
  }
  const int b = S.seq;
  if (b < 0) return;   // tb past the last block (not launched)
  const int s0 = a.node_offsets[b];
  const int n = a.node_offsets[b + 1] - s0;
  const int node_base = (tb - S.base) * bs;
  const uint16_t* kn = (const uint16_t*)a.k_node;
  const uint16_t* vn = (const uint16_t*)a.v_node;
  // the piece c = (head, slot, piece of the row) of the block, zero past the last node
  auto piece = [&](const uint16_t* src, int g0, int c) {
    const int g = g0 + c / (bs * CH), slot = (c / CH) % bs, ch = c % CH;
    const int node = node_base + slot;
    return node < n ? *(const uint4*)(src + ((size_t)(s0 + node) * Hkv + g) * D + ch * 8)
                    : make_uint4(0u, 0u, 0u, 0u);
  };
  // rounds of hg heads: their key and value pieces loaded together, the keys stored as they are
  // (piece c of the round's heads lands at piece c of their destination), the values staged in LDS
  // as [head, slot][d] and written d-major
  constexpr int kPer = 64 * CH / kPrepThreads;   // pieces per thread and round, of keys and of values
  static_assert(kPer * kPrepThreads == 64 * CH, "packing round shape");
  uint16_t* vt = (uint16_t*)a.v_tail;
  const int hg = 64 / bs, groups = bs / 8;
  for (int g0 = ga; g0 < gb; g0 += hg) {
    const int ng = min(hg, gb - g0);
    const int np = ng * bs * CH;
    uint4 kr[kPer], vr[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = threadIdx.x + i * kPrepThreads;
      if (c < np) {
        kr[i] = piece(kn, g0, c);
        vr[i] = piece(vn, g0, c);
      }
    }
    uint4* kt = (uint4*)a.k_tail + ((size_t)tb * Hkv + g0) * bs * CH;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = threadIdx.x + i * kPrepThreads;
      if (c < np) {
        kt[c] = kr[i];
        *(uint4*)&S.vs[c / CH][(c % CH) * 8] = vr[i];
      }
    }
    __syncthreads();
    for (int c = threadIdx.x; c < ng * D * groups; c += kPrepThreads) {
      const int gi = c / (D * groups), d = (c / groups) % D, sg = c % groups;
      const int row = gi * bs + sg * 8;
      uint32_t w4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w4[e] = (uint32_t)S.vs[row + 2 * e][d] | ((uint32_t)S.vs[row + 2 * e + 1][d] << 16);
      *(uint4*)(vt + (((size_t)tb * Hkv + g0 + gi) * D + d) * bs + sg * 8) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
    }
    __syncthreads();
  }
}

// The order in which the verification's workers take the nodes: nodes with a draft row (which
// stream their draft row too, three times the bytes of the others) first, in node order, then the
// others, so that the long items do not come last.
__device__ void order_block(const int32_t* draft_row, int R, int N, int32_t* order, OrderLds& S) {
  int* scan_s = S.scan;
  int hcarry = 0;
  for (int base = 0; base < N; base += blockDim.x) {
    const int v = base + threadIdx.x;
    const int dr = v < N ? draft_row[v] : -1;
    const int h = v < N && dr >= 0 && dr < R;
    int tot;
    const int ex = block_exclusive_scan(h, scan_s, &tot);
    if (v < N) order[h ? hcarry + ex : N - 1 - (v - hcarry - ex)] = v;
    hcarry += tot;
  }
}

// Start of a call: clears the status word, the workers' node counter and the per-sequence error
// words; with draft_row, builds the workers' node order.
__global__ __launch_bounds__(kPrepThreads) void start_kernel(uint32_t* status, uint32_t* seq_err, int B,
                                                             const int32_t* draft_row, int R, int N,
                                                             int32_t* order) {
  __shared__ OrderLds lds;
  if (threadIdx.x == 0) {
    status[0] = 0u;
    status[kCounterWord] = 0u;
  }
  if (seq_err)
    for (int b = threadIdx.x; b < B; b += blockDim.x) seq_err[b] = 0u;
  if (draft_row) order_block(draft_row, R, N, order, lds);
}

__global__ __launch_bounds__(kPrepThreads) void prep_kernel(PrepArgs a) {
  __shared__ PrepLds lds;
  prep_sequence(a, blockIdx.x, lds);
}

// Preparation with the call's start folded in (blocks [0, B): sequence blockIdx.x, each clearing and
// reporting into its own error word; block B: the status word and the workers' node counter; with
// an order to build, block B + 1: the verification workers' node order).
__global__ __launch_bounds__(kPrepThreads) void prep_start_kernel(PrepArgs a, int B, OrderArgs o) {
  __shared__ union {
    PrepLds prep;
    OrderLds order;
  } lds;
  const int bid = blockIdx.x;
  if (bid < B) {
    prep_sequence(a, bid, lds.prep);
  } else if (bid == B) {
    if (threadIdx.x == 0) {
      a.status[0] = 0u;
      a.status[kCounterWord] = 0u;
    }
  } else {
    order_block(o.draft_row, o.R, o.N, o.order, lds.order);
  }
}

// Blocks [0, B): preparation of sequence blockIdx.x; block B: the work plan; with an order to
// build, the last block: the verification workers' node order; the blocks between: hp KV heads of
// one packed node block each.  The jobs' LDS is overlaid.
template <int D>
__global__ __launch_bounds__(kPrepThreads) void prelude_kernel(PrepArgs pa, PlanArgs pl, AttnArgs a, OrderArgs o,
                                                               int hp) {
  __shared__ union {
    PrepLds prep;
    PlanLds plan;
    PackLds<D> pack;
    OrderLds order;
  } lds;
  const int bid = blockIdx.x;
  if (bid < pl.B) {
    prep_sequence(pa, bid, lds.prep);
  } else if (bid == pl.B) {
    plan_block(pl, a, lds.plan);
  } else if (o.order && bid == (int)gridDim.x - 1) {
    order_block(o.draft_row, o.R, o.N, o.order, lds.order);
  } else {
    const int i = bid - pl.B - 1, nhg = (a.Hkv + hp - 1) / hp;
    const int ga = (i % nhg) * hp;
    pack_block<D>(a, i / nhg, ga, min(a.Hkv, ga + hp), lds.pack);
  }
}

PrepArgs prep_args(const int32_t* node_offsets, const int32_t* prefix_len, const int32_t* parent,
                   uint8_t* chain_ws, uint64_t* mask_ws, const tav_tree_out* out, uint32_t* status,
                   uint32_t* seq_err) {
  PrepArgs a;
  a.node_offsets = node_offsets; a.prefix_len = prefix_len; a.parent = parent;
  a.chain_ws = chain_ws; a.mask_ws = mask_ws;
  a.depth_out = out ? out->depth : nullptr;
  a.pos_out = out ? out->position : nullptr;
  a.mask_out = out ? out->mask : nullptr;
  a.chain_out = out ? out->is_chain : nullptr;
  a.status = status;
  a.seq_err = seq_err;
  a.fused_start = 0;
  return a;
}

}  // namespace

hipError_t launch_start(uint32_t* status, uint32_t* seq_err, int B, const int32_t* draft_row, int R, int N,
                        int32_t* order, hipStream_t s) {
  start_kernel<<<1, kPrepThreads, 0, s>>>(status, seq_err, B, draft_row, R, N, order);
  return hipGetLastError();
}

hipError_t launch_prep(const Plan& p, const int32_t* node_offsets, const int32_t* prefix_len,
                       const int32_t* parent, uint8_t* chain_ws, uint64_t* mask_ws,
                       const tav_tree_out* out, uint32_t* status, uint32_t* seq_err, hipStream_t s) {
  prep_kernel<<<p.B, kPrepThreads, 0, s>>>(
      prep_args(node_offsets, prefix_len, parent, chain_ws, mask_ws, out, status, seq_err));
  return hipGetLastError();
}

hipError_t launch_prep_start(const Plan& p, const int32_t* node_offsets, const int32_t* prefix_len,
                             const int32_t* parent, uint8_t* chain_ws, uint64_t* mask_ws, const tav_tree_out* out,
                             uint32_t* status, uint32_t* seq_err, const OrderArgs& o, hipStream_t s) {
  PrepArgs pa = prep_args(node_offsets, prefix_len, parent, chain_ws, mask_ws, out, status, seq_err);
  pa.fused_start = 1;
  prep_start_kernel<<<p.B + 1 + (o.order ? 1 : 0), kPrepThreads, 0, s>>>(pa, p.B, o);
  return hipGetLastError();
}

hipError_t launch_prelude(const Plan& p, const int32_t* parent, const tav_tree_out* out, const AttnArgs& a,
                          const OrderArgs& o, bool fused_start, hipStream_t s) {
  PrepArgs pa = prep_args(a.node_offsets, a.prefix_len, parent, const_cast<uint8_t*>(a.is_chain),
                          const_cast<uint64_t*>(a.mask), out, a.status, a.seq_err);
  pa.fused_start = fused_start ? 1 : 0;
  PlanArgs pl;
  pl.fused_start = fused_start ? 1 : 0;
  pl.B = p.B; pl.NB = p.NB; pl.bs = p.bs; pl.total_rb_host = p.total_rb; pl.tiles_host = p.tiles_per_head;
  pl.tail_blocks_host = p.tail_blocks; pl.C = p.C; pl.W = p.W;
  // KV heads per packing block: one while (node block, head) pairs are few, more when they would be
  // tens of thousands of small blocks
  constexpr int64_t kPackBlocks = 2048;
  const int64_t pairs = (int64_t)p.tail_blocks * p.Hkv;
  const int hp = (int)std::min<int64_t>(p.Hkv, std::max<int64_t>(1, (pairs + kPackBlocks - 1) / kPackBlocks));
  const int grid = p.B + 1 + p.tail_blocks * ((p.Hkv + hp - 1) / hp) + (o.order ? 1 : 0);
  if (p.D == 128) prelude_kernel<128><<<grid, kPrepThreads, 0, s>>>(pa, pl, a, o, hp);
  else prelude_kernel<64><<<grid, kPrepThreads, 0, s>>>(pa, pl, a, o, hp);
  return hipGetLastError();
}

}  // namespace tav
