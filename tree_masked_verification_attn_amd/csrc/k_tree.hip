// Tree preparation and the attention work plan.
//
// Visibility follows Progressive Tree Drafting, Section 3.1 ("Tree
// Construction"): pi(v) = {v} U pi(P(v)), and a node's position is fixed by
// |pi(v)|; behind a cached prefix of L rows, position = L + depth(v).
#include "tav_internal.h"

namespace tav {
namespace {

// Clears the status word and the counter word that follows it in the status block.
__global__ void clear_status_kernel(uint32_t* status) {
  if (threadIdx.x == 0) { status[0] = 0u; status[kCounterWord] = 0u; }
}

// Exclusive scan of one int per thread over a 1024-thread block; also returns the total.
__device__ int block_exclusive_scan(int v, int* lds, int* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) lds[wid] = x;
  __syncthreads();
  if (wid == 0) {
    int s = lane < nw ? lds[lane] : 0;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      int y = __shfl_up(s, d, 64);
      if (lane >= d) s += y;
    }
    if (lane < nw) lds[lane] = s;
  }
  __syncthreads();
  int excl = (wid > 0 ? lds[wid - 1] : 0) + x - v;
  *total = lds[nw - 1];
  __syncthreads();
  return excl;
}

// One 1024-thread block: seq_rb_off[B+1] (row blocks per sequence), rb_seq,
// rb_tile[total_rb+1] (first key tile of each row block, per KV head) and
// tail_blk[B+1] (first packed node block of each sequence), identical to the
// host plan; a disagreement with the host's totals sets TAV_DEV_PLAN_MISMATCH.
__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* node_offsets,
                                                     const int32_t* prefix_len, int B, int NB,
                                                     int bs, int total_rb_host, int tiles_host,
                                                     int tail_blocks_host, int C, int W,
                                                     int32_t* seq_rb_off, int32_t* rb_seq,
                                                     int32_t* rb_tile, int32_t* tail_blk,
                                                     int32_t* wg_rb, int32_t* wg_tile,
                                                     const uint8_t* is_chain, int32_t* rb_meta,
                                                     uint32_t* status) {
  __shared__ int lds[16];
  int carry = 0, bcarry = 0;
  for (int base = 0; base < B; base += 1024) {
    const int b = base + threadIdx.x;
    int cnt = 0, nblk = 0;
    if (b < B) {
      const int n = node_offsets[b + 1] - node_offsets[b];
      cnt = (n + NB - 1) / NB;
      nblk = (n + bs - 1) / bs;
    }
    int tot, btot;
    const int ex = block_exclusive_scan(cnt, lds, &tot);
    const int bex = block_exclusive_scan(nblk, lds, &btot);
    if (b < B) {
      seq_rb_off[b] = carry + ex;
      tail_blk[b] = bcarry + bex;
    }
    carry += tot;
    bcarry += btot;
  }
  if (threadIdx.x == 0) {
    seq_rb_off[B] = carry;
    tail_blk[B] = bcarry;
  }
  const int total_rb = carry;
  if (total_rb != total_rb_host || bcarry != tail_blocks_host) {
    if (threadIdx.x == 0) atomicOr(status, (uint32_t)TAV_DEV_PLAN_MISMATCH);
    return;
  }
  __syncthreads();
  int tcarry = 0;
  for (int base = 0; base < total_rb; base += 1024) {
    const int r = base + threadIdx.x;
    int cnt = 0;
    if (r < total_rb) {
      int lo = 0, hi = B;  // largest b with seq_rb_off[b] <= r
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (seq_rb_off[mid] <= r) lo = mid; else hi = mid;
      }
      const int b = lo;
      const int n = node_offsets[b + 1] - node_offsets[b];
      cnt = rb_tiles(prefix_len[b], n, r - seq_rb_off[b], NB);
      rb_seq[r] = b;
    }
    int tot;
    const int ex = block_exclusive_scan(cnt, lds, &tot);
    if (r < total_rb) rb_tile[r] = tcarry + ex;
    tcarry += tot;
  }
  if (threadIdx.x == 0) {
    rb_tile[total_rb] = tcarry;
    if (tcarry != tiles_host) atomicOr(status, (uint32_t)TAV_DEV_PLAN_MISMATCH);
  }
  if (tcarry != tiles_host) return;
  __syncthreads();
  // each attention workgroup's first key tile (its share of the weighted tile axis: tile t of
  // row block r at t + kRbCost * r) and the row block holding it
  for (int w = threadIdx.x; w <= W; w += blockDim.x) {
    const int x = w * C;   // weighted position of the share's start
    int lo = 0, hi = total_rb;  // largest r with rb_tile[r] + kRbCost * r <= x
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (rb_tile[mid] + kRbCost * mid <= x) lo = mid; else hi = mid;
    }
    // a share starting inside a row block's fixed-cost gap starts at the next row block
    const int j = w == W ? tcarry : min(rb_tile[lo] + (x - rb_tile[lo] - kRbCost * lo), rb_tile[lo + 1]);
    wg_tile[w] = j;
    if (w < W) {
      int r = lo;   // the row block holding tile j (an empty share keeps any valid index)
      if (j >= rb_tile[lo + 1] && lo + 1 < total_rb) r = lo + 1;
      wg_rb[w] = r;
    }
  }
  // the attention kernel's record of each row block
  for (int r = threadIdx.x; r < total_rb; r += blockDim.x) {
    const int b = rb_seq[r];
    const int s0 = node_offsets[b];
    const int n = node_offsets[b + 1] - s0;
    const int node0 = (r - seq_rb_off[b]) * NB;
    const bool chain = is_chain[b] != 0;
    int32_t* m = rb_meta + (size_t)r * kMetaWords;
    m[kMetaTile0] = rb_tile[r];
    m[kMetaTileEnd] = rb_tile[r + 1];
    m[kMetaS0] = s0;
    m[kMetaN] = n;
    m[kMetaL] = prefix_len[b];
    m[kMetaNode0] = node0;
    m[kMetaTailN] = min(n, node0 + NB);
    m[kMetaFlags] = (chain ? 1 : 0) | ((chain || n <= kMaxTreeNodes) ? 2 : 0);
  }
}

// One block per sequence: validate parents, detect chains, and build depth,
// position and the 256-bit ancestor masks of non-chain trees.
__global__ __launch_bounds__(256) void prep_kernel(const int32_t* node_offsets,
                                                    const int32_t* prefix_len,
                                                    const int32_t* parent, uint8_t* chain_ws,
                                                    uint64_t* mask_ws, int32_t* depth_out,
                                                    int32_t* pos_out, uint64_t* mask_out,
                                                    uint8_t* chain_out, uint32_t* status) {
  __shared__ int par_s[kMaxTreeNodes];
  const int b = blockIdx.x;
  const int s0 = node_offsets[b];
  const int n = node_offsets[b + 1] - s0;
  const int L = prefix_len[b];
  int bad = 0, not_chain = 0;
  for (int v = threadIdx.x; v < n; v += blockDim.x) {
    int p = parent[s0 + v];
    if (v == 0 ? p != -1 : (p < 0 || p >= v)) bad = 1;
    if (v > 0 && p != v - 1) not_chain = 1;
  }
  bad = __syncthreads_or(bad);
  not_chain = __syncthreads_or(not_chain);
  if (bad) {
    if (threadIdx.x == 0) atomicOr(status, (uint32_t)TAV_DEV_BAD_PARENT);
    if (threadIdx.x == 0) chain_ws[b] = 0;
    return;
  }
  if (threadIdx.x == 0) {
    chain_ws[b] = not_chain ? 0 : 1;
    if (chain_out) chain_out[b] = not_chain ? 0 : 1;
  }
  if (!not_chain) {
    for (int v = threadIdx.x; v < n; v += blockDim.x) {
      if (depth_out) depth_out[s0 + v] = v;
      if (pos_out) pos_out[s0 + v] = L + v;
      if (mask_out) {
#pragma unroll
        for (int w = 0; w < kMaskWords; ++w) mask_out[(size_t)(s0 + v) * kMaskWords + w] = 0ull;
      }
    }
    return;
  }
  if (n > kMaxTreeNodes) {
    if (threadIdx.x == 0) atomicOr(status, (uint32_t)TAV_DEV_TREE_TOO_LARGE);
    return;
  }
  for (int v = threadIdx.x; v < n; v += blockDim.x) par_s[v] = parent[s0 + v];
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
      mask_ws[(size_t)(s0 + v) * kMaskWords + k] = w[k];
      if (mask_out) mask_out[(size_t)(s0 + v) * kMaskWords + k] = w[k];
    }
    if (depth_out) depth_out[s0 + v] = d;
    if (pos_out) pos_out[s0 + v] = L + d;
  }
}

}  // namespace

hipError_t launch_clear_status(uint32_t* status, hipStream_t s) {
  clear_status_kernel<<<1, 64, 0, s>>>(status);
  return hipGetLastError();
}

hipError_t launch_plan(const Plan& p, const int32_t* node_offsets, const int32_t* prefix_len,
                       const uint8_t* is_chain, int32_t* seq_rb_off, int32_t* rb_seq, int32_t* rb_tile,
                       int32_t* tail_blk, int32_t* wg_rb, int32_t* wg_tile, int32_t* rb_meta,
                       uint32_t* status, hipStream_t s) {
  plan_kernel<<<1, 1024, 0, s>>>(node_offsets, prefix_len, p.B, p.NB, p.bs, p.total_rb,
                                 p.tiles_per_head, p.tail_blocks, p.C, p.W, seq_rb_off, rb_seq,
                                 rb_tile, tail_blk, wg_rb, wg_tile, is_chain, rb_meta, status);
  return hipGetLastError();
}

hipError_t launch_prep(const Plan& p, const int32_t* node_offsets, const int32_t* prefix_len,
                       const int32_t* parent, uint8_t* chain_ws, uint64_t* mask_ws,
                       const tav_tree_out* out, uint32_t* status, hipStream_t s) {
  prep_kernel<<<p.B, 256, 0, s>>>(node_offsets, prefix_len, parent, chain_ws, mask_ws,
                                  out ? out->depth : nullptr, out ? out->position : nullptr,
                                  out ? out->mask : nullptr, out ? out->is_chain : nullptr, status);
  return hipGetLastError();
}

}  // namespace tav
