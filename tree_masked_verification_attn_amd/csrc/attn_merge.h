// Online-softmax merge of the pieces of attention row blocks cut between workgroups (merge_kernel),
// and the sentinel rows of sequences whose tree or prefix has a device-detected error (both paths).
#pragma once

#ifndef TAV_MERGE_ROWS
#define TAV_MERGE_ROWS 16
#endif

#include "tav_internal.h"

namespace tav {

constexpr int kMergeRows = TAV_MERGE_ROWS;   // rows of one merge workgroup (256 threads)

// out = sum_s exp(lse_s - LSE) O_s over the pieces of row block r, KV head g, rows [row0, row0 +
// nrows); the pieces O_s are normalised by their own sums and stored in bf16, lse_s in float.  Row
// block r's key tiles [A, E) were cut into the pieces of workgroups A/C .. (E-1)/C; the first piece
// sits in slot 2w+1 of its workgroup (its last segment), the others in slot 2w (their workgroup's
// first segment).  A thread owns 8 outputs at a time (16-byte loads and stores).
template <typename OutT>
__device__ inline void merge_rows(const AttnArgs& a, int D, int log2G, int r, int g, int row0, int nrows) {
  // the row block's record from the plan (one round of loads beside the status word)
  const int32_t* m = a.rb_meta + (size_t)r * kMetaWords;
  const int b = m[kMetaSeq], s0 = m[kMetaS0], n = m[kMetaN], node0 = m[kMetaNode0];
  const int wf = m[kMetaWf], wl = m[kMetaWl];
  if (a.status[0] & TAV_DEV_PLAN_MISMATCH) return;
  if (b < 0 || b >= a.B) return;
  const int NB = kRowsPerWG >> log2G;
  const int G = 1 << log2G;
  const int nodes_here = min(NB, n - node0);
  const int DQ = D / 8;
  const int ntask = nrows * DQ;   // a task: eight outputs of one row
  const bool cut = wf != wl;
  constexpr int kT = kMergeRows / 16;   // tasks per thread taken with their loads in flight together
                                        // (kMergeRows rows x D / 8 at D <= 128 on 256 threads); further
                                        // tasks go one by one
  constexpr int kPre = 4;    // pieces loaded together (a batch), folded in by an online softmax
  auto task_row = [&](int task) { return row0 + task / DQ; };
  auto task_ok = [&](int task) { return task < ntask && (task_row(task) >> log2G) < nodes_here; };
  auto base_of = [&](int w, int row) {
    const int slot = w == wf ? 2 * w + 1 : 2 * w;
    return ((size_t)slot * a.Hkv + g) * kRowsPerWG + row;
  };
  auto load_batch = [&](int task, int w0, float (&ls)[kPre], uint4 (&ob)[kPre]) {
    const int row = task_row(task), dq = task % DQ;
#pragma unroll
    for (int q = 0; q < kPre; ++q) {
      ls[q] = -INFINITY;
      ob[q] = make_uint4(0u, 0u, 0u, 0u);
      if (w0 + q <= wl) {
        const size_t base = base_of(w0 + q, row);
        ls[q] = a.part_lse[base];
        ob[q] = *(const uint4*)(a.part_o + base * D + dq * 8);   // 8 bf16
      }
    }
  };
  // second round: the first batch of this thread's first kT tasks, issued with the sequence's error
  // word (the pieces' slots are valid whatever the sequence's state; they are used only without errors)
  float ls0[kT][kPre];
  uint4 ob0[kT][kPre];
#pragma unroll
  for (int i = 0; i < kT; ++i) {
    const int task = threadIdx.x + i * blockDim.x;
    if (cut && task_ok(task)) {
      load_batch(task, wf, ls0[i], ob0[i]);
    } else {
#pragma unroll
      for (int q = 0; q < kPre; ++q) {
        ls0[i][q] = -INFINITY;
        ob0[i][q] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  }
  // (a sequence whose tree or prefix is unusable gets sentinel rows from sentinel_rows instead)
  if (a.seq_err[b] & kAttnErrBits) return;
  if (!cut) return;  // one workgroup held the whole row block
  // out = sum_s exp(lse_s - LSE) O_s / sum_s exp(lse_s - LSE), LSE the running maximum of the lse_s
  struct Acc {
    float M = -INFINITY, den = 0.f;
    float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  };
  auto fold = [](Acc& c, const float (&ls)[kPre], const uint4 (&ob)[kPre]) {
    float mb = c.M;
#pragma unroll
    for (int q = 0; q < kPre; ++q) mb = fmaxf(mb, ls[q]);
    if (mb > c.M) {
      const float sc = c.M == -INFINITY ? 0.f : __expf(c.M - mb);
      c.den *= sc;
#pragma unroll
      for (int e = 0; e < 8; ++e) c.o[e] *= sc;
      c.M = mb;
    }
#pragma unroll
    for (int q = 0; q < kPre; ++q) {
      if (ls[q] == -INFINITY) continue;
      const float wgt = __expf(ls[q] - c.M);
      c.den += wgt;
      const uint32_t w4[4] = {ob[q].x, ob[q].y, ob[q].z, ob[q].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        c.o[2 * e] += wgt * __uint_as_float(w4[e] << 16);
        c.o[2 * e + 1] += wgt * __uint_as_float(w4[e] & 0xFFFF0000u);
      }
    }
  };
  auto finish = [&](int task, const Acc& c) {
    const int row = task_row(task), dq = task % DQ;
    const int node = s0 + node0 + (row >> log2G);
    const int head = g * G + (row & (G - 1));
    const float inv = c.den > 0.f ? 1.f / c.den : 0.f;
    OutT* op = (OutT*)a.out + ((size_t)node * a.Hq + head) * D + dq * 8;
    if constexpr (sizeof(OutT) == 2) {
      union { OutT e[8]; uint4 u; } w;
#pragma unroll
      for (int e = 0; e < 8; ++e) w.e[e] = (OutT)(c.o[e] * inv);
      *(uint4*)op = w.u;
    } else {
      float4* o4 = (float4*)op;
      o4[0] = make_float4(c.o[0] * inv, c.o[1] * inv, c.o[2] * inv, c.o[3] * inv);
      o4[1] = make_float4(c.o[4] * inv, c.o[5] * inv, c.o[6] * inv, c.o[7] * inv);
    }
    if (dq == 0 && a.lse) a.lse[(size_t)node * a.Hq + head] = c.den > 0.f ? c.M + __logf(c.den) : -INFINITY;
  };
  auto rest = [&](int task, Acc& c) {   // the batches after the first
    for (int w0 = wf + kPre; w0 <= wl; w0 += kPre) {
      float ls[kPre];
      uint4 ob[kPre];
      load_batch(task, w0, ls, ob);
      fold(c, ls, ob);
    }
  };
#pragma unroll
  for (int i = 0; i < kT; ++i) {
    const int task = threadIdx.x + i * blockDim.x;
    if (!task_ok(task)) continue;
    Acc c;
    fold(c, ls0[i], ob0[i]);
    rest(task, c);
    finish(task, c);
  }
  for (int task = threadIdx.x + kT * blockDim.x; task < ntask; task += blockDim.x) {
    if (!task_ok(task)) continue;
    float ls[kPre];
    uint4 ob[kPre];
    load_batch(task, wf, ls, ob);
    Acc c;
    fold(c, ls, ob);
    rest(task, c);
    finish(task, c);
  }
}

// The sentinel rows of sequence b (out = 0, lse = -inf) when its tree or prefix has a device-detected
// error (every sequence when the call's plan disagreed with the host's).
template <typename OutT>
__device__ inline void sentinel_rows(const AttnArgs& a, int D, int b) {
  const bool all = (a.status[0] & TAV_DEV_PLAN_MISMATCH) != 0;
  if (!all && !(a.seq_err[b] & kAttnErrBits)) return;
  const int s0 = a.node_offsets[b], e0 = a.node_offsets[b + 1];
  const size_t row_elems = (size_t)a.Hq * D;
  OutT* out = (OutT*)a.out;
  for (size_t i = threadIdx.x; i < (size_t)(e0 - s0) * row_elems; i += blockDim.x)
    out[(size_t)s0 * row_elems + i] = (OutT)0.f;
  if (a.lse)
    for (int i = threadIdx.x; i < (e0 - s0) * a.Hq; i += blockDim.x) a.lse[(size_t)s0 * a.Hq + i] = -INFINITY;
}

// Merge workgroups: one per (unit, KV head, kMergeRows rows).  A unit is a row block when the launch covers
// every row block (few row blocks), else a boundary between consecutive workgroup shares (many row
// blocks: only a row block holding a share boundary strictly inside it was cut, and the first such
// boundary names it), so the launch's size does not grow with the number of row blocks.
struct MergeGrid {
  int units;          // row blocks or share boundaries
  bool by_boundary;
};
__host__ __device__ inline MergeGrid merge_grid(int total_rb, int W) {
  return total_rb > W - 1 ? MergeGrid{W - 1, true} : MergeGrid{total_rb, false};
}
// The row block that unit u merges, or -1.
__device__ inline int merge_unit_rb(const AttnArgs& a, int u, bool by_boundary) {
  if (!by_boundary) return u;
  const int w = u + 1;   // the boundary where workgroup w's share starts
  const int r = a.wg_rb[w];
  const int t = a.wg_tile[w];
  if (r < 0 || r >= a.total_rb || !(t > a.rb_tile[r] && t < a.rb_tile[r + 1])) return -1;
  return a.wg_tile[w - 1] > a.rb_tile[r] ? -1 : r;   // an earlier boundary inside r names it
}
// Merge workgroup i of a launch laid out by merge_grid (rows of 16 per (unit, KV head)).
template <typename OutT>
__device__ inline void merge_block(const AttnArgs& a, int D, int log2G, int i, bool by_boundary) {
  constexpr int kZ = kRowsPerWG / kMergeRows;
  if (a.status[0] & TAV_DEV_PLAN_MISMATCH) return;   // (the plan's arrays are not to be trusted)
  const int r = merge_unit_rb(a, i / (kZ * a.Hkv), by_boundary);
  if (r < 0) return;
  merge_rows<OutT>(a, D, log2G, r, (i / kZ) % a.Hkv, (i % kZ) * kMergeRows, kMergeRows);
}

}  // namespace tav
