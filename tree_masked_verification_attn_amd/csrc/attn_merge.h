// Online-softmax merge of the pieces of attention row blocks cut between workgroups (merge_kernel),
// and the sentinel rows of sequences whose tree or prefix has a device-detected error.
#pragma once

#include "tav_internal.h"

namespace tav {

// out = sum_s exp(lse_s - LSE) O_s over the pieces of row block r, KV head g, rows [row0, row0 +
// nrows); the pieces O_s are normalised by their own sums and stored in bf16, lse_s in float.  Row block r's key tiles [A, E) were cut into the pieces of workgroups A/C .. (E-1)/C;
// the first piece sits in slot 2w+1 of its workgroup (its last segment), the others in slot 2w
// (their workgroup's first segment).  A thread owns 4 outputs at a time.
template <typename OutT>
__device__ inline void merge_rows(const AttnArgs& a, int D, int log2G, int r, int g, int row0, int nrows) {
  // the row block's record from the plan (one round of loads beside the status words)
  const int32_t* m = a.rb_meta + (size_t)r * kMetaWords;
  const int b = m[kMetaSeq], s0 = m[kMetaS0], n = m[kMetaN], node0 = m[kMetaNode0];
  const int wf = m[kMetaWf], wl = m[kMetaWl];
  if (a.status[0] & TAV_DEV_PLAN_MISMATCH) return;
  if (b < 0 || b >= a.B) return;
  const int NB = kRowsPerWG >> log2G;
  const int G = 1 << log2G;
  const int nodes_here = min(NB, n - node0);
  if (a.seq_err[b] & kAttnErrBits) {
    // the sequence's tree or prefix is unusable: its rows become sentinels (out = 0, lse = -inf)
    for (int task = threadIdx.x; task < nrows * D; task += blockDim.x) {
      const int row = row0 + task / D, d = task % D;
      if ((row >> log2G) >= nodes_here) continue;
      const size_t orow = (size_t)(s0 + node0 + (row >> log2G)) * a.Hq + g * G + (row & (G - 1));
      ((OutT*)a.out)[orow * D + d] = (OutT)0.f;
      if (d == 0 && a.lse) a.lse[orow] = -INFINITY;
    }
    return;
  }
  if (wf == wl) return;  // one workgroup held the whole row block
  const int DQ = D / 4;
  constexpr int kPre = 4;   // pieces whose loads are all issued before any is used
  const int np = wl - wf + 1;
  for (int task = threadIdx.x; task < nrows * DQ; task += blockDim.x) {
    const int row = row0 + task / DQ, dq = task % DQ;
    if ((row >> log2G) >= nodes_here) continue;
    const int node = s0 + node0 + (row >> log2G);
    const int head = g * G + (row & (G - 1));
    float M = -INFINITY;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float den = 0.f;
    auto add_piece = [&](float ls, uint2 ob) {
      if (ls == -INFINITY) return;
      const float wgt = __expf(ls - M);
      den += wgt;
      acc.x += wgt * __uint_as_float(ob.x << 16);
      acc.y += wgt * __uint_as_float(ob.x & 0xFFFF0000u);
      acc.z += wgt * __uint_as_float(ob.y << 16);
      acc.w += wgt * __uint_as_float(ob.y & 0xFFFF0000u);
    };
    auto base_of = [&](int w) {
      const int slot = w == wf ? 2 * w + 1 : 2 * w;
      return ((size_t)slot * a.Hkv + g) * kRowsPerWG + row;
    };
    if (np <= kPre) {
      float ls[kPre];
      uint2 ob[kPre];
#pragma unroll
      for (int i = 0; i < kPre; ++i) {
        ls[i] = -INFINITY;
        ob[i] = make_uint2(0u, 0u);
        if (i < np) {
          const size_t base = base_of(wf + i);
          ls[i] = a.part_lse[base];
          ob[i] = *(const uint2*)(a.part_o + base * D + dq * 4);   // 4 bf16
        }
      }
#pragma unroll
      for (int i = 0; i < kPre; ++i) M = fmaxf(M, ls[i]);
#pragma unroll
      for (int i = 0; i < kPre; ++i) add_piece(ls[i], ob[i]);
    } else {
      for (int w = wf; w <= wl; ++w) M = fmaxf(M, a.part_lse[base_of(w)]);
      for (int w = wf; w <= wl; ++w) {
        const size_t base = base_of(w);
        add_piece(a.part_lse[base], *(const uint2*)(a.part_o + base * D + dq * 4));
      }
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

}  // namespace tav
