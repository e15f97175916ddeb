// Tree-masked attention over a paged prefix plus each node's ancestors.
//
// Every tree node attends to its sequence's cached prefix and to pi(v), the
// node itself and its ancestors (Progressive Tree Drafting, Section 3.1 "Tree
// Construction" and Section 3.2 "Candidate Verification"; RheoSampling scores
// its pruned draft tree in one target forward, Section 2.1; PreSTO's suffix
// requests share the cached prefix x_{0:c}, Section 3.2 and Appendix B.3
// Example 4).  Scores are scale * <q, k>, softmax over the visible keys.
//
// bf16 path (gfx950 MFMA).  A row block holds up to 256 query rows (nodes x
// the G query heads sharing a KV head), so every KV tile is read from HBM once
// and used by all rows.  Per KV head the 64-key tiles of all row blocks are
// concatenated and cut into equal ranges, one workgroup each (so every compute
// unit gets the same number of tiles); a workgroup walks its range across
// row-block boundaries, finishing a row block's output itself when it holds the
// whole block and leaving a partial (O, lse) for merge_kernel otherwise.
// Each of the 8 waves owns 32 rows and computes
//   S^T = K Q^T   (v_mfma_f32_32x32x16_bf16, keys x rows), online softmax per
//   row in registers (each lane holds one row's scores, so P^T feeds the next
//   MFMA directly), and O^T += V^T P^T.
// A tile is taken in two halves of 32 keys with one online-softmax update each,
// pipelined inside the wave: the scores of the second half run on the matrix
// cores while the first half's softmax runs on the vector ALU, and the first
// half's P V products run next to the second half's softmax.  Tiles reach LDS
// by global->LDS copies through a ring of four stages (three in flight while
// one is used, one barrier per tile).  The tree nodes' own keys and
// values are first packed into blocks of the cache layout (pack_tail_kernel), so
// tree-tail tiles take the same copy path as prefix tiles.  Block-table and
// plan entries are read through the scalar cache.  K tiles are row-major with
// an XOR swizzle, V tiles d-major in a layout whose operand reads are free of
// bank conflicts.  The softmax scale is folded into one FMA per score.
#include "tav_internal.h"
#include "attn_merge.h"

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
// a barrier, and compiler-only memory barriers around both.
// The source is a wave-uniform base (scalar registers) plus a per-lane byte offset, so a tile's
// copies need no per-lane address arithmetic: only the scalar base changes from tile to tile.
// lds_off: the wave's destination as an LDS address (wave-uniform).
__device__ inline void dma16(const void* gbase, uint32_t goff, uint32_t lds_off) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :: "v"(goff), "s"(gbase), "s"(__builtin_amdgcn_readfirstlane(lds_off)) : "memory", "m0");
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

constexpr int kStages = 5;            // ring stages in LDS (2 in use, 3 in flight)
constexpr float kSumLimit = 65536.f;  // keep a stale max while every probability stays <= 2^16

// Stored 16-byte position of chunk c of key row k in a K tile (bank spreading
// for the MFMA operand reads: rows are 256 B for D = 128 and 128 B for D = 64).
template <int D>
__device__ inline int kpos(int c, int key) {
  return D == 128 ? (c ^ (key & 15)) : (c ^ ((key >> 1) & 7));
}

typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;

// A kernel argument read again from the kernarg segment where it is used (one scalar load), for the
// arguments only row-block switches, segment ends and error paths need: the tile loop then keeps
// fewer scalar registers live (the rest no longer spill into vector-register lanes).
template <typename T>
__device__ __forceinline__ T cold_arg(size_t off) {
  const __attribute__((address_space(4))) char* kp =
      (const __attribute__((address_space(4))) char*)__builtin_amdgcn_kernarg_segment_ptr();
  return *(const volatile T __attribute__((address_space(4)))*)(kp + off);
}
#define TAV_COLD(field) cold_arg<decltype(AttnArgs::field)>(offsetof(AttnArgs, field))
typedef const __attribute__((address_space(4))) uint8_t* const_u8_ptr;

// Scalar-cache views of the work plan (wave-uniform reads).
struct PlanView {
  int total_rb;
};

// Where the tiles of one row block come from (wave-uniform).
struct TileCursor {
  int r;          // row block
  int seq;        // its sequence
  int t;          // tile within the row block
  int T;          // tiles of the row block
  int Tp;         // prefix tiles
  int L;          // prefix rows
  int tail_off;   // first packed node block of the sequence
  int tail_nblk;  // packed node blocks of the sequence
  int first_blk;  // block of prefix row 0 (a valid block for rows past the prefix)
  const_i32_ptr btab;
};

__device__ __forceinline__ void cursor_load(TileCursor& c, const PlanView& pv, int r) {
  const const_i32_ptr rb_seq = (const_i32_ptr)TAV_COLD(rb_seq);
  const const_i32_ptr rb_tile = (const_i32_ptr)TAV_COLD(rb_tile);
  const const_i32_ptr pref_len = (const_i32_ptr)TAV_COLD(prefix_len);
  const const_i32_ptr tail_blk = (const_i32_ptr)TAV_COLD(tail_blk);
  const int b = rb_seq[r];
  c.r = r;
  c.seq = b;
  c.T = rb_tile[r + 1] - rb_tile[r];
  c.L = pref_len[b];
  c.Tp = (c.L + kTileKeys - 1) / kTileKeys;
  c.tail_off = tail_blk[b];
  c.tail_nblk = tail_blk[b + 1] - c.tail_off;
  c.btab = (const_i32_ptr)(TAV_COLD(block_table) + (size_t)b * TAV_COLD(max_blocks));
  c.first_blk = c.L > 0 ? c.btab[0] : 0;
}

__device__ __forceinline__ void cursor_advance(TileCursor& c, const PlanView& pv) {
  if (++c.t == c.T) {
    c.t = 0;
    if (c.r + 1 < pv.total_rb) cursor_load(c, pv, c.r + 1);
  }
}

// Where the 16-key sub-block sb of the tile under cursor c lies: for a prefix tile the
// block-table entry (loaded now, checked when used, so the scalar load's latency overlaps the
// math) or a stand-in block for rows past the prefix; for a tree-node tile the packed block.
struct BlockRef {
  int blk, slot0, seq;
  bool tail;
};
__device__ __forceinline__ BlockRef cursor_block(const TileCursor& c, int sb, int lbs) {
  const int bs = 1 << lbs;
  BlockRef ref;
  ref.seq = c.seq;
  if (c.t < c.Tp) {
    const int r0 = c.t * kTileKeys + sb * 16;
    ref.blk = r0 < c.L ? c.btab[r0 >> lbs] : c.first_blk;
    ref.slot0 = r0 & (bs - 1);
    ref.tail = false;
  } else {
    const int j0 = (c.t - c.Tp) * kTileKeys + sb * 16;
    const int lb = j0 >> lbs;
    ref.blk = c.tail_off + (lb < c.tail_nblk ? lb : 0);
    ref.slot0 = j0 & (bs - 1);
    ref.tail = true;
  }
  return ref;
}

// x combined with its value in the other half of the wave (lane i ^ 32), by max
__device__ inline float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D, int LOG2G>
__global__ __launch_bounds__(512) void attn_bf16_kernel(AttnArgs a) {
  constexpr int G = 1 << LOG2G;
  constexpr int KS = D / 16;               // k-steps of S^T = K Q^T
  constexpr int DB = D / 32;               // 32-wide d blocks of O^T
  constexpr int CH = D / 8;                // 16-byte chunks per key row
  constexpr int NB = kRowsPerWG >> LOG2G;  // nodes per row block
  constexpr int TILE_BYTES = kTileKeys * D * 2;
  constexpr int SUB_BYTES = D * 32;                     // one 16-key sub-block of V^T
  constexpr int KEYS_PER_DMA = 1024 / (D * 2);          // key rows per 1 KB wave copy
  constexpr int DMA_PER_OPERAND = TILE_BYTES / 1024 / 8;  // per wave and tile, for K and for V
  constexpr int DMA_PER_TILE = 2 * DMA_PER_OPERAND;
  // LDS: per stage a K tile [64 keys][D] (16-byte chunk c of key k stored at kpos(c, k)) and
  // a V^T tile of 4 sub-blocks of 16 keys, each [32-d group][key half][32 d][8 keys].
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kStages][2 * TILE_BYTES];

  if (a.status[0] & TAV_DEV_PLAN_MISMATCH) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h32 = lane >> 5, l32 = lane & 31;
  // Workgroup L of the 1-D grid runs on XCD L % 8 (round-robin dispatch over the 8 XCDs); each XCD
  // is given a contiguous run of the head-major work list (logical id g * W + wg), so the row blocks
  // of one (sequence, KV head) -- which stream the same prefix tiles at the same time -- share one
  // XCD's L2 instead of reading the tiles once per XCD.
  int wg, g;
  {
    const int L = blockIdx.x, nwg = gridDim.x;
    const int vl = (nwg & 7) == 0 ? (L & 7) * (nwg >> 3) + (L >> 3) : L;
    g = vl / a.W;
    wg = vl - g * a.W;
  }
  const int j_begin = a.wg_tile[wg];
  const int j_end = a.wg_tile[wg + 1];
  if (j_begin >= j_end) return;
  const int Hq = a.Hq, Hkv = a.Hkv, bs = a.block_size;
  const int lbs = __builtin_ctz(bs);   // block sizes are powers of two
  const const_i32_ptr rb_tile = (const_i32_ptr)a.rb_tile;
  const uint16_t* kc = (const uint16_t*)a.k_cache;
  const uint16_t* vc = (const uint16_t*)a.v_cache;
  const uint16_t* ktl = (const uint16_t*)a.k_tail;
  const uint16_t* vtl = (const uint16_t*)a.v_tail;
  const PlanView pview{a.total_rb};
  const int sb = wave >> 1;   // 16-key sub-block of each tile this wave copies

  // ---- global -> LDS copies of tile j into ring slot (j - j_begin) % kStages.  Wave w copies
  // key rows 8w..8w+7 and d rows (w%2)*D/2 .. of V^T sub-block w/2.  Sources are resolved one
  // tile ahead of the issue, so the scalar loads overlap the math.
  const int r_first = a.wg_rb[wg];
  TileCursor cur;
  cursor_load(cur, pview, r_first);
  cur.t = j_begin - rb_tile[r_first];
  BlockRef nref;   // the next tile's sub-block (its block-table entry may still be loading)
  auto resolve = [&]() __attribute__((always_inline)) {   // the tile under cur, then advance
    nref = cursor_block(cur, sb, lbs);
    cursor_advance(cur, pview);
  };
  // this lane's byte offsets inside a block of the caches (the same for every tile): key rows
  // 8w..8w+7 of the tile (16-byte chunks permuted by kpos), value rows (w%2)*D/2 .. of sub-block w/2
  uint32_t k_off[DMA_PER_OPERAND], v_off[DMA_PER_OPERAND];
#pragma unroll
  for (int i = 0; i < DMA_PER_OPERAND; ++i) {
    const int kt = wave * 8 + i * KEYS_PER_DMA + lane / CH;   // key of the tile
    k_off[i] = (uint32_t)(((kt - sb * 16) * D + kpos<D>(lane % CH, kt) * 8) * 2);
    v_off[i] = (uint32_t)((((wave & 1) * (D / 2) + i * 32 + l32) * bs + h32 * 8) * 2);
  }
  // the ring's LDS address (taken once: per-tile destinations are then plain 32-bit sums) and the
  // slot the next copies go to (slot of tile j = (j - j_begin) % kStages, kept as a running count)
  const uint32_t lds_addr = (uint32_t)(size_t)(__attribute__((address_space(3))) uint8_t*)&lds[0][0];
  int issue_slot = 0;
  auto issue = [&]() __attribute__((always_inline)) {   // the next tile, next_issue
    // (wave-uniform: the block index and both bases stay in scalar registers)
    const bool bad = !nref.tail && (unsigned)nref.blk >= (unsigned)a.num_blocks;
    if (bad && lane == 0) {
      atomicOr(TAV_COLD(status), (uint32_t)TAV_DEV_BAD_BLOCK);
      atomicOr(TAV_COLD(seq_err) + nref.seq, (uint32_t)TAV_DEV_BAD_BLOCK);
    }
    const int blk = bad ? 0 : nref.blk;   // (the sequence's rows become sentinels after the kernel)
    const uint16_t* rk = (nref.tail ? ktl : kc) + (((size_t)blk * Hkv + g) * bs + nref.slot0) * D;
    const uint16_t* rv = (nref.tail ? vtl : vc) + ((size_t)blk * Hkv + g) * D * bs + nref.slot0;
    const uint32_t kbase = lds_addr + (uint32_t)issue_slot * (2 * TILE_BYTES);
    const uint32_t vbase = kbase + TILE_BYTES + sb * SUB_BYTES;
    issue_slot = issue_slot + 1 == kStages ? 0 : issue_slot + 1;
#pragma unroll
    for (int i = 0; i < DMA_PER_OPERAND; ++i) {
      dma16(rk, k_off[i], kbase + (wave * 8 + i * KEYS_PER_DMA) * (D * 2));
      dma16(rv, v_off[i], vbase + (((wave & 1) * (D / 2) + i * 32) >> 5) * 1024);
    }
  };

  // ---- the row block being computed (a segment of this workgroup's range)
  const int row = wave * 32 + l32;   // this lane's query row in the row block
  int seg_r = 0, seg_A = 0, seg_E = 0, seg_s0 = 0, seg_n = 0, seg_L = 0, seg_Tp = 0;
  int seg_node0 = 0, seg_tail_n = 0;
  bool seg_chain = false, seg_ok = true;
  int rnode = 0;
  bool rvalid = false;
  int rhead = 0;
  bf16x8_t qreg[KS];
  uint4 mwa = make_uint4(0u, 0u, 0u, 0u), mwb = mwa;   // this row's ancestor mask words (trees)
  // start_segment(r): row block r's record (one scalar load), this lane's row, and its query and
  // ancestor mask words in qreg / mwa, mwb.  The loads and the wait for them are one assembly
  // statement: a compiler-placed wait would sit at the registers' first use, after later copies
  // to LDS have been issued, and (the counts being in order) wait for those too.  The wait covers
  // every copy issued before it.  Rows past the block's nodes read node 0's query (finite values
  // whose outputs are dropped); rows without mask words read node 0's and clear them.
  auto start_segment = [&](int r) __attribute__((always_inline)) {
    const const_i32_ptr m = (const_i32_ptr)TAV_COLD(rb_meta) + (size_t)r * kMetaWords;
    const const_i32_ptr chain_w = (const_i32_ptr)TAV_COLD(is_chain);   // chain flags, 4 per word
    seg_r = r;
    seg_A = m[kMetaTile0];
    seg_E = m[kMetaTileEnd];
    seg_s0 = m[kMetaS0];
    seg_n = m[kMetaN];
    seg_L = m[kMetaL];
    seg_node0 = m[kMetaNode0];
    seg_tail_n = m[kMetaTailN];
    const int flags = m[kMetaFlags];
    const int sb_ = m[kMetaSeq];
    seg_chain = ((chain_w[sb_ >> 2] >> ((sb_ & 3) * 8)) & 0xff) != 0;
    seg_ok = seg_chain || (flags & 2) != 0;   // larger trees were rejected by preparation
    seg_Tp = (seg_L + kTileKeys - 1) / kTileKeys;
    rnode = seg_node0 + (row >> LOG2G);
    rvalid = (row >> LOG2G) < min(NB, seg_n - seg_node0);
    rhead = g * G + (row & (G - 1));
    const bool mask_rows = !seg_chain && seg_ok && rvalid;
    const int qnode = seg_s0 + (rvalid ? rnode : 0);
    const uint4* mp = (const uint4*)(TAV_COLD(mask) + (size_t)(mask_rows ? qnode : seg_s0) * kMaskWords);
    const uint16_t* qp = (const uint16_t*)TAV_COLD(q) + ((size_t)qnode * Hq + rhead) * D + h32 * 8;
    static_assert(KS == 4 || KS == 8, "query registers");
    if constexpr (KS == 8) {
      asm volatile(
          "global_load_dwordx4 %0, %10, off\n\t"
          "global_load_dwordx4 %1, %10, off offset:32\n\t"
          "global_load_dwordx4 %2, %10, off offset:64\n\t"
          "global_load_dwordx4 %3, %10, off offset:96\n\t"
          "global_load_dwordx4 %4, %10, off offset:128\n\t"
          "global_load_dwordx4 %5, %10, off offset:160\n\t"
          "global_load_dwordx4 %6, %10, off offset:192\n\t"
          "global_load_dwordx4 %7, %10, off offset:224\n\t"
          "global_load_dwordx4 %8, %11, off\n\t"
          "global_load_dwordx4 %9, %11, off offset:16\n\t"
          "s_waitcnt vmcnt(0)"
          : "=&v"(qreg[0]), "=&v"(qreg[1]), "=&v"(qreg[2]), "=&v"(qreg[3]), "=&v"(qreg[4]),
            "=&v"(qreg[5]), "=&v"(qreg[6]), "=&v"(qreg[7]), "=&v"(mwa), "=&v"(mwb)
          : "v"(qp), "v"(mp)
          : "memory");
    } else {
      asm volatile(
          "global_load_dwordx4 %0, %6, off\n\t"
          "global_load_dwordx4 %1, %6, off offset:32\n\t"
          "global_load_dwordx4 %2, %6, off offset:64\n\t"
          "global_load_dwordx4 %3, %6, off offset:96\n\t"
          "global_load_dwordx4 %4, %7, off\n\t"
          "global_load_dwordx4 %5, %7, off offset:16\n\t"
          "s_waitcnt vmcnt(0)"
          : "=&v"(qreg[0]), "=&v"(qreg[1]), "=&v"(qreg[2]), "=&v"(qreg[3]), "=&v"(mwa), "=&v"(mwb)
          : "v"(qp), "v"(mp)
          : "memory");
    }
    if (!mask_rows) mwa = mwb = make_uint4(0u, 0u, 0u, 0u);
  };

  const float c2 = a.scale * kLog2e;      // score -> log2 units
  float m_run = -INFINITY, l_run = 0.f;   // running max (log2 units) and sum of this lane's row
  f32x16_t acc[DB];
#pragma unroll
  for (int mb = 0; mb < DB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[mb][r] = 0.f;

  // raw scores S^T = K Q^T of key half kb (keys kb*32 .. kb*32+31 of the tile in ring slot
  // st); element r of this lane is key kb*32 + (r/8)*16 + h32*8 + r%8, query row `row`
  auto scores = [&](int st, int kb, f32x16_t& s) __attribute__((always_inline)) {
    const uint8_t* kbase = lds[st];
    const int key = kb * 32 + sigma(l32);
    const f32x16_t zero = {};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8_t ka = *(const bf16x8_t*)(kbase + key * (D * 2) + kpos<D>(ks * 2 + h32, key) * 16);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[ks], ks == 0 ? zero : s, 0, 0, 0);
    }
  };

  auto kread = [&](int st, int kb, int ks) __attribute__((always_inline)) -> bf16x8_t {
    const int key = kb * 32 + sigma(l32);
    return *(const bf16x8_t*)(lds[st] + key * (D * 2) + kpos<D>(ks * 2 + h32, key) * 16);
  };
  auto vread = [&](int st, int k2, int mb) __attribute__((always_inline)) -> bf16x8_t {
    return *(const bf16x8_t*)(lds[st] + TILE_BYTES + k2 * SUB_BYTES + mb * 1024 + h32 * 512 + l32 * 16);
  };

  auto rescale = [&](float alpha) __attribute__((always_inline)) {
#pragma unroll
    for (int mb = 0; mb < DB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][r] *= alpha;
  };

  // whether tile t of the current row block has keys some row must not see: the partial last
  // prefix tile, or a tree-node tile (except a chain's tiles wholly below every row)
  auto needs_mask = [&](int t) __attribute__((always_inline)) -> bool {
    if (t < seg_Tp - 1) return false;
    if (t == seg_Tp - 1) return (seg_L & (kTileKeys - 1)) != 0;
    const int j0 = (t - seg_Tp) * kTileKeys;
    return !(seg_chain && j0 + kTileKeys - 1 <= seg_node0 && j0 + kTileKeys - 1 < seg_tail_n);
  };

  // masking of the scores of half kb of tile t.  Element r is key kb*32 + (r/8)*16 + h32*8 +
  // r%8 of the tile: every test compares the compile-time part of that index with one
  // lane-adjusted bound.
  auto mask = [&](int t, int kb, f32x16_t& s) __attribute__((always_inline)) {
    if (t < seg_Tp) {
      const int x = seg_L - t * kTileKeys - h32 * 8;   // element visible iff its constant < x
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kc_ = kb * 32 + (r >> 3) * 16 + (r & 7);
        s[r] = kc_ < x ? s[r] : -INFINITY;
      }
    } else {
      const int j0 = (t - seg_Tp) * kTileKeys;  // first tree node of the tile
      const int wi = t - seg_Tp;
      // pick the word arithmetically (a select between the words could become a dynamically
      // indexed access)
      const uint64_t mw0 = (uint64_t)mwa.x | ((uint64_t)mwa.y << 32);
      const uint64_t mw1 = (uint64_t)mwa.z | ((uint64_t)mwa.w << 32);
      const uint64_t mw2 = (uint64_t)mwb.x | ((uint64_t)mwb.y << 32);
      const uint64_t mw3 = (uint64_t)mwb.z | ((uint64_t)mwb.w << 32);
      const uint64_t word = (mw0 & (0ull - (uint64_t)(wi == 0))) | (mw1 & (0ull - (uint64_t)(wi == 1))) |
                            (mw2 & (0ull - (uint64_t)(wi == 2))) | (mw3 & (0ull - (uint64_t)(wi >= 3)));
      const int xn = seg_tail_n - j0 - h32 * 8;          // node exists iff constant < xn
      const int xc = rnode - j0 - h32 * 8;               // chain: visible iff constant <= xc
      const uint64_t ml = word >> (h32 * 8);             // tree: bit `constant` of ml
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kc_ = kb * 32 + (r >> 3) * 16 + (r & 7);
        const bool vis = kc_ < xn && (seg_chain ? kc_ <= xc : ((ml >> kc_) & 1ull) != 0ull);
        s[r] = vis ? s[r] : -INFINITY;
      }
    }
  };

  // output of the finished segment: the whole row block -> out / lse; a cut one -> its slot
  struct OutRow { int A, E, s0, node; bool valid; };   // a finished segment's output row
  auto finish_segment = [&](const OutRow& o_) __attribute__((always_inline)) {
    const float l_tot = sum_halves(l_run);
    const float inv_l = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const float lse_nat = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    if (o_.A >= j_begin && o_.E <= j_end) {
      if (o_.valid) {
        uint16_t* op = (uint16_t*)TAV_COLD(out) + ((size_t)(o_.s0 + o_.node) * Hq + rhead) * D;
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
        float* lsep = TAV_COLD(lse);
        if (h32 == 0 && lsep) lsep[(size_t)(o_.s0 + o_.node) * Hq + rhead] = lse_nat;
      }
    } else {
      const int slot = o_.A < j_begin ? 2 * wg : 2 * wg + 1;
      const size_t prow = ((size_t)slot * Hkv + g) * kRowsPerWG + row;
      uint16_t* po = TAV_COLD(part_o) + prow * D;
#pragma unroll
      for (int mb = 0; mb < DB; ++mb) {
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          union { __bf16 e[4]; uint2 u; } o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o.e[e] = (__bf16)(acc[mb][rq * 4 + e] * inv_l);
          *(uint2*)(po + mb * 32 + rq * 8 + h32 * 4) = o.u;
        }
      }
      if (h32 == 0) TAV_COLD(part_lse)[prow] = lse_nat;
    }
    m_run = -INFINITY;
    l_run = 0.f;
#pragma unroll
    for (int mb = 0; mb < DB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][r] = 0.f;
  };

  // ---- prologue: the first kStages - 2 tiles in flight, the first segment
  const int n = j_end - j_begin;   // tiles of this workgroup
  int next_issue = j_begin;
  resolve();
  for (int k = 0; k < kStages - 2 && next_issue < j_end; ++k) {
    issue();
    ++next_issue;
    if (next_issue < j_end) resolve();
  }
  start_segment(r_first);
  int landed = next_issue - 1;   // tiles whose copies are known to have landed (this wave's)

  f32x16_t s0, s1;   // scores of the tile between its M and V phases (keys 0..31, 32..63)
  bf16x8_t pp[4];    // probabilities of the tile between its V phase and the next M phase,
                     // one MFMA operand per 16-key sub-block

  // M phase of tile k: P V of tile k-1 (then the segment's output if tile k-1 ended it), then
  // the scores S^T = K Q^T of tile k.  Only MFMAs and their operand reads from LDS: one stream
  // of operands (values of tile k-1, then keys of tile k) read PF ahead of the MFMAs (the order
  // is fixed by scheduling barriers).
  constexpr int PF = 3;
  constexpr int NPV = 4 * DB;   // P V MFMAs of a tile
  constexpr int NS = 2 * KS;    // score MFMAs of a tile (the two key halves interleaved)
  auto m_phase = [&](int k, int st_prev, int st_k) __attribute__((always_inline)) {
    if (k >= 1) {
      const int st = st_prev;
      bf16x8_t op[PF];
#pragma unroll
      for (int f = 0; f < PF; ++f) op[f] = vread(st, f / DB, f % DB);
#pragma unroll
      for (int i = 0; i < NPV; ++i) {
        acc[i % DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[i % PF], pp[i / DB], acc[i % DB], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (i + PF < NPV) op[i % PF] = vread(st, (i + PF) / DB, (i + PF) % DB);
        __builtin_amdgcn_sched_barrier(0);
      }
      const int j = j_begin + k - 1;
      if (j + 1 == min(seg_E, j_end)) {
        const OutRow orow{seg_A, seg_E, seg_s0, rnode, rvalid && seg_ok};
        if (j + 1 < j_end) {
          start_segment(seg_r + 1);
          landed = next_issue - 1;
        }
        finish_segment(orow);
      }
    }
    if (k < n) {
      const int st = st_k;
      bf16x8_t op[PF];
#pragma unroll
      for (int f = 0; f < PF; ++f) op[f] = kread(st, f & 1, f >> 1);
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const int ks = i >> 1;
        if (i & 1) s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[i % PF], qreg[ks], ks == 0 ? f32x16_t{} : s1, 0, 0, 0);
        else s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[i % PF], qreg[ks], ks == 0 ? f32x16_t{} : s0, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (i + PF < NS) op[i % PF] = kread(st, (i + PF) & 1, (i + PF) >> 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      s0 = f32x16_t{};
      s1 = f32x16_t{};
    }
  };

  // V phase of tile k: masking, one online-softmax update with all 64 keys, probabilities into
  // pp.  In the partial last prefix tile the first group also zeroes the values of keys past the
  // prefix (cache slots past it may hold anything, and 0 * NaN would reach the output); nobody
  // reads them before the next period.
  auto v_phase = [&](int k, int st_k) __attribute__((always_inline)) {
    const int t = j_begin + k - seg_A;
    const bool masked = needs_mask(t);
    if (masked && t < seg_Tp && tid < 256) {
      // 16-byte units of V^T are [sub-block][32-d group][key half][32 d] of 8 keys each
      const int lim = seg_L - t * kTileKeys;
      uint8_t* vbase = lds[st_k] + TILE_BYTES;
      for (int u = tid; u < 4 * (D / 32) * 2 * 32; u += 256) {
        const int k0 = (u / ((D / 32) * 64)) * 16 + ((u >> 5) & 1) * 8;   // first key of the unit
        if (k0 + 8 <= lim) continue;
        uint4* p = (uint4*)(vbase + u * 16);
        uint4 v = *p;
        const int x = lim - k0;   // keys k0 + e, e >= x, are zeroed
        v.x &= (0 < x ? 0xFFFFu : 0u) | (1 < x ? 0xFFFF0000u : 0u);
        v.y &= (2 < x ? 0xFFFFu : 0u) | (3 < x ? 0xFFFF0000u : 0u);
        v.z &= (4 < x ? 0xFFFFu : 0u) | (5 < x ? 0xFFFF0000u : 0u);
        v.w &= (6 < x ? 0xFFFFu : 0u) | (7 < x ? 0xFFFF0000u : 0u);
        *p = v;
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
    if (masked) {
      mask(t, 0, s0);
      mask(t, 1, s1);
    }
    // Exponentials against the running max (in log2 units), summed in float and packed to bf16
    // (a bf16 dot product would share the matrix cores with the other wave).  While every lane's sum
    // stays within 2^16 no probability exceeds 2^16 and the running max stands; otherwise (and
    // at a segment's first tile, whose running max is -inf) the row max is taken and the
    // exponentials are redone against it, with the accumulator rescaled.
    auto exps = [&](float mu) __attribute__((always_inline)) -> float {
      Bf16Pack8 q[4];   // built whole here, so the registers of the previous tile's pp are free
      float ps = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e0 = fast_exp2(fmaf(s0[r], c2, -mu)), e1 = fast_exp2(fmaf(s1[r], c2, -mu));
        ps += e0 + e1;
        q[r >> 3].e[r & 7] = (__bf16)e0;
        q[2 + (r >> 3)].e[r & 7] = (__bf16)e1;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) pp[i] = q[i].v;
      return ps;
    };
    float ps = exps(m_run == -INFINITY ? 0.f : m_run);
    if (__ballot(!(ps <= kSumLimit) || m_run == -INFINITY) != 0ull) {
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
      const float m_new = fmaxf(m_run, max_halves(mx) * c2);
      const float alpha = fast_exp2(m_run - (m_new == -INFINITY ? 0.f : m_new));
      m_run = m_new;
      ps = exps(m_new == -INFINITY ? 0.f : m_new);
      l_run *= alpha;
      rescale(alpha);
    }
    l_run += ps;
  };

  // Ping-pong: a wave takes the phases M(0) V(0) M(1) V(1) ... V(n-1) M(n); period m (between the
  // workgroup barriers that open tiles m and m+1) holds M(m) then V(m) for the first group of waves
  // and V(m-1) then M(m) for the second (4..7; wave w runs on SIMD w % 4), so on every SIMD one wave
  // feeds the matrix cores while the other does the softmax.  Tile m's keys are read in period m and
  // its values in period m + 1 (in the partial last prefix tile the first group zeroes the values
  // past the prefix in its V(m), in period m): before the barrier that opens period m every wave
  // waits for its copies of tile m, and after it issues tile m+3 into the slot of tile m-2, which
  // nobody reads any more.  One barrier per tile: the two groups' phases are not
  // otherwise synchronised (a second barrier between the phases kept them in step and cost 1-2 %).
  auto open_pair = [&](int m) __attribute__((always_inline)) {   // the barrier opening period m
    const int need = j_begin + m;
    asm volatile("" ::: "memory");
    if (need < j_end && need > landed) {
      // Past a segment start every copy issued before it has landed; later tiles wait by count
      // (the output stores of the finished segment, issued in between, are older than their
      // copies).
      const int after = next_issue - 1 - need;   // tiles issued after the one needed
      if (after >= 2) wait_vm<2 * DMA_PER_TILE>();
      else if (after == 1) wait_vm<DMA_PER_TILE>();
      else wait_vm<0>();
    }
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (next_issue < j_end) {
      issue();
      ++next_issue;
      if (next_issue < j_end) resolve();
    }
  };
  auto mid_pair = [&]() __attribute__((always_inline)) {   // between the phases: no LDS access moves across
    asm volatile("" ::: "memory");
  };
  // (each group as its own straight loop: the phases follow each other in a fixed order)
  // (st_m: ring slot of tile m, st_p: of tile m - 1, as running counts)
  if (wave < 4) {
    for (int m = 0, st_m = 0, st_p = kStages - 1; m <= n; ++m) {
      open_pair(m);
      __builtin_amdgcn_s_setprio(1);
      m_phase(m, st_p, st_m);
      __builtin_amdgcn_s_setprio(0);
      mid_pair();
      if (m < n) v_phase(m, st_m);
      st_p = st_m;
      st_m = st_m + 1 == kStages ? 0 : st_m + 1;
    }
  } else {
    for (int m = 0, st_m = 0, st_p = kStages - 1; m <= n; ++m) {
      open_pair(m);
      if (m >= 1) v_phase(m - 1, st_p);
      mid_pair();
      __builtin_amdgcn_s_setprio(1);
      m_phase(m, st_p, st_m);
      __builtin_amdgcn_s_setprio(0);
      st_p = st_m;
      st_m = st_m + 1 == kStages ? 0 : st_m + 1;
    }
  }
}

// Online-softmax merge of the split row blocks (attn_merge.h): nmerge workgroups laid out by
// merge_grid, then one workgroup per sequence for its sentinel rows.
template <typename OutT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(8))) void merge_kernel(AttnArgs a, int D, int log2G, int nmerge, int by_boundary) {
  const int i = blockIdx.x;
  if (i < nmerge) merge_block<OutT>(a, D, log2G, i, by_boundary != 0);
  else sentinel_rows<OutT>(a, D, i - nmerge);
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
        atomicOr(a.seq_err + b, (uint32_t)TAV_DEV_BAD_BLOCK);
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

// float32 path: the rows of a sequence whose tree or prefix has a device-detected error become
// sentinels (out = 0, lse = -inf); one block per sequence.
__global__ __launch_bounds__(256) void attn_sentinel_f32_kernel(AttnArgs a, int D) {
  sentinel_rows<float>(a, D, blockIdx.x);
}

template <int D>
hipError_t launch_bf16_d(const Plan& p, const AttnArgs& a, hipStream_t s) {
  const dim3 grid(p.W * p.Hkv);
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
  if (p.W == 0) return hipSuccess;
  return p.D == 128 ? launch_bf16_d<128>(p, a, s) : launch_bf16_d<64>(p, a, s);
}

hipError_t launch_attn_sentinel_f32(const Plan& p, const AttnArgs& a, hipStream_t s) {
  attn_sentinel_f32_kernel<<<p.B, 256, 0, s>>>(a, p.D);
  return hipGetLastError();
}

hipError_t launch_attn_f32(const Plan& p, const AttnArgs& a, hipStream_t s) {
  dim3 grid(p.N, p.Hq);
  if (p.D == 128) attn_f32_kernel<128><<<grid, 64, 0, s>>>(a);
  else attn_f32_kernel<64><<<grid, 64, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_merge(const Plan& p, const AttnArgs& a, bool bf16_out, hipStream_t s) {
  // (launched also when nothing was cut: it writes the sentinel rows of sequences with errors)
  const MergeGrid mg = merge_grid(p.total_rb, p.W);
  const int nmerge = mg.units * p.Hkv * (kRowsPerWG / kMergeRows);
  const int grid = nmerge + p.B;
  if (bf16_out) merge_kernel<__bf16><<<grid, 256, 0, s>>>(a, p.D, p.log2G, nmerge, mg.by_boundary ? 1 : 0);
  else merge_kernel<float><<<grid, 256, 0, s>>>(a, p.D, p.log2G, nmerge, mg.by_boundary ? 1 : 0);
  return hipGetLastError();
}

}  // namespace tav
