// Internal declarations shared by the host code and the gfx950 kernels of libtav.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "tav.h"

namespace tav {

constexpr int kTileKeys = 64;      // keys per attention tile (prefix or tree-tail)
constexpr int kRowsPerWG = 256;    // query rows (node x head-in-group) per attention workgroup
constexpr int kMaxTreeNodes = 256; // non-chain trees: ancestor sets are 256-bit masks
constexpr int kMaskWords = 4;
constexpr int kMaxChildren = 256;  // children of one node held by the verification kernels
constexpr int kMaxChunks = 2048;   // chunks of 64 sixteen-byte units per vocabulary row
                                   // (V <= 1 Mi bf16 / 512 Ki f32 tokens)
constexpr int kMaxDraftSupport = 128;  // tokens per sparse draft row
constexpr int kCounterWord = 16;   // status block: word 0 = status bits, word 16 = the workers' node counter
// Device-detected errors that make a sequence's attention rows sentinels (its tree or its prefix is
// unusable); any device-detected error of a sequence makes its verification outputs sentinels.
constexpr uint32_t kAttnErrBits = TAV_DEV_BAD_PARENT | TAV_DEV_TREE_TOO_LARGE | TAV_DEV_BAD_BLOCK;

// Work decomposition of the attention pass.  A "row block" is up to
// kRowsPerWG / G consecutive nodes of one sequence; it sees ceil(L / 64) prefix
// key tiles followed by the tiles of its sequence's tree nodes.  Per KV head,
// the key tiles of all row blocks are concatenated in row-block order
// (rb_tile[r] = first tile of row block r) and cut into W equal ranges of C
// tiles, one workgroup each; a workgroup crosses row-block boundaries, and a
// row block cut between workgroups is finished by the merge kernel.  The same
// integer formulas run on the host (grid sizes, workspace) and on the device
// (plan_kernel), so both agree.
struct Plan {
  int B = 0, N = 0, Hq = 0, Hkv = 0, D = 0, G = 0, log2G = 0, NB = 0;
  int bs = 16, lbs = 4;   // KV block size and its log2
  int total_rb = 0;       // row blocks over all sequences
  int tiles_per_head = 0; // key tiles per KV head over all row blocks
  int C = 0;              // key tiles per attention workgroup
  int W = 0;              // attention workgroups per KV head
  int tail_blocks = 0;    // packed blocks (block_size rows) of tree-node keys / values
  // workspace layout (byte offsets)
  size_t off_status = 0, off_chain = 0, off_mask = 0, off_seq_rb = 0, off_rb_seq = 0,
         off_rb_tile = 0, off_tail_blk = 0, off_wg_rb = 0, off_wg_tile = 0, off_rb_meta = 0, off_ktail = 0, off_vtail = 0, off_part_o = 0,
         off_part_lse = 0, off_stats = 0, off_term = 0, off_step = 0,
         off_presto = 0, off_order = 0, off_seq_err = 0, off_cw = 0, off_rec = 0, total = 0;
  int nch = 0;            // vocabulary chunks (64 sixteen-byte units) per row
};

__host__ __device__ static inline int ceil_div(int a, int b) { return (a + b - 1) / b; }
__host__ __device__ static inline int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Tiles of the key sequence seen by row block rb of a sequence with n nodes
// and L prefix rows: ceil(L / 64) prefix tiles, then the tree nodes 0 ..
// min(n, (rb+1) * NB) - 1 (every ancestor of a node has an id <= the node).
__host__ __device__ static inline int rb_tiles(int L, int n, int rb, int NB) {
  int tail = n < (rb + 1) * NB ? n : (rb + 1) * NB;
  return (L + kTileKeys - 1) / kTileKeys + (tail + kTileKeys - 1) / kTileKeys;
}

// What the attention kernel needs of a row block when it starts computing it, gathered by the
// plan into one record (scalar loads): its key tiles [tile0, tile_end) per KV head, the
// sequence's first node and node count, its prefix length, the block's first node, the bound on
// its nodes (min(n, node0 + nodes per block)), flags (2: the tree fits the ancestor masks) and
// the sequence index (whose chain flag the preparation writes).
// Work split of the attention kernel: every row block costs its key tiles plus kRbCost tiles'
// worth of fixed work (its partial prefix tile and masked tree tile, the output of the finished
// segment and the start of the next), and each workgroup takes an equal share Cv of that
// weighted length: tile t of row block r sits at t + kRbCost * r, and workgroup w holds the tiles
// whose position lies in [w Cv, (w+1) Cv).  The cost was measured per tile on MI355X.
constexpr int kRbCost = 4;

enum RbMeta { kMetaTile0 = 0, kMetaTileEnd, kMetaS0, kMetaN, kMetaL, kMetaNode0, kMetaTailN, kMetaFlags,
              kMetaSeq, kMetaWf, kMetaWl, kMetaWords };   // Wf / Wl: workgroups of the first / last tile

struct AttnArgs {
  const void* q;
  const void* k_node;
  const void* v_node;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  void* out;
  float* lse;
  const int32_t* node_offsets;
  const int32_t* prefix_len;
  const uint8_t* is_chain;
  const uint64_t* mask;
  const int32_t* seq_rb_off;  // [B+1] first row block of each sequence
  const int32_t* rb_seq;      // [total_rb] sequence of each row block
  const int32_t* rb_tile;     // [total_rb+1] first key tile (per KV head) of each row block
  const int32_t* tail_blk;    // [B+1] first packed node block of each sequence
  const int32_t* wg_rb;       // [W] row block holding the first key tile of each workgroup
  const int32_t* wg_tile;     // [W+1] first key tile of each workgroup (per KV head)
  const int32_t* rb_meta;     // [total_rb, kMetaWords] per row block, fields RbMeta
  void* k_tail;               // [tail_blocks, Hkv, bs, D] node keys in the cache layout
  void* v_tail;               // [tail_blocks, Hkv, D, bs] node values in the cache layout
  uint16_t* part_o;           // [2W, Hkv, 256, D] partial outputs of cut row blocks (bf16)
  float* part_lse;            // [2W, Hkv, 256]
  uint32_t* status;
  uint32_t* seq_err;          // [B] device-detected errors of each sequence (TAV_DEV_* bits)
  int B, Hq, Hkv, total_rb, tiles_per_head, C, W, tail_blocks, block_size, num_blocks, max_blocks;
  float scale;        // softmax scale (natural)
};

// What the vocabulary streaming kernel leaves for the pick kernel, per node.
struct NodeRec {
  double S;      // sum exp(l / T - M)
  double Z;      // sum (p - q~)+ over the row (dense draft rows with a sampled child)
  float M;       // max l / T (0 when no logit is finite); greedy rows: max l
  int A;         // greedy rows: the argmax (smallest id among equal maxima), else -1
  int b;         // the node's sequence
  uint32_t err;  // errors found while streaming (TAV_DEV_* bits)
  int flags;     // kRec* bits
  int s0, n;     // the sequence's first node and node count
  float T;       // the sequence's temperature
};
constexpr int kRecResidual = 1;   // the chunk weights are those of (p - q~)+
constexpr int kRecNoMass = 2;     // no finite logit
constexpr int kRecGreedy = 4;     // temperature 0: M and A are the row's max and argmax

// A node's verification step, taken by the pick for every node (it depends on the node's own values
// only); the walk follows the accepted children from the root.
struct StepRec {
  int next;       // the accepted child (sequence-local id), or -1: the path ends here
  int bonus;      // with next == -1: the token drawn at this node
  uint32_t err;   // TAV_DEV_* bits that count only if the walk reaches this node
  int pad;
};

struct VocabArgs {
  const void* logits;
  const float* temperature;
  const float* draft;          // [R, V] dense draft rows (K == 0)
  const int32_t* draft_idx;    // [R, K] sparse draft rows: support ids (ascending) ...
  const float* draft_val;      // [R, K] ... and q~ there
  int K;                       // sparse support size (0: dense rows)
  const int32_t* draft_row;
  const int32_t* node_offsets;
  const int32_t* parent;
  const int32_t* token;
  const uint8_t* sampled;
  const float* uniforms;
  float* stats;          // [N, 3]
  int32_t* term_token;   // [N]
  StepRec* step;         // [N] each node's verification step, for the walk
  uint8_t* node_status;  // [N] output; the pick writes 2 for every child its step rejects, else 0 (the walk
                         // keeps the 2 only where the parent lies on the accepted path)
  uint32_t* status;
  uint32_t* seq_err;     // [B] device-detected errors of each sequence
  int32_t* queue;        // node counter of the workers' queue (cleared with the status word)
  const int32_t* order;  // [N] the nodes in the order the workers take them (nodes with a draft row first)
  float* cw;             // [N, nch] chunk weights under p or (p - q~)+, from the streaming kernel
  NodeRec* rec;          // [N] from the streaming kernel
  int B, N, V, R, nch;
};

struct WalkArgs {
  const int32_t* node_offsets;
  const int32_t* parent;
  const StepRec* step;         // [N] each node's step, from the pick
  uint8_t* node_status;        // [N] the pick's rejection marks in, the walk's statuses out
  int32_t* path;
  int32_t* path_len;
  int32_t* bonus;
  uint32_t* status;
  const uint32_t* seq_err;     // [B] errors found by the earlier kernels of the call
  int B, max_path;
};

struct PrestoArgs {
  int T, R, M, max_transitions;
  double alpha;
  const float* root_lp0;
  const float* root_lq;
  const int32_t* cut;
  const int32_t* suffix_off;
  const float* lp0;
  const float* lq;
  const int32_t* pf_parent;
  const uint8_t* pf_is_accept;
  const int32_t* pf_request;
  const float* u;
  float* log_accept;
  double* log_accept64;
  int32_t* pf_path;
  int32_t* pf_path_len;
  uint32_t* status;
};

struct ScoreArgs {
  const void* logits;      // [N, V]
  const int32_t* token;    // [N] or null
  float tau;               // proposal temperature
  int kpow;                // 1 / tau when it is a whole number in 1..8, else 0
  float* lp0;              // [N] outputs (each may be null)
  float* lq;
  float* ent;
  int32_t* argmax;
  uint32_t* status;
  int N, V;
};

constexpr int kMaxDraftDepth = 32;           // draft-tree depths
constexpr int kMaxDraftCandidates = 2048;    // candidates of one draft tree (the root included)

// Draft-tree construction state (workspace) and sizes.  Candidate ids: the root 0, then per depth
// d the parents in rank order, each parent's slots in pool order: depth d holds ids
// [base[d], base[d + 1]), kcount[d] parents x slots of them.
struct DraftArgs {
  int B, V, S, K, Kd, C, slots, m, hybrid, R, D;
  float temperature, eps;
  int base[kMaxDraftDepth + 2];
  int kcount[kMaxDraftDepth + 2];
  int32_t* cand_parent;     // [B, C]
  int32_t* cand_token;      // [B, C]
  double* cand_score;       // [B, C]
  uint8_t* cand_sampled;    // [B, C]
  uint8_t* cand_depth;      // [B, C]
  int32_t* row_idx;         // [B, C, S] a hybrid parent's draft row: support ids ascending ...
  float* row_val;           // [B, C, S] ... and q~ there
  int32_t* frontier;        // [B, K] the parents of the next depth
  uint32_t* status;
  uint32_t* seq_err;        // [B]
};

struct DraftOut {
  int32_t* parent;          // [B, R + 1]
  int32_t* token;
  uint8_t* sampled;
  int32_t* cand_id;         // optional
  int32_t* draft_row;       // [B, R + 1]
  int32_t* draft_idx;       // [B * (R + 1), S]
  float* draft_val;
};

// The error message of the calling thread (tav_last_error) and the status to return, for host
// code outside tav_host.hip.
tav_status tav_host_fail(tav_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
tav_status tav_host_ok();

// Kernel launchers (defined next to their kernels).  They return the HIP error
// of the launch.
// Start of every call: status word, counters and the per-sequence error words seq_err[B] cleared;
// with draft_row (verification), the order in which the vocabulary workers take the nodes is built
// into order[N].
hipError_t launch_start(uint32_t* status, uint32_t* seq_err, int B, const int32_t* draft_row, int R, int N,
                        int32_t* order, hipStream_t s);
hipError_t launch_prep(const Plan& p, const int32_t* node_offsets, const int32_t* prefix_len,
                       const int32_t* parent, uint8_t* chain_ws, uint64_t* mask_ws,
                       const tav_tree_out* out, uint32_t* status, uint32_t* seq_err, hipStream_t s);
// bf16 attention: preparation, work plan and node packing in one launch.
// The verification workers' node order (built by the start kernel, or by one extra block of the
// prelude when the same call runs both): order null = none.
struct OrderArgs {
  const int32_t* draft_row;
  int R, N;
  int32_t* order;
};
hipError_t launch_prelude(const Plan& p, const int32_t* parent, const tav_tree_out* out, const AttnArgs& a,
                          const OrderArgs& o, bool fused_start, hipStream_t s);
// The float32 pass's preparation with the call's start folded in (status word, workers' counter, each
// sequence's error word; the workers' node order when o.order is set).
hipError_t launch_prep_start(const Plan& p, const int32_t* node_offsets, const int32_t* prefix_len,
                             const int32_t* parent, uint8_t* chain_ws, uint64_t* mask_ws, const tav_tree_out* out,
                             uint32_t* status, uint32_t* seq_err, const OrderArgs& o, hipStream_t s);
hipError_t launch_attn_bf16(const Plan& p, const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_f32(const Plan& p, const AttnArgs& a, hipStream_t s);
// Merge of the cut row blocks; also writes the sentinel rows (out = 0, lse = -inf) of every
// sequence whose tree or prefix has a device-detected error.
hipError_t launch_merge(const Plan& p, const AttnArgs& a, bool bf16_out, hipStream_t s);
// The same sentinel rows for the float32 path (one block per sequence).
hipError_t launch_attn_sentinel_f32(const Plan& p, const AttnArgs& a, hipStream_t s);
// Vocabulary workers: one 512-thread workgroup per compute unit, persistent over the node queue.
hipError_t launch_vocab(const VocabArgs& a, bool bf16_logits, int num_cus, hipStream_t s);
// The walk: one 256-thread workgroup per sequence; with attn != nullptr the same launch also runs, in
// further workgroups, the merge of the cut bf16 attention row blocks (launch_merge's work) or, with
// f32_sentinels, the float32 path's sentinel rows (launch_attn_sentinel_f32's work).
hipError_t launch_walk(const WalkArgs& a, const Plan* plan, const AttnArgs* attn, bool f32_sentinels,
                       hipStream_t s);
// Draft-tree construction: depth d's pools (one workgroup per (sequence, parent)) and the next
// parents (one workgroup per sequence); the global prune.
hipError_t launch_draft_expand(const DraftArgs& a, int d, const uint16_t* logits, const float* uniforms,
                               int32_t* frontier_out, hipStream_t s);
hipError_t launch_draft_prune(const DraftArgs& a, const DraftOut& o, hipStream_t s);
// Per-token scores: one 512-thread workgroup per row, persistent over the rows.
hipError_t launch_score(const ScoreArgs& a, bool bf16, int num_cus, hipStream_t s);
hipError_t launch_presto(const PrestoArgs& a, hipStream_t s);

}  // namespace tav
