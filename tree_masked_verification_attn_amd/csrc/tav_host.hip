// Host side of libtav: argument validation, the work plan, the workspace
// layout, kernel launches and error reporting.  Nothing here allocates device
// memory; every call only enqueues work on the caller's stream(s).
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>

#include <utility>
#include <vector>

#include <mutex>

#include "tav_internal.h"

// Workspace of tav_tree_attn_verify_noalloc: one device array per GPU the library runs on, held
// until the process ends.  Host code never passes this name to a kernel or a copy (on the host it
// is a stand-in, not a device address); it uses the address hipGetSymbolAddress returns for the
// current device (scratch_address below).
static __device__ __align__(256) uint8_t scratch[TAV_NOALLOC_SCRATCH_BYTES];

namespace tav {
namespace {

thread_local std::string g_last_error;

tav_status vfail(tav_status s, const char* fmt, va_list ap) {
  char buf[512];
  vsnprintf(buf, sizeof buf, fmt, ap);
  g_last_error = buf;
  return s;
}

tav_status fail(tav_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
tav_status fail(tav_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vfail(s, fmt, ap);
  va_end(ap);
  return s;
}

tav_status ok() {
  g_last_error.clear();
  return TAV_OK;
}

#define TAV_HIP(call)                                                                   \
  do {                                                                                  \
    hipError_t e_ = (call);                                                             \
    if (e_ != hipSuccess) return fail(TAV_ERR_HIP, "%s: %s", #call, hipGetErrorString(e_)); \
  } while (0)

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

constexpr int kMaxDevices = 64;
constexpr int kTargetWorkgroups = 256;  // one round of one workgroup per MI355X compute unit
constexpr int kMinTilesPerWG = 8;       // at least 512 keys per attention workgroup (more than kRbCost)

int log2_exact(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return (1 << l) == x ? l : -1;
}

tav_status check_problem(const tav_problem* p) {
  if (!p) return fail(TAV_ERR_NULL_POINTER, "problem is NULL");
  if (p->num_seqs < 1) return fail(TAV_ERR_BAD_SHAPE, "num_seqs must be >= 1 (got %d)", p->num_seqs);
  if (!p->node_offsets_host || !p->node_offsets || !p->prefix_len_host || !p->prefix_len)
    return fail(TAV_ERR_NULL_POINTER, "node_offsets / prefix_len (host and device copies) are required");
  const int32_t* off = p->node_offsets_host;
  if (off[0] != 0) return fail(TAV_ERR_BAD_SHAPE, "node_offsets[0] must be 0");
  for (int b = 0; b < p->num_seqs; ++b)
    if (off[b + 1] <= off[b])
      return fail(TAV_ERR_BAD_SHAPE, "sequence %d has no nodes (node_offsets must increase)", b);
  if (p->num_q_heads < 1 || p->num_kv_heads < 1 || p->num_q_heads % p->num_kv_heads)
    return fail(TAV_ERR_BAD_SHAPE, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                p->num_q_heads, p->num_kv_heads);
  const int G = p->num_q_heads / p->num_kv_heads;
  if (log2_exact(G) < 0 || G > 16)
    return fail(TAV_ERR_UNSUPPORTED, "query heads per KV head must be 1, 2, 4, 8 or 16 (got %d)", G);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(TAV_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", p->head_dim);
  if (p->dtype != TAV_F32 && p->dtype != TAV_BF16)
    return fail(TAV_ERR_UNSUPPORTED, "dtype must be TAV_F32 or TAV_BF16 (got %d)", p->dtype);
  if (!(p->sm_scale >= 0.f) || !isfinite(p->sm_scale))
    return fail(TAV_ERR_INVALID_ARGUMENT, "sm_scale must be finite and >= 0");
  if (p->block_size != 8 && p->block_size != 16 && p->block_size != 32 && p->block_size != 64)
    return fail(TAV_ERR_UNSUPPORTED, "block_size must be 8, 16, 32 or 64 (got %d)", p->block_size);
  if (p->dtype == TAV_BF16 && p->block_size < 16)
    return fail(TAV_ERR_UNSUPPORTED, "bf16 attention needs block_size 16, 32 or 64 (got %d)", p->block_size);
  if (p->max_blocks_per_seq < 1 || p->num_blocks < 0)
    return fail(TAV_ERR_BAD_SHAPE, "max_blocks_per_seq must be >= 1 and num_blocks >= 0");
  for (int b = 0; b < p->num_seqs; ++b) {
    const int L = p->prefix_len_host[b];
    if (L < 0 || (int64_t)L > (int64_t)p->max_blocks_per_seq * p->block_size)
      return fail(TAV_ERR_BAD_SHAPE, "prefix_len[%d] = %d outside [0, max_blocks_per_seq * block_size]", b, L);
  }
  if (p->vocab < 0) return fail(TAV_ERR_BAD_SHAPE, "vocab must be >= 0");
  return TAV_OK;
}

tav_status check_presto(const tav_presto_io* io) {
  if (!io->root_lp0 || !io->root_lq || !io->cut || !io->suffix_off || !io->lp0 || !io->lq ||
      !io->pf_parent || !io->pf_is_accept || !io->pf_request || !io->u || !io->log_accept ||
      !io->pf_path || !io->pf_path_len)
    return fail(TAV_ERR_NULL_POINTER, "a PreSTO array is NULL");
  if (io->T < 1 || io->num_requests < 1 || io->num_nodes < 1 || io->max_transitions < 0)
    return fail(TAV_ERR_BAD_SHAPE, "PreSTO sizes: T=%d requests=%d nodes=%d max_transitions=%d", io->T,
                io->num_requests, io->num_nodes, io->max_transitions);
  if (!isfinite(io->alpha)) return fail(TAV_ERR_INVALID_ARGUMENT, "alpha must be finite");
  return TAV_OK;
}

// The plan and workspace layout; identical integer formulas run in plan_kernel.  attn_wgs is the
// number of attention workgroups aimed at over all KV heads.
tav_status make_plan(const tav_problem* p, const tav_presto_io* pr, Plan* out,
                     int attn_wgs = kTargetWorkgroups) {
  tav_status st = check_problem(p);
  if (st != TAV_OK) return st;
  if (pr) {
    st = check_presto(pr);
    if (st != TAV_OK) return st;
  }
  Plan P;
  P.B = p->num_seqs;
  P.N = p->node_offsets_host[P.B];
  P.Hq = p->num_q_heads;
  P.Hkv = p->num_kv_heads;
  P.D = p->head_dim;
  P.G = P.Hq / P.Hkv;
  P.log2G = log2_exact(P.G);
  P.NB = kRowsPerWG >> P.log2G;
  P.bs = p->block_size;
  P.lbs = log2_exact(p->block_size);
  int64_t tiles = 0, tail_blocks = 0;
  for (int b = 0; b < P.B; ++b) {
    const int n = p->node_offsets_host[b + 1] - p->node_offsets_host[b];
    const int nrb = ceil_div(n, P.NB);
    P.total_rb += nrb;
    for (int rb = 0; rb < nrb; ++rb) tiles += rb_tiles(p->prefix_len_host[b], n, rb, P.NB);
    tail_blocks += ceil_div(n, P.bs);
  }
  if (tiles + (int64_t)kRbCost * P.total_rb > (int64_t)1 << 30 || tail_blocks > (int64_t)1 << 30)
    return fail(TAV_ERR_UNSUPPORTED, "problem too large: %lld key tiles per KV head", (long long)tiles);
  P.tiles_per_head = (int)tiles;
  P.tail_blocks = (int)tail_blocks;
  if (p->dtype == TAV_BF16) {
    // equal shares C of the weighted tile axis, about one workgroup per compute unit over all
    // KV heads
    const int64_t weighted = (int64_t)P.tiles_per_head + (int64_t)kRbCost * P.total_rb;
    const int target = attn_wgs / P.Hkv > 1 ? attn_wgs / P.Hkv : 1;
    P.C = (int)ceil_div64(weighted, target);
    if (P.C < kMinTilesPerWG) P.C = kMinTilesPerWG;
    static_assert(kMinTilesPerWG > kRbCost, "a share must not fit inside one row block's fixed cost");
    P.W = (int)ceil_div64(weighted, P.C);
  }
  size_t o = 0;
  P.off_status = o; o = align_up(o + 256);
  P.off_chain = o; o = align_up(o + (size_t)P.B);
  P.off_mask = o; o = align_up(o + (size_t)P.N * kMaskWords * 8);
  P.off_seq_rb = o; o = align_up(o + (size_t)(P.B + 1) * 4);
  P.off_rb_seq = o; o = align_up(o + (size_t)P.total_rb * 4);
  P.off_rb_tile = o; o = align_up(o + (size_t)(P.total_rb + 1) * 4);
  P.off_tail_blk = o; o = align_up(o + (size_t)(P.B + 1) * 4);
  P.off_wg_rb = o; o = align_up(o + (size_t)P.W * 4);
  P.off_wg_tile = o; o = align_up(o + (size_t)(P.W + 1) * 4);
  P.off_rb_meta = o; o = align_up(o + (size_t)P.total_rb * kMetaWords * 4);
  const size_t tail_bytes = (size_t)P.tail_blocks * P.Hkv * P.bs * P.D * 2;
  P.off_ktail = o;
  if (p->dtype == TAV_BF16) o = align_up(o + tail_bytes);
  P.off_vtail = o;
  if (p->dtype == TAV_BF16) o = align_up(o + tail_bytes);
  P.off_part_o = o;
  o = align_up(o + (size_t)2 * P.W * P.Hkv * kRowsPerWG * P.D * 2);
  P.off_part_lse = o;
  o = align_up(o + (size_t)2 * P.W * P.Hkv * kRowsPerWG * 4);
  P.off_stats = o; o = align_up(o + (size_t)P.N * 3 * 4);
  P.off_term = o; o = align_up(o + (size_t)P.N * 4);
  P.off_step = o; o = align_up(o + (size_t)P.N * sizeof(StepRec));
  P.off_presto = o; o = align_up(o + (size_t)(pr ? pr->num_requests : 0) * 8);
  P.off_order = o; o = align_up(o + (size_t)(p->vocab > 0 ? P.N : 0) * 4);
  P.off_seq_err = o; o = align_up(o + (size_t)P.B * 4);
  if (p->vocab > 0) P.nch = ceil_div(ceil_div(p->vocab, p->dtype == TAV_BF16 ? 8 : 4), 64);
  P.off_cw = o; o = align_up(o + (size_t)(p->vocab > 0 ? P.N : 0) * P.nch * 4);
  P.off_rec = o; o = align_up(o + (size_t)(p->vocab > 0 ? P.N : 0) * sizeof(NodeRec));
  P.total = o;
  *out = P;
  return TAV_OK;
}

template <typename T>
T* ws_at(void* ws, size_t off) {
  return (T*)((char*)ws + off);
}

tav_status check_ws(const Plan& P, void* ws, size_t bytes) {
  if (!ws) return fail(TAV_ERR_WORKSPACE, "workspace is NULL");
  if ((uintptr_t)ws & 255u) return fail(TAV_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (bytes < P.total)
    return fail(TAV_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", bytes, P.total);
  return TAV_OK;
}

tav_status check_tree(const tav_tree* t, bool verify) {
  if (!t || !t->parent) return fail(TAV_ERR_NULL_POINTER, "tree / tree.parent is NULL");
  if (verify && (!t->token || !t->sampled))
    return fail(TAV_ERR_NULL_POINTER, "verification needs tree.token and tree.sampled");
  return TAV_OK;
}

tav_status check_attn(const tav_problem* p, const tav_attn_io* io) {
  if (!io || !io->q || !io->k_node || !io->v_node || !io->out)
    return fail(TAV_ERR_NULL_POINTER, "attention q / k_node / v_node / out is NULL");
  bool any_prefix = false;
  for (int b = 0; b < p->num_seqs; ++b) any_prefix |= p->prefix_len_host[b] > 0;
  if (any_prefix && (!io->k_cache || !io->v_cache || !io->block_table))
    return fail(TAV_ERR_NULL_POINTER, "k_cache / v_cache / block_table are required when a prefix is present");
  if (any_prefix && p->num_blocks < 1) return fail(TAV_ERR_BAD_SHAPE, "num_blocks must be >= 1");
  if (!aligned16(io->q) || !aligned16(io->k_node) || !aligned16(io->v_node) || !aligned16(io->out) ||
      !aligned16(io->k_cache) || !aligned16(io->v_cache))
    return fail(TAV_ERR_INVALID_ARGUMENT, "attention arrays must be 16-byte aligned");
  return TAV_OK;
}

tav_status check_verify(const tav_problem* p, const tav_verify_io* io) {
  if (!io || !io->logits || !io->temperature || !io->draft_row || !io->uniforms || !io->node_status ||
      !io->path || !io->path_len || !io->bonus_token)
    return fail(TAV_ERR_NULL_POINTER, "a verification array is NULL");
  if (io->num_draft_rows < 0) return fail(TAV_ERR_BAD_SHAPE, "num_draft_rows must be >= 0");
  if (io->draft_k < 0 || io->draft_k > kMaxDraftSupport)
    return fail(TAV_ERR_UNSUPPORTED, "draft_k must be in [0, %d] (got %d)", kMaxDraftSupport, io->draft_k);
  if (io->num_draft_rows > 0 && io->draft_k == 0 && !io->draft) return fail(TAV_ERR_NULL_POINTER, "draft is NULL");
  if (io->num_draft_rows > 0 && io->draft_k > 0 && (!io->draft_idx || !io->draft_val))
    return fail(TAV_ERR_NULL_POINTER, "draft_idx / draft_val are NULL (sparse draft rows)");
  if (io->max_path < 1) return fail(TAV_ERR_BAD_SHAPE, "max_path must be >= 1");
  if (p->vocab < 1) return fail(TAV_ERR_BAD_SHAPE, "vocab must be >= 1 for verification");
  const int epu = p->dtype == TAV_BF16 ? 8 : 4;
  const int64_t cap = (int64_t)kMaxChunks * 64 * epu;
  if (p->vocab % epu)
    return fail(TAV_ERR_UNSUPPORTED, "vocab must be a multiple of %d for this logits dtype (got %d)", epu, p->vocab);
  if (p->vocab > cap)
    return fail(TAV_ERR_UNSUPPORTED, "vocab %d exceeds the %lld tokens supported for this dtype",
                p->vocab, (long long)cap);
  if (!aligned16(io->logits) || (io->draft_k == 0 && !aligned16(io->draft)))
    return fail(TAV_ERR_INVALID_ARGUMENT, "logits and draft must be 16-byte aligned");
  return TAV_OK;
}

AttnArgs attn_args(const tav_problem* p, const Plan& P, const tav_attn_io* io, void* ws) {
  AttnArgs a;
  a.q = io->q; a.k_node = io->k_node; a.v_node = io->v_node;
  a.k_cache = io->k_cache; a.v_cache = io->v_cache; a.block_table = io->block_table;
  a.out = io->out; a.lse = io->lse;
  a.node_offsets = p->node_offsets; a.prefix_len = p->prefix_len;
  a.is_chain = ws_at<uint8_t>(ws, P.off_chain);
  a.mask = ws_at<uint64_t>(ws, P.off_mask);
  a.seq_rb_off = ws_at<int32_t>(ws, P.off_seq_rb);
  a.rb_seq = ws_at<int32_t>(ws, P.off_rb_seq);
  a.rb_tile = ws_at<int32_t>(ws, P.off_rb_tile);
  a.tail_blk = ws_at<int32_t>(ws, P.off_tail_blk);
  a.wg_rb = ws_at<int32_t>(ws, P.off_wg_rb);
  a.wg_tile = ws_at<int32_t>(ws, P.off_wg_tile);
  a.rb_meta = ws_at<int32_t>(ws, P.off_rb_meta);
  a.k_tail = ws_at<void>(ws, P.off_ktail);
  a.v_tail = ws_at<void>(ws, P.off_vtail);
  a.part_o = ws_at<uint16_t>(ws, P.off_part_o);
  a.part_lse = ws_at<float>(ws, P.off_part_lse);
  a.status = ws_at<uint32_t>(ws, P.off_status);
  a.seq_err = ws_at<uint32_t>(ws, P.off_seq_err);
  a.B = P.B; a.Hq = P.Hq; a.Hkv = P.Hkv; a.total_rb = P.total_rb;
  a.tiles_per_head = P.tiles_per_head; a.C = P.C; a.W = P.W; a.tail_blocks = P.tail_blocks;
  a.block_size = p->block_size; a.num_blocks = p->num_blocks;
  a.max_blocks = p->max_blocks_per_seq;
  a.scale = p->sm_scale > 0.f ? p->sm_scale : 1.f / sqrtf((float)p->head_dim);
  return a;
}

tav_status enqueue_prep(const tav_problem* p, const Plan& P, const tav_tree* t,
                        const tav_tree_out* out, void* ws, hipStream_t s) {
  uint32_t* status = ws_at<uint32_t>(ws, P.off_status);
  TAV_HIP(launch_prep(P, p->node_offsets, p->prefix_len, t->parent, ws_at<uint8_t>(ws, P.off_chain),
                      ws_at<uint64_t>(ws, P.off_mask), out, status, ws_at<uint32_t>(ws, P.off_seq_err), s));
  return TAV_OK;
}

// Event pairs around one kernel of the pass (tav_kernel_timing): 1 = the bf16 attention kernel,
// 2 = the vocabulary workers' kernel.  Timing-only events: no system-scope fence on record.
struct KernelTiming {
  int which = 0;
  int device = -1;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pool;
  size_t used = 0;
};
thread_local KernelTiming g_timing;   // per calling host thread

void release_timing_events() {
  for (auto& e : g_timing.pool) {
    (void)hipEventDestroy(e.first);
    (void)hipEventDestroy(e.second);
  }
  g_timing.pool.clear();
  g_timing.used = 0;
  g_timing.device = -1;
}

tav_status timing_pair(hipEvent_t* start, hipEvent_t* stop) {
  int dev = 0;
  TAV_HIP(hipGetDevice(&dev));
  if (g_timing.device < 0) g_timing.device = dev;
  if (g_timing.device != dev)
    return fail(TAV_ERR_INVALID_ARGUMENT, "kernel timing events belong to device %d, not %d", g_timing.device, dev);
  if (g_timing.used == g_timing.pool.size()) {
    hipEvent_t a = nullptr, b = nullptr;
    TAV_HIP(hipEventCreateWithFlags(&a, hipEventDisableSystemFence));
    if (hipEventCreateWithFlags(&b, hipEventDisableSystemFence) != hipSuccess) {
      (void)hipEventDestroy(a);
      return fail(TAV_ERR_HIP, "hipEventCreate failed");
    }
    g_timing.pool.emplace_back(a, b);
  }
  *start = g_timing.pool[g_timing.used].first;
  *stop = g_timing.pool[g_timing.used].second;
  ++g_timing.used;
  return TAV_OK;
}

// Tree preparation and attention (bf16: preparation, plan and node packing in one launch, then the
// attention kernel and the merge of split row blocks; float32: preparation, the attention kernel and
// the sentinel rows).  fused_start: the call's start is folded into the preparation launch;
// defer_merge: the merge (bf16) or the sentinel rows (float32) run later, in the walk's launch.
tav_status enqueue_prep_attention(const tav_problem* p, const Plan& P, const tav_tree* t,
                                  const tav_tree_out* out, const tav_attn_io* io, void* ws, hipStream_t s,
                                  const OrderArgs& order = OrderArgs{nullptr, 0, 0, nullptr},
                                  bool fused_start = false, bool defer_merge = false) {
  const AttnArgs a = attn_args(p, P, io, ws);
  if (p->dtype == TAV_BF16) {
    TAV_HIP(launch_prelude(P, t->parent, out, a, order, fused_start, s));
    hipEvent_t ev0 = nullptr, ev1 = nullptr;
    if (g_timing.which == 1) {
      const tav_status st = timing_pair(&ev0, &ev1);
      if (st != TAV_OK) return st;
      TAV_HIP(hipEventRecord(ev0, s));
    }
    TAV_HIP(launch_attn_bf16(P, a, s));
    if (ev1) TAV_HIP(hipEventRecord(ev1, s));
    if (!defer_merge) TAV_HIP(launch_merge(P, a, true, s));
  } else {
    if (fused_start) {
      TAV_HIP(launch_prep_start(P, p->node_offsets, p->prefix_len, t->parent, ws_at<uint8_t>(ws, P.off_chain),
                                ws_at<uint64_t>(ws, P.off_mask), out, a.status, a.seq_err, order, s));
    } else {
      const tav_status st = enqueue_prep(p, P, t, out, ws, s);
      if (st != TAV_OK) return st;
    }
    TAV_HIP(launch_attn_f32(P, a, s));
    if (!defer_merge) TAV_HIP(launch_attn_sentinel_f32(P, a, s));
  }
  return TAV_OK;
}

VocabArgs vocab_args(const tav_problem* p, const Plan& P, const tav_tree* t, const tav_verify_io* io, void* ws) {
  uint32_t* status = ws_at<uint32_t>(ws, P.off_status);
  VocabArgs va;
  va.logits = io->logits; va.temperature = io->temperature; va.draft = io->draft;
  va.draft_idx = io->draft_idx; va.draft_val = io->draft_val; va.K = io->draft_k;
  va.draft_row = io->draft_row; va.node_offsets = p->node_offsets; va.parent = t->parent;
  va.token = t->token; va.sampled = t->sampled; va.uniforms = io->uniforms;
  va.stats = io->node_stats ? io->node_stats : ws_at<float>(ws, P.off_stats);
  va.term_token = io->node_term_token ? io->node_term_token : ws_at<int32_t>(ws, P.off_term);
  va.status = status;
  va.seq_err = ws_at<uint32_t>(ws, P.off_seq_err);
  va.step = ws_at<StepRec>(ws, P.off_step);
  va.node_status = io->node_status;
  va.B = P.B; va.N = P.N; va.V = p->vocab; va.R = io->num_draft_rows;
  va.queue = (int32_t*)(status + kCounterWord);
  va.order = ws_at<int32_t>(ws, P.off_order);
  va.cw = ws_at<float>(ws, P.off_cw);
  va.rec = ws_at<NodeRec>(ws, P.off_rec);
  va.nch = P.nch;
  return va;
}

tav_status enqueue_walk(const Plan& P, const tav_verify_io* io, const VocabArgs& va, hipStream_t s,
                        const AttnArgs* attn = nullptr, bool f32_sentinels = false) {
  WalkArgs wa;
  wa.node_offsets = va.node_offsets; wa.parent = va.parent; wa.step = va.step;
  wa.node_status = io->node_status; wa.path = io->path; wa.path_len = io->path_len; wa.bonus = io->bonus_token;
  wa.status = va.status; wa.seq_err = va.seq_err;
  wa.B = P.B; wa.max_path = io->max_path;
  TAV_HIP(launch_walk(wa, &P, attn, f32_sentinels, s));
  return TAV_OK;
}

tav_status num_compute_units(int* cus) {
  int dev = 0;
  TAV_HIP(hipGetDevice(&dev));
  TAV_HIP(hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev));
  if (*cus < 1) *cus = 1;
  return TAV_OK;
}

// Verification: the vocabulary streaming and pick kernels (the workers' node order was built earlier
// in the call: by the bf16 prelude's order block, else by the start kernel), then the walk (after
// wait_before, when given, on s).
tav_status enqueue_verify(const tav_problem* p, const Plan& P, const tav_tree* t,
                          const tav_verify_io* io, void* ws, hipStream_t s, hipEvent_t wait_before = nullptr,
                          const AttnArgs* attn = nullptr) {
  const VocabArgs va = vocab_args(p, P, t, io, ws);
  int cus = 0;
  tav_status st = num_compute_units(&cus);
  if (st != TAV_OK) return st;
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  if (g_timing.which == 2) {
    st = timing_pair(&ev0, &ev1);
    if (st != TAV_OK) return st;
    TAV_HIP(hipEventRecord(ev0, s));
  }
  TAV_HIP(launch_vocab(va, p->dtype == TAV_BF16, cus, s));
  if (ev1) TAV_HIP(hipEventRecord(ev1, s));
  if (wait_before) TAV_HIP(hipStreamWaitEvent(s, wait_before, 0));
  return enqueue_walk(P, io, va, s, attn, p->dtype != TAV_BF16);
}

tav_status enqueue_presto(const Plan& P, const tav_presto_io* io, void* ws, hipStream_t s) {
  PrestoArgs pa;
  pa.T = io->T; pa.R = io->num_requests; pa.M = io->num_nodes; pa.max_transitions = io->max_transitions;
  pa.alpha = (double)io->alpha;
  pa.root_lp0 = io->root_lp0; pa.root_lq = io->root_lq; pa.cut = io->cut; pa.suffix_off = io->suffix_off;
  pa.lp0 = io->lp0; pa.lq = io->lq; pa.pf_parent = io->pf_parent; pa.pf_is_accept = io->pf_is_accept;
  pa.pf_request = io->pf_request; pa.u = io->u; pa.log_accept = io->log_accept;
  pa.log_accept64 = ws_at<double>(ws, P.off_presto);
  pa.pf_path = io->pf_path; pa.pf_path_len = io->pf_path_len;
  pa.status = ws_at<uint32_t>(ws, P.off_status);
  TAV_HIP(launch_presto(pa, s));
  return TAV_OK;
}

// Events ordering the two streams of the whole-pass call (per host thread and device): device-scope
// release, no timing.
struct StreamEvents {
  int device = -1;
  hipEvent_t fork = nullptr, join = nullptr;
};
thread_local StreamEvents g_events;

tav_status get_events(hipEvent_t* fork, hipEvent_t* join) {
  int dev = 0;
  TAV_HIP(hipGetDevice(&dev));
  if (g_events.device != dev) {
    for (hipEvent_t* e : {&g_events.fork, &g_events.join}) {
      if (*e) (void)hipEventDestroy(*e);
      *e = nullptr;
    }
    g_events.device = -1;
    for (hipEvent_t* e : {&g_events.fork, &g_events.join})
      TAV_HIP(hipEventCreateWithFlags(e, hipEventDisableTiming | hipEventReleaseToDevice));
    g_events.device = dev;
  }
  *fork = g_events.fork;
  *join = g_events.join;
  return TAV_OK;
}

// Device address of the allocation-free call's array on the current device, looked up once per
// device (with that device current) and kept.
tav_status scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  TAV_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(TAV_ERR_INVALID_ARGUMENT, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(TAV_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    addr[dev] = p;
  }
  *out = addr[dev];
  return TAV_OK;
}

// The whole pass on a given workspace (shared by tav_tree_attn_verify and the allocation-free
// variant, which passes the library's own device array).
tav_status attn_verify_impl(const tav_problem* prob, const tav_tree* tree, const tav_attn_io* attn,
                            const tav_verify_io* verify, const tav_presto_io* presto,
                            const tav_tree_out* tree_out, void* workspace, size_t workspace_bytes,
                            void* attn_stream, void* verify_stream, const Plan* plan = nullptr) {
  const bool two = verify_stream != attn_stream && presto;
  Plan P;
  tav_status st = TAV_OK;
  if (plan) P = *plan;
  else st = make_plan(prob, presto, &P);
  if (st == TAV_OK) st = check_ws(P, workspace, workspace_bytes);
  if (st == TAV_OK) st = check_tree(tree, verify != nullptr);
  if (st == TAV_OK) st = check_attn(prob, attn);
  if (st == TAV_OK && verify) st = check_verify(prob, verify);
  if (st != TAV_OK) return st;
  hipStream_t sa = (hipStream_t)attn_stream;
  hipStream_t sv = (hipStream_t)verify_stream;
  hipEvent_t fork = nullptr, join = nullptr;
  if (two) {
    st = get_events(&fork, &join);
    if (st != TAV_OK) return st;
  }
  // attn_stream: start, preparation, attention, the verification's kernels, the walk (with the merge
  // of the cut row blocks in bf16, the sentinel rows in float32).  The attention kernel and the workers each take whole compute
  // units, so they run one after the other.  PreSTO is independent: on verify_stream (if different)
  // from the start.
  // the start of the call folded into the preparation launch (one launch fewer) when nothing else
  // starts before it: with verification (the walk then folds the sequences' error words into the
  // status word) and no PreSTO batch (which would run beside the preparation on its own stream)
  const bool fused_start = verify && !presto;
  // the workers' node order: built by an extra block of the preparation launch (the bf16 prelude, or
  // the float32 preparation when the start is folded into it), else by the start kernel
  const bool order_in_prelude = verify && (prob->dtype == TAV_BF16 || fused_start);
  const OrderArgs order{verify ? verify->draft_row : nullptr, verify ? verify->num_draft_rows : 0, P.N,
                        verify ? ws_at<int32_t>(workspace, P.off_order) : nullptr};
  if (!fused_start)
    TAV_HIP(launch_start(ws_at<uint32_t>(workspace, P.off_status), ws_at<uint32_t>(workspace, P.off_seq_err), P.B,
                         order_in_prelude ? nullptr : order.draft_row, order.R, P.N, order.order, sa));
  if (two) {
    TAV_HIP(hipEventRecord(fork, sa));
    TAV_HIP(hipStreamWaitEvent(sv, fork, 0));
  }
  if (presto) {
    st = enqueue_presto(P, presto, workspace, two ? sv : sa);
    if (st != TAV_OK) return st;
  }
  if (two) TAV_HIP(hipEventRecord(join, sv));
  // with verification the merge of the cut row blocks (bf16) or the sentinel rows (float32) run in
  // the walk's launch, beside the walks
  const bool defer_merge = verify != nullptr;
  st = enqueue_prep_attention(prob, P, tree, tree_out, attn, workspace, sa,
                              order_in_prelude ? order : OrderArgs{nullptr, 0, 0, nullptr}, fused_start,
                              defer_merge);
  if (st != TAV_OK) return st;
  if (verify) {
    const AttnArgs ma = attn_args(prob, P, attn, workspace);
    st = enqueue_verify(prob, P, tree, verify, workspace, sa, two ? join : nullptr, defer_merge ? &ma : nullptr);
    if (st != TAV_OK) return st;
  } else if (two) {
    TAV_HIP(hipStreamWaitEvent(sa, join, 0));
  }
  return ok();
}

}  // namespace

tav_status tav_host_fail(tav_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vfail(s, fmt, ap);
  va_end(ap);
  return s;
}

tav_status tav_host_ok() { return ok(); }

}  // namespace tav

using namespace tav;

extern "C" {

tav_status tav_workspace_size(const tav_problem* prob, const tav_presto_io* presto, size_t* bytes) {
  if (!bytes) return fail(TAV_ERR_NULL_POINTER, "bytes is NULL");
  Plan P;
  tav_status st = make_plan(prob, presto, &P);
  if (st != TAV_OK) return st;
  *bytes = P.total;
  return ok();
}

tav_status tav_tree_prep(const tav_problem* prob, const tav_tree* tree, const tav_tree_out* out,
                         void* workspace, size_t workspace_bytes, void* stream) {
  Plan P;
  tav_status st = make_plan(prob, nullptr, &P);
  if (st == TAV_OK) st = check_ws(P, workspace, workspace_bytes);
  if (st == TAV_OK) st = check_tree(tree, false);
  if (st != TAV_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  TAV_HIP(launch_start(ws_at<uint32_t>(workspace, P.off_status), ws_at<uint32_t>(workspace, P.off_seq_err), P.B,
                       nullptr, 0, 0, nullptr, s));
  st = enqueue_prep(prob, P, tree, out, workspace, s);
  return st == TAV_OK ? ok() : st;
}

tav_status tav_tree_attention(const tav_problem* prob, const tav_tree* tree, const tav_attn_io* io,
                              void* workspace, size_t workspace_bytes, void* stream) {
  Plan P;
  tav_status st = make_plan(prob, nullptr, &P);
  if (st == TAV_OK) st = check_ws(P, workspace, workspace_bytes);
  if (st == TAV_OK) st = check_tree(tree, false);
  if (st == TAV_OK) st = check_attn(prob, io);
  if (st != TAV_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  TAV_HIP(launch_start(ws_at<uint32_t>(workspace, P.off_status), ws_at<uint32_t>(workspace, P.off_seq_err), P.B,
                       nullptr, 0, 0, nullptr, s));
  st = enqueue_prep_attention(prob, P, tree, nullptr, io, workspace, s);
  return st == TAV_OK ? ok() : st;
}

tav_status tav_tree_verify(const tav_problem* prob, const tav_tree* tree, const tav_verify_io* io,
                           void* workspace, size_t workspace_bytes, void* stream) {
  Plan P;
  tav_status st = make_plan(prob, nullptr, &P);
  if (st == TAV_OK) st = check_ws(P, workspace, workspace_bytes);
  if (st == TAV_OK) st = check_tree(tree, true);
  if (st == TAV_OK) st = check_verify(prob, io);
  if (st != TAV_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  TAV_HIP(launch_start(ws_at<uint32_t>(workspace, P.off_status), ws_at<uint32_t>(workspace, P.off_seq_err), P.B,
                       io->draft_row, io->num_draft_rows, P.N, ws_at<int32_t>(workspace, P.off_order), s));
  st = enqueue_verify(prob, P, tree, io, workspace, s);
  return st == TAV_OK ? ok() : st;
}

tav_status tav_presto_accept(const tav_presto_io* io, void* workspace, size_t workspace_bytes,
                             void* stream) {
  if (!io) return fail(TAV_ERR_NULL_POINTER, "presto io is NULL");
  tav_status st = check_presto(io);
  if (st != TAV_OK) return st;
  Plan P;  // PreSTO alone needs only the status word and the fp64 log A buffer
  P.off_status = 0;
  P.off_presto = 256;
  P.total = 256 + align_up((size_t)io->num_requests * 8);
  st = check_ws(P, workspace, workspace_bytes);
  if (st != TAV_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  TAV_HIP(launch_start(ws_at<uint32_t>(workspace, P.off_status), nullptr, 0, nullptr, 0, 0, nullptr, s));
  st = enqueue_presto(P, io, workspace, s);
  return st == TAV_OK ? ok() : st;
}

tav_status tav_tree_attn_verify(const tav_problem* prob, const tav_tree* tree, const tav_attn_io* attn,
                                const tav_verify_io* verify, const tav_presto_io* presto,
                                const tav_tree_out* tree_out, void* workspace, size_t workspace_bytes,
                                void* attn_stream, void* verify_stream) {
  return attn_verify_impl(prob, tree, attn, verify, presto, tree_out, workspace, workspace_bytes, attn_stream,
                          verify_stream);
}

tav_status tav_tree_attn_verify_noalloc(const tav_problem* prob, const tav_tree* tree, const tav_attn_io* attn,
                                        const tav_verify_io* verify, const tav_presto_io* presto,
                                        const tav_tree_out* tree_out, uint32_t* status_out,
                                        void* attn_stream, void* verify_stream) {
  Plan P;
  tav_status st = make_plan(prob, presto, &P);
  if (st != TAV_OK) return st;
  if (P.total > (size_t)TAV_NOALLOC_SCRATCH_BYTES)
    return fail(TAV_ERR_WORKSPACE,
                "this problem needs %zu bytes of workspace; the allocation-free call has %zu (use "
                "tav_tree_attn_verify with a caller workspace)",
                P.total, (size_t)TAV_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != TAV_OK) return st;
  st = attn_verify_impl(prob, tree, attn, verify, presto, tree_out, ws, (size_t)TAV_NOALLOC_SCRATCH_BYTES,
                        attn_stream, verify_stream, &P);
  if (st != TAV_OK) return st;
  if (status_out)   // the status word (written by this call's kernels) into the caller's buffer
    TAV_HIP(hipMemcpyAsync(status_out, ws_at<uint32_t>(ws, P.off_status), sizeof(uint32_t),
                           hipMemcpyDeviceToDevice, (hipStream_t)attn_stream));
  return ok();
}

tav_status tav_token_scores(const tav_score_io* io, void* workspace, size_t workspace_bytes, void* stream) {
  if (!io) return fail(TAV_ERR_NULL_POINTER, "score io is NULL");
  if (io->num_rows < 0 || io->vocab < 1) return fail(TAV_ERR_BAD_SHAPE, "num_rows must be >= 0 and vocab >= 1");
  if (io->dtype != TAV_F32 && io->dtype != TAV_BF16)
    return fail(TAV_ERR_UNSUPPORTED, "dtype must be TAV_F32 or TAV_BF16 (got %d)", io->dtype);
  const int epu = io->dtype == TAV_BF16 ? 8 : 4;
  if (io->vocab % epu)
    return fail(TAV_ERR_UNSUPPORTED, "vocab must be a multiple of %d for this dtype (got %d)", epu, io->vocab);
  if (io->num_rows > 0 && !io->logits) return fail(TAV_ERR_NULL_POINTER, "logits is NULL");
  if (!aligned16(io->logits)) return fail(TAV_ERR_INVALID_ARGUMENT, "logits must be 16-byte aligned");
  if (!(io->tau > 0.f) || !isfinite(io->tau)) return fail(TAV_ERR_INVALID_ARGUMENT, "tau must be finite and > 0");
  Plan P;
  P.off_status = 0;
  P.total = 256;
  tav_status st = check_ws(P, workspace, workspace_bytes);
  if (st != TAV_OK) return st;
  int cus = 0;
  st = num_compute_units(&cus);
  if (st != TAV_OK) return st;
  ScoreArgs a;
  a.logits = io->logits; a.token = io->token; a.tau = io->tau;
  const float inv = 1.f / io->tau;
  const int k = (int)lrintf(inv);
  a.kpow = (k >= 1 && k <= 8 && fabsf(inv - (float)k) <= 1e-6f * inv) ? k : 0;
  a.lp0 = io->token ? io->log_p0 : nullptr;
  a.lq = io->token ? io->log_q : nullptr;
  a.ent = io->entropy; a.argmax = io->argmax;
  a.status = ws_at<uint32_t>(workspace, 0);
  a.N = io->num_rows; a.V = io->vocab;
  hipStream_t s = (hipStream_t)stream;
  TAV_HIP(launch_start(a.status, nullptr, 0, nullptr, 0, 0, nullptr, s));
  TAV_HIP(launch_score(a, io->dtype == TAV_BF16, cus, s));
  return ok();
}

namespace {

// Sizes, candidate-id ranges and workspace layout of a draft-tree construction.
tav_status draft_plan(const tav_draft_params* p, DraftArgs* a, size_t* total) {
  if (!p) return fail(TAV_ERR_NULL_POINTER, "draft params are NULL");
  if (p->num_seqs < 1 || p->vocab < 8 || p->vocab % 8)
    return fail(TAV_ERR_BAD_SHAPE, "draft: num_seqs >= 1 and vocab a positive multiple of 8 (got %d, %d)",
                p->num_seqs, p->vocab);
  if (p->depth < 1 || p->depth > kMaxDraftDepth || p->expand_k < 1 || p->expand_k > 64)
    return fail(TAV_ERR_UNSUPPORTED, "draft: depth in [1, %d], expand_k in [1, 64] (got %d, %d)", kMaxDraftDepth,
                p->depth, p->expand_k);
  if (p->support < 1 || p->support > kMaxDraftSupport || p->support > p->vocab || p->slots < 1 ||
      p->slots > p->support || p->lead_m < 0 || p->lead_m >= p->slots)
    return fail(TAV_ERR_UNSUPPORTED, "draft: need 0 <= lead_m < slots <= support <= min(128, vocab) (got %d, %d, %d)",
                p->lead_m, p->slots, p->support);
  if (p->hybrid < TAV_DRAFT_HYBRID_NONE || p->hybrid > TAV_DRAFT_HYBRID_ALL)
    return fail(TAV_ERR_INVALID_ARGUMENT, "draft: hybrid must be TAV_DRAFT_HYBRID_NONE, _FIRST or _ALL");
  if (!(p->temperature > 0.f) || !isfinite(p->temperature) || !(p->eps >= 0.f) || !isfinite(p->eps))
    return fail(TAV_ERR_INVALID_ARGUMENT, "draft: temperature must be finite and > 0, eps finite and >= 0");
  DraftArgs A{};
  A.B = p->num_seqs; A.V = p->vocab; A.S = p->support; A.K = p->expand_k; A.slots = p->slots; A.m = p->lead_m;
  A.hybrid = p->hybrid; A.R = p->budget; A.D = p->depth; A.temperature = p->temperature; A.eps = p->eps;
  A.kcount[0] = 0;
  A.base[0] = 0;
  A.kcount[1] = 1;
  A.base[1] = 1;
  for (int d = 1; d <= A.D; ++d) {
    const int nd = A.kcount[d] * A.slots;
    A.base[d + 1] = A.base[d] + nd;
    A.kcount[d + 1] = d < A.D ? (nd < A.K ? nd : A.K) : 0;
    if (A.base[d + 1] > kMaxDraftCandidates)
      return fail(TAV_ERR_UNSUPPORTED, "draft: more than %d candidates per tree", kMaxDraftCandidates);
  }
  A.C = A.base[A.D + 1];
  if (p->budget < 1 || p->budget > A.C - 1)
    return fail(TAV_ERR_BAD_SHAPE, "draft: budget must be in [1, %d] (got %d)", A.C - 1, p->budget);
  const size_t B = (size_t)A.B, C = (size_t)A.C, S = (size_t)A.S;
  size_t o = 0;
  A.status = (uint32_t*)o; o = align_up(o + 256);
  A.seq_err = (uint32_t*)o; o = align_up(o + B * 4);
  A.cand_parent = (int32_t*)o; o = align_up(o + B * C * 4);
  A.cand_token = (int32_t*)o; o = align_up(o + B * C * 4);
  A.cand_score = (double*)o; o = align_up(o + B * C * 8);
  A.cand_sampled = (uint8_t*)o; o = align_up(o + B * C);
  A.cand_depth = (uint8_t*)o; o = align_up(o + B * C);
  A.row_idx = (int32_t*)o; o = align_up(o + B * C * S * 4);
  A.row_val = (float*)o; o = align_up(o + B * C * S * 4);
  A.frontier = (int32_t*)o; o = align_up(o + B * (size_t)A.K * 4);
  *a = A;
  *total = o;
  return TAV_OK;
}

// The layout's offsets turned into addresses inside the workspace.
void draft_bind(DraftArgs* a, void* ws) {
  char* w = (char*)ws;
  a->status = (uint32_t*)(w + (size_t)a->status);
  a->seq_err = (uint32_t*)(w + (size_t)a->seq_err);
  a->cand_parent = (int32_t*)(w + (size_t)a->cand_parent);
  a->cand_token = (int32_t*)(w + (size_t)a->cand_token);
  a->cand_score = (double*)(w + (size_t)a->cand_score);
  a->cand_sampled = (uint8_t*)(w + (size_t)a->cand_sampled);
  a->cand_depth = (uint8_t*)(w + (size_t)a->cand_depth);
  a->row_idx = (int32_t*)(w + (size_t)a->row_idx);
  a->row_val = (float*)(w + (size_t)a->row_val);
  a->frontier = (int32_t*)(w + (size_t)a->frontier);
}

}  // namespace

tav_status tav_draft_workspace_size(const tav_draft_params* p, size_t* bytes) {
  if (!bytes) return fail(TAV_ERR_NULL_POINTER, "bytes is NULL");
  DraftArgs a;
  size_t total = 0;
  const tav_status st = draft_plan(p, &a, &total);
  if (st != TAV_OK) return st;
  *bytes = total;
  return ok();
}

tav_status tav_draft_expand(const tav_draft_params* p, int32_t d, const void* draft_logits, const float* uniforms,
                            int32_t* frontier_out, void* workspace, size_t workspace_bytes, void* stream) {
  DraftArgs a;
  size_t total = 0;
  tav_status st = draft_plan(p, &a, &total);
  if (st != TAV_OK) return st;
  if (d < 1 || d > a.D) return fail(TAV_ERR_INVALID_ARGUMENT, "draft: depth %d outside [1, %d]", d, a.D);
  if (!draft_logits || !uniforms) return fail(TAV_ERR_NULL_POINTER, "draft logits / uniforms are NULL");
  if (!aligned16(draft_logits)) return fail(TAV_ERR_INVALID_ARGUMENT, "draft logits must be 16-byte aligned");
  Plan P;
  P.total = total;
  st = check_ws(P, workspace, workspace_bytes);
  if (st != TAV_OK) return st;
  draft_bind(&a, workspace);
  a.Kd = a.kcount[d];
  hipStream_t s = (hipStream_t)stream;
  if (d == 1) TAV_HIP(launch_start(a.status, a.seq_err, a.B, nullptr, 0, 0, nullptr, s));
  TAV_HIP(launch_draft_expand(a, d, (const uint16_t*)draft_logits, uniforms, frontier_out, s));
  return ok();
}

tav_status tav_draft_prune(const tav_draft_params* p, int32_t* parent, int32_t* token, uint8_t* sampled,
                           int32_t* cand_id, int32_t* draft_row, int32_t* draft_idx, float* draft_val,
                           void* workspace, size_t workspace_bytes, void* stream) {
  DraftArgs a;
  size_t total = 0;
  tav_status st = draft_plan(p, &a, &total);
  if (st != TAV_OK) return st;
  if (!parent || !token || !sampled || !draft_row || !draft_idx || !draft_val)
    return fail(TAV_ERR_NULL_POINTER, "draft prune: an output array is NULL");
  Plan P;
  P.total = total;
  st = check_ws(P, workspace, workspace_bytes);
  if (st != TAV_OK) return st;
  draft_bind(&a, workspace);
  DraftOut o{parent, token, sampled, cand_id, draft_row, draft_idx, draft_val};
  TAV_HIP(launch_draft_prune(a, o, (hipStream_t)stream));
  return ok();
}

tav_status tav_read_status(const void* workspace, void* stream, uint32_t* status_bits) {
  if (!workspace || !status_bits) return fail(TAV_ERR_NULL_POINTER, "workspace / status_bits is NULL");
  TAV_HIP(hipStreamSynchronize((hipStream_t)stream));
  TAV_HIP(hipMemcpy(status_bits, workspace, sizeof(uint32_t), hipMemcpyDeviceToHost));
  return ok();
}

tav_status tav_kernel_timing(int which) {
  if (which < 0 || which > 2) return fail(TAV_ERR_INVALID_ARGUMENT, "tav_kernel_timing: which must be 0, 1 or 2");
  release_timing_events();
  g_timing.which = which;
  return ok();
}

tav_status tav_kernel_timing_read(double* total_ms, int32_t* launches) {
  if (!total_ms || !launches) return fail(TAV_ERR_NULL_POINTER, "total_ms / launches is NULL");
  double total = 0.0;
  for (size_t i = 0; i < g_timing.used; ++i) {
    TAV_HIP(hipEventSynchronize(g_timing.pool[i].second));
    float ms = 0.f;
    TAV_HIP(hipEventElapsedTime(&ms, g_timing.pool[i].first, g_timing.pool[i].second));
    total += ms;
  }
  *total_ms = total;
  *launches = (int32_t)g_timing.used;
  g_timing.used = 0;
  return ok();
}

const char* tav_status_string(tav_status s) {
  switch (s) {
    case TAV_OK: return "TAV_OK";
    case TAV_ERR_NULL_POINTER: return "TAV_ERR_NULL_POINTER";
    case TAV_ERR_BAD_SHAPE: return "TAV_ERR_BAD_SHAPE";
    case TAV_ERR_UNSUPPORTED: return "TAV_ERR_UNSUPPORTED";
    case TAV_ERR_WORKSPACE: return "TAV_ERR_WORKSPACE";
    case TAV_ERR_HIP: return "TAV_ERR_HIP";
    case TAV_ERR_INVALID_ARGUMENT: return "TAV_ERR_INVALID_ARGUMENT";
  }
  return "unknown tav_status";
}

const char* tav_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
