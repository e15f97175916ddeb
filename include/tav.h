/*
 * tav.h -- C ABI of the tree-masked scoring pass on AMD MI355X (gfx950).
 *
 * One batched pass over B token trees: every tree node is a query that attends
 * to its sequence's cached prefix (paged KV) plus only its own root-to-node
 * ancestors, followed by per-node verification of the tree against the target
 * distribution, and (optionally) PreSTO's log-acceptance and MH walk over a
 * prefetched subtree.
 *
 * Sources (the method is defined on these pages; the numbering is the pages'):
 *  - Progressive Tree Drafting (arXiv 2607.10661), Section 3.1 "Tree
 *    Construction": pi(v) = {v} U pi(P(v)); position from |pi(v)|.
 *    Section 3.2 "Candidate Verification" and Appendix E / F: sequential
 *    rejection with renormalisation; accepted sequence X' = (n0..nk, V_nk).
 *  - RheoSampling (arXiv 2609.21827), Section 3.3 Algorithm 1
 *    (RheoVerification), Section 5.4 (temperature decoupling).
 *  - PreSTO (arXiv 2610.13171), Section 3.2 Example 3 / Equation 6
 *    (log-acceptance), Appendix B.1 (Equations 7-9), Appendix B.3 Example 5
 *    (walk over the prefetched subtree).
 *
 * Conventions shared by every entry point
 *  - All array arguments are device pointers unless the field name ends in
 *    _host.  Arrays are dense, row-major, and 16-byte aligned.
 *  - The caller owns every buffer.  The library never allocates device memory
 *    and keeps no pointer after a call returns; scratch lives in a caller-owned
 *    workspace of at least tav_workspace_size() bytes (256-byte aligned).
 *  - Calls are asynchronous on the given stream(s): host-checkable problems
 *    return a tav_status synchronously and enqueue nothing; problems only the
 *    device can see set bits in a status word inside the workspace
 *    (tav_read_status) and the affected sequence's outputs become sentinels:
 *      - an error of its tree or its prefix (TAV_DEV_BAD_PARENT,
 *        TAV_DEV_TREE_TOO_LARGE, TAV_DEV_BAD_BLOCK) zeroes its attention rows
 *        (out = 0, lse = -inf);
 *      - any device-detected error of the sequence (those and the verification
 *        ones: tokens, siblings, sampled children, draft rows, logits,
 *        temperature, residual mass, path length) makes its verification
 *        outputs path_len = 0, path = -1, bonus_token = -1, node_status = 0;
 *      - TAV_DEV_PLAN_MISMATCH (device copies of node_offsets / prefix_len
 *        differ from the host copies) leaves attention outputs unwritten and
 *        makes every sequence's verification outputs sentinels;
 *      - PreSTO errors (TAV_DEV_PRESTO_BAD_TREE) give NaN log_accept for the
 *        affected request.
 *    Every kernel checks an index before it uses it, so a bad input never
 *    causes an out-of-bounds access.
 *  - Streams are passed as void* and are hipStream_t values (NULL = the null
 *    stream).  Calls on different workspaces are independent; two calls that
 *    share a workspace must be ordered by the caller.
 *
 * Tree layout
 *  - Sequence b owns nodes [node_offsets[b], node_offsets[b+1]) (at least one).
 *  - parent[] is sequence-local: node 0 of a sequence is its root (parent -1,
 *    the last committed token); every other node's parent is an earlier node
 *    of the same sequence.  Hence every ancestor of node v has an id <= v.
 *  - A sequence whose every node's parent is the node just before it is a
 *    chain (causal attention, any length).  Any other tree may have at most
 *    256 nodes (ancestor sets are 256-bit masks).
 *  - A forest whose roots share one cached prefix up to different lengths
 *    (PreSTO's suffix requests, each keeping the state's prefix up to its own
 *    cut: Section 3.2 step (2), Appendix B.3 Example 4) is passed as one
 *    sequence per root: prefix_len of each is its root's prefix length, and
 *    their block-table rows name the same physical blocks, so the shared
 *    prefix is stored once.
 */
#ifndef TAV_H
#define TAV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum tav_status {
  TAV_OK = 0,
  TAV_ERR_NULL_POINTER = 1,      /* a required pointer is NULL */
  TAV_ERR_BAD_SHAPE = 2,         /* sizes inconsistent (offsets, heads, prefix vs block table, ...) */
  TAV_ERR_UNSUPPORTED = 3,       /* valid but not implemented (head_dim, dtype, group size, vocab) */
  TAV_ERR_WORKSPACE = 4,         /* workspace NULL, misaligned or smaller than tav_workspace_size() */
  TAV_ERR_HIP = 5,               /* a HIP runtime call or kernel launch failed */
  TAV_ERR_INVALID_ARGUMENT = 6   /* other invalid scalar argument (temperature field, counts, ...) */
} tav_status;

typedef enum tav_dtype {
  TAV_F32 = 0,   /* float32 q/k/v/cache/out/logits */
  TAV_BF16 = 1   /* bfloat16 q/k/v/cache/out/logits; fp32 accumulation */
} tav_dtype;

/* Device status bits (OR-ed into the workspace status word). */
enum {
  TAV_DEV_BAD_PARENT = 1u << 0,         /* parent not in [-1, v) or node 0 not a root */
  TAV_DEV_TREE_TOO_LARGE = 1u << 1,     /* non-chain tree with more than 256 nodes */
  TAV_DEV_BAD_BLOCK = 1u << 2,          /* block-table entry outside [0, num_blocks) */
  TAV_DEV_BAD_TOKEN = 1u << 3,          /* a child token outside [0, vocab) */
  TAV_DEV_DUP_SIBLING_TOKEN = 1u << 4,  /* two children of one node carry the same token */
  TAV_DEV_MULTI_SAMPLED = 1u << 5,      /* more than one sampled child under one node */
  TAV_DEV_NO_DRAFT = 1u << 6,           /* sampled child but draft_row of its parent < 0 or >= R */
  TAV_DEV_ZERO_DRAFT_MASS = 1u << 7,    /* the sampled token has zero draft probability */
  TAV_DEV_NONFINITE_LOGITS = 1u << 8,   /* NaN or +inf logit (-inf is allowed: zero mass) */
  TAV_DEV_EMPTY_RESIDUAL = 1u << 9,     /* the final residual of the walk has no mass */
  TAV_DEV_PATH_OVERFLOW = 1u << 10,     /* accepted path longer than max_path */
  TAV_DEV_TOO_MANY_CHILDREN = 1u << 11, /* a node with more than 256 children */
  TAV_DEV_PRESTO_BAD_TREE = 1u << 12,   /* malformed prefetching tree / request ids */
  TAV_DEV_PLAN_MISMATCH = 1u << 13,     /* internal: device work plan differs from the host's */
  TAV_DEV_BAD_TEMPERATURE = 1u << 14,   /* a temperature that is not finite and > 0 */
  TAV_DEV_BAD_DRAFT = 1u << 15,         /* sparse draft row: id outside [0, V), ids not strictly
                                           ascending, or a value not finite and >= 0 */
  TAV_DEV_DRAFT_TIES = 1u << 16         /* draft-tree construction: more than 2048 tokens share the
                                           logit at the support's edge (support then unspecified) */
};

/* Problem description (host struct). */
typedef struct tav_problem {
  int32_t num_seqs;                  /* B >= 1 */
  const int32_t* node_offsets_host;  /* [B+1] host copy; node_offsets[0] = 0, strictly increasing */
  const int32_t* node_offsets;       /* [B+1] device copy of the same */
  const int32_t* prefix_len_host;    /* [B] host copy; cached prefix rows of each sequence (>= 0) */
  const int32_t* prefix_len;         /* [B] device copy of the same */
  int32_t num_q_heads;               /* Hq */
  int32_t num_kv_heads;              /* Hkv; query head h reads KV head h / (Hq / Hkv) */
  int32_t head_dim;                  /* 64 or 128 */
  int32_t dtype;                     /* tav_dtype of q, k, v, caches, out and logits */
  float sm_scale;                    /* softmax scale; 0 means 1/sqrt(head_dim) */
  int32_t block_size;                /* prefix rows per KV block: 16, 32 or 64 (bf16); 8 also for f32 */
  int32_t num_blocks;                /* physical blocks in k_cache / v_cache */
  int32_t max_blocks_per_seq;        /* row stride of block_table; prefix_len <= this * block_size */
  int32_t vocab;                     /* V for verification (0 when no verification is run) */
} tav_problem;

/* Tree arrays (device). token and sampled are only read by verification. */
typedef struct tav_tree {
  const int32_t* parent;    /* [N] sequence-local parent, -1 at each sequence's node 0 */
  const int32_t* token;     /* [N] token of each node (the root's token is not read) */
  const uint8_t* sampled;   /* [N] 1 if the node was drawn from its parent's draft distribution */
} tav_tree;

/* Optional outputs of tree preparation (each may be NULL). */
typedef struct tav_tree_out {
  int32_t* depth;       /* [N] |pi(v)| - 1 */
  int32_t* position;    /* [N] prefix_len + depth (0-based position of the node's token) */
  uint64_t* mask;       /* [N][4] bit j set iff node j (sequence-local) is in pi(v); zero for chains */
  uint8_t* is_chain;    /* [B] 1 for a chain sequence */
} tav_tree_out;

/* Attention inputs and outputs.  Layouts:
 *   q [N, Hq, D];  k_node, v_node [N, Hkv, D] (the tree nodes' own keys/values);
 *   k_cache [num_blocks, Hkv, block_size, D] and v_cache [num_blocks, Hkv, D, block_size]
 *     (values d-major inside a block): prefix row r of sequence b is slot
 *     r % block_size of block block_table[b * max_blocks_per_seq + r / block_size];
 *   out [N, Hq, D] in the problem dtype; lse [N, Hq] float (natural log), optional. */
typedef struct tav_attn_io {
  const void* q;
  const void* k_node;
  const void* v_node;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  void* out;
  float* lse;
} tav_attn_io;

/* Verification inputs and outputs.
 *   logits [N, V] (problem dtype): target logits at each node (the distribution
 *     over the token that follows the node);
 *   temperature [B] >= 0: p = softmax(logits / T); T = 0 is greedy decoding (Progressive
 *     Tree Drafting, Section 3.2: the child whose token is the argmax of its parent's logits
 *     is accepted, the last node's argmax is the bonus token; draft rows are not read);
 *   draft [R, V] float and draft_row [N]: row draft_row[v] is the (already
 *     tempered) distribution v's sampled child was drawn from; -1 if none;
 *   or, with draft_k > 0, sparse rows (RheoSampling Section 3.2: the draft truncated to
 *     its top entries before the softmax, so q~ is zero off a support of at most 128
 *     tokens): draft_idx [R, draft_k] int32 support token ids in strictly ascending
 *     order and draft_val [R, draft_k] float q~ at those ids (zeros allowed); draft is
 *     then not read.  Verification reads K entries per row instead of V;
 *   uniforms [N, 2] in [0, 1): uniforms[c][0] tests node c as a candidate,
 *     uniforms[v][1] drives the final draw at v.
 * Outputs:
 *   node_status [N]: 0 not reached, 1 accepted (the root always), 2 rejected;
 *   path [B, max_path]: accepted sequence-local node ids from the root, -1 padded;
 *   path_len [B]; bonus_token [B]: the final token drawn at the last path node.
 *   node_stats [N, 3] float (optional): M = max l/T, S = sum exp(l/T - M), Z = sum (p - q~)+;
 *   node_term_token [N] (optional): the token the final draw would give if the walk ended at v. */
typedef struct tav_verify_io {
  const void* logits;
  const float* temperature;
  const float* draft;
  int32_t num_draft_rows;
  const int32_t* draft_row;
  const int32_t* draft_idx;
  const float* draft_val;
  int32_t draft_k;
  const float* uniforms;
  uint8_t* node_status;
  int32_t* path;
  int32_t max_path;
  int32_t* path_len;
  int32_t* bonus_token;
  float* node_stats;
  int32_t* node_term_token;
} tav_verify_io;

/* PreSTO prefetch round.  Per-token arrays hold tokens t = 1..T at index t-1.
 *   root_lp0 / root_lq [T]: log p0 and log q_tau of the current state's tokens;
 *   request i (0..R-1): cut[i] in [0, T); its suffix (tokens cut[i]+1..T) occupies
 *     lp0/lq[suffix_off[i] .. suffix_off[i+1]) with suffix_off[i+1]-suffix_off[i] = T - cut[i];
 *   prefetching tree over M nodes (node 0 = current state): pf_parent[v] < v;
 *     pf_is_accept[v] = 1 for an acceptance child; pf_request[v] = its request id,
 *     or -1 for a rejection child or a deferred request; u[v] = the MH uniform
 *     used for the decision taken at node v.
 * Outputs: log_accept [R] (Equation 6, computed in float64, stored as float);
 *   pf_path [M] tree nodes visited from the root, -1 padded; pf_path_len [1]
 *   = completed transitions + 1. */
typedef struct tav_presto_io {
  int32_t T;
  float alpha;
  const float* root_lp0;
  const float* root_lq;
  int32_t num_requests;
  const int32_t* cut;
  const int32_t* suffix_off;
  const float* lp0;
  const float* lq;
  int32_t num_nodes;
  const int32_t* pf_parent;
  const uint8_t* pf_is_accept;
  const int32_t* pf_request;
  const float* u;
  int32_t max_transitions;
  float* log_accept;
  int32_t* pf_path;
  int32_t* pf_path_len;
} tav_presto_io;

/* Per-token scores of sampled tokens (PreSTO, Appendix D.3: the patched sampler returns, for
 * each sampled token, its proposal log-probability under q_tau = softmax(l / tau), its base-model
 * log-probability under p0 = softmax(l) from the unprocessed logits, and the full-vocabulary
 * entropy of p0 in natural log -- the per-token inputs of log A, PreSTO Section 3.2 Example 3;
 * Progressive Tree Drafting, Section 3.2: a node's greedy verification token is the argmax).
 *   logits [num_rows, vocab] (dtype TAV_BF16 or TAV_F32, 16-byte aligned, vocab a multiple of 8
 *     for bf16 and 4 for f32): the unprocessed logits of each row;
 *   token [num_rows] (may be NULL: then log_p0 / log_q are not written): the sampled token;
 *   tau > 0 finite: the proposal temperature;
 * outputs (each may be NULL): log_p0 [num_rows], log_q [num_rows], entropy [num_rows] (float),
 *   argmax [num_rows] (int32, smallest id among equal maxima; -1 for a row with no finite logit).
 * Device-detected errors: a token outside [0, vocab) (TAV_DEV_BAD_TOKEN) or a NaN / +inf logit or
 * a row with no finite logit (TAV_DEV_NONFINITE_LOGITS) make that row's scores NaN.  workspace:
 * at least 256 bytes, 256-byte aligned (the status word; tav_read_status reads it). */
typedef struct tav_score_io {
  int32_t num_rows;
  int32_t vocab;
  int32_t dtype;
  const void* logits;
  const int32_t* token;
  float tau;
  float* log_p0;
  float* log_q;
  float* entropy;
  int32_t* argmax;
} tav_score_io;

tav_status tav_token_scores(const tav_score_io* io, void* workspace, size_t workspace_bytes, void* stream);

/* PreSTO's prefetching tree for one batch (host only, no HIP call; PreSTO Section 3.2 step (1)
 * and Appendix C).  Node v holds an MH state with cut c_v (node 0, the root: the current state,
 * cut T); expanding v creates an acceptance child carrying a suffix-resampling request whose cut
 * is drawn uniformly from {0..T-1}, and a rejection child that keeps v's state and cut; the request
 * joins this batch iff its cut <= c_v (Condition 1), else it is deferred.
 *   TAV_PREFETCH_BFS: breadth-first expansion until `budget` requests or an empty queue (a deferred
 *     acceptance child is created but not expanded; the rejection child is always queued).
 *   TAV_PREFETCH_PREDICTIVE: the selection of at most `budget` candidate nodes (depth < depth_cap,
 *     Condition 1 at the node and at every ancestor) maximising the predicted number of completed
 *     transitions (Equation 17: the sum of predicted reaching weights, Equation 11, with branch
 *     probability (1 + P(accept) - P(reject)) / 2, Equation 14, from a three-class logistic
 *     regression on the cut fraction c/T); the tree is the root and both children of each
 *     selected node.  The optimum of Equation 19.
 * Nodes are named by heap index (root 1, acceptance child 2h, rejection child 2h + 1) and listed in
 * ascending heap index (so parent < child); the cut of the acceptance child with heap index h is
 * floor(U * T) with U the top 53 bits, over 2^53, of SplitMix64 (Steele, Lea and Flood) at state
 * seed + h * 0x9E3779B97F4A7C15.  Requests are numbered in node order.  The output arrays feed
 * tav_presto_io (pf_parent, pf_is_accept, pf_request; request_cut = cut of each request).
 * Errors: NULL arrays, budget outside [1, 62], T or depth_cap < 1, capacity < 2 * budget + 1 or
 * outgrown, non-finite class weights (all host-checked). */
enum { TAV_PREFETCH_BFS = 0, TAV_PREFETCH_PREDICTIVE = 1 };

typedef struct tav_prefetch_params {
  int32_t T;           /* state length */
  int32_t budget;      /* N_pf: at most this many requests */
  int32_t depth_cap;   /* K' = K - k: only nodes of depth < K' are expanded */
  int32_t rule;        /* TAV_PREFETCH_BFS or TAV_PREFETCH_PREDICTIVE */
  uint64_t seed;       /* cut draws */
  float class_w[6];    /* (bias, slope) on c/T for the classes certain reject, certain accept, uncertain */
} tav_prefetch_params;

typedef struct tav_prefetch_out {
  int32_t capacity;               /* entries of the node arrays: 2 * budget + 1 suffices for the
                                     predictive rule; a BFS expansion whose request is deferred adds
                                     two nodes but no request, so BFS trees can be larger
                                     (TAV_ERR_BAD_SHAPE when the tree outgrows capacity) */
  int32_t num_nodes;              /* out */
  int32_t num_requests;           /* out */
  int32_t* parent;                /* [capacity] host arrays */
  uint8_t* is_accept;
  int32_t* request;               /* request id of an acceptance child in this batch, else -1 */
  int32_t* cut;                   /* cut of every node (the root: T) */
  int64_t* heap;                  /* [capacity] optional: heap index of every node */
  int32_t* request_cut;           /* [budget] optional: cut of every request */
  double predicted_transitions;   /* out: sum of predicted reaching weights of the expanded nodes */
} tav_prefetch_out;

tav_status tav_prefetch_build(const tav_prefetch_params* params, tav_prefetch_out* out);

/* After scoring (host only): epsilon-rounded branch probabilities h(v+) = 0 if A <= eps, 1 if
 * A >= 1 - eps, else A with A = exp(log_accept) (PreSTO Appendix C Equation 10), reaching weights
 * R(root) = 1, R(v+-) = R(v) h(v+-) (Equation 11) and the expected number of completed transitions
 * F = sum of R over the nodes whose acceptance child carries a request of this batch (Lemma 1,
 * Equation 12).  parent < child, node 0 the root; reach [num_nodes] optional.  eps in [0, 1/2). */
tav_status tav_prefetch_reach(int32_t num_nodes, const int32_t* parent, const uint8_t* is_accept,
                              const int32_t* request, int32_t num_requests, const float* log_accept,
                              float eps, double* reach, double* expected_transitions);

/* Draft-tree construction on the GPU (RheoSampling Section 2.1: EAGLE's expand-then-rerank;
 * Section 3.2 and Appendix C.1: the hybrid pool with the sampled token's proxy, the sparse draft,
 * global pruning with its tie-break).  B trees are built at once, one depth per tav_draft_expand
 * call (the drafter's forward pass on the selected parents happens between calls), then
 * tav_draft_prune writes the pruned trees in the layout tav_tree / tav_verify_io take.
 * Per parent: the drafter's bf16 logits z are truncated to their `support` largest entries (ties at
 * the edge to the smaller token ids); q = softmax(z) over the support ranks tokens (path score =
 * product of proxies); a hybrid pool takes the top lead_m tokens (proxy q), one token Y drawn from
 * the tail of softmax(z / temperature) off the leads with the parent's uniform (inverse CDF in
 * token-id order; proxy min{q(x_m), 1 - sum of the leads' q}, or q(x_1) + eps when lead_m = 0),
 * then the highest remaining tokens (proxy q); a plain pool takes the top `slots` tokens.  Depth d
 * expands the top min(expand_k, candidates of depth d - 1) candidates of depth d - 1 by score (ties:
 * smaller candidate id); depth 1 expands the root.  The prune keeps the `budget` candidates with the
 * highest scores (ties: shallower, then smaller id), numbered by (depth, id) after the root. */
enum { TAV_DRAFT_HYBRID_NONE = 0, TAV_DRAFT_HYBRID_FIRST = 1, TAV_DRAFT_HYBRID_ALL = 2 };

typedef struct tav_draft_params {
  int32_t num_seqs;     /* B */
  int32_t vocab;        /* V, a multiple of 8 (bf16 logits) */
  int32_t depth;        /* D in [1, 32] */
  int32_t expand_k;     /* parents expanded per depth, in [1, 64] */
  int32_t slots;        /* pool slots per parent, in [1, support] */
  int32_t lead_m;       /* hybrid pool: lead tokens, in [0, slots) */
  int32_t hybrid;       /* TAV_DRAFT_HYBRID_ALL, _FIRST (the rank-0 parent of each depth) or _NONE */
  int32_t support;      /* S in [slots, 128], <= V */
  int32_t budget;       /* R: nodes kept besides the root, <= the number of candidates */
  float temperature;    /* > 0: the sampled token's distribution is softmax(z / temperature) */
  float eps;            /* lead_m = 0: the sampled token's proxy is q(x_1) + eps */
} tav_draft_params;

/* Workspace bytes of a construction (host only).  Errors: parameters outside the ranges above,
 * more than 2048 candidates per tree. */
tav_status tav_draft_workspace_size(const tav_draft_params* p, size_t* bytes);

/* Depth d in [1, depth]: draft_logits [B, K_d, V] bf16 are the drafter's logits at the parents of
 * depth d (K_1 = 1: the root; then the parents this call's predecessor listed), uniforms [B, K_d]
 * the parents' uniforms in [0, 1).  frontier_out [B, expand_k] (optional): the candidate ids of
 * the parents of depth d + 1 in rank order, -1 padded -- the nodes the drafter runs on next.
 * Calls for one construction are issued in depth order on one stream with one workspace.  Device
 * errors: non-finite draft logits (TAV_DEV_NONFINITE_LOGITS), TAV_DEV_DRAFT_TIES. */
tav_status tav_draft_expand(const tav_draft_params* p, int32_t d, const void* draft_logits, const float* uniforms,
                            int32_t* frontier_out, void* workspace, size_t workspace_bytes, void* stream);

/* After depth D: the pruned trees, budget + 1 nodes per tree (node 0 the root), rows b * (budget
 * + 1) ...: parent (-1 at roots, sequence-local), token (-1 at roots), sampled, cand_id (optional:
 * the candidate id of each node), draft_row (the node's own index if its sampled child was kept,
 * else -1) and the draft rows draft_idx / draft_val [B * (budget + 1), support] (support ids
 * ascending and q~, written for the rows draft_row names) -- tav_verify_io's sparse draft rows with
 * num_draft_rows = B * (budget + 1). */
tav_status tav_draft_prune(const tav_draft_params* p, int32_t* parent, int32_t* token, uint8_t* sampled,
                           int32_t* cand_id, int32_t* draft_row, int32_t* draft_idx, float* draft_val,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace the calls below need for this problem (host only; no HIP
 * call).  presto may be NULL.  Errors: NULL pointer, bad shape. */
tav_status tav_workspace_size(const tav_problem* prob, const tav_presto_io* presto, size_t* bytes);

/* Tree preparation: validation, depth, position, ancestor masks, chain flags
 * (Progressive Tree Drafting, Section 3.1).  Also clears the status word. */
tav_status tav_tree_prep(const tav_problem* prob, const tav_tree* tree, const tav_tree_out* out,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Tree-masked attention (prep + split-KV prefix/tail attention + merge). */
tav_status tav_tree_attention(const tav_problem* prob, const tav_tree* tree, const tav_attn_io* io,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Verification (vocabulary statistics + walk) of every sequence.  Clears the
 * status word first. */
tav_status tav_tree_verify(const tav_problem* prob, const tav_tree* tree, const tav_verify_io* io,
                           void* workspace, size_t workspace_bytes, void* stream);

/* PreSTO log-acceptance of every request and the MH walk. */
tav_status tav_presto_accept(const tav_presto_io* io, void* workspace, size_t workspace_bytes,
                             void* stream);

/* The whole pass, on attn_stream: tree prep, attention, then (if verify != NULL) the
 * verification's vocabulary work and walk.  PreSTO (if presto != NULL) runs on verify_stream from the
 * start when that differs from attn_stream (attn_stream then waits for it before the call returns),
 * else on attn_stream.  tree_out may be NULL.  Returns after enqueueing; synchronising attn_stream
 * covers the whole pass. */
tav_status tav_tree_attn_verify(const tav_problem* prob, const tav_tree* tree,
                                const tav_attn_io* attn, const tav_verify_io* verify,
                                const tav_presto_io* presto, const tav_tree_out* tree_out,
                                void* workspace, size_t workspace_bytes,
                                void* attn_stream, void* verify_stream);

/* Bytes of the device array that serves as workspace of tav_tree_attn_verify_noalloc (64 MiB, one
 * array per GPU the library runs on, held until the process ends). */
#define TAV_NOALLOC_SCRATCH_BYTES (64u << 20)

/* The whole pass exactly as tav_tree_attn_verify, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation): the
 * workspace is the library's own device array of TAV_NOALLOC_SCRATCH_BYTES on the current GPU
 * instead of a caller buffer, and the call allocates nothing (no hipMalloc / hipFree, no
 * allocating library routine).  The caller still passes every input and output.
 *   status_out: optional device pointer; the call's device status word is copied there (on
 *     attn_stream, after the pass) -- the array itself is not exposed.
 * Errors: as tav_tree_attn_verify; TAV_ERR_WORKSPACE when tav_workspace_size() of the problem
 * exceeds TAV_NOALLOC_SCRATCH_BYTES (nothing enqueued).  The array's address is looked up on the
 * first call on each device.  Every call on one GPU uses that GPU's one array and the array keeps
 * the last call's contents (each call clears what must start at zero): calls that may overlap on
 * one GPU -- different streams without ordering, or several host threads -- race and must be
 * ordered by the caller. */
tav_status tav_tree_attn_verify_noalloc(const tav_problem* prob, const tav_tree* tree,
                                        const tav_attn_io* attn, const tav_verify_io* verify,
                                        const tav_presto_io* presto, const tav_tree_out* tree_out,
                                        uint32_t* status_out, void* attn_stream, void* verify_stream);

/* Waits for stream, then copies the device status word to *status_bits. */
tav_status tav_read_status(const void* workspace, void* stream, uint32_t* status_bits);

/* Optional timing of one kernel of the pass, for benchmarks (the only host state the library keeps
 * besides the per-thread error message and per-thread fork/join events of the two-stream call;
 * it is per calling host thread).  tav_kernel_timing(which) with
 * which = 1 records a pair of HIP events on the attention stream immediately before and after
 * every bf16 tree-attention kernel launch (not around the preparation or merge launches); with
 * which = 2 before every launch of the verification's vocabulary streaming kernel and after the
 * pick kernel that follows it, on the stream the verification runs on; which = 0 stops recording
 * and releases the events.
 * tav_kernel_timing_read waits for the recorded events, returns the summed elapsed milliseconds
 * and the number of launches recorded since the previous read or enable, and starts a new
 * record.  The events are timing-only (no system-scope fence when recorded).  They belong to the
 * device current at the first recording; recording on another device returns
 * TAV_ERR_INVALID_ARGUMENT, and so does a which outside 0..2.  The record belongs to the calling
 * host thread: only calls made on that thread are timed, and threads do not share it. */
tav_status tav_kernel_timing(int which);
tav_status tav_kernel_timing_read(double* total_ms, int32_t* launches);

/* Static description of a status code. */
const char* tav_status_string(tav_status s);

/* Message of the last error returned on the calling thread ("" if none). */
const char* tav_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TAV_H */
