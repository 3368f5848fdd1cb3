/*
 * tree_attn.h - C ABI of the MI355X (gfx950) split tree-verify attention library
 * (libtreeattn.so).
 *
 * What it computes.  In the verify step of tree speculative decoding the draft
 * tree's tokens are flattened into one sequence after the committed prefix.
 * Each tree token's attention is computed in two pieces: one over the committed
 * prefix, which needs no custom mask, and one among the tree tokens, which
 * needs the tree mask.  The two partial results are combined exactly by their
 * log-sum-exp (merge_attentions).  [pith.science review of arXiv 2508.08192,
 * "What carries the argument"; the merge of attention over disjoint KV chunks
 * is credited to Hydragen (Juravsky et al. 2024) in the pith.science verdict
 * record, pith_extraction.supporting_citations]
 *
 * Readings of what the pages leave open (all fixed here, for every call):
 *   - tree mask = ancestor-or-self: tree node i attends to tree node j iff j is
 *     i or an ancestor of i (SpecInfer tree verification);
 *   - every tree node attends to all prefix_lens[b] prefix tokens;
 *   - grouped-query attention: query head h reads KV head h / G, G = Hq / Hkv;
 *   - scores s = softmax_scale * dot(q, k), no positional encoding applied;
 *   - lse outputs are natural logarithms; a row with no visible key gets
 *     o = 0 and lse = -inf.
 *
 * Conventions shared by every entry point.
 *   - Every pointer argument except `shape` is a DEVICE pointer owned by the
 *     caller.  The library never allocates or frees device memory and never
 *     synchronises, except tree_attn_get_error (documented below).  All calls
 *     are asynchronous on `stream`.
 *   - All tensors are dense, row-major, contiguous, at least 16-byte aligned.
 *   - Element type of q, k_cache, v_cache, k_tree, v_tree and `out` is
 *     shape->dtype (bf16 = raw 16-bit patterns, or fp32).  Partial outputs
 *     (o_prefix, o_suffix, lse_*) are fp32.
 *   - Layouts (N = total_tree_nodes, Hq, Hkv, D = head_dim, 64-token blocks):
 *       q, out            [N, Hq, D]
 *       lse_out, lse_*    [N, Hq]            fp32
 *       o_prefix, o_suffix[N, Hq, D]         fp32
 *       k_cache, v_cache  [num_blocks, Hkv, 64, D]
 *       block_table       int32 [batch, max_blocks_per_seq]; token t of
 *                         sequence b is slot t % 64 of block block_table[b][t/64]
 *                         (PagedAttention layout, Kwon et al. 2023, named in the
 *                         same supporting_citations field as the scheme adapted
 *                         for tree attention)
 *       prefix_lens       int32 [batch]
 *       k_tree, v_tree    [N, Hkv, D]
 *       parents           int32 [N]; local index of the parent inside its own
 *                         sequence's tree, -1 for a root, parent[i] < i
 *       tree_offsets      int32 [batch + 1]; tree of sequence b is rows
 *                         [tree_offsets[b], tree_offsets[b+1]); tree_offsets[0]
 *                         = 0 and tree_offsets[batch] = N
 *       mask              uint64 [N, W], W = ceil(max_tree_nodes / 64) words per
 *                         node (W = 1 up to 64 nodes); bit j % 64 of word j / 64
 *                         of row tree_offsets[b] + i is set iff local node j is
 *                         i or an ancestor of i
 *   - Return codes report what the host can see: bad scalars, null or
 *     misaligned pointers, unsupported shapes, a workspace that is too small,
 *     launch failures.  Properties of device data (a bad parent array, a prefix
 *     length beyond max_prefix_len, a block id outside [0, num_blocks), bad
 *     tree_offsets) are checked by the kernels, which never read out of bounds
 *     because of them; they set a flag in the workspace that
 *     tree_attn_get_error reports.  Outputs of an affected sequence are then
 *     unspecified.
 *   - Thread safety: calls may come from any host thread.  Calls that run
 *     concurrently (different streams) must use different workspaces.  A
 *     call never needs the whole GPU to itself: the work items of one
 *     launch that meet to combine their partial results wait only for items
 *     that are already running, so concurrent calls, or other kernels
 *     holding some of the CUs, delay a call but cannot stall it.
 *   - Graph capture: after a first call of a shape outside any capture (it
 *     sets a kernel attribute once), every call issues only kernel launches,
 *     so a sequence of calls can be captured into a HIP graph and replayed
 *     with new data in the same buffers.
 */
#ifndef TREE_ATTN_H_
#define TREE_ATTN_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TA_OK = 0,
  TA_ERR_INVALID_ARG = 1,  /* bad scalar, null or misaligned pointer */
  TA_ERR_UNSUPPORTED = 2,  /* shape outside what the kernels implement */
  TA_ERR_BAD_TREE = 3,     /* device-detected: parent array or tree_offsets invalid */
  TA_ERR_WORKSPACE = 4,    /* workspace null or smaller than tree_attn_workspace_size */
  TA_ERR_HIP = 5,          /* a HIP runtime call or kernel launch failed */
  TA_ERR_BAD_PREFIX = 6,   /* device-detected: prefix length or block id out of range */
  TA_ERR_TIMEOUT = 7,      /* device-detected: a bounded cross-workgroup wait gave up */
  TA_ERR_NO_BLOCKS = 8,    /* device-detected: free list or block-table row too small */
  TA_ERR_SCRATCH = 9       /* the shape needs more workspace than tree_attn_verify_noalloc's
                              static scratch holds */
} ta_status;

typedef enum { TA_DTYPE_F32 = 0, TA_DTYPE_BF16 = 1 } ta_dtype;

/* Host-side description of one call.  Everything here is a host value; the
 * per-sequence data (prefix lengths, trees) stays on the device. */
typedef struct {
  int32_t batch;              /* B >= 1 (B <= 2048; and at most 2^18 groups:
                                 B * Hkv * ceil(max_tree_nodes * Hq / Hkv / 64)) */
  int32_t num_q_heads;        /* Hq, a multiple of num_kv_heads */
  int32_t num_kv_heads;       /* Hkv >= 1 */
  int32_t head_dim;           /* D in {64, 128} */
  int32_t block_size;         /* tokens per KV block; must be 64 */
  int32_t max_blocks_per_seq; /* row stride of block_table, >= 1 */
  int32_t max_tree_nodes;     /* upper bound on any sequence's tree size, 1..256 (up to
                                 64 nodes a tree takes one 64-bit mask word per node,
                                 beyond that ceil(T/64) words) */
  int32_t max_prefix_len;     /* upper bound on prefix_lens[b], 0..64*max_blocks_per_seq */
  int32_t total_tree_nodes;   /* N = tree_offsets[B] */
  int32_t num_blocks;         /* pool size: valid block ids are [0, num_blocks) */
  int32_t split_tokens;       /* prefix tokens per work item: 0 = library heuristic
                                 (short prefixes in one chunk per sequence: up to
                                 3 blocks for one sequence, 6 for a batch, 8 for
                                 a batch of 32 groups or more),
                                 else a positive multiple of 64 */
  float softmax_scale;        /* <= 0 selects 1/sqrt(head_dim) */
  ta_dtype dtype;             /* element type of q, caches, tree K/V and out */
} ta_shape;

/* Bytes of device workspace tree_attn_prefix / tree_attn_verify /
 * tree_attn_build_mask need for `shape` (0 if the shape is invalid).
 * A workspace must be zero-filled before its first use (tree_attn_workspace_init
 * does that).  A call that completes without a device-detected error leaves
 * the workspace's counters ready for the next call, so one workspace serves
 * call after call on one stream, whatever each call's shape (as long as the
 * workspace is large enough for it); after TA_ERR_TIMEOUT it must be
 * zero-filled again. */
size_t tree_attn_workspace_size(const ta_shape* shape);

/* Zero-fill a workspace with a kernel (no hipMemset, so graph capture is safe). */
ta_status tree_attn_workspace_init(void* ws, size_t ws_bytes, hipStream_t stream);

/* Build the ancestor-or-self mask words of every tree:
 * mask[i] = (parent[i] < 0 ? 0 : mask[parent[i]]) | (1 << i), per sequence,
 * over W = ceil(max_tree_nodes / 64) words per node (trees of up to 256 nodes;
 * one wave per tree up to 64 nodes, one 256-thread workgroup above).
 * Validates each parent (-1 or an earlier node of the same tree) and each tree
 * size (1..max_tree_nodes); a violation raises TA_ERR_BAD_TREE in the
 * workspace flag and that tree's words are zero.
 * [pith.science review, "What carries the argument": the draft-token piece
 * "needs the tree mask"] */
ta_status tree_attn_build_mask(const ta_shape* shape, const int32_t* parents,
                               const int32_t* tree_offsets, uint64_t* mask_out,
                               void* ws, size_t ws_bytes, hipStream_t stream);

/* Prefix pass: attention of every tree query over its sequence's whole
 * committed prefix (no mask), read through the block table.  Writes the
 * normalised output o_prefix and lse_prefix (fp32).  A sequence with
 * prefix_lens[b] == 0 gets o = 0, lse = -inf.
 * [pith.science review, "What carries the argument": query-to-prefix piece] */
ta_status tree_attn_prefix(const ta_shape* shape, const void* q, const void* k_cache,
                           const void* v_cache, const int32_t* block_table,
                           const int32_t* prefix_lens, const int32_t* tree_offsets,
                           float* o_prefix, float* lse_prefix, void* ws, size_t ws_bytes,
                           hipStream_t stream);

/* Suffix pass: attention of every tree query over the tree tokens whose bit is
 * set in its mask words (normally from tree_attn_build_mask; W words per node
 * as above).  Bits at or above the tree size are ignored.  Trees of more than
 * 64 nodes are scored in segments of 64 keys folded by their log-sum-exps.
 * Writes o_suffix, lse_suffix (fp32).
 * [pith.science review, "What carries the argument": draft-token piece] */
ta_status tree_attn_suffix(const ta_shape* shape, const void* q, const void* k_tree,
                           const void* v_tree, const uint64_t* mask,
                           const int32_t* tree_offsets, float* o_suffix, float* lse_suffix,
                           hipStream_t stream);

/* merge_attentions for two results over disjoint key sets, row by row:
 * lse = log(exp(lse_a) + exp(lse_b)),
 * out = exp(lse_a - lse) * o_a + exp(lse_b - lse) * o_b.
 * rows = N * Hq; o_* are fp32 [rows, head_dim]; out is out_dtype; lse_out fp32.
 * Both inputs -inf gives out = 0, lse = -inf.  `out` may alias o_a only when
 * out_dtype is fp32.
 * [pith.science verdict record, pith_extraction.supporting_citations, Juravsky
 * et al. 2024] */
ta_status tree_attn_merge(int64_t rows, int32_t head_dim, ta_dtype out_dtype,
                          const float* o_a, const float* lse_a, const float* o_b,
                          const float* lse_b, void* out, float* lse_out,
                          hipStream_t stream);

/* Fused verify: prefix pass + mask build + suffix pass + merge in one kernel
 * launch; for one sequence whose (KV head, row pass) groups have several
 * prefix chunks, all running at once (the 8k-context verify), in two launches
 * on `stream`: the attention kernel storing every chunk's partial result in
 * the workspace, then a combine kernel merging them (tree_attn_launch_info
 * mode 3).  Writes out (shape->dtype) and lse_out (fp32, may be NULL).  Trees
 * of up to 256 nodes (max_tree_nodes <= 256, else TA_ERR_UNSUPPORTED).  Up to
 * 64 nodes the tree rows sit in LDS beside the KV ring; larger trees stream
 * through the ring in 64-node segments after the last chunk's KV blocks,
 * under mask words the kernel builds in LDS.
 * [pith.science review, "What carries the argument"] */
ta_status tree_attn_verify(const ta_shape* shape, const void* q, const void* k_cache,
                           const void* v_cache, const int32_t* block_table,
                           const int32_t* prefix_lens, const void* k_tree,
                           const void* v_tree, const int32_t* parents,
                           const int32_t* tree_offsets, void* out, float* lse_out,
                           void* ws, size_t ws_bytes, hipStream_t stream);

/* Fused verify for the in-cache tree layout ("tree padding"): the tree K/V
 * rows of sequence b are not separate tensors but sit in the paged cache right
 * after its prefix, node i at position prefix_lens[b] + i (slot (P+i) % 64 of
 * block block_table[b][(P+i)/64]).  The prefix piece covers positions
 * [0, P) as in tree_attn_verify; the tree piece reads its rows through the
 * block table, so the tree K/V need no separate write.  Each table row must
 * cover P + T positions (a region of up to 5 blocks for 256 nodes); a region
 * block id outside [0, num_blocks) or a row too short raises
 * TA_ERR_BAD_PREFIX.  Same shape, workspace, outputs and tree sizes (up to 256
 * nodes) as tree_attn_verify.  [pith.science verdict record: desk editor letter (paged
 * KV with tree padding) and referee summary (paged/persistent KV-cache
 * handling for tree attention)] */
ta_status tree_attn_verify_incache(const ta_shape* shape, const void* q, const void* k_cache,
                                   const void* v_cache, const int32_t* block_table,
                                   const int32_t* prefix_lens, const int32_t* parents,
                                   const int32_t* tree_offsets, void* out, float* lse_out,
                                   void* ws, size_t ws_bytes, hipStream_t stream);

/* Commit for the in-cache layout: the accepted path (root first, as
 * tree_attn_accept_greedy writes it) is compacted in place -- position P + t
 * takes the row that was at P + accept_path[b][t], for every KV head -- and
 * prefix_lens[b] becomes P + accept_len[b].  No block is allocated (the tree
 * region's blocks are already in the table); rows past the new prefix are
 * left as they are and are no longer history.  A path that is not a root
 * path: TA_ERR_BAD_TREE; a region running past the table row or a region
 * block id out of range: TA_ERR_BAD_PREFIX; either way that sequence is left
 * as it was.  One kernel launch, one workgroup per sequence.  Only the
 * workspace header is used.  [same sources; fdeinterviews.com summary,
 * paragraph on hidden correctness obligations] */
ta_status tree_attn_commit_incache(const ta_shape* shape, const int32_t* parents,
                                   const int32_t* tree_offsets, const int32_t* accept_len,
                                   const int32_t* accept_path, void* k_cache, void* v_cache,
                                   const int32_t* block_table, int32_t* prefix_lens, void* ws,
                                   size_t ws_bytes, hipStream_t stream);

/* Greedy acceptance after verification, one sequence per wave.  For tree
 * node i of sequence b (local index), draft_tokens[i] is the token the node
 * stands for and target_argmax[i] the target model's greedy next token at it
 * (both int32 [N], packed like the tree rows).  A root is accepted; node i is
 * accepted iff its parent p is and draft_tokens[i] == target_argmax[p].  Trees
 * of up to 64 nodes take one wave each, larger ones (up to 256) one 256-thread
 * workgroup with multi-word ancestor sets.  The
 * accepted path ends at the deepest accepted node (the smallest index among
 * equally deep ones) and runs root first:
 *   accept_len[b]       number of path nodes (>= 1; 0 for an invalid tree)
 *   accept_path[b][t]   int32 [batch, max_tree_nodes], local node indices,
 *                       -1 after the path
 *   bonus_token[b]      target_argmax at the path's last node (-1 if invalid)
 * Every tree must have 1..max_tree_nodes nodes; a bad parent array or bad
 * tree_offsets raise TA_ERR_BAD_TREE in the workspace flag.  Only the
 * workspace header is used: any workspace of at least 768 bytes will do.
 * [the service commits an accepted path: fdeinterviews.com summary, opening
 * paragraph; greedy draft decoding: pith.science verdict record, referee
 * summary.  The pages print no acceptance rule; this is the plain greedy
 * reading.] */
ta_status tree_attn_accept_greedy(const ta_shape* shape, const int32_t* parents,
                                  const int32_t* tree_offsets, const int32_t* draft_tokens,
                                  const int32_t* target_argmax, int32_t* accept_len,
                                  int32_t* accept_path, int32_t* bonus_token, void* ws,
                                  size_t ws_bytes, hipStream_t stream);

/* Commit accepted paths into the paged cache.  For every sequence b with
 * P = prefix_lens[b] and A = accept_len[b] (0 <= A <= tree size; A = 0 commits
 * nothing), the K/V rows of tree nodes accept_path[b][0..A) (a root path, root
 * first, as tree_attn_accept_greedy writes it) go, for every KV head, to
 * prefix positions P .. P+A-1 (slot (P+t) % 64 of block block_table[b][(P+t)/64]),
 * and prefix_lens[b] becomes P + A.  No other cache slot is written: rejected
 * nodes leave no trace.  Blocks needed beyond the cdiv(P, 64) the sequence
 * holds are taken from the front of free_blocks (int32 [free_count], pool
 * block ids), sequences in batch order, and written into block_table;
 * *blocks_taken (device int32, may be NULL) receives how many were taken.
 * Device checks (workspace flag, first error wins):
 *   - a path that is not a root path of its tree, or bad tree_offsets:
 *     TA_ERR_BAD_TREE, that sequence is left as it was;
 *   - P outside [0, 64 * max_blocks_per_seq]: TA_ERR_BAD_PREFIX, likewise;
 *   - a block-table row too short for P + A, or more blocks needed than
 *     free_count: TA_ERR_NO_BLOCKS and nothing at all is committed;
 *   - a free-list entry outside [0, num_blocks): TA_ERR_BAD_PREFIX and
 *     nothing is committed; an entry of the sequence's own row outside it:
 *     TA_ERR_BAD_PREFIX, the rows bound for that block are not written.
 * Uses shape's batch, num_kv_heads, head_dim, dtype, max_blocks_per_seq,
 * max_tree_nodes, total_tree_nodes and num_blocks.  The workspace must hold at
 * least tree_attn_workspace_size(shape) bytes (its scratch area holds the
 * per-sequence plan; the counters are not touched).  Two kernel launches.
 * [fdeinterviews.com summary, opening paragraph and the paragraph on hidden
 * correctness obligations; pith.science verdict record, minor comment on
 * Section 3.3 (KV-cache bookkeeping rewound to the accepted tokens)] */
ta_status tree_attn_commit(const ta_shape* shape, const void* k_tree, const void* v_tree,
                           const int32_t* parents, const int32_t* tree_offsets,
                           const int32_t* accept_len, const int32_t* accept_path,
                           void* k_cache, void* v_cache, int32_t* block_table,
                           int32_t* prefix_lens, const int32_t* free_blocks, int32_t free_count,
                           int32_t* blocks_taken, void* ws, size_t ws_bytes,
                           hipStream_t stream);

/* tree_attn_verify without a caller workspace, for callers that cannot
 * allocate device memory: code under HIP-graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same inputs, outputs, semantics and
 * kernels as tree_attn_verify; the workspace is instead a static device array
 * of the library (32 MiB, one per GPU the library runs on, held until the
 * process ends; its address is taken once per device on the first call there).
 * The call allocates and frees nothing.  Shapes whose tree_attn_workspace_size
 * exceeds 32 MiB return TA_ERR_SCRATCH before anything is launched (e.g. a
 * batch of 256 long ragged sequences: use tree_attn_verify there).
 * device_status (device int32, may be NULL) receives the call's device-side
 * error code (TA_OK, TA_ERR_BAD_TREE, TA_ERR_BAD_PREFIX or TA_ERR_TIMEOUT)
 * when the call's kernels have run; a second small kernel on the stream
 * writes it, clears the flag and, after an error, clears the static array's
 * counters.  Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (two streams, two host threads) race and must not be
 * made; calls in order on one stream are fine. */
ta_status tree_attn_verify_noalloc(const ta_shape* shape, const void* q, const void* k_cache,
                                   const void* v_cache, const int32_t* block_table,
                                   const int32_t* prefix_lens, const void* k_tree,
                                   const void* v_tree, const int32_t* parents,
                                   const int32_t* tree_offsets, void* out, float* lse_out,
                                   int32_t* device_status, hipStream_t stream);

/* Synchronises `stream`, reads and clears the device error flag of workspace
 * `ws` and returns it (TA_OK if no kernel flagged anything).  This is the only
 * entry point that blocks the host. */
ta_status tree_attn_get_error(void* ws, hipStream_t stream);

/* Static description of a status code. */
const char* tree_attn_status_string(ta_status status);

/* Work-item size (prefix tokens per work item) the library would use for
 * `shape`; 0 if the shape is invalid.  For inspection and benchmarking. */
int32_t tree_attn_split_tokens(const ta_shape* shape);

/* How tree_attn_verify would launch for `shape` (host values only; no device
 * call beyond cached device attributes).  info (host int32 [4]) receives:
 *   info[0]  prefix tokens per work item (a multiple of 64; the kernel may
 *            pick another from the actual prefix lengths when info[3] is 2
 *            and split_tokens is 0: one chunk per sequence if the longest
 *            has at most 6 blocks (8 with 32 groups of sequence, KV head and
 *            row pass or more), else the smallest that fits the grid)
 *   info[1]  workgroups of the launch (one per CU at most)
 *   info[2]  bound on the work items (workspace partial slots)
 *   info[3]  0: every item runs in the first round and the chunks of a group
 *               split the final combine (they meet at a barrier, waiting only
 *               for chunks that have started);
 *            1: more items than workgroups: items are handed out by ticket
 *               and the last chunk of each group to arrive combines it alone;
 *            2: decided on the device from the actual prefix lengths (0 when
 *               the items fit the first round, else 1);
 *            3: one sequence, every item in the first round, more than one
 *               chunk a group: two launches on the stream, the attention
 *               kernel storing every chunk's partial and a combine kernel
 *               folding them (no chunk waits for another).
 * TA_ERR_INVALID_ARG for a null info; shape errors as tree_attn_verify. */
ta_status tree_attn_launch_info(const ta_shape* shape, int32_t* info);

#ifdef __cplusplus
}
#endif

#endif /* TREE_ATTN_H_ */
