/*
 * eagle3.h — C ABI of the MI355X (gfx950) EAGLE-3 speculative-decoding step.
 *
 * One step has five parts, each behind one call:
 *   eagle3_draft_tree   the EAGLE-3 head (fused 3d->d FC over three target taps,
 *                       [input_norm(e) ; hidden_norm(x)] into one decoder layer,
 *                       shared LM head) drafts a tree by top-k expansion
 *                       ("EAGLE-3: Engineering Implementation of LLM Inference
 *                       Acceleration", VIII-IX and XI.1-XI.2; EAGLE-2's dynamic
 *                       tree, VI.7 Draft Sequence);
 *   eagle3_verify_tree  one target pass over every tree node with tree-masked
 *                       attention at position prefix + depth ("Advanced
 *                       speculative decoding: tree drafts and EAGLE", Why trees,
 *                       Implementation: forward_with_mask);
 *   eagle3_accept       greedy longest-path acceptance, or sequential rejection
 *                       sampling with residual norm(max(0, p - q)) and a bonus
 *                       token ("EAGLE-3: Engineering Implementation ...", III.5,
 *                       X.3-X.6), over a chain or level by level over a tree
 *                       ("Advanced speculative decoding ...", Exercises);
 *   eagle3_compact_kv   the accepted nodes' K/V move to contiguous positions and
 *                       the next catch-up inputs are gathered ("Advanced
 *                       speculative decoding ...", Implementation, the note on
 *                       compacting KV slots).
 *
 * Conventions
 *   - Every pointer argument is a DEVICE pointer unless marked (host).
 *   - The caller allocates every buffer (weights, KV caches, workspace, I/O) and
 *     keeps it alive for the context's lifetime; the library borrows pointers,
 *     never frees them and never allocates device memory.
 *   - All calls are asynchronous on the context's stream, except where a
 *     function says it synchronises.  One context serves one stream and is not
 *     thread-safe; calls that overlap on one context race.
 *   - Element type "T" is the shape's storage dtype: float for EAGLE3_F32,
 *     bfloat16 (uint16 bits, round-to-nearest-even) for EAGLE3_BF16.
 *   - Linear weights W are [out_features, in_features] (y = x W^T): row-major
 *     for EAGLE3_F32, and for EAGLE3_BF16 in the packed slab layout that
 *     eagle3_pack_linear produces (the embedding table and the norm vectors
 *     are never packed).
 *   - Errors: synchronous argument checks return a nonzero eagle3_status and
 *     launch nothing.  Data-dependent faults found on the device (a capacity
 *     overflow, a malformed tree) set bits in the context's device status word
 *     (read by eagle3_device_status) and the affected sequence's work is
 *     skipped; no call traps or faults on such input.
 */
#ifndef EAGLE3_H
#define EAGLE3_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  EAGLE3_OK = 0,
  EAGLE3_EINVAL = 1,       /* bad argument: NULL, size out of range, bad shape */
  EAGLE3_ECAPACITY = 2,    /* request exceeds max_batch / max_rows / workspace */
  EAGLE3_EUNSUPPORTED = 3, /* valid but not supported (e.g. > 64 tree rows)     */
  EAGLE3_EHIP = 4          /* a HIP runtime call failed                         */
} eagle3_status;

/* Device status bits (eagle3_device_status). */
#define EAGLE3_DEV_KV_OVERFLOW   0x1  /* seq_len + rows exceeded the KV capacity  */
#define EAGLE3_DEV_BAD_TREE      0x2  /* parent index >= child index, or < 0      */
#define EAGLE3_DEV_BAD_TOKEN     0x4  /* token id outside [0, vocab)              */
#define EAGLE3_DEV_BAD_PATH      0x8  /* path length 0 or > depth + 1             */

enum { EAGLE3_F32 = 0, EAGLE3_BF16 = 1 };
enum { EAGLE3_GREEDY_TREE = 0, EAGLE3_SAMPLE_CHAIN = 1, EAGLE3_SAMPLE_TREE = 2 };
enum { EAGLE3_LM_ALL = 0, EAGLE3_LM_LAST = 1, EAGLE3_LM_NONE = 2 };

/* LLaMA-shaped target (also the draft layer's head layout: Hq, Hkv, hd, ffn). */
typedef struct {
  int32_t n_layers, d_model, n_heads, n_kv_heads, head_dim, ffn, vocab;  /* head_dim % 4 == 0, <= 256 */
  float rope_theta;   /* rotate-half RoPE, inverse frequencies theta^(-2i/hd)      */
  float rms_eps;      /* RMSNorm epsilon                                          */
  int32_t dtype;      /* EAGLE3_F32 or EAGLE3_BF16: weights, activations, KV, aux */
  int32_t taps[3];    /* residual stream entering 0-indexed layer taps[i], i.e.
                         HF hidden_states[taps[i]] ("EAGLE-3: Engineering ...",
                         IX.1-IX.3); concatenated as [l ; m ; h]                 */
  int32_t draft_vocab; /* 0: the draft head shares the target's full-vocabulary
                          LM head; else V_d in [topk, vocab]: the draft owns a head
                          over V_d ids mapped to target ids by d2t ("EAGLE-3:
                          Engineering ...", VIII.6).  Draft top-k, scores and
                          draws are over the draft ids; trees hold target ids;
                          sampled chains return q scattered into the target
                          vocabulary (zero off d2t), so p and q share a support
                          (X.2).                                                   */
} eagle3_shape;

/* Draft policy.  GREEDY_TREE: dynamic tree of `depth` levels, top-`topk` per
 * expansion, `n_nodes` kept (root excluded), ranked by cumulative draft
 * log-probability.  SAMPLE_CHAIN: chain of `depth` drafts each drawn from
 * q = softmax(draft logits / temperature) (or its argmax when draft_greedy);
 * requires topk == 1 and n_nodes == depth.  SAMPLE_TREE: the GREEDY_TREE
 * draft, accepted by level-by-level rejection sampling at `temperature` > 0
 * ("Advanced speculative decoding: tree drafts and EAGLE", Exercises, trees
 * under sampling). */
typedef struct {
  int32_t mode, depth, topk, n_nodes;
  float temperature;
  int32_t draft_greedy;
} eagle3_spec_cfg;

typedef struct {
  const void *attn_norm;           /* [d]                 */
  const void *wq, *wk, *wv;        /* [Hq*hd, d], [Hkv*hd, d], [Hkv*hd, d] */
  const void *wo;                  /* [d, Hq*hd]          */
  const void *ffn_norm;            /* [d]                 */
  const void *w_gate, *w_up;       /* [ffn, d]            */
  const void *w_down;              /* [d, ffn]            */
} eagle3_layer_weights;

typedef struct {
  const void *embed;                    /* [V, d], shared with the draft head       */
  const eagle3_layer_weights *layers;   /* (host) array [n_layers], copied at create */
  const void *final_norm;               /* [d]                                      */
  const void *lm_head;                  /* [V, d], shared with the draft head       */
} eagle3_target_weights;

/* EAGLE-3 head ("EAGLE-3: Engineering ...", VIII.1-VIII.5, IX.5). */
typedef struct {
  const void *fc;                  /* [d, 3d]  fusion FC, bias-free         */
  const void *input_norm;          /* [d]      RMSNorm of the embedding e   */
  const void *hidden_norm;         /* [d]      RMSNorm of the feature x     */
  const void *wq, *wk, *wv;        /* [Hq*hd, 2d], [Hkv*hd, 2d], [Hkv*hd, 2d] */
  const void *wo;                  /* [d, Hq*hd]                            */
  const void *post_norm;           /* [d]                                   */
  const void *w_gate, *w_up;       /* [ffn, d]                              */
  const void *w_down;              /* [d, ffn]                              */
  const void *final_norm;          /* [d]      norm before the head         */
  const void *lm_head;             /* [draft_vocab, d] the draft-owned head (draft_vocab > 0; NULL otherwise) */
  const int32_t *d2t;              /* [draft_vocab] strictly ascending target ids in [0, vocab) (draft_vocab > 0;
                                      NULL otherwise); checked at create: a violation raises BAD_TOKEN */
} eagle3_head_weights;

typedef struct eagle3_ctx eagle3_ctx;

/* Bytes of the two KV caches for max_batch sequences of max_seq slots.
 *   target: [n_layers][2 (K,V)][max_batch][Hkv][max_seq][hd] of T
 *   draft : [2 (K,V)][max_batch][Hkv][max_seq][hd] of T
 * A sequence needs max_seq >= committed length + n_nodes + 1 (target) and
 * >= committed length + (depth - 1) * topk (draft). */
eagle3_status eagle3_kv_bytes(const eagle3_shape *shape, int32_t max_batch, int32_t max_seq,
                              size_t *target_bytes /* host */, size_t *draft_bytes /* host */);

/* Workspace bytes for calls of at most max_batch sequences and max_rows rows
 * (B * rows of one verify, B * (depth+1) catch-up rows, or one prefill chunk). */
eagle3_status eagle3_workspace_bytes(const eagle3_shape *shape, const eagle3_spec_cfg *cfg,
                                     int32_t max_batch, int32_t max_rows, int32_t max_seq,
                                     size_t *bytes /* host */);

/* Create a context.  All pointers are borrowed.  `stream` is a hipStream_t
 * (NULL = the null stream).  Returns EINVAL for an inconsistent shape or cfg
 * (among them a tree of more nodes than its topk + (depth - 1) * topk^2
 * candidates) and EUNSUPPORTED for n_nodes + 1 > 64 or (depth - 1) * topk > 64. */
eagle3_status eagle3_create(const eagle3_shape *shape /* host */, const eagle3_spec_cfg *cfg /* host */,
                            const eagle3_target_weights *target /* host struct */,
                            const eagle3_head_weights *head /* host struct */,
                            int32_t max_batch, int32_t max_rows, int32_t max_seq,
                            void *workspace, size_t workspace_bytes,
                            void *kv_target, void *kv_draft, void *stream,
                            eagle3_ctx **out /* host */);
eagle3_status eagle3_destroy(eagle3_ctx *ctx);

/* Paged KV cache ("Speculative Decoding (EAGLE3) in the vLLM Neuron
 * Framework", The propose() Method: a position's cache slot comes from its
 * sequence's block table).  Position pos of context sequence s lives in block
 * block_table[s * blocks_per_seq + pos / block_size] at offset
 * pos % block_size; every call of the context (prefill, draft, verify,
 * compaction) reads and writes K/V through the table.  Pools:
 *   target: [n_layers][2 (K,V)][n_blocks][Hkv][block_size][hd] of T
 *   draft : [2 (K,V)][n_blocks][Hkv][block_size][hd] of T
 * (the draft layer's cache uses the same table).  block_size is a power of
 * two >= 64, so one 64-key attention tile never spans two blocks.  The table
 * is caller-owned device memory, read at every launch (it may change between
 * steps; a graph replay sees its current contents): the caller allocates
 * blocks for every position a call touches (committed + n_nodes + 1 for the
 * target, committed + (depth - 1) * topk for the draft).  Entries outside
 * [0, n_blocks) are never dereferenced: a write through one is dropped and
 * raises EAGLE3_DEV_KV_OVERFLOW, a read is clamped into the pool. */
typedef struct {
  int32_t block_size;           /* positions per block: a power of two, >= 64 */
  int32_t n_blocks;             /* blocks in each pool */
  int32_t blocks_per_seq;       /* table entries per sequence; the logical capacity is blocks_per_seq * block_size */
  const int32_t *block_table;   /* device [max_batch, blocks_per_seq] */
} eagle3_kv_pages;

/* Bytes of the two paged pools. */
eagle3_status eagle3_paged_kv_bytes(const eagle3_shape *shape, int32_t block_size, int32_t n_blocks,
                                    size_t *target_bytes /* host */, size_t *draft_bytes /* host */);

/* eagle3_create for a paged cache: max_seq is pages->blocks_per_seq *
 * pages->block_size; kv_target / kv_draft are the pools above.  EINVAL for a
 * block size that is not a power of two >= 64 or sizes < 1. */
eagle3_status eagle3_create_paged(const eagle3_shape *shape /* host */, const eagle3_spec_cfg *cfg /* host */,
                                  const eagle3_target_weights *target /* host struct */,
                                  const eagle3_head_weights *head /* host struct */,
                                  int32_t max_batch, int32_t max_rows, const eagle3_kv_pages *pages /* host */,
                                  void *workspace, size_t workspace_bytes,
                                  void *kv_target, void *kv_draft, void *stream,
                                  eagle3_ctx **out /* host */);

/* Per-request draft lengths ("Speculative Decoding (EAGLE3) in the vLLM
 * Neuron Framework", SpecDecodeMetadata and Design Choices: requests verify
 * different numbers of drafts; one near its length limit verifies none and
 * decodes a single token).  n_draft: device [max_batch] int32, indexed by
 * context sequence, read at every later launch; NULL restores the full
 * budget.  Sequence s verifies the root and its first min(n_draft[s],
 * n_rows - 1) tree nodes (node order: parents precede children, so they form
 * a tree); for a chain, its first n_draft[s] drafts.  eagle3_verify_tree
 * with a mask (a draft's verify; prefill chunks are not affected) writes no
 * K/V for the other rows and their outputs are unspecified (the capacity
 * check covers only the active rows); eagle3_accept ignores them;
 * in chain mode the final draw still uses uniforms[b, depth].  Negative
 * values count as 0. */
eagle3_status eagle3_set_draft_lengths(eagle3_ctx *ctx, const int32_t *n_draft);

/* Index bookkeeping of one flat verify batch ("Speculative Decoding (EAGLE3)
 * in the vLLM Neuron Framework", SpecDecodeMetadata: Index Bookkeeping).
 * Request b owns flat input positions [cu[b-1], cu[b]) (cu[-1] = 0), the
 * last num_draft_tokens[b] of which are drafts; its logits are needed at the
 * nd + 1 positions that end it.  Outputs (device int32):
 *   cu_num_draft_tokens [batch]: running total of drafts;
 *   logits_indices [batch + total drafts]: those positions, request by request;
 *   target_logits_indices [total drafts]: entries of logits_indices that verify a draft;
 *   bonus_logits_indices [batch]: each request's last entry;
 *   draft_token_ids [total drafts] (NULL to skip): input_ids at the draft
 *     positions (input_ids may be NULL when it is skipped).
 * max_drafts is the capacity of target_logits_indices and draft_token_ids
 * (logits_indices holds batch + max_drafts).  One workgroup, any batch;
 * cu_num_scheduled_tokens and num_draft_tokens are device [batch].  A
 * request with nd < 0, an empty request, nd + 1 > its scheduled tokens, or a
 * total above max_drafts sets *error (device int32, NULL allowed) to 1 (else
 * 0); nd is then clamped into [0, scheduled - 1], entries past the
 * capacities are not written and the outputs are unspecified.
 * Asynchronous on `stream` (a hipStream_t; NULL = null stream). */
eagle3_status eagle3_spec_decode_metadata(int32_t batch, int32_t max_drafts, const int32_t *cu_num_scheduled_tokens,
                                          const int32_t *num_draft_tokens, const int32_t *input_ids,
                                          int32_t *cu_num_draft_tokens, int32_t *logits_indices,
                                          int32_t *target_logits_indices, int32_t *bonus_logits_indices,
                                          int32_t *draft_token_ids, int32_t *error, void *stream);

/* Convert one linear weight W [rows, cols] (row-major, out_features x
 * in_features) into the layout the context's GEMM kernels stream.
 *   EAGLE3_BF16: cols % 128 == 0 (else EUNSUPPORTED); dst receives
 *     R16 * cols elements, R16 = 16 ceil(rows / 16) (rows >= rows are zero
 *     padding).  The columns are cut into 128-wide slabs stored one after the
 *     other; slab t holds the 16-row blocks in order, each as four 16 x 32
 *     MFMA operand fragments of 64 lanes x 8 consecutive bf16 (lane l: row
 *     l % 16, columns 8 (l / 16) .. + 7 of the fragment).  Element (n, k)
 *     lands at index
 *     ((k / 128 * (R16 / 16) + n / 16) * 4 + (k % 128) / 32) * 512
 *       + ((n % 16) + 16 * ((k % 32) / 8)) * 8 + k % 8.
 *     This lets every weight load of the bf16 GEMMs be one contiguous 1 KiB
 *     fragment per wave, with all workgroups sweeping the same slab at once.
 *   EAGLE3_F32: a plain copy of rows * cols floats (fp32 weights are used
 *     row-major).
 * src and dst are caller-owned device buffers that must not overlap (EINVAL).
 * Asynchronous on `stream` (a hipStream_t; NULL = null stream).  Which
 * weights take this layout: wq, wk, wv, wo, w_gate, w_up, w_down of every
 * target layer and of the head, the head's fc, and the shared lm_head. */
eagle3_status eagle3_pack_linear(int32_t dtype, const void *src, void *dst, int32_t rows, int32_t cols,
                                 void *stream);

/* Target pass over n_rows new rows of each of `batch` sequences (cache slots
 * [seq_begin, seq_begin + batch)).  Row i of sequence b has token
 * tokens[b*n_rows+i] at RoPE position pos[b*n_rows+i] (pos NULL: seq_lens[b]+i)
 * and writes its K/V to slot seq_lens[b] + i.  It sees every committed slot
 * [0, seq_lens[b]) and, when mask is given, the rows whose bit is set in
 * mask[b*n_rows+i] (bit j = row j; tree mode, n_rows <= 64); mask NULL is the
 * causal chain (prefill): row i sees rows 0..i.  seq_lens is not changed.
 * Outputs (each may be NULL):
 *   logits [B*n_rows, V] float (lm_mode ALL) or [B, V] (LM_LAST: last row of
 *          each sequence); argmax / margin [B*n_rows] or [B] likewise: the
 *          largest logit's index (lowest index on ties) and top1 - top2;
 *   aux    [B*n_rows, 3d] of T: the storage-rounded residual entering each tap. */
eagle3_status eagle3_verify_tree(eagle3_ctx *ctx, int32_t seq_begin, int32_t batch,
                                 const int32_t *seq_lens, int32_t n_rows,
                                 const int32_t *tokens, const int32_t *pos, const uint64_t *mask,
                                 int32_t lm_mode, float *logits, int32_t *argmax, float *margin,
                                 void *aux);

/* Draft catch-up over committed positions without drafting (the draft's
 * prefill phase, "Speculative Decoding (EAGLE3) in the vLLM Neuron Framework",
 * The propose() Method).  For sequence b (slot seq_begin + b) the n_rows rows
 * are positions start[b] .. start[b]+n_rows-1; row j pairs aux[b*n_rows+j]
 * (target taps at that position, [3d] of T) with the embedding of
 * next_tok[b*n_rows+j] (the token at the following position).  Writes the
 * draft K/V of those positions. */
eagle3_status eagle3_draft_prefill(eagle3_ctx *ctx, int32_t seq_begin, int32_t batch,
                                   const int32_t *start, int32_t n_rows,
                                   const void *aux, const int32_t *next_tok);

/* Draft stage of one step for sequences [0, batch).
 *   seq_lens [B]   committed target length P_b; the root sits at position P_b.
 *   new_len  [B]   catch-up rows c_b in [1, depth+1]: positions P_b - c_b .. P_b - 1.
 *   aux_new  [B, depth+1, 3d] of T and next_tok [B, depth+1]: catch-up inputs
 *                  (row j of b valid for j < c_b); next_tok[b][c_b - 1] is the root.
 *   uniforms [B, depth] float in [0,1) (SAMPLE_CHAIN only, else NULL).
 * Outputs, [B, n_nodes+1] each, root first, nodes ordered by (depth, creation):
 *   tokens, parents (root -1), depth, pos (= P_b + depth), mask (bit j of row i
 *   set iff j is i or an ancestor of i), score (cumulative draft log-prob,
 *   root 0).  q [B, depth, V] float (SAMPLE_CHAIN: the draft distributions the
 *   drafts were drawn from; else NULL). */
eagle3_status eagle3_draft_tree(eagle3_ctx *ctx, int32_t batch, const int32_t *seq_lens,
                                const int32_t *new_len, const void *aux_new, const int32_t *next_tok,
                                const float *uniforms,
                                int32_t *tokens, int32_t *parents, int32_t *depth, int32_t *pos,
                                uint64_t *mask, float *score, float *q);

/* Residual stream of every later eagle3_verify_tree call ("Advanced
 * speculative decoding: tree drafts and EAGLE", Implementation: the target
 * pass over the tree rows; "EAGLE-3: Engineering ...", IX.1: hidden_states[i]
 * is the stream entering decoder layer i).  buf: device float [n_layers + 1,
 * R, d] with R = batch * n_rows of the call: entry l is the fp32 residual
 * entering layer l (entry 0 the embedding rows), entry n_layers the stream
 * leaving the last layer (the final norm's input).  The caller sizes it for
 * the calls it makes.  NULL stops the copies.  A parity output: the pass
 * never reads it; the copies run on the context's stream as the pass goes. */
eagle3_status eagle3_set_hidden_out(eagle3_ctx *ctx, float *buf);

/* Draft logits of every later eagle3_draft_tree call ("EAGLE-3: Engineering
 * Implementation ...", VIII.5-VIII.6: the draft head's LM-head output, the
 * distribution the tree is ranked and drawn from).  table: device float
 * [max_batch, 1 + E, V_d] (V_d = draft_vocab, or vocab when the head is
 * shared; E = (depth - 1) * topk for trees, depth - 1 for a sampled chain),
 * laid out as eagle3_tree_from_logits reads it: row 0 of sequence b is the
 * root's draft row (the last catch-up row's logits), row 1 + r expansion row
 * r in creation order (trees: depth-major, frontier rank within a depth;
 * chains: the row that drew draft r + 2).  Rows of a sequence the call does
 * not reach keep their old contents.  NULL stops the copies.  The copies are
 * launched on the context's stream right after each LM-head pass, so a
 * captured step writes them on every replay.  This is a parity output: the
 * step itself never reads it. */
eagle3_status eagle3_set_draft_logits_out(eagle3_ctx *ctx, float *table);

/* Tree construction alone, from given draft logits (no draft model): the same
 * kernels as eagle3_draft_tree with logits_table [B, 1 + (depth-1)*topk, V_d]
 * float (V_d = draft_vocab, or vocab when the head is shared), where row 0 is
 * the root's draft row and row 1 + r is expansion row r
 * (expansion rows are numbered in creation order across depths).  roots [B].
 * Outputs as eagle3_draft_tree. */
eagle3_status eagle3_tree_from_logits(eagle3_ctx *ctx, int32_t batch, const int32_t *roots,
                                      const int32_t *seq_lens, const float *logits_table,
                                      const float *uniforms,
                                      int32_t *tokens, int32_t *parents, int32_t *depth, int32_t *pos,
                                      uint64_t *mask, float *score, float *q);

/* Acceptance over trees of n_rows = n_nodes + 1 rows per sequence.
 *   GREEDY_TREE: argmax [B, n_rows] (target argmax per tree row); logits, q,
 *                uniforms unused (NULL).
 *   SAMPLE_CHAIN: logits [B, n_rows, V] target logits; q [B, depth, V];
 *                uniforms [B, depth+1]: uniforms[b][i] decides draft i+1,
 *                uniforms[b][depth] drives the one residual or bonus draw.
 *   SAMPLE_TREE: logits [B, n_rows, V] target logits (p = softmax(logits /
 *                temperature)); parents as from eagle3_draft_tree; q unused;
 *                uniforms [B, depth*topk + 1] in [0, 1).  From the root, the
 *                current node's children are tested in row order: child i (a
 *                top-k pick, so its draft distribution is the point mass at
 *                its token x) is accepted iff u < p'(x), p' the node's
 *                residual, with u = uniforms[b][d*topk + i] (d = the node's
 *                depth); a rejection removes x from p'.  An accepted child
 *                becomes the current node; when every child is rejected, or
 *                the node has none, next_root is drawn from the residual with
 *                uniforms[b][depth*topk] and the walk ends.  Decisions use the
 *                samplers' fixed point: W_v = floor(p(v) * 2^48), accept iff
 *                floor(u * S) < W_x with S the integer mass not yet removed.
 *                A malformed tree or token raises BAD_TREE / BAD_TOKEN.
 * Outputs: path [B, depth+1] (tree row indices, root first, -1 padded),
 * path_len [B], next_root [B], emitted [B, depth+1] (committed tokens, -1
 * padded; may be NULL). */
eagle3_status eagle3_accept(eagle3_ctx *ctx, int32_t batch, int32_t n_rows,
                            const int32_t *tokens, const int32_t *parents, const int32_t *argmax,
                            const float *logits, const float *q, const float *uniforms,
                            int32_t *path, int32_t *path_len, int32_t *next_root, int32_t *emitted);

/* Compaction after acceptance.  For sequence b and j < path_len[b]: target
 * K/V of slot seq_lens[b] + path[b][j] moves to slot seq_lens[b] + j in every
 * layer and KV head (all sources are read before any destination is written).
 * Then aux_new[b][j] = aux_tree[b][path[b][j]], next_tok[b][j] =
 * tokens[b][path[b][j+1]] (next_root[b] for the last), new_len[b] =
 * path_len[b] and seq_lens[b] += path_len[b].  The draft cache needs no move:
 * its speculative entries are simply overwritten by the next step.
 *   aux_tree [B, n_rows, 3d] of T (from eagle3_verify_tree); aux_new
 *   [B, depth+1, 3d] of T; next_tok [B, depth+1]; new_len [B].
 *   src_dst [B, depth+1, 2] int32 or NULL: the moves of sequence b as
 *   (source position, destination position) pairs, i.e. (P + path[b][j],
 *   P + j) with P the committed length before the call, for j < path_len[b];
 *   (-1, -1) after them and for every j of a sequence whose path is malformed
 *   (which moves nothing and raises EAGLE3_DEV_BAD_PATH).  These are the
 *   index lists of the page's cache update over the accepted path. */
eagle3_status eagle3_compact_kv(eagle3_ctx *ctx, int32_t batch, int32_t *seq_lens, int32_t n_rows,
                                const int32_t *path, const int32_t *path_len, const int32_t *tokens,
                                const int32_t *next_root, const void *aux_tree,
                                void *aux_new, int32_t *next_tok, int32_t *new_len, int32_t *src_dst);

/* Rebind the context to another stream (a hipStream_t; NULL = null stream).
 * Later calls launch there.  The step's calls (eagle3_draft_tree,
 * eagle3_verify_tree, eagle3_accept, eagle3_compact_kv) make no host
 * synchronisation, allocate nothing and keep every variable quantity in
 * device memory, so a step can be captured into a HIP graph on a capturing
 * stream and replayed; replays see the device state as it is at replay time. */
eagle3_status eagle3_set_stream(eagle3_ctx *ctx, void *stream);

/* One token per row from softmax(logits / temperature), drawn by the same
 * integer inverse CDF as the acceptance sampler (temperature > 0), or the
 * argmax (lowest index on ties) when temperature == 0.  logits [n, V] float,
 * uniforms [n] in [0, 1) (unused at temperature 0), tokens [n] out; n <= the
 * context's max_rows.  This is vanilla decoding's sampling step and the root
 * draw after a prefill. */
eagle3_status eagle3_sample(eagle3_ctx *ctx, int32_t n, const float *logits, float temperature,
                            const float *uniforms, int32_t *tokens);

/* Training-time-test attention forward ("EAGLE-3: Engineering Implementation
 * ...", VII.5 Attention Mask and the draft layer's forward_ttt): the draft
 * layer's attention while it is trained on its own predictions.  T positions
 * of one sequence; the native step's keys are attended causally (query i sees
 * native keys 0..i), and each of the S simulated steps adds one key per
 * position that only the query at that position sees (the diagonal); all
 * scores of a query share one softmax, scaled by 1/sqrt(head_dim).  Query head
 * h reads KV head h / (n_heads / n_kv_heads).  No context is needed.
 *   dtype: EAGLE3_F32 or EAGLE3_BF16 (every tensor); head_dim % 4 == 0, <= 256
 *   q, out [T, n_heads, head_dim]; k0, v0 [n_kv_heads, T, head_dim];
 *   ks, vs [S, n_kv_heads, T, head_dim] (S >= 0; NULL allowed when S == 0)
 *   ws: caller-owned device workspace of eagle3_ttt_workspace_bytes() bytes,
 *   256-byte aligned.  Asynchronous on `stream` (a hipStream_t; NULL = null
 *   stream).  Bad sizes or pointers return EAGLE3_EINVAL and launch nothing. */
eagle3_status eagle3_ttt_workspace_bytes(int32_t T, int32_t n_heads, int32_t head_dim, size_t *bytes /* host */);
eagle3_status eagle3_ttt_attention(int32_t dtype, int32_t T, int32_t S, int32_t n_heads, int32_t n_kv_heads,
                                   int32_t head_dim, const void *q, const void *k0, const void *v0, const void *ks,
                                   const void *vs, void *out, void *ws, size_t ws_bytes, void *stream);

/* eagle3_ttt_attention for callers that cannot allocate device memory: code
 * under HIP graph capture, serving loops and harnesses that forbid
 * allocation.  Same computation and arguments, without ws / ws_bytes: the
 * scratch is a fixed array of EAGLE3_TTT_STATIC_SCRATCH_BYTES inside the
 * library, one per GPU, held until the process ends.  The bf16 path at
 * head_dim 64 or 128 uses none of it; fp32 and other head sizes need
 * eagle3_ttt_workspace_bytes(T, n_heads, head_dim), and a call that needs
 * more than the array returns EAGLE3_ECAPACITY and launches nothing.  Nothing
 * must start at zero: every call writes all the scratch it reads.  Every call
 * on one GPU shares that GPU's array, so calls that overlap on one GPU (other
 * streams or threads) race; calls on one stream are ordered.  No device
 * memory is allocated or freed. */
#define EAGLE3_TTT_STATIC_SCRATCH_BYTES ((size_t)32 << 20)
eagle3_status eagle3_ttt_attention_static(int32_t dtype, int32_t T, int32_t S, int32_t n_heads, int32_t n_kv_heads,
                                          int32_t head_dim, const void *q, const void *k0, const void *v0,
                                          const void *ks, const void *vs, void *out, void *stream);

/* Human-readable name of a status code (static string). */
const char *eagle3_status_string(eagle3_status s);

/* Reads and clears the device status word; synchronises the context's stream. */
eagle3_status eagle3_device_status(eagle3_ctx *ctx, int32_t *flags /* host */);

/* Per-kernel timing.  eagle3_profile(ctx, 1) clears the counters and makes
 * every later launch of the weight-streaming GEMM and attention kernels record
 * a HIP event pair on the context's stream; eagle3_profile(ctx, 0) stops.
 * eagle3_profile_read synchronises the stream and returns, for kernel id
 * `kernel` (EAGLE3_PROF_*), the number of launches, their summed duration in
 * ms, and the summed algorithmic bytes (weights + activations + outputs each
 * read or written once) and flops of those launches. */
enum {
  EAGLE3_PROF_GEMM_M64 = 0,  /* MFMA GEMM, 64-row tiles (verify, prefill)     */
  EAGLE3_PROF_GEMM_M16 = 1,  /* MFMA GEMM, 16-row tiles (draft, last-row LM)  */
  EAGLE3_PROF_ATTN = 2,      /* tree-masked attention (all modes)             */
  EAGLE3_PROF_GEMM_BIG = 3,  /* MFMA GEMM, 128 x 128 tiles (more than 64 rows) */
  EAGLE3_PROF_COUNT = 4
};
eagle3_status eagle3_profile(eagle3_ctx *ctx, int32_t enable);
eagle3_status eagle3_profile_read(eagle3_ctx *ctx, int32_t kernel, int64_t *launches /* host */,
                                  double *total_ms /* host */, double *bytes /* host */,
                                  double *flops /* host */);

#ifdef __cplusplus
}
#endif
#endif /* EAGLE3_H */
