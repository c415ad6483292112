/*
 * psa.h - shared-prefix (prefix-tree) block-sparse attention on MI355X (gfx950).
 *
 * C ABI of libpsa.so.  Plain pointers and sizes only.  Every call returns a
 * psa_status; a failing call writes nothing the caller owns and launches nothing,
 * and psa_last_error() gives a detail string for the calling thread.  No exception
 * or abort crosses this boundary.
 *
 * What is computed (sources are web pages; each is named by its title):
 *
 *  - The mask.  unsloth "prefix_grouper_kernel.py", function _make_mask_mod and its
 *    docstring: q may attend to kv iff both are in the same group, kv <= q, and
 *    either kv is a prompt (prefix) token or q is a completion (suffix) token of the
 *    same completion as kv.  Prompt rows are therefore causal, and every completion
 *    row sees its whole prompt.  Pad tokens (negative group id) see nothing and are
 *    seen by nothing (same page, the comment above _pad_len).
 *  - The prefix tree.  Automodel PR #2564, "Changelog": the tree is carried as
 *    node_lengths and sample_paths; a token sees every token of its node's strict
 *    ancestors and the tokens of its own node at or before itself.
 *  - The attention.  unsloth "prefix_grouper_kernel.py", flex_shared_prefix_attention:
 *    Q/K/V are [T, heads, head_dim] (the page's [1, T, H, D] without the batch),
 *    K/V carry the KV-head count (GQA), the softmax scale defaults to 1/sqrt(head_dim).
 *    q head h reads kv head h / (hq / hkv).
 *  - The block sparsity.  Same page, module docstring: tiles that the mask empties
 *    are never computed.  A tile map classifies every (q-tile, kv-tile) pair as
 *    empty (0), partial (1) or full (2); kernels apply the per-element mask only on
 *    partial tiles.
 *
 * Layouts (all row-major, contiguous):
 *   q, o, dq, dout : [T, hq, d]      k, v, dk, dv : [T, hkv, d]
 *   lse            : [hq, T] float32, natural log; -inf on rows that see no key.
 * Element type: PSA_FP32 -> float, PSA_BF16 -> bfloat16 (raw 16-bit storage).
 * Outputs are overwritten in full, pad rows included (O = 0, LSE = -inf, grads 0).
 */
#ifndef PSA_H
#define PSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PSA_ABI_VERSION 6  /* 5: PSA_FP8_E4M3 forward; 6: psa_unfold_rows takes dst_bytes */

typedef enum {
  PSA_OK = 0,
  PSA_ERR_NULL = 1,         /* a required pointer is NULL                              */
  PSA_ERR_SHAPE = 2,        /* T, head counts or tile sizes out of range; hq % hkv != 0 */
  PSA_ERR_LAYOUT = 3,       /* metadata that defines no prefix forest (see the builders) */
  PSA_ERR_DTYPE = 4,        /* unknown psa_dtype                                        */
  PSA_ERR_UNSUPPORTED = 5,  /* head_dim / dtype combination not compiled                */
  PSA_ERR_MAP_MISMATCH = 6, /* map built for another T, tile shape or device            */
  PSA_ERR_WORKSPACE = 7,    /* workspace NULL or smaller than psa_bwd_workspace_size    */
  PSA_ERR_HIP = 8,          /* a HIP runtime call failed (text in psa_last_error)       */
  PSA_ERR_ALLOC = 9,        /* a device or host allocation failed                       */
  PSA_ERR_VALUE = 10        /* a scalar argument is invalid (e.g. non-finite scale)     */
} psa_status;

/* Element types.  PSA_FP8_E4M3 (OCP e4m3 Q, K, V; O written in bf16) is taken by
 * psa_fwd only, for forwards without gradient. */
typedef enum { PSA_FP32 = 0, PSA_BF16 = 1, PSA_FP8_E4M3 = 2 } psa_dtype;
typedef enum { PSA_PASS_FWD = 0, PSA_PASS_BWD = 1 } psa_pass;

/* Opaque, library-owned, immutable after it is built. */
typedef struct psa_tile_map psa_tile_map;

typedef struct {
  int64_t T;           /* tokens, pads included                                  */
  int32_t block_m;     /* q rows per tile                                         */
  int32_t block_n;     /* kv columns per tile                                     */
  int64_t n_qtiles;    /* ceil(T / block_m)                                       */
  int64_t n_ktiles;    /* ceil(T / block_n)                                       */
  int64_t nnz;         /* non-empty tiles                                         */
  int64_t n_full;      /* tiles whose every pair is kept                          */
  int64_t n_partial;   /* non-empty tiles that are not full                       */
  int32_t form;        /* PSA_FORM_INTERVAL or PSA_FORM_NODES (mask encoding)     */
  int32_t causal;      /* 1: kv <= q is part of the mask; 0: a bidirectional draft map */
} psa_tile_map_info;

/* Mask encodings a map can carry (psa_tile_map_info.form). */
#define PSA_FORM_INTERVAL 0 /* packed layouts: kv visible to q iff kv <= q < end[kv]    */
#define PSA_FORM_NODES 1    /* any layout: per-token node numbers (psa_tile_map_export_nodes) */

/* Build flags (the _ex builders). */
#define PSA_MAP_NODE_FORM 1 /* build the node form even where the interval form exists */
/* Flag of psa_build_tile_map_draft. */
#define PSA_DRAFT_CAUSAL 1 /* draft blocks attend causally within the block */

/* Library ABI version (PSA_ABI_VERSION of the build). */
int32_t psa_abi_version(void);
/* Static text for a status code. */
const char* psa_status_string(psa_status s);
/* Detail of the last failing call on this thread ("" if none). */
const char* psa_last_error(void);

/*
 * Tile shape (block_m, block_n) that psa_fwd (pass PSA_PASS_FWD) or psa_bwd
 * (PSA_PASS_BWD) needs its map built with, for this dtype and head_dim.
 * Errors: PSA_ERR_NULL, PSA_ERR_DTYPE, PSA_ERR_UNSUPPORTED.
 */
psa_status psa_tile_shape(psa_pass pass, psa_dtype dtype, int32_t d, int32_t* block_m,
                          int32_t* block_n);

/*
 * Build a tile map from per-token labels (device pointers, T entries each):
 *   group[t]     >= 0 group id, < 0 pad token;
 *   suffix[t]    completion id (ignored on prompt and pad tokens);
 *   is_prefix[t] 1 on prompt tokens, 0 on completion tokens (ignored on pads).
 * Any labelling is accepted; the mask is the rule above, token by token.  The packed
 * layout (reading of unsloth "prefix_grouper_kernel.py", build_seg_info_multigroup,
 * which always packs this way: each group one contiguous run, group ids increasing
 * from run to run, a group's prompt tokens before its completion tokens, each
 * completion one contiguous run with completion ids increasing within the group,
 * pads between groups or at either end) gets the interval form (one int per token);
 * every other labelling (interleaved groups or completions, prompt tokens after
 * completion tokens, ids out of order) gets the node form (three ints per token:
 * each token's node - its group's prompt, or one completion - numbered in
 * depth-first order, and each node's subtree range), built by a sort of the node
 * keys.  Both give the same mask; the node form costs one more classification pass
 * and reads two more ints per key on partial tiles.
 * 1 <= block_m, block_n <= 1024.  T may be 0 (an empty map).
 * Work is enqueued on `stream` (a hipStream_t, NULL = default); the call waits once
 * on that stream to size the sparse lists.  The map may be used on `stream` at once;
 * on another stream, after synchronising with `stream`.
 * Ownership: *out belongs to the caller until psa_tile_map_destroy.
 * Errors: PSA_ERR_NULL, PSA_ERR_SHAPE, PSA_ERR_HIP, PSA_ERR_ALLOC.
 */
psa_status psa_build_tile_map_tokens(int64_t T, const int32_t* group, const int32_t* suffix,
                                     const uint8_t* is_prefix, int32_t block_m,
                                     int32_t block_n, void* stream, psa_tile_map** out);
/* The same with flags (0 or PSA_MAP_NODE_FORM); PSA_ERR_VALUE for an unknown bit. */
psa_status psa_build_tile_map_tokens_ex(int64_t T, const int32_t* group, const int32_t* suffix,
                                        const uint8_t* is_prefix, int32_t block_m,
                                        int32_t block_n, int32_t flags, void* stream,
                                        psa_tile_map** out);

/*
 * Build a tile map from a prefix tree (host pointers):
 *   node_lengths[n_nodes]  tokens of each node; node n owns the n-th contiguous run;
 *   path_ptr[n_paths + 1], path_nodes[path_ptr[n_paths]]  sample path s lists node
 *   indices root -> leaf in path_nodes[path_ptr[s] .. path_ptr[s+1]).
 * Required (reading of Automodel PR #2564, whose fold emits a prompt before its
 * continuations): every node lies on a path; a node has one parent across all paths;
 * a parent comes before its children (a smaller node index), so every token a node
 * sees sits before it.  Otherwise PSA_ERR_LAYOUT.  Nodes in depth-first pre-order
 * (each subtree one contiguous run of nodes) get the interval form; any other order
 * (breadth-first, interleaved branches) the node form, numbered on the host.
 * Several roots pack several trees.  Zero-length nodes are allowed.
 * T >= sum(node_lengths); tokens past the sum are pads.
 * Same stream, ownership and error rules as psa_build_tile_map_tokens.
 */
psa_status psa_build_tile_map_tree(int64_t n_nodes, const int32_t* node_lengths,
                                   int64_t n_paths, const int32_t* path_ptr,
                                   const int32_t* path_nodes, int64_t T, int32_t block_m,
                                   int32_t block_n, void* stream, psa_tile_map** out);
/* The same with flags (0 or PSA_MAP_NODE_FORM); PSA_ERR_VALUE for an unknown bit. */
psa_status psa_build_tile_map_tree_ex(int64_t n_nodes, const int32_t* node_lengths,
                                      int64_t n_paths, const int32_t* path_ptr,
                                      const int32_t* path_nodes, int64_t T, int32_t block_m,
                                      int32_t block_n, int32_t flags, void* stream,
                                      psa_tile_map** out);

/*
 * Build a tile map for the packed-document draft mask of block-diffusion drafters
 * (Automodel PR #3023, PR description and the review comment listing the mask
 * builder's arguments; Model-Optimizer PR #2757, the commit note on the generation
 * mask).  The flat layout is the context, positions [0, ctx_len), then n_blocks
 * blocks of block_size draft tokens (block b's token j at ctx_len + b * block_size
 * + j), then pads up to T.  The queries that matter are the draft tokens: a draft
 * token of block b sees the context positions c < anchors[b] whose ctx_doc[c] equals
 * anchor_doc[b], and its own block's tokens (all of them; with PSA_DRAFT_CAUSAL only
 * those at or before itself).  A block with keep[b] == 0 sees nothing and is seen by
 * nothing; context rows and pads see nothing (O = 0, LSE = -inf).  The caller passes
 * Q, K, V for all T positions (context query rows are ignored).
 * Device pointers: anchors[n_blocks] int32 in [0, ctx_len] (else PSA_ERR_LAYOUT),
 * keep[n_blocks] uint8 (NULL: every block kept), ctx_doc[ctx_len] and
 * anchor_doc[n_blocks] int32 document ids (both NULL: one document; ignored when
 * there is no context or no block).  Needs
 * T >= ctx_len + n_blocks * block_size and (ctx_len + 1) * n_blocks <= 2^32.
 * The map takes the node form with causal = 0 unless PSA_DRAFT_CAUSAL is set.
 * Same stream and ownership rules as psa_build_tile_map_tokens.
 * Errors: PSA_ERR_NULL, PSA_ERR_SHAPE, PSA_ERR_LAYOUT, PSA_ERR_VALUE, PSA_ERR_HIP,
 * PSA_ERR_ALLOC.
 */
psa_status psa_build_tile_map_draft(int64_t ctx_len, int32_t block_size, int64_t n_blocks,
                                    const int32_t* anchors, const uint8_t* keep,
                                    const int32_t* ctx_doc, const int32_t* anchor_doc,
                                    int32_t flags, int64_t T, int32_t block_m, int32_t block_n,
                                    void* stream, psa_tile_map** out);

/* Sizes of a built map.  Errors: PSA_ERR_NULL. */
psa_status psa_tile_map_info_get(const psa_tile_map* map, psa_tile_map_info* out);

/*
 * Copy a map to host buffers (NULL arguments are skipped); waits for the map's
 * build stream.  Sizes: end[T] (int32: key t is visible to rows q with
 * t <= q < end[t]), kinds[n_qtiles * n_ktiles] (row-major, 0/1/2), row_ptr[n_qtiles+1],
 * col[nnz], kind[nnz] (CSR: per q-tile its kv-tiles ascending), col_ptr[n_ktiles+1],
 * row[nnz], kind_csc[nnz] (CSC: per kv-tile its q-tiles ascending).
 * end must be NULL for a node-form map.
 * Errors: PSA_ERR_NULL, PSA_ERR_HIP, PSA_ERR_VALUE (end of a node-form map).
 */
psa_status psa_tile_map_export(const psa_tile_map* map, int32_t* end, uint8_t* kinds,
                               int32_t* row_ptr, int32_t* col, uint8_t* kind,
                               int32_t* col_ptr, int32_t* row, uint8_t* kind_csc);

/*
 * Copy the mask encoding as nodes to host buffers of T int32 each (NULL skipped):
 * kv is visible to q iff kv <= q (only when the map is causal) and
 * lo[kv] <= key[q] < lo[kv] + w[kv].  For a
 * node-form map these are its arrays (key: the token's node number from 1, 0 on a
 * pad; [lo, lo + w): the numbers of the node's subtree, w = 0 on a pad); an
 * interval-form map is written as key = lo = t, w = end[t] - t.  Waits for the
 * build stream.  Errors: PSA_ERR_NULL, PSA_ERR_HIP.
 */
psa_status psa_tile_map_export_nodes(const psa_tile_map* map, int32_t* key, int32_t* lo,
                                     int32_t* w);

/* Free a map (NULL is a no-op).  Work that uses it must have completed. */
void psa_tile_map_destroy(psa_tile_map* map);

/*
 * Forward: O = softmax(scale * Q K^T masked) V per q head, and LSE.
 * Defined by unsloth "prefix_grouper_kernel.py": flex_shared_prefix_attention (the
 * call: Q, K, V and the block mask; GQA through enable_gqa; the default scale
 * 1/sqrt(head_dim) of _run_flex) with the mask of _make_mask_mod; its module docstring
 * (masked blocks are skipped) and the comment on the flash block sizes (a completion
 * row's prompt run and own run go through one softmax).  The result is the dense
 * masked softmax of that definition; the block skipping only leaves out tiles whose
 * every pair is masked.
 * Supported: d in {64, 128, 256} for PSA_FP32 and PSA_BF16 (and PSA_FP8_E4M3 here).
 * Device pointers: q, k, v (inputs), o, lse (outputs, fully overwritten).  lse may be
 * NULL for a forward whose LSE is not needed (no backward follows, e.g. the extra
 * no-grad log-prob passes of a policy-gradient step): then only O is written.
 * scale <= 0 selects 1/sqrt(d).  T must equal the map's T; the map's tile shape must
 * be psa_tile_shape(PSA_PASS_FWD, dtype, d).  With PSA_FP8_E4M3, q, k, v hold OCP
 * e4m3 bytes taken at face value (no per-tensor scale; fold one into `scale` for Q K^T
 * and into O afterwards for V), products accumulate in fp32, P is rounded to bf16 for
 * P V as in the bf16 path, and o is bf16.  Asynchronous on `stream`.
 * Errors: PSA_ERR_NULL, PSA_ERR_SHAPE, PSA_ERR_DTYPE, PSA_ERR_UNSUPPORTED,
 * PSA_ERR_MAP_MISMATCH, PSA_ERR_VALUE, PSA_ERR_HIP.
 */
psa_status psa_fwd(const psa_tile_map* map, psa_dtype dtype, int64_t T, int32_t hq,
                   int32_t hkv, int32_t d, float scale, const void* q, const void* k,
                   const void* v, void* o, float* lse, void* stream);

/* Bytes of device workspace psa_bwd needs for these sizes.  Errors as psa_fwd. */
psa_status psa_bwd_workspace_size(const psa_tile_map* map, psa_dtype dtype, int64_t T,
                                  int32_t hq, int32_t hkv, int32_t d, size_t* bytes);

/*
 * Backward (FlashAttention-2 style): dQ, dK, dV of sum(dO * O) given the forward's
 * O and LSE.  The pages give no backward of their own: the unsloth page's
 * flex_shared_prefix_attention is differentiated by autograd, so this is the exact
 * gradient of the forward above (the analytic softmax-attention gradient,
 * dS = P * (dP - rowsum(dO * O)), restricted to the kept pairs).  dK and dV sum over
 * the q heads that share a kv head (the gradient of enable_gqa).  Supported: d in
 * {64, 128, 256} for PSA_FP32 and PSA_BF16.  Device pointers:
 * q, k, v, o, lse, dout (inputs, element type `dtype`), dq, dk, dv (outputs, element
 * type `grad_dtype`, fully overwritten), workspace (caller-owned scratch of at least
 * psa_bwd_workspace_size bytes, contents undefined on entry and exit).
 * grad_dtype is PSA_FP32 (the fp32 accumulators as they are; with bf16 inputs this is
 * the form that meets the bf16 parity bar for any gradient magnitude) or `dtype`.
 * The map's tile shape must be psa_tile_shape(PSA_PASS_BWD, ...).  Asynchronous on
 * `stream`.  Errors: as psa_fwd, plus PSA_ERR_WORKSPACE; PSA_ERR_DTYPE for a
 * grad_dtype that is neither PSA_FP32 nor `dtype`.
 */
psa_status psa_bwd(const psa_tile_map* map, psa_dtype dtype, psa_dtype grad_dtype, int64_t T,
                   int32_t hq, int32_t hkv, int32_t d, float scale, const void* q,
                   const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * psa_bwd without a workspace argument and without any allocation, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  It runs what psa_bwd runs, with the workspace in
 * a fixed device array that the library holds on each GPU it runs on until the
 * process ends (looked up, not allocated, on a device's first call).  Limit: the
 * backward's workspace, 2 x T x hq x 4 bytes (each plane rounded up to 256 bytes),
 * must fit in 32 MiB (T x hq <= 4,194,240), else PSA_ERR_WORKSPACE before any launch.
 * Every call on one GPU uses that GPU's one array: calls that overlap on one GPU (on
 * different streams without ordering) race and must not be issued.  The array keeps
 * the last call's contents, every byte a call reads is written by that call first.
 * Arguments and other errors as psa_bwd.
 */
psa_status psa_bwd_noalloc(const psa_tile_map* map, psa_dtype dtype, psa_dtype grad_dtype,
                           int64_t T, int32_t hq, int32_t hkv, int32_t d, float scale,
                           const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           void* stream);

/*
 * The backward in stages, for callers that time or overlap them (psa_bwd runs all
 * three), with options.  flags is the OR of a nonzero set of stages:
 *   PSA_STAGE_PREPARE  -D = -rowsum(dO * O) and LSE in log2 units, into the workspace
 *                      (reads o, lse, dout);
 *   PSA_STAGE_DKDV     dK, dV (reads q, k, v, dout and the prepared workspace);
 *   PSA_STAGE_DQ       dQ (reads q, k, v, dout and the prepared workspace).
 * DKDV and DQ depend only on PREPARE, not on each other.  When PREPARE and DQ are
 * requested together (as psa_bwd does), the dQ kernel does the preparation of its own
 * rows (it holds dO for exactly those rows) and runs first, and DKDV, if requested,
 * runs after it; the results are those of the three stages run one by one, up to the
 * order of the fp32 sums that form D.  And optionally:
 *   PSA_BWD_SPLIT_PDS  carry P and dS into the dV, dK and dQ products as a pair of
 *                      bf16 fragments hi + lo (about 16 significant bits instead of
 *                      8, at two MFMAs per product instead of one).  Without it P
 *                      and dS are rounded to bf16 once before those products, as in
 *                      FlashAttention-2; psa_bwd runs without it.  No effect on fp32
 *                      inputs, whose products are fp32 throughout.
 * Arguments and errors as psa_bwd (pointers a requested stage does not read may be
 * NULL), plus PSA_ERR_VALUE for an empty stage set or an unknown bit.
 */
#define PSA_STAGE_PREPARE 1
#define PSA_STAGE_DKDV 2
#define PSA_STAGE_DQ 4
#define PSA_STAGE_ALL 7
#define PSA_BWD_SPLIT_PDS 16
psa_status psa_bwd_stages(const psa_tile_map* map, psa_dtype dtype, psa_dtype grad_dtype,
                          int64_t T, int32_t hq, int32_t hkv, int32_t d, float scale,
                          const void* q, const void* k, const void* v, const void* o,
                          const float* lse, const void* dout, void* dq, void* dk, void* dv,
                          void* workspace, size_t workspace_bytes, int32_t flags,
                          void* stream);

/*
 * Fold of rollout groups into the flat shared-prefix layout (Automodel PR #2564 page:
 * PR description and "Changelog", fold_shared_prefix_rollouts; the commit note on
 * pre-shifted labels).  Group g, one prompt and the completions sampled from it, is
 * stored once as [prompt_g | c_g0 | c_g1 | ...]; groups follow one another; positions
 * from the folded length up to T are pad tokens.
 *   n_groups; host tables: prompt_len[n_groups]; comp_ptr[n_groups + 1] (group g owns
 *     completions comp_ptr[g] .. comp_ptr[g+1]-1, comp_ptr[0] = 0); comp_len[n_comp],
 *     n_comp = comp_ptr[n_groups].  Lengths may be 0.
 *   device inputs: prompt_tok (int32, the prompts' tokens concatenated in group order),
 *     comp_tok (int32, the completions' tokens concatenated in completion order).
 *   T >= the folded length (sum of all lengths).
 *   device outputs, [T] each, fully written; NULL skips one (at least one is given):
 *     input_ids   the flat tokens (pad_id on pads);
 *     labels      pre-shifted next-token labels: the next flat token of the same group,
 *                 except ignore_index on the last token of every completion, on a
 *                 prompt's last token when the group has no completion token, and on
 *                 pads (a prompt's last token is labelled with the first token of the
 *                 group's first non-empty completion, its flat successor);
 *     position_ids  a prompt's tokens 0 .. P-1; a completion's P .. P+R-1 (each
 *                 completion continues its prompt as if alone); 0 on pads;
 *     group, suffix, is_prefix  the token-form input of psa_build_tile_map_tokens: group
 *                 g, suffix -1 and is_prefix 1 on prompt tokens, suffix = the global
 *                 completion index on completion tokens, -1 / -1 / 0 on pads.
 *   workspace: device scratch of psa_fold_workspace_size bytes (contents undefined on
 *     entry and exit; the call uploads its segment table there, on `stream`).
 * Asynchronous on `stream`.  Errors (nothing is launched): PSA_ERR_NULL, PSA_ERR_SHAPE (T
 * too short or out of range), PSA_ERR_LAYOUT (negative lengths, comp_ptr not starting
 * at 0 or decreasing), PSA_ERR_WORKSPACE, PSA_ERR_VALUE (a capturing stream),
 * PSA_ERR_HIP.
 */
psa_status psa_fold_workspace_size(int64_t n_groups, int64_t n_comp, size_t* bytes);
psa_status psa_fold_rollouts(int64_t n_groups, const int32_t* prompt_len,
                             const int32_t* comp_ptr, const int32_t* comp_len,
                             const int32_t* prompt_tok, const int32_t* comp_tok, int64_t T,
                             int32_t pad_id, int32_t ignore_index, int32_t* input_ids,
                             int32_t* labels, int32_t* position_ids, int32_t* group,
                             int32_t* suffix, uint8_t* is_prefix, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * Unfold: the rows of a folded per-token tensor (src, T rows of row_bytes bytes, the
 * layout psa_fold_rollouts writes for the same tables) gathered into the per-sample
 * layout, to hand per-token outputs or log-probabilities back to the samples: sample
 * (g, i) is [prompt_g | c_gi]; samples follow in completion order; dst receives
 * sum over completions of (P_g + R_gi) rows.  A group without completions gives no
 * sample.  row_bytes: a positive multiple of 4 (rows move as 16-byte words when
 * row_bytes, src and dst allow it).  Device pointers src, dst (4-byte aligned);
 * dst_bytes: the bytes dst holds (at least the unfolded rows times row_bytes, else
 * PSA_ERR_SHAPE); workspace as psa_fold_rollouts.  Asynchronous on `stream`.  Errors as
 * psa_fold_rollouts.
 *
 * Fold and unfold copy their segment table from library-owned pinned host memory to
 * the workspace on `stream`; they refuse a stream that is being captured into a graph
 * (PSA_ERR_VALUE), since a replay would copy that host memory again.
 */
psa_status psa_unfold_rows(int64_t n_groups, const int32_t* prompt_len,
                           const int32_t* comp_ptr, const int32_t* comp_len, int64_t T,
                           int64_t row_bytes, const void* src, void* dst, size_t dst_bytes,
                           void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PSA_H */
