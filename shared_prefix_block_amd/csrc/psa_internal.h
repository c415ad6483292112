// Internal declarations shared by the C ABI (api.cpp) and the HIP kernel files.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>
#include <vector>

#include "psa.h"

// The tile map: the per-token mask encoding plus the full/partial/empty
// classification of every (q-tile, kv-tile) pair, as a dense kinds matrix and as
// CSR / CSC lists.
//
// Two encodings of keep(q, kv):
//  - interval form (packed layouts): kv <= q < end[kv];
//  - node form (any layout): kv <= q and lo[kv] <= key[q] < lo[kv] + w[kv], where
//    key[t] is the pre-order number (from 1) of t's node in the prefix forest and
//    [lo, lo + w) the pre-order numbers of the node's subtree; pads have key 0 and
//    w 0, so they see nothing and are seen by nothing.
// A map that is not causal (draft blocks attending both ways) drops kv <= q: the
// ranges alone decide, and they already keep context keys before their queries.
constexpr int32_t kFormInterval = 0, kFormNodes = 1;
struct psa_tile_map {
  int64_t T = 0;
  int32_t bm = 0, bn = 0;
  int64_t nq = 0, nk = 0;
  int64_t nnz = 0, n_full = 0, n_partial = 0;
  int32_t form = kFormInterval;
  int32_t causal = 1;  // 0: node form without the kv <= q conjunct
  int device = 0;
  hipStream_t stream = nullptr;  // build stream (export waits on it; buffers freed on it)
  size_t buf1_bytes = 0, buf2_bytes = 0, buf3_bytes = 0;  // sizes of the device buffers
  hipEvent_t ev1 = nullptr, ev2 = nullptr, ev3 = nullptr;  // their reuse events

  // node form (buf3): key | lo | w, T int32 each
  void* buf3 = nullptr;
  int32_t* nkey = nullptr;
  int32_t* nlo = nullptr;
  int32_t* nw = nullptr;

  // phase-1 allocation (sized before the sync)
  void* buf1 = nullptr;
  int32_t* end = nullptr;      // [T]      key t visible to rows q in [t, end[t])
  uint8_t* kinds = nullptr;    // [nq*nk]  0 empty, 1 partial, 2 full (row-major)
  int32_t* row_ptr = nullptr;  // [nq+1]
  int32_t* col_ptr = nullptr;  // [nk+1]
  // phase-2 allocation (sized after the sync)
  void* buf2 = nullptr;
  int32_t* col = nullptr;       // [nnz] CSR kv-tile index
  uint8_t* kind = nullptr;      // [nnz] CSR kind
  int32_t* row = nullptr;       // [nnz] CSC q-tile index
  uint8_t* kind_csc = nullptr;  // [nnz] CSC kind
  int32_t* qorder = nullptr;    // [nq]  q-tiles by descending CSR row length
  int32_t* korder = nullptr;    // [nk]  kv-tiles by descending CSC column length
};

// Error helpers (api.cpp)
psa_status psa_set_error(psa_status s, const std::string& msg);
psa_status psa_hip_error(hipError_t e, const char* what);

// ---------------------------------------------------------------------------
// tilemap.hip
// ---------------------------------------------------------------------------
// Zero the pointer arrays' counts and info (info[3], the first layout error, = -1).
hipError_t launch_map_init(int64_t nk, int32_t* row_ptr, int32_t* col_ptr, int64_t* info,
                           hipStream_t stream);
// Per-token interval ends from labels.  info[3] receives the first layout error as
// position * 8 + code (codes 1..4), or stays -1.  scratch: tokens_scratch_ints(T) ints.
int64_t tokens_scratch_ints(int64_t T);
hipError_t launch_tokens_end(int64_t T, const int32_t* group, const int32_t* suffix,
                             const uint8_t* is_prefix, int32_t* end, int32_t* scratch,
                             int64_t* info, hipStream_t stream);
// Per-token interval ends from a per-node table (node token start, node subtree end).
hipError_t launch_tree_end(int64_t T, int64_t n_nodes, const int64_t* node_start,
                           const int64_t* node_subtree_end, int64_t t_real, int32_t* end,
                           hipStream_t stream);
// Node form from labels: key / lo / w per token (see psa_tile_map).  Nodes are the
// groups' prompts and completions, numbered in the order of (group id, prompt first,
// then completion ids).  scratch: tokens_nodes_scratch_bytes(T) bytes.
size_t tokens_nodes_scratch_bytes(int64_t T);
hipError_t launch_tokens_nodes(int64_t T, const int32_t* group, const int32_t* suffix,
                               const uint8_t* is_prefix, int32_t* key, int32_t* lo,
                               int32_t* w, void* scratch, size_t scratch_bytes,
                               hipStream_t stream);
// Node form from a per-node table (node token start, pre-order number, subtree size).
hipError_t launch_tree_nodes(int64_t T, int64_t n_nodes, const int64_t* node_start,
                             const int64_t* node_pre, const int64_t* node_size, int64_t t_real,
                             int32_t* key, int32_t* lo, int32_t* w, hipStream_t stream);
// Classification + counts + pointer scans (after launch_map_init).  info (device,
// 8 x int64) receives nnz, n_full, n_partial.
hipError_t launch_classify(int64_t T, int32_t bm, int32_t bn, int64_t nq, int64_t nk,
                           const int32_t* end, uint8_t* kinds, int32_t* row_ptr,
                           int32_t* col_ptr, int32_t* ktile_min_end, int32_t* ktile_max_end,
                           int64_t* info, hipStream_t stream);
// Node form of a packed-document draft layout (context [0, S), then n_blocks blocks
// of bs draft tokens): a block's number orders it by (document, anchor, index); a
// context key's range holds the kept blocks of its document anchored after it; a
// draft key's range is its own block.  anchors out of [0, S] set info[3] to
// block * 8 + 5.  scratch: draft_scratch_bytes(n_blocks) bytes.
size_t draft_scratch_bytes(int64_t n_blocks);
hipError_t launch_draft_nodes(int64_t T, int64_t S, int32_t bs, int64_t n_blocks,
                              const int32_t* anchors, const uint8_t* keep,
                              const int32_t* ctx_doc, const int32_t* anchor_doc, int32_t* key,
                              int32_t* lo, int32_t* w, void* scratch, size_t scratch_bytes,
                              int64_t* info, hipStream_t stream);
// The same from the node form.  ksum: 4 * align64(nk) ints of scratch.  causal = 0
// drops the kv <= q conjunct.
hipError_t launch_classify_nodes(int64_t T, int32_t bm, int32_t bn, int64_t nq, int64_t nk,
                                 const int32_t* key, const int32_t* lo, const int32_t* w,
                                 int32_t causal, uint8_t* kinds, int32_t* row_ptr,
                                 int32_t* col_ptr, int32_t* ksum, int64_t* info,
                                 hipStream_t stream);
// CSR and CSC lists (ordered compaction of kinds) and the two length orders.
hipError_t launch_fill_lists(int64_t nq, int64_t nk, const uint8_t* kinds,
                             const int32_t* row_ptr, const int32_t* col_ptr, int32_t* col,
                             uint8_t* kind, int32_t* row, uint8_t* kind_csc, int32_t* qorder,
                             int32_t* korder, hipStream_t stream);

// ---------------------------------------------------------------------------
// attention kernels
// ---------------------------------------------------------------------------
struct AttnShape {
  int64_t T;
  int32_t hq, hkv, d;
  float scale;  // resolved softmax scale
};

// Kernel tile shapes (the map's block_m, block_n must equal these).
constexpr int32_t kTileM = 128;
constexpr int32_t kTileN = 128;

bool fwd_supported(psa_dtype dt, int32_t d);
bool bwd_supported(psa_dtype dt, int32_t d);

hipError_t launch_fwd(const psa_tile_map& map, psa_dtype dt, const AttnShape& s,
                      const void* q, const void* k, const void* v, void* o, float* lse,
                      hipStream_t stream);

size_t bwd_workspace_bytes(const AttnShape& s);
// The fixed device scratch of psa_bwd_noalloc (attn_bwd.hip): its size, and its
// address on the current device (looked up once per device, never allocated).
constexpr size_t kBwdScratchBytes = size_t{32} << 20;
hipError_t bwd_scratch(void** ptr);
hipError_t launch_bwd(const psa_tile_map& map, psa_dtype dt, psa_dtype grad_dt, const AttnShape& s,
                      const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dout, void* dq, void* dk, void* dv,
                      void* workspace, int stages, bool split, hipStream_t stream);

// ---------------------------------------------------------------------------
// fold.hip
// ---------------------------------------------------------------------------
// One run of flat positions of the folded layout: a group's prompt, a completion, or
// the pad tail.  src indexes prompt_tok (prompt) or comp_tok (completion); last_src
// is the comp_tok index of the label of the run's last token, or -1 (masked).
constexpr int32_t kFoldPrompt = 0, kFoldComp = 1, kFoldPad = 2;
struct FoldSeg {
  int64_t flat_start, len, src, last_src;
  int32_t kind, group, suffix, pos_base;
};
// One contiguous byte range copied by the unfold.
struct UnfoldSeg {
  int64_t src_byte, dst_byte, bytes, unused;
};
constexpr int64_t kUnfoldChunk = 16384;  // bytes per work-group
hipError_t launch_fold(const FoldSeg* segs, int64_t n_segs, int64_t max_len,
                       const int32_t* prompt_tok, const int32_t* comp_tok, int32_t pad_id,
                       int32_t ignore, int32_t* input_ids, int32_t* labels,
                       int32_t* position_ids, int32_t* group, int32_t* suffix,
                       uint8_t* is_prefix, hipStream_t stream);
hipError_t launch_unfold(const UnfoldSeg* segs, int64_t n_segs, int64_t max_bytes,
                         const void* src, void* dst, bool words16, hipStream_t stream);
