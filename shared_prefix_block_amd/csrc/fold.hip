// The steps on either side of the attention: folding rollout groups (one prompt and
// the completions sampled from it) into the flat shared-prefix layout, and unfolding
// per-token rows of that layout back to the samples.
//
// Source: Automodel PR #2564 page (PR description; "Changelog" entry for
// fold_shared_prefix_rollouts: deduplicated flat input_ids, pre-shifted next-token
// labels, per-completion position_ids; the commit note on pre-shifted labels: token t
// predicts t + 1, a completion's last token masked).  The attention metadata written
// beside them is the token form of the unsloth prefix_grouper_kernel.py page
// (build_seg_info_multigroup: prefix tokens of a group, suffix ids counted over all
// groups).
//
// Both kernels walk a small segment table the host builds from the lengths: one
// work-group per (segment, chunk), coalesced along the segment.  They move bytes and
// do no arithmetic worth the name, so their bound is HBM bandwidth.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "psa_internal.h"

namespace {

// fold: one thread per flat position of a segment; work-group b takes chunk
// b % n_chunks of segment b / n_chunks
__global__ __launch_bounds__(256) void k_fold(const FoldSeg* __restrict__ segs, int64_t n_chunks,
                                              const int32_t* __restrict__ prompt_tok,
                                              const int32_t* __restrict__ comp_tok,
                                              int32_t pad_id, int32_t ignore,
                                              int32_t* __restrict__ input_ids,
                                              int32_t* __restrict__ labels,
                                              int32_t* __restrict__ position_ids,
                                              int32_t* __restrict__ group,
                                              int32_t* __restrict__ suffix,
                                              uint8_t* __restrict__ is_prefix) {
  const FoldSeg sg = segs[blockIdx.x / n_chunks];
  const int64_t j = int64_t(blockIdx.x % n_chunks) * 256 + threadIdx.x;
  if (j >= sg.len) return;
  const int64_t t = sg.flat_start + j;
  int32_t id, lab, pos, g, s;
  uint8_t pre;
  if (sg.kind == kFoldPad) {
    id = pad_id;
    lab = ignore;
    pos = 0;
    g = -1;
    s = -1;
    pre = 0;
  } else {
    const int32_t* src = sg.kind == kFoldPrompt ? prompt_tok : comp_tok;
    id = src[sg.src + j];
    // token t predicts t + 1 of its own segment; a segment's last token takes the
    // label the host resolved for it (a completion's: masked; a prompt's: the first
    // token of the group's first non-empty completion, or masked)
    if (j + 1 < sg.len)
      lab = src[sg.src + j + 1];
    else
      lab = sg.last_src >= 0 ? comp_tok[sg.last_src] : ignore;
    pos = sg.pos_base + int32_t(j);
    g = sg.group;
    s = sg.suffix;
    pre = sg.kind == kFoldPrompt ? 1 : 0;
  }
  if (input_ids) input_ids[t] = id;
  if (labels) labels[t] = lab;
  if (position_ids) position_ids[t] = pos;
  if (group) group[t] = g;
  if (suffix) suffix[t] = s;
  if (is_prefix) is_prefix[t] = pre;
}

// unfold: a segment is one contiguous byte range on both sides; each work-group moves
// kUnfoldChunk bytes of it in 16-byte (or 4-byte) words
template <typename W>
__global__ __launch_bounds__(256) void k_unfold(const UnfoldSeg* __restrict__ segs,
                                                int64_t n_chunks,
                                                const char* __restrict__ src,
                                                char* __restrict__ dst) {
  const UnfoldSeg sg = segs[blockIdx.x / n_chunks];
  constexpr int64_t kWords = kUnfoldChunk / int64_t(sizeof(W));
  const int64_t n_words = sg.bytes / int64_t(sizeof(W));
  const int64_t w0 = int64_t(blockIdx.x % n_chunks) * kWords;
  if (w0 >= n_words) return;
  const W* s = reinterpret_cast<const W*>(src + sg.src_byte);
  W* d = reinterpret_cast<W*>(dst + sg.dst_byte);
#pragma unroll
  for (int k = 0; k < int(kWords / 256); ++k) {
    const int64_t w = w0 + k * 256 + threadIdx.x;
    if (w < n_words) d[w] = s[w];
  }
}

}  // namespace

hipError_t launch_fold(const FoldSeg* segs, int64_t n_segs, int64_t max_len,
                       const int32_t* prompt_tok, const int32_t* comp_tok, int32_t pad_id,
                       int32_t ignore, int32_t* input_ids, int32_t* labels,
                       int32_t* position_ids, int32_t* group, int32_t* suffix,
                       uint8_t* is_prefix, hipStream_t stream) {
  if (n_segs == 0 || max_len == 0) return hipSuccess;
  const int64_t n_chunks = (max_len + 255) / 256;
  if (n_segs * n_chunks > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_fold, dim3(unsigned(n_segs * n_chunks)), dim3(256), 0, stream, segs,
                     n_chunks, prompt_tok, comp_tok, pad_id, ignore, input_ids, labels,
                     position_ids, group, suffix, is_prefix);
  return hipGetLastError();
}

hipError_t launch_unfold(const UnfoldSeg* segs, int64_t n_segs, int64_t max_bytes,
                         const void* src, void* dst, bool words16, hipStream_t stream) {
  if (n_segs == 0 || max_bytes == 0) return hipSuccess;
  const int64_t n_chunks = (max_bytes + kUnfoldChunk - 1) / kUnfoldChunk;
  if (n_segs * n_chunks > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid(unsigned(n_segs * n_chunks));
  if (words16)
    hipLaunchKernelGGL(k_unfold<uint4>, grid, dim3(256), 0, stream, segs, n_chunks,
                       static_cast<const char*>(src), static_cast<char*>(dst));
  else
    hipLaunchKernelGGL(k_unfold<uint32_t>, grid, dim3(256), 0, stream, segs, n_chunks,
                       static_cast<const char*>(src), static_cast<char*>(dst));
  return hipGetLastError();
}
