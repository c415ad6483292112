// Tile-map builder kernels (gfx950).
//
// Step 1 turns either metadata form into one int32 per token, end[t], such that key t
// is visible to exactly the rows q with t <= q < end[t].  This interval form is exact
// for the accepted layouts (see psa.h): a prompt token of a group is seen by every
// later token of its group, so end = the group's end; a completion token is seen by
// the later tokens of its own completion, so end = the completion's end; in a prefix
// tree laid out in depth-first pre-order a token is seen by the later tokens of its
// node and by every token of the node's subtree, so end = the subtree's end; a pad is
// seen by nobody, so end = t.  (Mask rule: unsloth "prefix_grouper_kernel.py",
// _make_mask_mod; tree: Automodel PR #2564, "Changelog".)
//
// Step 2 classifies every (q-tile, kv-tile) pair as empty / partial / full, which is
// the block sparsity the unsloth page's module docstring relies on (masked blocks are
// never computed), then lays the non-empty tiles out as CSR (per q-tile) and CSC
// (per kv-tile) lists in ascending order.  Everything is integer work with scans or
// integer atomics whose sums do not depend on order, so the map is deterministic.
//
// Layouts that are not packed this way (groups or completions interleaved, a prompt
// token after a completion token, group or completion ids out of order, a prefix tree
// whose subtrees are not contiguous) have no interval form; they get the node form
// instead (psa_tile_map): every token carries the pre-order number of its node in the
// prefix forest (a group's prompt is the parent of its completions), every key the
// pre-order range of its node's subtree, and keep(q, kv) is kv <= q with q's node in
// kv's subtree, which is the same rule written on nodes.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>
#include <cstring>

#include <rocprim/device/device_radix_sort.hpp>
#include <rocprim/device/device_select.hpp>

#include "psa_internal.h"

namespace {

constexpr int kScanThreads = 1024;

// Inclusive scan over the 1024 threads of a block (Hillis-Steele in LDS), each
// thread sitting at position `slot` (a permutation of the thread ids).  On return
// sh[] holds the whole inclusive scan by slot; callers read what they need and pass
// a barrier before the next use of sh.
template <typename T, typename Op>
__device__ T scan_slot(T v, int slot, T* sh, Op op) {
  sh[slot] = v;
  __syncthreads();
  for (int off = 1; off < kScanThreads; off <<= 1) {
    T other = slot >= off ? sh[slot - off] : v;
    __syncthreads();
    if (slot >= off) v = op(v, other);
    sh[slot] = v;
    __syncthreads();
  }
  return v;
}

struct AddOp {
  __device__ long long operator()(long long a, long long b) const { return a + b; }
};

// ---------------------------------------------------------------------------
// Step 1a: labels -> end[], with the layout checks, in two passes over chunks of
// kTokChunk tokens (one block each).  A "group break" at e (0 < e <= T) means tokens
// e-1 and e are not of the same group (or either is a pad, or e = T); a "run break"
// is a group break or a change of completion.  end[t] is the first group break after
// t for a prompt token, the first run break after t for a completion token, and t for
// a pad.
// ---------------------------------------------------------------------------
constexpr int kTokThreads = 256;
constexpr int kTokItems = 4;
constexpr int kTokChunk = kTokThreads * kTokItems;
constexpr int32_t kNone = INT_MAX;

__device__ inline bool group_break(int64_t T, const int32_t* group, int64_t e) {
  if (e >= T) return true;
  const int32_t a = group[e - 1], b = group[e];
  return a < 0 || b < 0 || a != b;
}
__device__ inline bool run_break(int64_t T, const int32_t* group, const int32_t* suffix,
                                 const uint8_t* is_prefix, int64_t e) {
  return group_break(T, group, e) || is_prefix[e] != is_prefix[e - 1] ||
         suffix[e] != suffix[e - 1];
}

// Minimum of v over the threads of the block with a larger thread id (kNone if none).
__device__ inline int32_t block_min_after(int32_t v, int32_t* sh) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int32_t x = v;  // inclusive minimum over lanes >= lane of this wave
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t y = __shfl_down(x, off);
    if (lane + off < 64) x = y < x ? y : x;
  }
  const int32_t nxt = __shfl_down(x, 1);  // every lane takes part in the shuffle
  const int32_t after_in_wave = lane < 63 ? nxt : kNone;
  if (lane == 0) sh[w] = x;
  __syncthreads();
  int32_t r = after_in_wave;
  for (int k = w + 1; k < kTokThreads / 64; ++k) r = sh[k] < r ? sh[k] : r;
  __syncthreads();
  return r;
}

// Pass 1: layout checks (the first offending position and its code, atomically
// minimised into *err as position * 8 + code) and, per chunk, its first group break
// and first run break (kNone if none).
__global__ __launch_bounds__(kTokThreads) void k_tokens_check(
    int64_t T, const int32_t* __restrict__ group, const int32_t* __restrict__ suffix,
    const uint8_t* __restrict__ is_prefix, int32_t* first_g, int32_t* first_r,
    unsigned long long* err) {
  __shared__ int32_t sh[kTokThreads / 64];
  const int64_t t0 = int64_t(blockIdx.x) * kTokChunk + int64_t(threadIdx.x) * kTokItems;
  unsigned long long my_err = ~0ull;
  int32_t fg = kNone, fr = kNone;
  for (int i = 0; i < kTokItems; ++i) {
    const int64_t t = t0 + i;
    if (t >= T) break;
    const int32_t g = group[t];
    if (g >= 0 && t > 0 && my_err == ~0ull) {
      int code = 0;
      const int32_t gp = group[t - 1];
      if (gp >= 0) {
        if (g < gp) {
          code = 1;
        } else if (g == gp) {  // the same group continues
          const bool pf = is_prefix[t] != 0, ppf = is_prefix[t - 1] != 0;
          if (pf && !ppf) code = 3;
          else if (!pf && !ppf && suffix[t] < suffix[t - 1]) code = 4;
        }
      } else {  // after a pad run: compare with the last real token before it
        int64_t pr = t - 2;
        while (pr >= 0 && group[pr] < 0) --pr;
        if (pr >= 0) {
          const int32_t gr = group[pr];
          if (g < gr) code = 1;
          else if (g == gr) code = 2;
        }
      }
      if (code) my_err = (unsigned long long)t * 8 + code;
    }
    const int64_t e = t + 1;  // break between t and t + 1 ?
    if (fg == kNone && group_break(T, group, e)) fg = int32_t(e);
    if (fr == kNone && run_break(T, group, suffix, is_prefix, e)) fr = int32_t(e);
  }
  if (my_err != ~0ull) atomicMin(err, my_err);
  // the chunk's first breaks: the minimum over its threads
  const int32_t g_after = block_min_after(fg, sh);
  const int32_t r_after = block_min_after(fr, sh);
  if (threadIdx.x == 0) {
    first_g[blockIdx.x] = fg < g_after ? fg : g_after;
    first_r[blockIdx.x] = fr < r_after ? fr : r_after;
  }
}

// First break at or after chunk c + 1 (T if none): wave 0 scans 64 chunks at a time.
__device__ inline int32_t next_break(const int32_t* first, int64_t c, int64_t n_chunks,
                                     int64_t T, int32_t* sh) {
  if (threadIdx.x < 64) {
    int32_t found = kNone;
    for (int64_t c0 = c + 1; c0 < n_chunks && found == kNone; c0 += 64) {
      const int64_t cc = c0 + threadIdx.x;
      int32_t v = cc < n_chunks ? first[cc] : kNone;
      for (int off = 32; off >= 1; off >>= 1) {
        const int32_t y = __shfl_xor(v, off);
        v = y < v ? y : v;
      }
      found = v;  // wave-uniform
    }
    if (threadIdx.x == 0) sh[0] = found == kNone ? int32_t(T) : found;
  }
  __syncthreads();
  const int32_t r = sh[0];
  __syncthreads();
  return r;
}

// Pass 2: end[] per chunk, from the breaks inside the chunk and the first ones after.
__global__ __launch_bounds__(kTokThreads) void k_tokens_end(
    int64_t T, const int32_t* __restrict__ group, const int32_t* __restrict__ suffix,
    const uint8_t* __restrict__ is_prefix, const int32_t* __restrict__ first_g,
    const int32_t* __restrict__ first_r, int32_t* __restrict__ end) {
  __shared__ int32_t sh[kTokThreads / 64];
  const int64_t c = blockIdx.x, n_chunks = gridDim.x;
  const int64_t t0 = c * kTokChunk + int64_t(threadIdx.x) * kTokItems;
  bool gb[kTokItems], rb[kTokItems];
  int32_t fg = kNone, fr = kNone;
  for (int i = 0; i < kTokItems; ++i) {
    const int64_t t = t0 + i, e = t + 1;
    gb[i] = t < T && group_break(T, group, e);
    rb[i] = t < T && run_break(T, group, suffix, is_prefix, e);
    if (fg == kNone && gb[i]) fg = int32_t(e);
    if (fr == kNone && rb[i]) fr = int32_t(e);
  }
  const int32_t later_g = next_break(first_g, c, n_chunks, T, sh);
  const int32_t later_r = next_break(first_r, c, n_chunks, T, sh);
  int32_t ng = block_min_after(fg, sh), nr = block_min_after(fr, sh);
  ng = later_g < ng ? later_g : ng;
  nr = later_r < nr ? later_r : nr;
  for (int i = kTokItems - 1; i >= 0; --i) {
    const int64_t t = t0 + i;
    if (t >= T) continue;
    if (gb[i]) ng = int32_t(t + 1);
    if (rb[i]) nr = int32_t(t + 1);
    end[t] = group[t] < 0 ? int32_t(t) : (is_prefix[t] ? ng : nr);
  }
}

// Step 1b: per-node table -> end[].  node_start non-decreasing (zero-length nodes
// share a start; the last of them is the one that owns the tokens).
__global__ void k_tree_end(int64_t T, int64_t n_nodes, const int64_t* __restrict__ node_start,
                           const int64_t* __restrict__ sub_end, int64_t t_real,
                           int32_t* __restrict__ end) {
  for (int64_t t = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; t < T;
       t += int64_t(gridDim.x) * blockDim.x) {
    if (t >= t_real) {
      end[t] = int32_t(t);
      continue;
    }
    int64_t lo = 0, hi = n_nodes;  // first index with node_start > t
    while (lo < hi) {
      int64_t mid = (lo + hi) >> 1;
      if (node_start[mid] <= t) lo = mid + 1;
      else hi = mid;
    }
    end[t] = int32_t(sub_end[lo - 1]);
  }
}

// ---------------------------------------------------------------------------
// Step 1c: labels -> node form.  A node is (group, prompt) or (group, completion s);
// its sort key is group * 2^33 + (0 for the prompt, 1 + s as unsigned 32-bit for a
// completion), so a group's nodes are one contiguous run of sorted keys with the
// prompt first.  The node number is the rank among the distinct keys, plus 1; a
// prompt's subtree is every node of its group, a completion's is itself.
// ---------------------------------------------------------------------------
constexpr uint64_t kPadComposite = ~0ull;  // above every real key: sorts last

__device__ inline uint64_t node_composite(int32_t g, int32_t s, uint8_t pf) {
  return (uint64_t(uint32_t(g)) << 33) | (pf ? 0ull : uint64_t(uint32_t(s)) + 1ull);
}

__global__ void k_node_composite(int64_t T, const int32_t* __restrict__ group,
                                 const int32_t* __restrict__ suffix,
                                 const uint8_t* __restrict__ is_prefix,
                                 uint64_t* __restrict__ comp) {
  for (int64_t t = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; t < T;
       t += int64_t(gridDim.x) * blockDim.x) {
    const int32_t g = group[t];
    comp[t] = g < 0 ? kPadComposite : node_composite(g, suffix[t], is_prefix[t]);
  }
}

// first index in uniq[0, n) whose value is > x (x < x_limit is not assumed)
__device__ inline int64_t upper_index(const uint64_t* __restrict__ uniq, int64_t n, uint64_t x) {
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if (uniq[mid] <= x) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

__global__ void k_node_number(int64_t T, const int32_t* __restrict__ group,
                              const uint8_t* __restrict__ is_prefix,
                              const uint64_t* __restrict__ comp,
                              const uint64_t* __restrict__ uniq,
                              const int64_t* __restrict__ n_uniq, int32_t* __restrict__ key,
                              int32_t* __restrict__ lo, int32_t* __restrict__ w) {
  const int64_t n = *n_uniq;
  for (int64_t t = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; t < T;
       t += int64_t(gridDim.x) * blockDim.x) {
    const uint64_t c = comp[t];
    if (c == kPadComposite) {
      key[t] = 0;
      lo[t] = 0;
      w[t] = 0;
      continue;
    }
    const int64_t r = upper_index(uniq, n, c) - 1;  // rank of c itself
    int64_t width = 1;
    if (is_prefix[t]) {  // every key of the group: up to group * 2^33 + (2^33 - 1)
      const uint64_t last = (uint64_t(uint32_t(group[t])) << 33) | ((1ull << 33) - 1);
      width = upper_index(uniq, n, last) - r;
    }
    key[t] = int32_t(r + 1);
    lo[t] = int32_t(r + 1);
    w[t] = int32_t(width);
  }
}

// Step 1d: per-node table -> node form (the tree's pre-order numbering is the host's).
__global__ void k_tree_nodes(int64_t T, int64_t n_nodes, const int64_t* __restrict__ node_start,
                             const int64_t* __restrict__ pre, const int64_t* __restrict__ size,
                             int64_t t_real, int32_t* __restrict__ key, int32_t* __restrict__ lo,
                             int32_t* __restrict__ w) {
  for (int64_t t = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; t < T;
       t += int64_t(gridDim.x) * blockDim.x) {
    if (t >= t_real) {
      key[t] = 0;
      lo[t] = 0;
      w[t] = 0;
      continue;
    }
    int64_t a = 0, b = n_nodes;  // first node with node_start > t; the one before owns t
    while (a < b) {
      const int64_t mid = (a + b) >> 1;
      if (node_start[mid] <= t) a = mid + 1;
      else b = mid;
    }
    const int64_t node = a - 1;
    key[t] = int32_t(pre[node] + 1);
    lo[t] = int32_t(pre[node] + 1);
    w[t] = int32_t(size[node]);
  }
}

// ---------------------------------------------------------------------------
// Step 2: classification
// ---------------------------------------------------------------------------
// info[0..2] = nnz, n_full, n_partial; info[3] = first layout error (all ones: none).
__global__ void k_map_init(int64_t nk, int32_t* row_ptr, int32_t* col_ptr, int64_t* info) {
  for (int64_t j = threadIdx.x; j <= nk; j += blockDim.x) col_ptr[j] = 0;
  if (threadIdx.x < 8) info[threadIdx.x] = threadIdx.x == 3 ? -1 : 0;
  if (threadIdx.x == 0) row_ptr[0] = 0;
}

// One wave per kv-tile: min of end[] over its columns, and the furthest row any of
// its columns reaches (-1 if every column is a pad).
__global__ __launch_bounds__(64) void k_ktile_summary(int64_t T, int32_t bn, int64_t nk,
                                                      const int32_t* __restrict__ end,
                                                      int32_t* kmin, int32_t* kmax) {
  const int64_t j = blockIdx.x;
  if (j >= nk) return;
  const int64_t k0 = j * bn;
  const int64_t k1 = k0 + bn < T ? k0 + bn : T;
  int mn = INT_MAX, mx = -1;
  for (int64_t kv = k0 + threadIdx.x; kv < k1; kv += 64) {
    int e = end[kv];
    mn = e < mn ? e : mn;
    if (e > kv && e > mx) mx = e;
  }
  for (int off = 32; off >= 1; off >>= 1) {
    int a = __shfl_xor(mn, off), b = __shfl_xor(mx, off);
    mn = a < mn ? a : mn;
    mx = b > mx ? b : mx;
  }
  if (threadIdx.x == 0) {
    kmin[j] = mn;
    kmax[j] = mx;
  }
}

constexpr int kClassifyThreads = 256;

__global__ __launch_bounds__(kClassifyThreads) void k_classify_rows(
    int64_t T, int32_t bm, int32_t bn, int64_t nq, int64_t nk, const int32_t* __restrict__ end,
    const int32_t* __restrict__ kmin, const int32_t* __restrict__ kmax, uint8_t* kinds,
    int32_t* row_ptr, int32_t* col_ptr, int64_t* info) {
  __shared__ int red[3][kClassifyThreads / 64];
  const int64_t i = blockIdx.x;
  const int64_t q0 = i * bm;
  const int64_t q_last = (q0 + bm < T ? q0 + bm : T) - 1;  // last row inside [0, T)
  const bool rows_in = q0 + bm <= T;
  int cnt = 0, nfull = 0, npart = 0;
  for (int64_t j = threadIdx.x; j < nk; j += kClassifyThreads) {
    const int64_t k0 = j * bn;
    const int64_t k_last = (k0 + bn < T ? k0 + bn : T) - 1;
    const bool cols_in = k0 + bn <= T;
    uint8_t kind = 0;
    if (k0 <= q_last && kmax[j] > q0) {
      if (rows_in && cols_in && k_last <= q0 && kmin[j] > q0 + bm - 1) {
        kind = 2;
      } else {
        for (int64_t kv = k0; kv <= k_last && kv <= q_last; ++kv) {
          int64_t e = end[kv];
          int64_t lo = kv > q0 ? kv : q0;
          if (e - 1 >= lo) {
            kind = 1;
            break;
          }
        }
      }
    }
    kinds[i * nk + j] = kind;
    if (kind) {
      ++cnt;
      if (kind == 2) ++nfull;
      else ++npart;
      atomicAdd(&col_ptr[j + 1], 1);
    }
  }
  for (int off = 32; off >= 1; off >>= 1) {
    cnt += __shfl_xor(cnt, off);
    nfull += __shfl_xor(nfull, off);
    npart += __shfl_xor(npart, off);
  }
  const int w = threadIdx.x / 64;
  if ((threadIdx.x & 63) == 0) {
    red[0][w] = cnt;
    red[1][w] = nfull;
    red[2][w] = npart;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int a = 0, b = 0, c = 0;
    for (int k = 0; k < kClassifyThreads / 64; ++k) {
      a += red[0][k];
      b += red[1][k];
      c += red[2][k];
    }
    row_ptr[i + 1] = a;
    atomicAdd(reinterpret_cast<unsigned long long*>(&info[1]), (unsigned long long)b);
    atomicAdd(reinterpret_cast<unsigned long long*>(&info[2]), (unsigned long long)c);
  }
}

// Step 1e: draft layout -> node form.  Block b's sort key is
// order(anchor document) * 2^32 + a_b * n_blocks + b (the host checks that the low
// word fits), or all ones for a block not kept; its number is its rank, from 1.
__device__ inline uint64_t doc_order(int32_t d) { return uint64_t(uint32_t(d) ^ 0x80000000u); }

__global__ void k_draft_composite(int64_t S, int64_t n, const int32_t* __restrict__ anchors,
                                  const uint8_t* __restrict__ keep,
                                  const int32_t* __restrict__ anchor_doc,
                                  uint64_t* __restrict__ comp, int32_t* __restrict__ idx,
                                  unsigned long long* err) {
  for (int64_t b = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; b < n;
       b += int64_t(gridDim.x) * blockDim.x) {
    const int32_t a = anchors[b];
    idx[b] = int32_t(b);
    if (a < 0 || a > S) {
      atomicMin(err, (unsigned long long)b * 8 + 5);
      comp[b] = kPadComposite;
      continue;
    }
    const bool live = keep ? keep[b] != 0 : true;
    const uint64_t d = anchor_doc ? doc_order(anchor_doc[b]) : doc_order(0);
    comp[b] = live ? (d << 32) | (uint64_t(a) * uint64_t(n) + uint64_t(b)) : kPadComposite;
  }
}

__global__ void k_draft_rank(int64_t n, const uint64_t* __restrict__ sorted,
                             const int32_t* __restrict__ order, int32_t* __restrict__ rank) {
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < n;
       i += int64_t(gridDim.x) * blockDim.x)
    rank[order[i]] = sorted[i] == kPadComposite ? 0 : int32_t(i + 1);
}

// first index in sorted[0, n) whose value is >= x
__device__ inline int64_t lower_index(const uint64_t* __restrict__ v, int64_t n, uint64_t x) {
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if (v[mid] < x) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

__global__ void k_draft_tokens(int64_t T, int64_t S, int32_t bs, int64_t n,
                               const int32_t* __restrict__ ctx_doc,
                               const uint64_t* __restrict__ sorted,
                               const int32_t* __restrict__ rank, int32_t* __restrict__ key,
                               int32_t* __restrict__ lo, int32_t* __restrict__ w) {
  for (int64_t t = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; t < T;
       t += int64_t(gridDim.x) * blockDim.x) {
    int32_t k = 0, a = 0, width = 0;
    if (t < S) {  // a context key: the kept blocks of its document anchored after it
      const uint64_t d = (ctx_doc ? doc_order(ctx_doc[t]) : doc_order(0)) << 32;
      const int64_t first = lower_index(sorted, n, d | (uint64_t(t + 1) * uint64_t(n)));
      const int64_t past = upper_index(sorted, n, d | 0xffffffffull);
      a = int32_t(first + 1);
      width = int32_t(past - first);
    } else if (t < S + int64_t(bs) * n) {  // a draft token: its own block
      k = rank[(t - S) / bs];
      a = k;
      width = k > 0 ? 1 : 0;
    }
    key[t] = k;
    lo[t] = a;
    w[t] = width;
  }
}

// Node form.  One wave per kv-tile: over its keys with w > 0, the smallest lo and the
// largest lo + w (INT_MAX / 0 if none); and, for the full test, the largest lo and
// the smallest lo + w over all its columns, or INT_MAX / 0 if a column is a pad or
// lies past T (such a tile is never full).
__global__ __launch_bounds__(64) void k_ktile_summary_nodes(int64_t T, int32_t bn, int64_t nk,
                                                            const int32_t* __restrict__ lo,
                                                            const int32_t* __restrict__ w,
                                                            int32_t* ksum, int64_t stride) {
  const int64_t j = blockIdx.x;
  if (j >= nk) return;
  const int64_t k0 = j * bn;
  const int64_t k1 = k0 + bn < T ? k0 + bn : T;
  int mn = INT_MAX, mx = 0, flo = 0, fhi = INT_MAX;
  bool all = k0 + bn <= T;
  for (int64_t kv = k0 + threadIdx.x; kv < k1; kv += 64) {
    const int a = lo[kv], n = w[kv];
    if (n > 0) {
      mn = a < mn ? a : mn;
      mx = a + n > mx ? a + n : mx;
      flo = a > flo ? a : flo;
      fhi = a + n < fhi ? a + n : fhi;
    } else {
      all = false;
    }
  }
  for (int off = 32; off >= 1; off >>= 1) {
    const int a = __shfl_xor(mn, off), b = __shfl_xor(mx, off);
    const int c = __shfl_xor(flo, off), d = __shfl_xor(fhi, off);
    mn = a < mn ? a : mn;
    mx = b > mx ? b : mx;
    flo = c > flo ? c : flo;
    fhi = d < fhi ? d : fhi;
  }
  all = __all(all);
  if (threadIdx.x == 0) {
    ksum[j] = mn;
    ksum[stride + j] = mx;
    ksum[2 * stride + j] = all ? flo : INT_MAX;
    ksum[3 * stride + j] = all ? fhi : 0;
  }
}

// One block per q-tile, its keys in LDS as runs of equal node numbers (number, last
// row); each wave takes every fourth kv-tile.  A tile is empty when it lies wholly
// after the q-tile (kv > q everywhere; causal maps only) or when the keys' subtree
// ranges miss the q-tile's key range; full when it lies wholly at or before the
// q-tile (causal maps) and every range holds every key; otherwise the wave searches
// it exactly, one column per lane: a key is seen by some row iff a run's number lies
// in its range (and, causal, the run ends at or after the key).
__global__ __launch_bounds__(kClassifyThreads) void k_classify_nodes_rows(
    int64_t T, int32_t bm, int32_t bn, int64_t nq, int64_t nk, const int32_t* __restrict__ key,
    const int32_t* __restrict__ lo, const int32_t* __restrict__ w, int32_t causal,
    const int32_t* __restrict__ ksum, int64_t stride, uint8_t* kinds, int32_t* row_ptr,
    int32_t* col_ptr, int64_t* info) {
  __shared__ int32_t qk[1024];
  __shared__ int32_t runk[1024], runl[1024];  // run number, run's last row (absolute)
  __shared__ int red[3][kClassifyThreads / 64];
  __shared__ int n_runs;
  const int64_t i = blockIdx.x;
  const int64_t q0 = i * bm;
  const int64_t q_last = (q0 + bm < T ? q0 + bm : T) - 1;
  const bool rows_in = q0 + bm <= T;
  const int nrow = int(q_last - q0 + 1);
  int kmin = INT_MAX, kmax = 0;  // over real rows (key > 0)
  bool all_real = rows_in;
  for (int r = threadIdx.x; r < nrow; r += kClassifyThreads) {
    const int k = key[q0 + r];
    qk[r] = k;
    if (k > 0) {
      kmin = k < kmin ? k : kmin;
      kmax = k > kmax ? k : kmax;
    } else {
      all_real = false;
    }
  }
  for (int off = 32; off >= 1; off >>= 1) {
    const int a = __shfl_xor(kmin, off), b = __shfl_xor(kmax, off);
    kmin = a < kmin ? a : kmin;
    kmax = b > kmax ? b : kmax;
  }
  all_real = __all(all_real);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  if (lane == 0) {
    red[0][wv] = kmin;
    red[1][wv] = kmax;
    red[2][wv] = all_real ? 1 : 0;
  }
  __syncthreads();
  for (int k = 0; k < kClassifyThreads / 64; ++k) {
    kmin = red[0][k] < kmin ? red[0][k] : kmin;
    kmax = red[1][k] > kmax ? red[1][k] : kmax;
    all_real = all_real && red[2][k];
  }
  if (wv == 0) {  // run-length encoding of the rows' node numbers, 64 rows at a time
    int count = 0;
    for (int base = 0; base < nrow; base += 64) {
      const int r = base + lane;
      const bool start = r < nrow && (r == 0 || qk[r] != qk[r - 1]);
      const unsigned long long m = __ballot(start);
      const int at = count + __popcll(m & ((1ull << lane) - 1)) - 1;  // run of row r
      if (start) runk[at + 1] = qk[r];
      count += __popcll(m);
      // the row before a run start ends the previous run
      if (start && r > 0) runl[at] = int(q0) + r - 1;
    }
    if (lane == 0) {
      if (count > 0) runl[count - 1] = int(q0) + nrow - 1;
      n_runs = count;
    }
  }
  __syncthreads();
  const int m_runs = n_runs;

  int cnt = 0, nfull = 0, npart = 0;  // lane 0 of each wave counts its tiles
  for (int64_t j = wv; j < nk; j += kClassifyThreads / 64) {
    const int64_t k0 = j * bn;
    const int64_t k_last = (k0 + bn < T ? k0 + bn : T) - 1;
    const int mn = ksum[j], mx = ksum[stride + j];
    uint8_t kind = 0;
    if ((k0 <= q_last || !causal) && kmax > 0 && mn != INT_MAX && mx > kmin && mn <= kmax) {
      if (all_real && k0 + bn <= T && (k_last <= q0 || !causal) && ksum[2 * stride + j] <= kmin &&
          kmax < ksum[3 * stride + j]) {
        kind = 2;
      } else {
        bool found = false;
        for (int64_t kv = k0 + lane; kv <= k_last && !found; kv += 64) {
          const int a = lo[kv], n = w[kv];
          if (n <= 0) continue;
          for (int e = 0; e < m_runs; ++e) {
            if (uint32_t(runk[e] - a) < uint32_t(n) && (!causal || runl[e] >= kv)) {
              found = true;
              break;
            }
          }
        }
        kind = __any(found) ? 1 : 0;
      }
    }
    if (lane == 0) {
      kinds[i * nk + j] = kind;
      if (kind) {
        ++cnt;
        if (kind == 2) ++nfull;
        else ++npart;
        atomicAdd(&col_ptr[j + 1], 1);
      }
    }
  }
  if (lane == 0) {
    red[0][wv] = cnt;
    red[1][wv] = nfull;
    red[2][wv] = npart;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int a = 0, b = 0, c = 0;
    for (int k = 0; k < kClassifyThreads / 64; ++k) {
      a += red[0][k];
      b += red[1][k];
      c += red[2][k];
    }
    row_ptr[i + 1] = a;
    atomicAdd(reinterpret_cast<unsigned long long*>(&info[1]), (unsigned long long)b);
    atomicAdd(reinterpret_cast<unsigned long long*>(&info[2]), (unsigned long long)c);
  }
}

// In-place inclusive scan of counts ptr[1..n] (one block), both pointer arrays.
__global__ __launch_bounds__(kScanThreads) void k_scan_ptrs(int64_t nq, int64_t nk,
                                                            int32_t* row_ptr, int32_t* col_ptr,
                                                            int64_t* info) {
  __shared__ long long sh[kScanThreads];
  for (int which = 0; which < 2; ++which) {
    int32_t* p = which == 0 ? row_ptr : col_ptr;
    const int64_t n = which == 0 ? nq : nk;
    long long carry = 0;
    for (int64_t c0 = 0; c0 < n; c0 += kScanThreads) {
      int64_t idx = c0 + threadIdx.x;
      long long v = idx < n ? p[idx + 1] : 0;
      __syncthreads();
      long long incl = scan_slot(v, int(threadIdx.x), sh, AddOp());
      if (idx < n) p[idx + 1] = int32_t(carry + incl);
      long long total = sh[kScanThreads - 1];
      __syncthreads();
      carry += total;
    }
    if (threadIdx.x == 0) {
      p[0] = 0;
      if (which == 0) info[0] = carry;
    }
    __syncthreads();
  }
}

// Ordered compaction of one CSR row (one block per q-tile).
constexpr int kFillThreads = 256;

__device__ inline int block_excl_count(bool f, int* sh_w, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  unsigned long long m = __ballot(f);
  int before_in_wave = __popcll(m & ((1ull << lane) - 1));
  if (lane == 0) sh_w[w] = __popcll(m);
  __syncthreads();
  int before = 0, all = 0;
  for (int k = 0; k < kFillThreads / 64; ++k) {
    if (k < w) before += sh_w[k];
    all += sh_w[k];
  }
  __syncthreads();
  *total = all;
  return before + before_in_wave;
}

// Rank of list i among n lists by descending length, ties by index (a stable sort):
// the number of lists that come before it.  One block; O(n) work.
__device__ inline int32_t length_rank(const int32_t* __restrict__ ptr, int64_t n, int64_t i,
                                      int* sh_w) {
  const int64_t li = ptr[i + 1] - ptr[i];
  int cnt = 0;
  for (int64_t j = threadIdx.x; j < n; j += kFillThreads) {
    const int64_t lj = ptr[j + 1] - ptr[j];
    cnt += (lj > li || (lj == li && j < i)) ? 1 : 0;
  }
  for (int off = 32; off >= 1; off >>= 1) cnt += __shfl_xor(cnt, off);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh_w[w] = cnt;
  __syncthreads();
  int total = 0;
  for (int k = 0; k < kFillThreads / 64; ++k) total += sh_w[k];
  return total;
}

// Blocks [0, nq): CSR row b, ordered compaction of row b of kinds, and its place in
// qorder (q-tiles by descending list length).  Blocks [nq, nq + nk): the same for CSC
// column b - nq and korder.
__global__ __launch_bounds__(kFillThreads) void k_fill_lists(
    int64_t nq, int64_t nk, const uint8_t* __restrict__ kinds,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_ptr, int32_t* col,
    uint8_t* kind, int32_t* row, uint8_t* kind_csc, int32_t* qorder, int32_t* korder) {
  __shared__ int sh_w[kFillThreads / 64];
  const bool csr = blockIdx.x < nq;
  const int64_t i = csr ? int64_t(blockIdx.x) : int64_t(blockIdx.x) - nq;
  const int64_t n_other = csr ? nk : nq;
  const int32_t* ptr = csr ? row_ptr : col_ptr;
  int32_t* idx = csr ? col : row;
  uint8_t* kd = csr ? kind : kind_csc;
  int64_t base = ptr[i];
  for (int64_t j0 = 0; j0 < n_other; j0 += kFillThreads) {
    const int64_t j = j0 + threadIdx.x;
    const uint8_t k = j < n_other ? (csr ? kinds[i * nk + j] : kinds[j * nk + i]) : 0;
    int total;
    const int pos = block_excl_count(k != 0, sh_w, &total);
    if (k) {
      idx[base + pos] = int32_t(j);
      kd[base + pos] = k;
    }
    base += total;
  }
  const int32_t r = length_rank(ptr, csr ? nq : nk, i, sh_w);
  if (threadIdx.x == 0) (csr ? qorder : korder)[r] = int32_t(i);
}

}  // namespace

hipError_t launch_map_init(int64_t nk, int32_t* row_ptr, int32_t* col_ptr, int64_t* info,
                           hipStream_t stream) {
  hipLaunchKernelGGL(k_map_init, dim3(1), dim3(1024), 0, stream, nk, row_ptr, col_ptr, info);
  return hipGetLastError();
}

int64_t tokens_scratch_ints(int64_t T) { return 2 * ((T + kTokChunk - 1) / kTokChunk); }

hipError_t launch_tokens_end(int64_t T, const int32_t* group, const int32_t* suffix,
                             const uint8_t* is_prefix, int32_t* end, int32_t* scratch,
                             int64_t* info, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int64_t n_chunks = (T + kTokChunk - 1) / kTokChunk;
  int32_t* first_g = scratch;
  int32_t* first_r = scratch + n_chunks;
  unsigned long long* err = reinterpret_cast<unsigned long long*>(info + 3);
  hipLaunchKernelGGL(k_tokens_check, dim3(unsigned(n_chunks)), dim3(kTokThreads), 0, stream, T,
                     group, suffix, is_prefix, first_g, first_r, err);
  hipLaunchKernelGGL(k_tokens_end, dim3(unsigned(n_chunks)), dim3(kTokThreads), 0, stream, T,
                     group, suffix, is_prefix, first_g, first_r, end);
  return hipGetLastError();
}

hipError_t launch_tree_end(int64_t T, int64_t n_nodes, const int64_t* node_start,
                           const int64_t* node_subtree_end, int64_t t_real, int32_t* end,
                           hipStream_t stream) {
  if (T == 0) return hipSuccess;
  int64_t blocks = (T + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_tree_end, dim3(unsigned(blocks)), dim3(256), 0, stream, T, n_nodes,
                     node_start, node_subtree_end, t_real, end);
  return hipGetLastError();
}

hipError_t launch_classify(int64_t T, int32_t bm, int32_t bn, int64_t nq, int64_t nk,
                           const int32_t* end, uint8_t* kinds, int32_t* row_ptr,
                           int32_t* col_ptr, int32_t* kmin, int32_t* kmax, int64_t* info,
                           hipStream_t stream) {
  if (nk > 0) {
    hipLaunchKernelGGL(k_ktile_summary, dim3(unsigned(nk)), dim3(64), 0, stream, T, bn, nk, end,
                       kmin, kmax);
  }
  if (nq > 0) {
    hipLaunchKernelGGL(k_classify_rows, dim3(unsigned(nq)), dim3(kClassifyThreads), 0, stream, T,
                       bm, bn, nq, nk, end, kmin, kmax, kinds, row_ptr, col_ptr, info);
  }
  hipLaunchKernelGGL(k_scan_ptrs, dim3(1), dim3(kScanThreads), 0, stream, nq, nk, row_ptr,
                     col_ptr, info);
  return hipGetLastError();
}

size_t tokens_nodes_scratch_bytes(int64_t T) {
  const size_t n = size_t(T > 0 ? T : 1);
  size_t sort_b = 0, uniq_b = 0;
  uint64_t* none = nullptr;
  int64_t* cnt = nullptr;
  (void)rocprim::radix_sort_keys(nullptr, sort_b, none, none, n, 0, 64);
  (void)rocprim::unique(nullptr, uniq_b, none, none, cnt, n);
  const size_t arr = (n * 8 + 255) / 256 * 256;
  return 3 * arr + 256 + (sort_b > uniq_b ? sort_b : uniq_b);
}

hipError_t launch_tokens_nodes(int64_t T, const int32_t* group, const int32_t* suffix,
                               const uint8_t* is_prefix, int32_t* key, int32_t* lo,
                               int32_t* w, void* scratch, size_t scratch_bytes,
                               hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const size_t arr = (size_t(T) * 8 + 255) / 256 * 256;
  char* base = static_cast<char*>(scratch);
  uint64_t* comp = reinterpret_cast<uint64_t*>(base);
  uint64_t* sorted = reinterpret_cast<uint64_t*>(base + arr);
  uint64_t* uniq = reinterpret_cast<uint64_t*>(base + 2 * arr);
  int64_t* n_uniq = reinterpret_cast<int64_t*>(base + 3 * arr);
  void* tmp = base + 3 * arr + 256;
  if (scratch_bytes < 3 * arr + 256) return hipErrorInvalidValue;
  size_t tmp_bytes = scratch_bytes - (3 * arr + 256);
  int64_t blocks = (T + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_node_composite, dim3(unsigned(blocks)), dim3(256), 0, stream, T, group,
                     suffix, is_prefix, comp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  size_t b = tmp_bytes;
  e = rocprim::radix_sort_keys(tmp, b, comp, sorted, size_t(T), 0, 64, stream);
  if (e != hipSuccess) return e;
  b = tmp_bytes;
  e = rocprim::unique(tmp, b, sorted, uniq, n_uniq, size_t(T), rocprim::equal_to<uint64_t>(),
                      stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_node_number, dim3(unsigned(blocks)), dim3(256), 0, stream, T, group,
                     is_prefix, comp, uniq, n_uniq, key, lo, w);
  return hipGetLastError();
}

hipError_t launch_tree_nodes(int64_t T, int64_t n_nodes, const int64_t* node_start,
                             const int64_t* node_pre, const int64_t* node_size, int64_t t_real,
                             int32_t* key, int32_t* lo, int32_t* w, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  int64_t blocks = (T + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_tree_nodes, dim3(unsigned(blocks)), dim3(256), 0, stream, T, n_nodes,
                     node_start, node_pre, node_size, t_real, key, lo, w);
  return hipGetLastError();
}

size_t draft_scratch_bytes(int64_t n_blocks) {
  const size_t n = size_t(n_blocks > 0 ? n_blocks : 1);
  size_t sort_b = 0;
  uint64_t* none = nullptr;
  int32_t* ni = nullptr;
  (void)rocprim::radix_sort_pairs(nullptr, sort_b, none, none, ni, ni, n, 0, 64);
  const size_t a8 = (n * 8 + 255) / 256 * 256, a4 = (n * 4 + 255) / 256 * 256;
  return 2 * a8 + 3 * a4 + sort_b;
}

hipError_t launch_draft_nodes(int64_t T, int64_t S, int32_t bs, int64_t n_blocks,
                              const int32_t* anchors, const uint8_t* keep,
                              const int32_t* ctx_doc, const int32_t* anchor_doc, int32_t* key,
                              int32_t* lo, int32_t* w, void* scratch, size_t scratch_bytes,
                              int64_t* info, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const size_t n = size_t(n_blocks > 0 ? n_blocks : 1);
  const size_t a8 = (n * 8 + 255) / 256 * 256, a4 = (n * 4 + 255) / 256 * 256;
  if (scratch_bytes < 2 * a8 + 3 * a4) return hipErrorInvalidValue;
  char* base = static_cast<char*>(scratch);
  uint64_t* comp = reinterpret_cast<uint64_t*>(base);
  uint64_t* sorted = reinterpret_cast<uint64_t*>(base + a8);
  int32_t* idx = reinterpret_cast<int32_t*>(base + 2 * a8);
  int32_t* order = reinterpret_cast<int32_t*>(base + 2 * a8 + a4);
  int32_t* rank = reinterpret_cast<int32_t*>(base + 2 * a8 + 2 * a4);
  void* tmp = base + 2 * a8 + 3 * a4;
  size_t tmp_bytes = scratch_bytes - (2 * a8 + 3 * a4);
  hipError_t e = hipSuccess;
  if (n_blocks > 0) {
    const int64_t blocks = (n_blocks + 255) / 256 < 4096 ? (n_blocks + 255) / 256 : 4096;
    unsigned long long* err = reinterpret_cast<unsigned long long*>(info + 3);
    hipLaunchKernelGGL(k_draft_composite, dim3(unsigned(blocks)), dim3(256), 0, stream, S,
                       n_blocks, anchors, keep, anchor_doc, comp, idx, err);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    e = rocprim::radix_sort_pairs(tmp, tmp_bytes, comp, sorted, idx, order, size_t(n_blocks), 0,
                                  64, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_draft_rank, dim3(unsigned(blocks)), dim3(256), 0, stream, n_blocks,
                       sorted, order, rank);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  int64_t tb = (T + 255) / 256;
  if (tb > 4096) tb = 4096;
  hipLaunchKernelGGL(k_draft_tokens, dim3(unsigned(tb)), dim3(256), 0, stream, T, S, bs,
                     n_blocks, ctx_doc, sorted, rank, key, lo, w);
  return hipGetLastError();
}

hipError_t launch_classify_nodes(int64_t T, int32_t bm, int32_t bn, int64_t nq, int64_t nk,
                                 const int32_t* key, const int32_t* lo, const int32_t* w,
                                 int32_t causal, uint8_t* kinds, int32_t* row_ptr,
                                 int32_t* col_ptr, int32_t* ksum, int64_t* info,
                                 hipStream_t stream) {
  const int64_t stride = (nk + 63) / 64 * 64;
  if (nk > 0) {
    hipLaunchKernelGGL(k_ktile_summary_nodes, dim3(unsigned(nk)), dim3(64), 0, stream, T, bn,
                       nk, lo, w, ksum, stride);
  }
  if (nq > 0) {
    hipLaunchKernelGGL(k_classify_nodes_rows, dim3(unsigned(nq)), dim3(kClassifyThreads), 0,
                       stream, T, bm, bn, nq, nk, key, lo, w, causal, ksum, stride, kinds,
                       row_ptr, col_ptr, info);
  }
  hipLaunchKernelGGL(k_scan_ptrs, dim3(1), dim3(kScanThreads), 0, stream, nq, nk, row_ptr,
                     col_ptr, info);
  return hipGetLastError();
}

hipError_t launch_fill_lists(int64_t nq, int64_t nk, const uint8_t* kinds,
                             const int32_t* row_ptr, const int32_t* col_ptr, int32_t* col,
                             uint8_t* kind, int32_t* row, uint8_t* kind_csc, int32_t* qorder,
                             int32_t* korder, hipStream_t stream) {
  if (nq + nk == 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_lists, dim3(unsigned(nq + nk)), dim3(kFillThreads), 0, stream, nq,
                     nk, kinds, row_ptr, col_ptr, col, kind, row, kind_csc, qorder, korder);
  return hipGetLastError();
}
