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
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

#include "psa_internal.h"

namespace {

constexpr int kScanThreads = 1024;
constexpr int kScanItems = 4;
constexpr int kChunk = kScanThreads * kScanItems;

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

struct MaxOp {
  __device__ long long operator()(long long a, long long b) const { return a > b ? a : b; }
};
struct MinOp {
  __device__ long long operator()(long long a, long long b) const { return a < b ? a : b; }
};
struct AddOp {
  __device__ long long operator()(long long a, long long b) const { return a + b; }
};

// ---------------------------------------------------------------------------
// Step 1a: labels -> end[], with the layout checks.  One block, chunked scans.
// flag[0] = error code (0 ok), flag[1] = first offending position + 1.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kScanThreads) void k_tokens_end(
    int64_t T, const int32_t* __restrict__ group, const int32_t* __restrict__ suffix,
    const uint8_t* __restrict__ is_prefix, int32_t* __restrict__ end, int32_t* flag) {
  __shared__ long long sh[kScanThreads];
  const int tid = threadIdx.x;
  const int rt = kScanThreads - 1 - tid;  // reversed slot for suffix scans

  // Forward pass: pr = last real index before t; layout checks.
  long long carry_prev = -1;
  for (int64_t c0 = 0; c0 < T; c0 += kChunk) {
    const int64_t t0 = c0 + int64_t(tid) * kScanItems;
    long long local_last = -1;
    for (int i = 0; i < kScanItems; ++i) {
      int64_t t = t0 + i;
      if (t < T && group[t] >= 0) local_last = t;
    }
    __syncthreads();
    scan_slot(local_last, tid, sh, MaxOp());
    long long excl = tid > 0 ? sh[tid - 1] : -1;
    const long long chunk_max = sh[kScanThreads - 1];
    __syncthreads();
    long long pr = excl > carry_prev ? excl : carry_prev;
    long long err = LLONG_MAX;  // position * 8 + code
    for (int i = 0; i < kScanItems; ++i) {
      int64_t t = t0 + i;
      if (t >= T) break;
      int32_t g = group[t];
      if (g < 0) continue;
      int code = 0;
      if (pr >= 0) {
        int32_t gp = group[pr];
        if (g < gp) code = 1;
        else if (g == gp && pr != t - 1) code = 2;
      }
      if (code == 0 && t > 0 && group[t - 1] == g) {  // the same group continues
        bool p = is_prefix[t] != 0, pp = is_prefix[t - 1] != 0;
        if (p && !pp) code = 3;
        else if (!p && !pp && suffix[t] < suffix[t - 1]) code = 4;
      }
      if (code && err == LLONG_MAX) err = (long long)t * 8 + code;
      pr = t;
    }
    scan_slot(err, tid, sh, MinOp());
    const long long first_err = sh[kScanThreads - 1];
    __syncthreads();
    if (first_err != LLONG_MAX) {  // uniform branch: every thread read the same value
      if (tid == 0) {
        flag[0] = int32_t(first_err & 7);
        flag[1] = int32_t(first_err >> 3) + 1;
      }
      return;
    }
    if (chunk_max > carry_prev) carry_prev = chunk_max;
  }
  if (tid == 0) {
    flag[0] = 0;
    flag[1] = 0;
  }

  // Backward pass: first group break / completion break after each t.
  long long carry_g = T, carry_s = T;
  const int64_t n_chunks = (T + kChunk - 1) / kChunk;
  for (int64_t c = n_chunks - 1; c >= 0; --c) {
    const int64_t t0 = c * kChunk + int64_t(tid) * kScanItems;
    bool gb[kScanItems], sb[kScanItems];
    long long lg = LLONG_MAX, ls = LLONG_MAX;  // first break position in this thread
    for (int i = 0; i < kScanItems; ++i) {
      const int64_t t = t0 + i, e = t + 1;  // break between t and t+1 ?
      gb[i] = sb[i] = false;
      if (t >= T) continue;
      if (e >= T) {
        gb[i] = sb[i] = true;
      } else {
        const int32_t ge = group[e], gt = group[t];
        gb[i] = ge < 0 || gt < 0 || ge != gt;
        sb[i] = gb[i] || is_prefix[e] != is_prefix[t] || suffix[e] != suffix[t];
      }
      if (gb[i] && lg == LLONG_MAX) lg = e;
      if (sb[i] && ls == LLONG_MAX) ls = e;
    }
    __syncthreads();
    scan_slot(lg, rt, sh, MinOp());
    long long after_g = rt > 0 ? sh[rt - 1] : LLONG_MAX;  // threads with larger tid
    const long long all_g = sh[kScanThreads - 1];
    __syncthreads();
    scan_slot(ls, rt, sh, MinOp());
    long long after_s = rt > 0 ? sh[rt - 1] : LLONG_MAX;
    const long long all_s = sh[kScanThreads - 1];
    long long ng = after_g < carry_g ? after_g : carry_g;
    long long ns = after_s < carry_s ? after_s : carry_s;
    for (int i = kScanItems - 1; i >= 0; --i) {
      const int64_t t = t0 + i;
      if (t >= T) continue;
      if (gb[i]) ng = t + 1;
      if (sb[i]) ns = t + 1;
      end[t] = group[t] < 0 ? int32_t(t) : int32_t(is_prefix[t] ? ng : ns);
    }
    if (all_g < carry_g) carry_g = all_g;
    if (all_s < carry_s) carry_s = all_s;
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
// Step 2: classification
// ---------------------------------------------------------------------------
__global__ void k_map_init(int64_t nk, int32_t* row_ptr, int32_t* col_ptr, int64_t* info) {
  for (int64_t j = threadIdx.x; j <= nk; j += blockDim.x) col_ptr[j] = 0;
  if (threadIdx.x < 8) info[threadIdx.x] = 0;
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

__global__ __launch_bounds__(kFillThreads) void k_fill_csr(int64_t nq, int64_t nk,
                                                           const uint8_t* __restrict__ kinds,
                                                           const int32_t* __restrict__ row_ptr,
                                                           int32_t* col, uint8_t* kind) {
  __shared__ int sh_w[kFillThreads / 64];
  const int64_t i = blockIdx.x;
  int64_t base = row_ptr[i];
  for (int64_t j0 = 0; j0 < nk; j0 += kFillThreads) {
    int64_t j = j0 + threadIdx.x;
    uint8_t k = j < nk ? kinds[i * nk + j] : 0;
    int total;
    int pos = block_excl_count(k != 0, sh_w, &total);
    if (k) {
      col[base + pos] = int32_t(j);
      kind[base + pos] = k;
    }
    base += total;
  }
}

__global__ __launch_bounds__(kFillThreads) void k_fill_csc(int64_t nq, int64_t nk,
                                                           const uint8_t* __restrict__ kinds,
                                                           const int32_t* __restrict__ col_ptr,
                                                           int32_t* row, uint8_t* kind_csc) {
  __shared__ int sh_w[kFillThreads / 64];
  const int64_t j = blockIdx.x;
  int64_t base = col_ptr[j];
  for (int64_t i0 = 0; i0 < nq; i0 += kFillThreads) {
    int64_t i = i0 + threadIdx.x;
    uint8_t k = i < nq ? kinds[i * nk + j] : 0;
    int total;
    int pos = block_excl_count(k != 0, sh_w, &total);
    if (k) {
      row[base + pos] = int32_t(i);
      kind_csc[base + pos] = k;
    }
    base += total;
  }
}

}  // namespace

hipError_t launch_tokens_end(int64_t T, const int32_t* group, const int32_t* suffix,
                             const uint8_t* is_prefix, int32_t* end, int32_t* flag,
                             hipStream_t stream) {
  hipLaunchKernelGGL(k_tokens_end, dim3(1), dim3(kScanThreads), 0, stream, T, group, suffix,
                     is_prefix, end, flag);
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
  hipLaunchKernelGGL(k_map_init, dim3(1), dim3(1024), 0, stream, nk, row_ptr, col_ptr, info);
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

hipError_t launch_fill_lists(int64_t nq, int64_t nk, const uint8_t* kinds,
                             const int32_t* row_ptr, const int32_t* col_ptr, int32_t* col,
                             uint8_t* kind, int32_t* row, uint8_t* kind_csc,
                             hipStream_t stream) {
  hipLaunchKernelGGL(k_fill_csr, dim3(unsigned(nq)), dim3(kFillThreads), 0, stream, nq, nk,
                     kinds, row_ptr, col, kind);
  hipLaunchKernelGGL(k_fill_csc, dim3(unsigned(nk)), dim3(kFillThreads), 0, stream, nq, nk,
                     kinds, col_ptr, row, kind_csc);
  return hipGetLastError();
}
