// C ABI of libpsa.so: argument validation, tile-map lifetime, kernel dispatch.
//
// Every validation runs before the first launch of a call, so a failing call writes
// nothing the caller owns.  The map builder is the one call that waits on its
// stream (once), to size the sparse lists.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <new>
#include <numeric>
#include <string>
#include <utility>
#include <vector>

#include "psa.h"
#include "psa_internal.h"

namespace {
thread_local std::string g_last_error;

constexpr int64_t kMaxT = (int64_t{1} << 31) - 4096;
constexpr int64_t kMaxTiles = int64_t{1} << 32;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Carver {  // carves one allocation into 256-byte aligned pieces
  size_t off = 0;
  template <typename T>
  size_t take(size_t count) {
    size_t at = off;
    off = align_up(off + count * sizeof(T), 256);
    return at;
  }
};

psa_status check_tiles(int64_t T, int32_t bm, int32_t bn) {
  if (T < 0 || T > kMaxT) return psa_set_error(PSA_ERR_SHAPE, "T out of range [0, 2^31-4096]");
  if (bm < 1 || bm > 1024 || bn < 1 || bn > 1024)
    return psa_set_error(PSA_ERR_SHAPE, "block_m and block_n must lie in [1, 1024]");
  int64_t nq = (T + bm - 1) / bm, nk = (T + bn - 1) / bn;
  if (nq * nk > kMaxTiles) return psa_set_error(PSA_ERR_SHAPE, "too many tiles (T / block too large)");
  return PSA_OK;
}

// Device memory of maps comes from a library-owned stream-ordered pool per device:
// a map's buffers are allocated and freed on its build stream, so a map built after
// another is destroyed reuses that memory without a device-wide wait.  If the pool
// cannot be created the plain allocator is used instead.
hipMemPool_t pool_for(int dev) {
  static std::mutex mu;
  static std::vector<hipMemPool_t> pools;
  static std::vector<bool> tried;
  std::lock_guard<std::mutex> lock(mu);
  if (dev < 0) return nullptr;
  if (pools.size() <= size_t(dev)) {
    pools.resize(dev + 1, nullptr);
    tried.resize(dev + 1, false);
  }
  if (!tried[dev]) {
    tried[dev] = true;
    hipMemPoolProps props;
    std::memset(&props, 0, sizeof(props));
    props.allocType = hipMemAllocationTypePinned;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    hipMemPool_t pool = nullptr;
    if (hipMemPoolCreate(&pool, &props) == hipSuccess) {
      uint64_t keep = uint64_t{1} << 30;  // bytes kept for reuse across syncs
      (void)hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
      pools[dev] = pool;
    } else {
      (void)hipGetLastError();
    }
  }
  return pools[dev];
}

// Buffers of destroyed maps are kept in a small cache and handed to later builds on
// the same device (a buffer at least as large as asked and at most twice as large):
// a steady stream of build / destroy pairs then does no allocation at all.  Each
// cached buffer carries an event recorded on its last map's stream at destroy time;
// a build that takes it makes its own stream wait on that event first.
struct CachedBuf {
  int dev;
  size_t bytes;
  void* p;
  hipEvent_t ev;
};
std::mutex g_cache_mu;
std::vector<CachedBuf> g_cache;
constexpr size_t kCacheMaxBytes = size_t{256} << 20;
constexpr size_t kCacheMaxCount = 16;

void raw_free(int dev, void* p, hipEvent_t ev, hipStream_t s) {
  // after the work ordered before ev, back to the pool (or the plain allocator)
  if (ev) {
    (void)hipStreamWaitEvent(s, ev, 0);
    (void)hipEventDestroy(ev);
  }
  if (pool_for(dev)) (void)hipFreeAsync(p, s);
  else (void)hipFree(p);
}

hipError_t map_alloc(psa_tile_map* m, void** p, size_t bytes, size_t* got, hipEvent_t* ev) {
  bytes = align_up(std::max<size_t>(bytes, 1), size_t{1} << 16);
  *ev = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_cache_mu);
    int best = -1;
    for (size_t k = 0; k < g_cache.size(); ++k) {
      const CachedBuf& c = g_cache[k];
      if (c.dev == m->device && c.bytes >= bytes && c.bytes <= 2 * bytes &&
          (best < 0 || c.bytes < g_cache[best].bytes))
        best = int(k);
    }
    if (best >= 0) {
      const CachedBuf c = g_cache[best];
      g_cache.erase(g_cache.begin() + best);
      *p = c.p;
      *got = c.bytes;
      *ev = c.ev;
      return c.ev ? hipStreamWaitEvent(m->stream, c.ev, 0) : hipSuccess;
    }
  }
  *got = bytes;
  hipMemPool_t pool = pool_for(m->device);
  if (pool) return hipMallocFromPoolAsync(p, bytes, pool, m->stream);
  return hipMalloc(p, bytes);
}

void map_release(const psa_tile_map* m, void* p, size_t bytes, hipEvent_t ev) {
  if (!p) return;
  if (!ev && hipEventCreateWithFlags(&ev, hipEventDisableTiming) != hipSuccess) {
    (void)hipGetLastError();
    ev = nullptr;
  }
  if (ev && hipEventRecord(ev, m->stream) == hipSuccess) {
    std::vector<CachedBuf> evicted;
    {
      std::lock_guard<std::mutex> lock(g_cache_mu);
      g_cache.push_back({m->device, bytes, p, ev});
      size_t total = 0;
      for (const CachedBuf& c : g_cache) total += c.bytes;
      while (!g_cache.empty() && (g_cache.size() > kCacheMaxCount || total > kCacheMaxBytes)) {
        total -= g_cache.front().bytes;  // the oldest goes back to the allocator
        evicted.push_back(g_cache.front());
        g_cache.erase(g_cache.begin());
      }
    }
    for (const CachedBuf& c : evicted) raw_free(c.dev, c.p, c.ev, m->stream);
    return;
  }
  (void)hipGetLastError();
  raw_free(m->device, p, ev, m->stream);
}

void free_map(psa_tile_map* m) {
  if (!m) return;
  map_release(m, m->buf1, m->buf1_bytes, m->ev1);
  map_release(m, m->buf2, m->buf2_bytes, m->ev2);
  map_release(m, m->buf3, m->buf3_bytes, m->ev3);
  delete m;
}

// Phase-1 allocation.  Layout: end | kinds | scratch | info (8 x int64) | row_ptr |
// col_ptr.
struct Phase1 {
  int32_t* scratch = nullptr;  // per-k-tile summaries (4 x align64(nk) ints)
  int32_t* tok_scratch = nullptr;
  int64_t* info = nullptr;     // nnz, n_full, n_partial, first layout error
};

psa_status alloc_phase1(psa_tile_map* m, Phase1* ph) {
  Carver c;
  const int64_t nk1 = std::max<int64_t>(m->nk, 1);
  size_t o_end = c.take<int32_t>(std::max<int64_t>(m->T, 1));
  size_t o_kinds = c.take<uint8_t>(std::max<int64_t>(m->nq * m->nk, 1));
  size_t o_scr = c.take<int32_t>(4 * align_up(nk1, 64));
  size_t o_tok = c.take<int32_t>(std::max<int64_t>(tokens_scratch_ints(m->T), 1));
  size_t o_info = c.take<int64_t>(8);
  size_t o_rp = c.take<int32_t>(m->nq + 1);
  size_t o_cp = c.take<int32_t>(m->nk + 1);
  const size_t total = c.off;
  hipError_t e = map_alloc(m, &m->buf1, total, &m->buf1_bytes, &m->ev1);
  if (e != hipSuccess) {
    m->buf1 = nullptr;
    (void)hipGetLastError();
    return psa_set_error(PSA_ERR_ALLOC, "device allocation of the tile map failed");
  }
  char* b = static_cast<char*>(m->buf1);
  m->end = reinterpret_cast<int32_t*>(b + o_end);
  m->kinds = reinterpret_cast<uint8_t*>(b + o_kinds);
  m->row_ptr = reinterpret_cast<int32_t*>(b + o_rp);
  m->col_ptr = reinterpret_cast<int32_t*>(b + o_cp);
  ph->scratch = reinterpret_cast<int32_t*>(b + o_scr);
  ph->tok_scratch = reinterpret_cast<int32_t*>(b + o_tok);
  ph->info = reinterpret_cast<int64_t*>(b + o_info);
  e = launch_map_init(m->nk, m->row_ptr, m->col_ptr, ph->info, m->stream);
  if (e != hipSuccess) return psa_hip_error(e, "tile map init launch");
  return PSA_OK;
}

// Classification of the map's encoding (interval or node form) and the one wait: the
// counts and the layout verdict land in info_h.
psa_status classify_and_wait(psa_tile_map* m, const Phase1& ph, int64_t* info_h) {
  const size_t stride = align_up(std::max<int64_t>(m->nk, 1), 64);
  hipError_t e;
  if (m->form == kFormNodes)
    e = launch_classify_nodes(m->T, m->bm, m->bn, m->nq, m->nk, m->nkey, m->nlo, m->nw,
                              m->causal, m->kinds, m->row_ptr, m->col_ptr, ph.scratch, ph.info,
                              m->stream);
  else
    e = launch_classify(m->T, m->bm, m->bn, m->nq, m->nk, m->end, m->kinds, m->row_ptr,
                        m->col_ptr, ph.scratch, ph.scratch + stride, ph.info, m->stream);
  if (e != hipSuccess) return psa_hip_error(e, "tile classification launch");
  if ((e = hipMemcpyAsync(info_h, ph.info, 8 * sizeof(int64_t), hipMemcpyDeviceToHost,
                          m->stream)) != hipSuccess ||
      (e = hipStreamSynchronize(m->stream)) != hipSuccess)
    return psa_hip_error(e, "tile map readback");
  return PSA_OK;
}

// The node-form arrays (key | lo | w) in their own buffer.
psa_status alloc_nodes(psa_tile_map* m) {
  const size_t arr = align_up(size_t(std::max<int64_t>(m->T, 1)) * 4, 256);
  if (map_alloc(m, &m->buf3, 3 * arr, &m->buf3_bytes, &m->ev3) != hipSuccess) {
    m->buf3 = nullptr;
    (void)hipGetLastError();
    return psa_set_error(PSA_ERR_ALLOC, "device allocation of the node arrays failed");
  }
  char* b = static_cast<char*>(m->buf3);
  m->nkey = reinterpret_cast<int32_t*>(b);
  m->nlo = reinterpret_cast<int32_t*>(b + arr);
  m->nw = reinterpret_cast<int32_t*>(b + 2 * arr);
  m->form = kFormNodes;
  return PSA_OK;
}

// Sparse lists from a classified map (info_h from classify_and_wait).
psa_status finish_lists(psa_tile_map* m, const int64_t* info_h, psa_tile_map** out) {
  hipError_t e;
  m->nnz = info_h[0];
  m->n_full = info_h[1];
  m->n_partial = info_h[2];

  Carver c;
  size_t o_col = c.take<int32_t>(std::max<int64_t>(m->nnz, 1));
  size_t o_kind = c.take<uint8_t>(std::max<int64_t>(m->nnz, 1));
  size_t o_row = c.take<int32_t>(std::max<int64_t>(m->nnz, 1));
  size_t o_kc = c.take<uint8_t>(std::max<int64_t>(m->nnz, 1));
  size_t o_qo = c.take<int32_t>(std::max<int64_t>(m->nq + m->nk, 1));  // qorder | korder
  if ((e = map_alloc(m, &m->buf2, c.off, &m->buf2_bytes, &m->ev2)) != hipSuccess) {
    m->buf2 = nullptr;
    (void)hipGetLastError();
    return psa_set_error(PSA_ERR_ALLOC, "device allocation of the tile lists failed");
  }
  char* b2 = static_cast<char*>(m->buf2);
  m->col = reinterpret_cast<int32_t*>(b2 + o_col);
  m->kind = reinterpret_cast<uint8_t*>(b2 + o_kind);
  m->row = reinterpret_cast<int32_t*>(b2 + o_row);
  m->kind_csc = reinterpret_cast<uint8_t*>(b2 + o_kc);
  m->qorder = reinterpret_cast<int32_t*>(b2 + o_qo);
  m->korder = m->qorder + m->nq;

  e = launch_fill_lists(m->nq, m->nk, m->kinds, m->row_ptr, m->col_ptr, m->col, m->kind,
                        m->row, m->kind_csc, m->qorder, m->korder, m->stream);
  if (e != hipSuccess) return psa_hip_error(e, "tile list launch");
  *out = m;
  return PSA_OK;
}

psa_status check_attn_args(const psa_tile_map* map, psa_dtype dtype, int64_t T, int32_t hq,
                           int32_t hkv, int32_t d, float scale, psa_pass pass) {
  if (!map) return psa_set_error(PSA_ERR_NULL, "map is NULL");
  if (dtype != PSA_FP32 && dtype != PSA_BF16 && dtype != PSA_FP8_E4M3)
    return psa_set_error(PSA_ERR_DTYPE, "unknown dtype");
  if (T < 0 || T > kMaxT) return psa_set_error(PSA_ERR_SHAPE, "T out of range");
  if (hq < 1 || hkv < 1 || hq % hkv != 0)
    return psa_set_error(PSA_ERR_SHAPE, "need hq >= 1, hkv >= 1 and hq % hkv == 0");
  if (T * int64_t{hq} * d > (int64_t{1} << 40))
    return psa_set_error(PSA_ERR_SHAPE, "tensor too large");
  bool ok = pass == PSA_PASS_FWD ? fwd_supported(dtype, d) : bwd_supported(dtype, d);
  if (!ok) return psa_set_error(PSA_ERR_UNSUPPORTED, "head_dim " + std::to_string(d) +
                                                          " is not compiled for this dtype");
  if (!std::isfinite(scale)) return psa_set_error(PSA_ERR_VALUE, "scale is not finite");
  if (T != map->T)
    return psa_set_error(PSA_ERR_MAP_MISMATCH, "T = " + std::to_string(T) +
                                                   " but the map was built for T = " +
                                                   std::to_string(map->T));
  if (map->bm != kTileM || map->bn != kTileN)
    return psa_set_error(PSA_ERR_MAP_MISMATCH,
                         "map tile shape " + std::to_string(map->bm) + "x" +
                             std::to_string(map->bn) + " is not the kernel tile shape " +
                             std::to_string(kTileM) + "x" + std::to_string(kTileN));
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != map->device)
    return psa_set_error(PSA_ERR_MAP_MISMATCH, "map was built on another device");
  return PSA_OK;
}

}  // namespace

psa_status psa_set_error(psa_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

psa_status psa_hip_error(hipError_t e, const char* what) {
  g_last_error = std::string(what) + ": " + hipGetErrorString(e);
  return PSA_ERR_HIP;
}

extern "C" {

int32_t psa_abi_version(void) { return PSA_ABI_VERSION; }

const char* psa_status_string(psa_status s) {
  switch (s) {
    case PSA_OK: return "ok";
    case PSA_ERR_NULL: return "null pointer";
    case PSA_ERR_SHAPE: return "shape out of range";
    case PSA_ERR_LAYOUT: return "metadata layout not accepted";
    case PSA_ERR_DTYPE: return "unknown dtype";
    case PSA_ERR_UNSUPPORTED: return "unsupported head_dim / dtype";
    case PSA_ERR_MAP_MISMATCH: return "tile map does not match the call";
    case PSA_ERR_WORKSPACE: return "workspace missing or too small";
    case PSA_ERR_HIP: return "HIP runtime error";
    case PSA_ERR_ALLOC: return "allocation failed";
    case PSA_ERR_VALUE: return "invalid scalar argument";
  }
  return "unknown status";
}

const char* psa_last_error(void) { return g_last_error.c_str(); }

psa_status psa_tile_shape(psa_pass pass, psa_dtype dtype, int32_t d, int32_t* block_m,
                          int32_t* block_n) {
  if (!block_m || !block_n) return psa_set_error(PSA_ERR_NULL, "output pointer is NULL");
  if (dtype != PSA_FP32 && dtype != PSA_BF16 && dtype != PSA_FP8_E4M3)
    return psa_set_error(PSA_ERR_DTYPE, "unknown dtype");
  bool ok = pass == PSA_PASS_FWD ? fwd_supported(dtype, d)
                                 : pass == PSA_PASS_BWD ? bwd_supported(dtype, d) : false;
  if (!ok) return psa_set_error(PSA_ERR_UNSUPPORTED, "no kernel for this pass / dtype / head_dim");
  *block_m = kTileM;
  *block_n = kTileN;
  return PSA_OK;
}

psa_status psa_build_tile_map_tokens(int64_t T, const int32_t* group, const int32_t* suffix,
                                     const uint8_t* is_prefix, int32_t block_m,
                                     int32_t block_n, void* stream, psa_tile_map** out) {
  return psa_build_tile_map_tokens_ex(T, group, suffix, is_prefix, block_m, block_n, 0, stream,
                                      out);
}

psa_status psa_build_tile_map_tokens_ex(int64_t T, const int32_t* group, const int32_t* suffix,
                                        const uint8_t* is_prefix, int32_t block_m,
                                        int32_t block_n, int32_t flags, void* stream,
                                        psa_tile_map** out) {
  if (!out) return psa_set_error(PSA_ERR_NULL, "out is NULL");
  psa_status st = check_tiles(T, block_m, block_n);
  if (st != PSA_OK) return st;
  if ((flags & ~PSA_MAP_NODE_FORM) != 0) return psa_set_error(PSA_ERR_VALUE, "unknown flag bit");
  if (T > 0 && (!group || !suffix || !is_prefix))
    return psa_set_error(PSA_ERR_NULL, "label pointer is NULL");
  psa_tile_map* m = new (std::nothrow) psa_tile_map();
  if (!m) return psa_set_error(PSA_ERR_ALLOC, "host allocation failed");
  m->T = T;
  m->bm = block_m;
  m->bn = block_n;
  m->nq = (T + block_m - 1) / block_m;
  m->nk = (T + block_n - 1) / block_n;
  m->stream = static_cast<hipStream_t>(stream);
  hipError_t e = hipGetDevice(&m->device);
  if (e != hipSuccess) {
    free_map(m);
    return psa_hip_error(e, "hipGetDevice");
  }
  Phase1 ph;
  if ((st = alloc_phase1(m, &ph)) != PSA_OK) {
    free_map(m);
    return st;
  }
  int64_t info_h[8];
  if (!(flags & PSA_MAP_NODE_FORM)) {
    // the interval form, when the layout is packed (the verdict comes with the counts)
    e = launch_tokens_end(T, group, suffix, is_prefix, m->end, ph.tok_scratch, ph.info,
                          m->stream);
    if (e != hipSuccess) {
      free_map(m);
      return psa_hip_error(e, "label scan launch");
    }
    if ((st = classify_and_wait(m, ph, info_h)) != PSA_OK) {
      free_map(m);
      return st;
    }
  }
  if ((flags & PSA_MAP_NODE_FORM) || info_h[3] != -1) {
    // any other layout: the node form (numbering by a sort of the node keys)
    void* scr = nullptr;
    size_t scr_bytes = 0;
    hipEvent_t scr_ev = nullptr;
    const size_t need = tokens_nodes_scratch_bytes(T);
    if ((st = alloc_nodes(m)) != PSA_OK) {
      free_map(m);
      return st;
    }
    if (map_alloc(m, &scr, need, &scr_bytes, &scr_ev) != hipSuccess) {
      (void)hipGetLastError();
      free_map(m);
      return psa_set_error(PSA_ERR_ALLOC, "device allocation of the node sort scratch failed");
    }
    e = launch_map_init(m->nk, m->row_ptr, m->col_ptr, ph.info, m->stream);
    if (e == hipSuccess)
      e = launch_tokens_nodes(T, group, suffix, is_prefix, m->nkey, m->nlo, m->nw, scr,
                              scr_bytes, m->stream);
    map_release(m, scr, scr_bytes, scr_ev);  // reusable once the launches are done
    if (e != hipSuccess) {
      free_map(m);
      return psa_hip_error(e, "label numbering launch");
    }
    if ((st = classify_and_wait(m, ph, info_h)) != PSA_OK) {
      free_map(m);
      return st;
    }
  }
  st = finish_lists(m, info_h, out);
  if (st != PSA_OK) free_map(m);
  return st;
}

psa_status psa_build_tile_map_tree(int64_t n_nodes, const int32_t* node_lengths,
                                   int64_t n_paths, const int32_t* path_ptr,
                                   const int32_t* path_nodes, int64_t T, int32_t block_m,
                                   int32_t block_n, void* stream, psa_tile_map** out) {
  return psa_build_tile_map_tree_ex(n_nodes, node_lengths, n_paths, path_ptr, path_nodes, T,
                                    block_m, block_n, 0, stream, out);
}

psa_status psa_build_tile_map_tree_ex(int64_t n_nodes, const int32_t* node_lengths,
                                      int64_t n_paths, const int32_t* path_ptr,
                                      const int32_t* path_nodes, int64_t T, int32_t block_m,
                                      int32_t block_n, int32_t flags, void* stream,
                                      psa_tile_map** out) {
  if (!out) return psa_set_error(PSA_ERR_NULL, "out is NULL");
  psa_status st = check_tiles(T, block_m, block_n);
  if (st != PSA_OK) return st;
  if ((flags & ~PSA_MAP_NODE_FORM) != 0) return psa_set_error(PSA_ERR_VALUE, "unknown flag bit");
  if (n_nodes < 0 || n_paths < 0) return psa_set_error(PSA_ERR_SHAPE, "negative count");
  if (n_nodes > 0 && (!node_lengths || !path_ptr || (!path_nodes && n_paths > 0)))
    return psa_set_error(PSA_ERR_NULL, "tree pointer is NULL");
  if (n_nodes > 0 && n_paths == 0)
    return psa_set_error(PSA_ERR_LAYOUT, "nodes given but no sample path");

  // --- host validation: parents (each before its children), subtree extents ---
  std::vector<int64_t> parent(n_nodes, -2);
  std::vector<int64_t> start(n_nodes + 1, 0);
  for (int64_t n = 0; n < n_nodes; ++n) {
    if (node_lengths[n] < 0) return psa_set_error(PSA_ERR_LAYOUT, "negative node length");
    start[n + 1] = start[n] + node_lengths[n];
  }
  if (start[n_nodes] > T)
    return psa_set_error(PSA_ERR_SHAPE, "T is shorter than sum(node_lengths)");
  if (n_paths > 0 && path_ptr[0] != 0) return psa_set_error(PSA_ERR_LAYOUT, "path_ptr[0] != 0");
  for (int64_t s = 0; s < n_paths; ++s) {
    int64_t a = path_ptr[s], b = path_ptr[s + 1];
    if (b <= a) return psa_set_error(PSA_ERR_LAYOUT, "empty or decreasing sample path");
    int64_t prev = -1;
    for (int64_t k = a; k < b; ++k) {
      int64_t node = path_nodes[k];
      if (node < 0 || node >= n_nodes)
        return psa_set_error(PSA_ERR_LAYOUT, "path node index out of range");
      if (parent[node] == -2)
        parent[node] = prev;
      else if (parent[node] != prev)
        return psa_set_error(PSA_ERR_LAYOUT,
                             "node " + std::to_string(node) + " has two different parents");
      prev = node;
    }
  }
  for (int64_t n = 0; n < n_nodes; ++n) {
    if (parent[n] == -2)
      return psa_set_error(PSA_ERR_LAYOUT, "node " + std::to_string(n) + " lies on no path");
    if (parent[n] >= n)
      return psa_set_error(PSA_ERR_LAYOUT, "node " + std::to_string(n) +
                                               " comes before its parent " +
                                               std::to_string(parent[n]));
  }
  // depth-first pre-order (every subtree one contiguous run of nodes) has the
  // interval form; any other order of parents before children gets the node form
  bool dfs = true;
  {
    std::vector<int64_t> stack;
    for (int64_t n = 0; n < n_nodes && dfs; ++n) {
      if (parent[n] == -1) {
        stack.clear();
      } else {
        while (!stack.empty() && stack.back() != parent[n]) stack.pop_back();
        dfs = !stack.empty();
      }
      stack.push_back(n);
    }
  }
  const bool nodes = !dfs || (flags & PSA_MAP_NODE_FORM);
  std::vector<int64_t> table;
  if (!nodes) {  // node start | token end of the node's subtree
    std::vector<int64_t> sub_end(n_nodes);
    for (int64_t n = 0; n < n_nodes; ++n) sub_end[n] = n + 1;
    for (int64_t n = n_nodes - 1; n >= 0; --n)
      if (parent[n] >= 0) sub_end[parent[n]] = std::max(sub_end[parent[n]], sub_end[n]);
    table.assign(2 * std::max<int64_t>(n_nodes, 1), 0);
    for (int64_t n = 0; n < n_nodes; ++n) {
      table[n] = start[n];
      table[n_nodes + n] = start[sub_end[n]];
    }
  } else {  // node start | pre-order number | subtree size (in nodes)
    std::vector<int64_t> first_child(n_nodes, -1), next_sib(n_nodes, -1), last_child(n_nodes, -1);
    std::vector<int64_t> roots;
    for (int64_t n = 0; n < n_nodes; ++n) {
      const int64_t p = parent[n];
      if (p < 0) {
        roots.push_back(n);
      } else {
        if (last_child[p] < 0) first_child[p] = n;
        else next_sib[last_child[p]] = n;
        last_child[p] = n;
      }
    }
    table.assign(3 * std::max<int64_t>(n_nodes, 1), 0);
    int64_t* pre = table.data() + n_nodes;
    int64_t* size = table.data() + 2 * n_nodes;
    int64_t counter = 0;
    std::vector<int64_t> stack;
    for (int64_t r : roots) {  // iterative depth-first walk, children in index order
      stack.push_back(r);
      while (!stack.empty()) {
        const int64_t n = stack.back();
        stack.pop_back();
        pre[n] = counter++;
        std::vector<int64_t> kids;
        for (int64_t c = first_child[n]; c >= 0; c = next_sib[c]) kids.push_back(c);
        for (auto it = kids.rbegin(); it != kids.rend(); ++it) stack.push_back(*it);
      }
    }
    for (int64_t n = 0; n < n_nodes; ++n) size[n] = 1;
    for (int64_t n = n_nodes - 1; n >= 0; --n)  // children come after their parent
      if (parent[n] >= 0) size[parent[n]] += size[n];
    for (int64_t n = 0; n < n_nodes; ++n) table[n] = start[n];
  }

  psa_tile_map* m = new (std::nothrow) psa_tile_map();
  if (!m) return psa_set_error(PSA_ERR_ALLOC, "host allocation failed");
  m->T = T;
  m->bm = block_m;
  m->bn = block_n;
  m->nq = (T + block_m - 1) / block_m;
  m->nk = (T + block_n - 1) / block_n;
  m->stream = static_cast<hipStream_t>(stream);
  hipError_t e = hipGetDevice(&m->device);
  if (e != hipSuccess) {
    free_map(m);
    return psa_hip_error(e, "hipGetDevice");
  }
  Phase1 ph;
  if ((st = alloc_phase1(m, &ph)) != PSA_OK) {
    free_map(m);
    return st;
  }
  void* d_table = nullptr;
  size_t table_bytes = 0;
  hipEvent_t table_ev = nullptr;
  if (n_nodes > 0) {
    if ((e = map_alloc(m, &d_table, table.size() * sizeof(int64_t), &table_bytes, &table_ev)) !=
        hipSuccess) {
      (void)hipGetLastError();
      free_map(m);
      return psa_set_error(PSA_ERR_ALLOC, "device allocation of the node table failed");
    }
    if ((e = hipMemcpyAsync(d_table, table.data(), table.size() * sizeof(int64_t),
                            hipMemcpyHostToDevice, m->stream)) != hipSuccess) {
      map_release(m, d_table, table_bytes, table_ev);
      free_map(m);
      return psa_hip_error(e, "node table upload");
    }
  }
  const int64_t* dt = static_cast<const int64_t*>(d_table);
  if (nodes) {
    if ((st = alloc_nodes(m)) != PSA_OK) {
      map_release(m, d_table, table_bytes, table_ev);
      free_map(m);
      return st;
    }
    e = launch_tree_nodes(T, n_nodes, dt, dt ? dt + n_nodes : nullptr,
                          dt ? dt + 2 * n_nodes : nullptr, start[n_nodes], m->nkey, m->nlo,
                          m->nw, m->stream);
  } else {
    e = launch_tree_end(T, n_nodes, dt, dt ? dt + n_nodes : nullptr, start[n_nodes], m->end,
                        m->stream);
  }
  map_release(m, d_table, table_bytes, table_ev);  // reusable once the launch is done
  if (e != hipSuccess) {
    free_map(m);
    return psa_hip_error(e, "tree expansion launch");
  }
  int64_t info_h[8];
  if ((st = classify_and_wait(m, ph, info_h)) != PSA_OK) {
    free_map(m);
    return st;
  }
  st = finish_lists(m, info_h, out);
  if (st != PSA_OK) free_map(m);
  return st;
}

psa_status psa_build_tile_map_draft(int64_t ctx_len, int32_t block_size, int64_t n_blocks,
                                    const int32_t* anchors, const uint8_t* keep,
                                    const int32_t* ctx_doc, const int32_t* anchor_doc,
                                    int32_t flags, int64_t T, int32_t block_m, int32_t block_n,
                                    void* stream, psa_tile_map** out) {
  if (!out) return psa_set_error(PSA_ERR_NULL, "out is NULL");
  psa_status st = check_tiles(T, block_m, block_n);
  if (st != PSA_OK) return st;
  if ((flags & ~PSA_DRAFT_CAUSAL) != 0) return psa_set_error(PSA_ERR_VALUE, "unknown flag bit");
  if (ctx_len < 0 || n_blocks < 0 || block_size < 1)
    return psa_set_error(PSA_ERR_SHAPE, "need ctx_len >= 0, n_blocks >= 0, block_size >= 1");
  if (n_blocks > (int64_t{1} << 31) || ctx_len + n_blocks * int64_t(block_size) > T)
    return psa_set_error(PSA_ERR_SHAPE, "T is shorter than ctx_len + n_blocks * block_size");
  if ((ctx_len + 1) * n_blocks > (int64_t{1} << 32))
    return psa_set_error(PSA_ERR_SHAPE, "(ctx_len + 1) * n_blocks must not exceed 2^32");
  if (n_blocks > 0 && !anchors) return psa_set_error(PSA_ERR_NULL, "anchors is NULL");
  if (ctx_len > 0 && n_blocks > 0 && (ctx_doc == nullptr) != (anchor_doc == nullptr))
    return psa_set_error(PSA_ERR_NULL, "ctx_doc and anchor_doc are given together or not at all");
  if (ctx_len == 0 || n_blocks == 0) ctx_doc = anchor_doc = nullptr;  // nothing to compare
  psa_tile_map* m = new (std::nothrow) psa_tile_map();
  if (!m) return psa_set_error(PSA_ERR_ALLOC, "host allocation failed");
  m->T = T;
  m->bm = block_m;
  m->bn = block_n;
  m->nq = (T + block_m - 1) / block_m;
  m->nk = (T + block_n - 1) / block_n;
  m->causal = (flags & PSA_DRAFT_CAUSAL) ? 1 : 0;
  m->stream = static_cast<hipStream_t>(stream);
  hipError_t e = hipGetDevice(&m->device);
  if (e != hipSuccess) {
    free_map(m);
    return psa_hip_error(e, "hipGetDevice");
  }
  Phase1 ph;
  if ((st = alloc_phase1(m, &ph)) != PSA_OK || (st = alloc_nodes(m)) != PSA_OK) {
    free_map(m);
    return st;
  }
  void* scr = nullptr;
  size_t scr_bytes = 0;
  hipEvent_t scr_ev = nullptr;
  if (map_alloc(m, &scr, draft_scratch_bytes(n_blocks), &scr_bytes, &scr_ev) != hipSuccess) {
    (void)hipGetLastError();
    free_map(m);
    return psa_set_error(PSA_ERR_ALLOC, "device allocation of the block sort scratch failed");
  }
  e = launch_draft_nodes(T, ctx_len, block_size, n_blocks, anchors, keep, ctx_doc, anchor_doc,
                         m->nkey, m->nlo, m->nw, scr, scr_bytes, ph.info, m->stream);
  map_release(m, scr, scr_bytes, scr_ev);  // reusable once the launches are done
  if (e != hipSuccess) {
    free_map(m);
    return psa_hip_error(e, "draft numbering launch");
  }
  int64_t info_h[8];
  if ((st = classify_and_wait(m, ph, info_h)) != PSA_OK) {
    free_map(m);
    return st;
  }
  if (info_h[3] != -1) {
    free_map(m);
    return psa_set_error(PSA_ERR_LAYOUT, "anchor of block " +
                                             std::to_string(uint64_t(info_h[3]) >> 3) +
                                             " lies outside [0, ctx_len]");
  }
  st = finish_lists(m, info_h, out);
  if (st != PSA_OK) free_map(m);
  return st;
}

psa_status psa_tile_map_info_get(const psa_tile_map* map, psa_tile_map_info* out) {
  if (!map || !out) return psa_set_error(PSA_ERR_NULL, "map or out is NULL");
  out->T = map->T;
  out->block_m = map->bm;
  out->block_n = map->bn;
  out->n_qtiles = map->nq;
  out->n_ktiles = map->nk;
  out->nnz = map->nnz;
  out->n_full = map->n_full;
  out->n_partial = map->n_partial;
  out->form = map->form;
  out->causal = map->causal;
  return PSA_OK;
}

psa_status psa_tile_map_export(const psa_tile_map* map, int32_t* end, uint8_t* kinds,
                               int32_t* row_ptr, int32_t* col, uint8_t* kind,
                               int32_t* col_ptr, int32_t* row, uint8_t* kind_csc) {
  if (!map) return psa_set_error(PSA_ERR_NULL, "map is NULL");
  if (end && map->form != kFormInterval && map->T > 0)
    return psa_set_error(PSA_ERR_VALUE, "a node-form map has no end[] (export its nodes)");
  hipError_t e = hipStreamSynchronize(map->stream);
  if (e != hipSuccess) return psa_hip_error(e, "hipStreamSynchronize");
  struct Item {
    void* dst;
    const void* src;
    size_t bytes;
  } items[] = {
      {end, map->end, size_t(map->T) * 4},
      {kinds, map->kinds, size_t(map->nq * map->nk)},
      {row_ptr, map->row_ptr, size_t(map->nq + 1) * 4},
      {col, map->col, size_t(map->nnz) * 4},
      {kind, map->kind, size_t(map->nnz)},
      {col_ptr, map->col_ptr, size_t(map->nk + 1) * 4},
      {row, map->row, size_t(map->nnz) * 4},
      {kind_csc, map->kind_csc, size_t(map->nnz)},
  };
  for (const Item& it : items) {
    if (!it.dst || it.bytes == 0) continue;
    if ((e = hipMemcpy(it.dst, it.src, it.bytes, hipMemcpyDeviceToHost)) != hipSuccess)
      return psa_hip_error(e, "tile map export");
  }
  return PSA_OK;
}

psa_status psa_tile_map_export_nodes(const psa_tile_map* map, int32_t* key, int32_t* lo,
                                     int32_t* w) {
  if (!map) return psa_set_error(PSA_ERR_NULL, "map is NULL");
  hipError_t e = hipStreamSynchronize(map->stream);
  if (e != hipSuccess) return psa_hip_error(e, "hipStreamSynchronize");
  const size_t n = size_t(map->T);
  if (n == 0) return PSA_OK;
  if (map->form == kFormNodes) {
    const std::pair<int32_t*, const int32_t*> items[] = {
        {key, map->nkey}, {lo, map->nlo}, {w, map->nw}};
    for (const auto& it : items) {
      if (!it.first) continue;
      if ((e = hipMemcpy(it.first, it.second, n * 4, hipMemcpyDeviceToHost)) != hipSuccess)
        return psa_hip_error(e, "tile map export");
    }
    return PSA_OK;
  }
  // interval form written as nodes: key t, range [t, end[t]) (kv <= q < end[kv])
  std::vector<int32_t> end(n);
  if ((e = hipMemcpy(end.data(), map->end, n * 4, hipMemcpyDeviceToHost)) != hipSuccess)
    return psa_hip_error(e, "tile map export");
  for (size_t t = 0; t < n; ++t) {
    if (key) key[t] = int32_t(t);
    if (lo) lo[t] = int32_t(t);
    if (w) w[t] = end[t] - int32_t(t);
  }
  return PSA_OK;
}

void psa_tile_map_destroy(psa_tile_map* map) { free_map(map); }

psa_status psa_fwd(const psa_tile_map* map, psa_dtype dtype, int64_t T, int32_t hq,
                   int32_t hkv, int32_t d, float scale, const void* q, const void* k,
                   const void* v, void* o, float* lse, void* stream) {
  psa_status st = check_attn_args(map, dtype, T, hq, hkv, d, scale, PSA_PASS_FWD);
  if (st != PSA_OK) return st;
  if (T == 0) return PSA_OK;
  // lse may be NULL: a forward whose LSE nobody reads (no backward follows)
  if (!q || !k || !v || !o) return psa_set_error(PSA_ERR_NULL, "tensor pointer is NULL");
  AttnShape s{T, hq, hkv, d, scale > 0.f ? scale : 1.0f / std::sqrt(float(d))};
  hipError_t e = launch_fwd(*map, dtype, s, q, k, v, o, lse, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return psa_hip_error(e, "forward launch");
  return PSA_OK;
}

psa_status psa_bwd_workspace_size(const psa_tile_map* map, psa_dtype dtype, int64_t T,
                                  int32_t hq, int32_t hkv, int32_t d, size_t* bytes) {
  if (!bytes) return psa_set_error(PSA_ERR_NULL, "bytes is NULL");
  psa_status st = check_attn_args(map, dtype, T, hq, hkv, d, 1.0f, PSA_PASS_BWD);
  if (st != PSA_OK) return st;
  *bytes = bwd_workspace_bytes(AttnShape{T, hq, hkv, d, 1.0f});
  return PSA_OK;
}

psa_status psa_bwd_stages(const psa_tile_map* map, psa_dtype dtype, psa_dtype grad_dtype,
                          int64_t T, int32_t hq, int32_t hkv, int32_t d, float scale,
                          const void* q, const void* k, const void* v, const void* o,
                          const float* lse, const void* dout, void* dq, void* dk, void* dv,
                          void* workspace, size_t workspace_bytes, int32_t flags,
                          void* stream) {
  psa_status st = check_attn_args(map, dtype, T, hq, hkv, d, scale, PSA_PASS_BWD);
  if (st != PSA_OK) return st;
  if (grad_dtype != PSA_FP32 && grad_dtype != dtype)
    return psa_set_error(PSA_ERR_DTYPE, "grad_dtype must be PSA_FP32 or the input dtype");
  const int32_t stages = flags & PSA_STAGE_ALL;
  const bool split = (flags & PSA_BWD_SPLIT_PDS) != 0;
  if (stages == 0 || (flags & ~(PSA_STAGE_ALL | PSA_BWD_SPLIT_PDS)) != 0)
    return psa_set_error(PSA_ERR_VALUE,
                         "flags must hold a nonzero set of stages and no unknown bit");
  if (T == 0) return PSA_OK;
  const bool pre = stages & PSA_STAGE_PREPARE, kv = stages & PSA_STAGE_DKDV,
             dqs = stages & PSA_STAGE_DQ;
  if ((pre && (!o || !lse || !dout)) || ((kv || dqs) && (!q || !k || !v || !dout)) ||
      (kv && (!dk || !dv)) || (dqs && !dq))
    return psa_set_error(PSA_ERR_NULL, "tensor pointer is NULL");
  AttnShape s{T, hq, hkv, d, scale > 0.f ? scale : 1.0f / std::sqrt(float(d))};
  size_t need = bwd_workspace_bytes(s);
  if (!workspace || workspace_bytes < need)
    return psa_set_error(PSA_ERR_WORKSPACE, "workspace needs " + std::to_string(need) + " bytes");
  hipError_t e = launch_bwd(*map, dtype, grad_dtype, s, q, k, v, o, lse, dout, dq, dk, dv,
                            workspace, stages, split, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return psa_hip_error(e, "backward launch");
  return PSA_OK;
}

psa_status psa_bwd(const psa_tile_map* map, psa_dtype dtype, psa_dtype grad_dtype, int64_t T,
                   int32_t hq, int32_t hkv, int32_t d, float scale, const void* q,
                   const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv, void* workspace,
                   size_t workspace_bytes, void* stream) {
  return psa_bwd_stages(map, dtype, grad_dtype, T, hq, hkv, d, scale, q, k, v, o, lse, dout,
                        dq, dk, dv, workspace, workspace_bytes, PSA_STAGE_ALL, stream);
}

psa_status psa_bwd_noalloc(const psa_tile_map* map, psa_dtype dtype, psa_dtype grad_dtype,
                           int64_t T, int32_t hq, int32_t hkv, int32_t d, float scale,
                           const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           void* stream) {
  psa_status st = check_attn_args(map, dtype, T, hq, hkv, d, scale, PSA_PASS_BWD);
  if (st != PSA_OK) return st;
  if (grad_dtype != PSA_FP32 && grad_dtype != dtype)
    return psa_set_error(PSA_ERR_DTYPE, "grad_dtype must be PSA_FP32 or the input dtype");
  const size_t need = bwd_workspace_bytes(AttnShape{T, hq, hkv, d, 1.0f});
  if (need > kBwdScratchBytes)
    return psa_set_error(PSA_ERR_WORKSPACE,
                         "psa_bwd_noalloc: these sizes need " + std::to_string(need) +
                             " bytes of scratch, above its fixed " +
                             std::to_string(kBwdScratchBytes) +
                             " (2 x T x hq x 4 bytes); use psa_bwd with a workspace");
  if (T == 0) return PSA_OK;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv)
    return psa_set_error(PSA_ERR_NULL, "tensor pointer is NULL");
  void* ws = nullptr;
  hipError_t e = bwd_scratch(&ws);
  if (e != hipSuccess) return psa_hip_error(e, "device scratch of psa_bwd_noalloc");
  AttnShape s{T, hq, hkv, d, scale > 0.f ? scale : 1.0f / std::sqrt(float(d))};
  e = launch_bwd(*map, dtype, grad_dtype, s, q, k, v, o, lse, dout, dq, dk, dv, ws,
                 PSA_STAGE_ALL, false, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return psa_hip_error(e, "backward launch");
  return PSA_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Fold / unfold of rollout groups (fold.hip).  The host checks the length tables and
// builds the segment table; it goes to the caller's workspace on the stream.
// ---------------------------------------------------------------------------
namespace {

struct Rollouts {
  int64_t n_groups = 0, n_comp = 0, folded = 0;
};

psa_status check_rollouts(int64_t n_groups, const int32_t* prompt_len, const int32_t* comp_ptr,
                          const int32_t* comp_len, Rollouts* r) {
  if (n_groups < 0) return psa_set_error(PSA_ERR_SHAPE, "negative n_groups");
  if (n_groups > 0 && (!prompt_len || !comp_ptr))
    return psa_set_error(PSA_ERR_NULL, "length table is NULL");
  if (n_groups > 0 && comp_ptr[0] != 0) return psa_set_error(PSA_ERR_LAYOUT, "comp_ptr[0] != 0");
  int64_t folded = 0;
  for (int64_t g = 0; g < n_groups; ++g) {
    if (prompt_len[g] < 0) return psa_set_error(PSA_ERR_LAYOUT, "negative prompt length");
    if (comp_ptr[g + 1] < comp_ptr[g])
      return psa_set_error(PSA_ERR_LAYOUT, "comp_ptr decreases at group " + std::to_string(g));
    folded += prompt_len[g];
  }
  const int64_t n_comp = n_groups > 0 ? comp_ptr[n_groups] : 0;
  if (n_comp > 0 && !comp_len) return psa_set_error(PSA_ERR_NULL, "comp_len is NULL");
  for (int64_t c = 0; c < n_comp; ++c) {
    if (comp_len[c] < 0) return psa_set_error(PSA_ERR_LAYOUT, "negative completion length");
    folded += comp_len[c];
  }
  if (folded > kMaxT) return psa_set_error(PSA_ERR_SHAPE, "folded length out of range");
  r->n_groups = n_groups;
  r->n_comp = n_comp;
  r->folded = folded;
  return PSA_OK;
}

size_t fold_table_bytes(int64_t n_groups, int64_t n_comp) {
  const size_t fold = size_t(n_groups + n_comp + 1) * sizeof(FoldSeg);
  const size_t unfold = size_t(2 * n_comp) * sizeof(UnfoldSeg);
  return align_up(std::max<size_t>(std::max(fold, unfold), 1), 256);
}

// Host staging of the segment tables: library-owned pinned buffers.  A buffer is
// handed out again only once the copy that last read it has completed (an event
// recorded after that copy), so the caller's table can be a temporary and the copy is
// a true asynchronous DMA.  The copy reads host memory when it runs, which a captured
// graph would repeat on every replay: fold and unfold refuse stream capture.
struct Staging {
  void* h = nullptr;
  size_t bytes = 0;
  hipEvent_t ev = nullptr;
};
std::mutex g_stage_mu;
std::vector<Staging> g_stage;
constexpr size_t kStageCount = 4;

psa_status check_not_capturing(hipStream_t stream) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(stream, &cs);
  if (e != hipSuccess) return psa_hip_error(e, "hipStreamIsCapturing");
  if (cs != hipStreamCaptureStatusNone)
    return psa_set_error(PSA_ERR_VALUE,
                         "fold / unfold upload a host table and cannot be captured in a graph");
  return PSA_OK;
}

template <typename S>
psa_status upload_table(const std::vector<S>& table, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  const size_t need = table.size() * sizeof(S);
  if (!workspace || workspace_bytes < need)
    return psa_set_error(PSA_ERR_WORKSPACE, "workspace smaller than psa_fold_workspace_size");
  psa_status st = check_not_capturing(stream);
  if (st != PSA_OK) return st;
  std::lock_guard<std::mutex> lock(g_stage_mu);
  // a buffer whose last copy is done (the smallest one that fits), else a new one,
  // else wait for the first
  int pick = -1;
  for (size_t i = 0; i < g_stage.size(); ++i) {
    const Staging& b = g_stage[i];
    if (b.bytes < need) continue;
    if (b.ev && hipEventQuery(b.ev) != hipSuccess) continue;
    if (pick < 0 || b.bytes < g_stage[pick].bytes) pick = int(i);
  }
  hipError_t e = hipSuccess;
  if (pick < 0) {
    if (g_stage.size() < kStageCount) {
      g_stage.push_back(Staging{});
      pick = int(g_stage.size()) - 1;
    } else {
      pick = 0;
      if (g_stage[0].ev && (e = hipEventSynchronize(g_stage[0].ev)) != hipSuccess)
        return psa_hip_error(e, "segment table staging wait");
    }
  }
  (void)hipGetLastError();  // a query of an unfinished event leaves hipErrorNotReady
  Staging& b = g_stage[pick];
  if (b.bytes < need) {
    if (b.h) (void)hipHostFree(b.h);
    b.h = nullptr;
    b.bytes = 0;
    const size_t bytes = align_up(std::max<size_t>(need, 1), 4096);
    if ((e = hipHostMalloc(&b.h, bytes, hipHostMallocPortable)) != hipSuccess) {
      b.h = nullptr;
      return psa_hip_error(e, "pinned staging allocation");
    }
    b.bytes = bytes;
  }
  if (!b.ev && (e = hipEventCreateWithFlags(&b.ev, hipEventDisableTiming)) != hipSuccess) {
    b.ev = nullptr;
    return psa_hip_error(e, "staging event");
  }
  std::memcpy(b.h, table.data(), need);
  if ((e = hipMemcpyAsync(workspace, b.h, need, hipMemcpyHostToDevice, stream)) != hipSuccess ||
      (e = hipEventRecord(b.ev, stream)) != hipSuccess)
    return psa_hip_error(e, "segment table upload");
  return PSA_OK;
}

}  // namespace

extern "C" {

psa_status psa_fold_workspace_size(int64_t n_groups, int64_t n_comp, size_t* bytes) {
  if (!bytes) return psa_set_error(PSA_ERR_NULL, "bytes is NULL");
  if (n_groups < 0 || n_comp < 0) return psa_set_error(PSA_ERR_SHAPE, "negative count");
  *bytes = fold_table_bytes(n_groups, n_comp);
  return PSA_OK;
}

psa_status psa_fold_rollouts(int64_t n_groups, const int32_t* prompt_len, const int32_t* comp_ptr,
                             const int32_t* comp_len, const int32_t* prompt_tok,
                             const int32_t* comp_tok, int64_t T, int32_t pad_id,
                             int32_t ignore_index, int32_t* input_ids, int32_t* labels,
                             int32_t* position_ids, int32_t* group, int32_t* suffix,
                             uint8_t* is_prefix, void* workspace, size_t workspace_bytes,
                             void* stream) {
  Rollouts r;
  psa_status st = check_rollouts(n_groups, prompt_len, comp_ptr, comp_len, &r);
  if (st != PSA_OK) return st;
  if (T < r.folded || T > kMaxT)
    return psa_set_error(PSA_ERR_SHAPE, "T must lie in [folded length, 2^31-4096]");
  int64_t n_prompt_tok = 0, n_comp_tok = 0;
  for (int64_t g = 0; g < n_groups; ++g) n_prompt_tok += prompt_len[g];
  n_comp_tok = r.folded - n_prompt_tok;
  if ((n_prompt_tok > 0 && !prompt_tok) || (n_comp_tok > 0 && !comp_tok))
    return psa_set_error(PSA_ERR_NULL, "token buffer is NULL");
  if (!input_ids && !labels && !position_ids && !group && !suffix && !is_prefix)
    return psa_set_error(PSA_ERR_NULL, "no output requested");

  // segments in flat order: each group's prompt, then its completions; the pad tail
  std::vector<FoldSeg> segs;
  segs.reserve(size_t(n_groups + r.n_comp + 1));
  int64_t flat = 0, psrc = 0, csrc = 0, max_len = 0;
  for (int64_t g = 0; g < n_groups; ++g) {
    // the label of the prompt's last token: the first token of the group's first
    // non-empty completion (its flat successor), if any
    int64_t first = -1, c_off = csrc;
    for (int32_t c = comp_ptr[g]; c < comp_ptr[g + 1]; ++c) {
      if (comp_len[c] > 0) {
        first = c_off;
        break;
      }
      c_off += comp_len[c];
    }
    FoldSeg p{flat, prompt_len[g], psrc, first, kFoldPrompt, int32_t(g), -1, 0};
    segs.push_back(p);
    flat += prompt_len[g];
    psrc += prompt_len[g];
    max_len = std::max<int64_t>(max_len, prompt_len[g]);
    for (int32_t c = comp_ptr[g]; c < comp_ptr[g + 1]; ++c) {
      FoldSeg s{flat, comp_len[c], csrc, -1, kFoldComp, int32_t(g), c, prompt_len[g]};
      segs.push_back(s);
      flat += comp_len[c];
      csrc += comp_len[c];
      max_len = std::max<int64_t>(max_len, comp_len[c]);
    }
  }
  segs.push_back(FoldSeg{flat, T - flat, 0, -1, kFoldPad, -1, -1, 0});
  max_len = std::max<int64_t>(max_len, T - flat);

  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = upload_table(segs, workspace, workspace_bytes, s)) != PSA_OK) return st;
  hipError_t e = launch_fold(static_cast<const FoldSeg*>(workspace), int64_t(segs.size()),
                             max_len, prompt_tok, comp_tok, pad_id, ignore_index, input_ids,
                             labels, position_ids, group, suffix, is_prefix, s);
  if (e != hipSuccess) return psa_hip_error(e, "fold launch");
  return PSA_OK;
}

psa_status psa_unfold_rows(int64_t n_groups, const int32_t* prompt_len, const int32_t* comp_ptr,
                           const int32_t* comp_len, int64_t T, int64_t row_bytes,
                           const void* src, void* dst, size_t dst_bytes, void* workspace,
                           size_t workspace_bytes, void* stream) {
  Rollouts r;
  psa_status st = check_rollouts(n_groups, prompt_len, comp_ptr, comp_len, &r);
  if (st != PSA_OK) return st;
  if (T < r.folded || T > kMaxT)
    return psa_set_error(PSA_ERR_SHAPE, "T must lie in [folded length, 2^31-4096]");
  if (row_bytes <= 0 || row_bytes % 4 != 0)
    return psa_set_error(PSA_ERR_SHAPE, "row_bytes must be a positive multiple of 4");
  if (r.n_comp > 0 && (!src || !dst)) return psa_set_error(PSA_ERR_NULL, "src or dst is NULL");

  // per sample (g, i): its prompt rows, then its completion rows
  std::vector<UnfoldSeg> segs;
  segs.reserve(size_t(2 * r.n_comp));
  int64_t flat = 0, out = 0, max_bytes = 0;
  for (int64_t g = 0; g < n_groups; ++g) {
    const int64_t p_start = flat;
    int64_t c_start = flat + prompt_len[g];
    for (int32_t c = comp_ptr[g]; c < comp_ptr[g + 1]; ++c) {
      const int64_t pb = int64_t(prompt_len[g]) * row_bytes, cb = int64_t(comp_len[c]) * row_bytes;
      if (pb > 0) segs.push_back(UnfoldSeg{p_start * row_bytes, out * row_bytes, pb, 0});
      out += prompt_len[g];
      if (cb > 0) segs.push_back(UnfoldSeg{c_start * row_bytes, out * row_bytes, cb, 0});
      out += comp_len[c];
      c_start += comp_len[c];
      max_bytes = std::max(max_bytes, std::max(pb, cb));
    }
    flat = c_start;
  }
  if (uint64_t(out) * uint64_t(row_bytes) > dst_bytes)
    return psa_set_error(PSA_ERR_SHAPE, "dst holds " + std::to_string(dst_bytes) +
                                            " bytes, the unfolded rows take " +
                                            std::to_string(out * row_bytes));
  if (segs.empty()) return PSA_OK;
  const bool w16 = row_bytes % 16 == 0 && reinterpret_cast<uintptr_t>(src) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(dst) % 16 == 0;
  if (!w16 && (reinterpret_cast<uintptr_t>(src) % 4 != 0 || reinterpret_cast<uintptr_t>(dst) % 4 != 0))
    return psa_set_error(PSA_ERR_SHAPE, "src and dst must be 4-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = upload_table(segs, workspace, workspace_bytes, s)) != PSA_OK) return st;
  hipError_t e = launch_unfold(static_cast<const UnfoldSeg*>(workspace), int64_t(segs.size()),
                               max_bytes, src, dst, w16, s);
  if (e != hipSuccess) return psa_hip_error(e, "unfold launch");
  return PSA_OK;
}

}  // extern "C"
