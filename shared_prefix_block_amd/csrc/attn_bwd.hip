// Backward kernels (FlashAttention-2 style gradients of the block-sparse forward).
//
//   bwd_pre : Dl[h, q] = sum_d dO[q, h, d] * O[q, h, d];  L2[h, q] = LSE * log2(e)
//             (+inf on rows that saw no key, so their probabilities come out 0).
//   dkdv    : one work-group per (kv-tile of 128 keys, kv head).  K and V stay in
//             registers; the CSC list of the kv-tile's non-empty q-tiles is walked for
//             every q head of the GQA group, so dK and dV are summed over the group
//             inside the work-group (no atomics, no repeated K/V).  Per q sub-step:
//             S = Q K^T and dP = dO V^T (Q, dO from LDS), P = exp2(S c - L2), masked on
//             partial tiles, dS = P (dP - Dl), dV^T += dO^T P, dK^T += Q^T dS.
//   dq      : one work-group per (q-tile, q head), walking the CSR list like the
//             forward: S^T = K Q^T and dP^T = V dO^T (Q, dO in registers), the same
//             P and dS, dQ^T += K^T dS^T.  Recomputing P here costs two extra
//             products but keeps dQ free of atomics and deterministic.
// dK and dQ are scaled by the softmax scale on the way out.
//
// Source of the gradient formulas: the analytic softmax-attention backward
// (FlashAttention-2); the mask, layout and GQA conventions are the forward's
// (unsloth "prefix_grouper_kernel.py", _make_mask_mod, flex_shared_prefix_attention).
#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>
#include <type_traits>

#include "attn_common.h"
#include "psa_internal.h"

namespace psa {
namespace {

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* Dl;  // [hq, T]
  float* L2;  // [hq, T]
  const int32_t* end;   // interval form
  const int32_t* nkey;  // node form
  const int32_t* nlo;
  const int32_t* nw;
  int32_t causal;  // node form: 0 drops the kv <= q conjunct
  const int32_t* row_ptr;
  const int32_t* col;
  const uint8_t* kind;
  const int32_t* col_ptr;
  const int32_t* row;
  const uint8_t* kind_csc;
  const int32_t* qorder;
  const int32_t* korder;
  int64_t T;
  int32_t hq, hkv;
  float c;      // scale * log2(e)
  float scale;  // softmax scale
  int64_t n_work;
  int32_t chunk;
  int32_t c0;  // first output column of a launch that accumulates a column slice
};

// ---------------------------------------------------------------------------
// Precision of P and dS in the products that form dV, dK and dQ (bf16 inputs).
// kSplitAdaptive: a wave's fragment (16 queries x 32 keys) is rounded to bf16 once,
// unless its largest P exceeds kTauP or its largest |dS| exceeds kTauS; then the
// residual (frag_residual) goes through a second MFMA per product.  A rounded element
// is off by at most 2^-9 of itself, so a rounded fragment adds at most 2^-9 * tau per
// element times the other operand to a gradient, while the few large entries (rows
// that see few keys, where the softmax concentrates) keep about 16 bits.
// kSplitAll: every fragment gets the residual pass.  fp32 inputs have nothing to split.
// ---------------------------------------------------------------------------
constexpr int kSplitAdaptive = 0, kSplitAll = 1;
constexpr float kTauP = 0.125f, kTauS = 1.0f;

template <typename T, int MODE, bool WITH_P, bool WITH_S = true>
__device__ __forceinline__ bool split_wanted(const float* p8, const float* s8) {
  if constexpr (!std::is_same<T, bf16_t>::value) {
    return false;
  } else if constexpr (MODE == kSplitAll) {
    return true;
  } else {
    float mp = 0.f, ms = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if constexpr (WITH_P) mp = fmaxf(mp, p8[j]);  // P >= 0
      if constexpr (WITH_S) ms = fmaxf(ms, fabsf(s8[j]));
    }
    return __any(mp > kTauP || ms > kTauS);  // wave-uniform
  }
}

// ---------------------------------------------------------------------------
// bwd_pre: 16 lanes per (row, head); 16 rows per 256-thread block.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdParams p) {
  const int64_t rid = int64_t(blockIdx.x) * 16 + (threadIdx.x >> 4);  // = q * hq + h
  const int sub = threadIdx.x & 15;
  const int64_t n = p.T * p.hq;
  const bool valid = rid < n;
  const T* O = static_cast<const T*>(p.o);
  const T* dO = static_cast<const T*>(p.dout);
  float acc = 0.f;
  if (valid) {
    const T* op = O + rid * D;
    const T* gp = dO + rid * D;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
      const int d = sub + 16 * i;
      acc += to_f32(op[d]) * to_f32(gp[d]);
    }
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 16);
  if (valid && sub == 0) {
    const int64_t q = rid / p.hq;
    const int h = int(rid % p.hq);
    p.Dl[int64_t(h) * p.T + q] = acc;
    const float lse = p.lse[int64_t(h) * p.T + q];
    p.L2[int64_t(h) * p.T + q] = lse == -INFINITY ? INFINITY : lse * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// dkdv: K and V of this work-group's 32 keys per wave stay in registers; the q
// sub-steps (CSC entries x q heads of the group x BMS-row slices) are staged in a
// double-buffered LDS pipeline.  bf16 needs only row-major Q and dO tiles: the
// transposed operands of dV^T += dO^T P and dK^T += Q^T dS come from the LDS
// transpose read.  fp32 stages transposed copies instead, and only the tiles its
// PART uses; where two buffers would not fit in LDS (fp32, d = 256) it stages one.
// CS > 1 (fp32, d = 256) splits the accumulated output into CS column slices, one
// per launch (columns c0 .. c0 + D / CS - 1), so that K, V and the accumulators fit.
// ---------------------------------------------------------------------------
template <typename T, int D, bool NODES, int PART = 0, int CS = 1>
struct DkdvCfg {
  static constexpr bool kBf16 = std::is_same<T, bf16_t>::value;
  static constexpr int NW = 4;
  static constexpr int NT = NW * 64;
  static constexpr int BK = 32 * NW;  // keys per work-group
  static_assert(BK == kTileN, "kv-tile must match the map");
  static constexpr int EB = int(sizeof(T));
  static constexpr int BMS = (D * EB > 256) ? 32 : 64;  // q rows per sub-step
  static constexpr int NSUB = kTileM / BMS;
  // row-major tile stride: bf16 tiles are read both as rows (16 B per lane) and
  // through the transpose read; a 32-byte pad keeps both free of bank conflicts
  static constexpr int NS = D + (kBf16 ? 32 : 16) / EB;
  static constexpr int TS = BMS + 16 / EB;  // transposed tile stride (fp32 only)
  static constexpr bool kDV = PART != 2, kDK = PART != 1;
  static constexpr int DC = D / CS;  // accumulated output columns per launch
  static constexpr int N_ELEMS = BMS * NS;
  static constexpr int T_ELEMS = kBf16 ? 0 : DC * TS;
  // register-path buffer (fp32): Q | dO (for dP) | Q^T (for dK) | dO^T (for dV)
  static constexpr int OFF_G = N_ELEMS;
  static constexpr int OFF_QT = OFF_G + (kDK ? N_ELEMS : 0);
  static constexpr int OFF_GT = OFF_QT + (kDK ? T_ELEMS : 0);
  static constexpr int BUF_ELEMS = OFF_GT + (kDV ? T_ELEMS : 0);
  // bf16: Q | dO | L2 | D (| node numbers) stages filled by direct-to-LDS loads into
  // swizzled, unpadded tiles (as the forward's K and V); fp32: through registers.
  static constexpr bool kDma = kBf16;
  static constexpr int LW = NODES ? 3 : 2;  // per-row words: L2, D (, key)
  static constexpr int TILE_BYTES = BMS * D * 2;
  static constexpr int STAGE_BYTES = 2 * TILE_BYTES + LW * BMS * 4;
  static constexpr int NBUF = 2 * BUF_ELEMS * EB + 2 * LW * BMS * 4 <= kLdsMax ? 2 : 1;
  static constexpr int LDS_BYTES = kDma ? 2 * STAGE_BYTES : NBUF * BUF_ELEMS * EB + 2 * LW * BMS * 4;
  static_assert(CS == 1 || !kDma, "column slices exist on the register path only");
  static_assert(LDS_BYTES <= kLdsMax, "LDS");
};

// PART: 0 computes dK and dV together; 1 only dV, 2 only dK.  At d = 256 K, V and
// both accumulators do not fit one wave's registers, so the pair is split into two
// passes (dV: S and P only; dK: S, dP and dS), at the price of recomputing S; fp32
// inputs take the two passes from d = 128 on (room for their partial sums).
template <typename T, typename G, int D, int MODE, int PART, bool NODES, int CS = 1>
__global__ __launch_bounds__(256) void dkdv_kernel(BwdParams p) {
  using C = DkdvCfg<T, D, NODES, PART, CS>;
  constexpr bool kDV = C::kDV, kDK = C::kDK;
  constexpr int DC = C::DC;
  constexpr bool kSingle = !C::kDma && C::NBUF == 1;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS_BYTES];
  T* const buf0 = reinterpret_cast<T*>(smem);
  float* const ld0 = reinterpret_cast<float*>(smem + C::NBUF * C::BUF_ELEMS * C::EB);  // [2][LW][BMS]

  const int64_t w_id = xcd_remap(blockIdx.x, p.chunk);
  if (w_id >= p.n_work) return;
  const int64_t ntok = p.T;
  const int hq = p.hq, hkv = p.hkv, rep = hq / hkv;
  const int hk = int(w_id % hkv);
  const int kt = p.korder[w_id / hkv];

  const int lane = threadIdx.x & 63, wave = wave_id();
  const int half = lane >> 5, l32 = lane & 31;
  const int64_t kvrow = int64_t(kt) * C::BK + 32 * wave + l32;
  const bool kvvalid = kvrow < ntok;
  const int kvrow_i = int(kvrow);
  // interval form: rows kv .. kv+reach-1; node form: this key's subtree range
  int32_t reach = 0, klo = 0, kw = 0;
  if constexpr (NODES) {
    klo = kvvalid ? p.nlo[kvrow] : 0;
    kw = kvvalid ? p.nw[kvrow] : 0;
  } else {
    reach = kvvalid ? p.end[kvrow] - kvrow_i : 0;
  }

  const T* Kg = static_cast<const T*>(p.k);
  const T* Vg = static_cast<const T*>(p.v);
  const T* Qg = static_cast<const T*>(p.q);
  const T* Gg = static_cast<const T*>(p.dout);

  Frag<T> kf[D / 16], vf[D / 16];  // loaded below, once the first tile's loads are in flight
  f32x16 adk[DC / 32], adv[DC / 32];
#pragma unroll
  for (int db = 0; db < DC / 32; ++db) {
    adk[db] = zero16();
    adv[db] = zero16();
  }
  const int c0 = CS > 1 ? p.c0 : 0;
  const float c = p.c;
  const int64_t ldq = int64_t(hq) * D;

  // Steps: (CSC entry, q head of the group, BMS-row slice).  Only the last entry's
  // q-tile can cross T; it keeps the slices below T.
  const int e0 = p.col_ptr[kt], e1 = p.col_ptr[kt + 1];
  int ns_last = C::NSUB;
  if (e1 > e0) {
    const int64_t left = ntok - int64_t(p.row[e1 - 1]) * kTileM;
    if (left < kTileM) ns_last = int((left + C::BMS - 1) / C::BMS);
  }
  const int full_steps = (e1 - e0 - 1) * rep * C::NSUB;
  const int n_steps = e1 > e0 ? full_steps + rep * ns_last : 0;
  // Step cursor (CSC entry, q head, slice), advanced without divisions.
  struct Cursor {
    int e, h, sub;
  };
  auto advance = [&](Cursor u) {
    const int ns = u.e == e1 - 1 ? ns_last : C::NSUB;
    if (++u.sub == ns) {
      u.sub = 0;
      if (++u.h == (hk + 1) * rep) {
        u.h = hk * rep;
        ++u.e;
      }
    }
    return u;
  };

  // CSC entries (q-tile index | kind << 30) of a 64-entry window in one register,
  // lane i holding entry e0 + wbase + i; read with readlane, so the loop issues no
  // scalar loads and the explicit wait counts see only the tile loads.
  int wbase = 0;
  uint32_t wreg = 0;
  auto window_load = [&](int base) {
    wbase = base;
    const int e = e0 + base + lane;
    wreg = e < e1 ? uint32_t(p.row[e]) | (uint32_t(p.kind_csc[e]) << 30) : 0u;
  };
  auto entry = [&](int e) {  // packed entry e (inside the window)
    return uint32_t(__builtin_amdgcn_readlane(int(wreg), e - e0 - wbase));
  };
  window_load(0);
  mark_ready(*reinterpret_cast<int32_t*>(&wreg));

  RowStage<T, C::BMS, D, C::NS, C::NT> qst, gst;
  using TStage = TransStage<T, C::BMS, DC, C::TS, C::NT>;
  typename std::conditional<C::kBf16, int, TStage>::type qtst, gtst;
  float l2_reg = INFINITY, dl_reg = 0.f;
  int32_t qk_reg = 0;
  bool l2_valid = false;
  DmaTile<C::BMS, D, C::NT> dt;
  const int pitch = int(ldq) * 2;
  if constexpr (C::kDma) dt.init(pitch);

  // DMA path: a stage's tile loads are not issued in one burst (the wave would stall
  // on the memory-request queue) but one per reduction step of the next sub-step's
  // first S/dP product, where the MFMAs hide their issue cost.  Without a next stage
  // the descriptors cover 0 bytes and the loads only write zeros into the idle buffer.
  constexpr int NT_LOADS = DmaTile<C::BMS, D, C::NT>::N;  // per tile and wave
  DmaRsrc rq{}, rg{};
  const uint32_t smem_u = lds_addr_u(smem);
  uint32_t st_next = smem_u;  // LDS address of the stage being filled
  auto dma_part = [&](int j) {
    if constexpr (C::kDma) {
      const int w = wave;
      if (j < NT_LOADS)
        dma_load16(rq, dt.voff[j], st_next + (j * (C::NT / 64) + w) * 1024);
      else
        dma_load16(rg, dt.voff[j - NT_LOADS],
                   st_next + C::TILE_BYTES + ((j - NT_LOADS) * (C::NT / 64) + w) * 1024);
    }
  };
  auto issue = [&](int n, const Cursor& u, int q_tile) {
    const int h = u.h, sub = u.sub;
    const int64_t q0 = int64_t(q_tile) * kTileM + sub * C::BMS;
    const int nvalid = ntok - q0 < C::BMS ? int(ntok - q0) : C::BMS;
    const T* qp = Qg + q0 * ldq + int64_t(h) * D;
    const T* gp = Gg + q0 * ldq + int64_t(h) * D;
    const int64_t at = int64_t(h) * ntok + q0;
    if constexpr (C::kDma) {  // into LDS stage n & 1: Q | dO | L2 | D
      const uint32_t st = smem_u + (n & 1) * C::STAGE_BYTES;
      st_next = st;
      rq = dma_rsrc(qp, nvalid * pitch);
      rg = dma_rsrc(gp, nvalid * pitch);
      // rows past T read L2 = D = 0; they sit in a partial tile and are masked
      if (wave == 0 && lane < C::BMS)
        dma_load4(dma_rsrc(p.L2 + at, nvalid * 4), lane * 4, st + 2 * C::TILE_BYTES);
      if (wave == 1 && lane < C::BMS)
        dma_load4(dma_rsrc(p.Dl + at, nvalid * 4), lane * 4,
                  st + 2 * C::TILE_BYTES + C::BMS * 4);
      if constexpr (NODES)  // rows past T read node 0: never visible
        if (wave == 2 && lane < C::BMS)
          dma_load4(dma_rsrc(p.nkey + q0, nvalid * 4), lane * 4,
                    st + 2 * C::TILE_BYTES + 2 * C::BMS * 4);
    } else {
      {  // the per-row values first, loaded by every lane; rows past the end read 0
        const int rr = int(threadIdx.x) & (C::BMS - 1);
        l2_reg = __builtin_bit_cast(float, buf_load4(buf_rsrc(p.L2 + at, nvalid * 4), rr * 4));
        dl_reg = __builtin_bit_cast(float, buf_load4(buf_rsrc(p.Dl + at, nvalid * 4), rr * 4));
        if constexpr (NODES) qk_reg = int32_t(buf_load4(buf_rsrc(p.nkey + q0, nvalid * 4), rr * 4));
        l2_valid = rr < nvalid;
      }
      qst.load(qp, ldq, nvalid);
      if constexpr (kDK) gst.load(gp, ldq, nvalid);
      if constexpr (!C::kBf16) {
        if constexpr (kDK) qtst.load(qp + c0, ldq, nvalid);
        if constexpr (kDV) gtst.load(gp + c0, ldq, nvalid);
      }
    }
  };
  auto commit = [&](int b) {  // register path
    T* base = buf0 + b * C::BUF_ELEMS;
    qst.store(base);
    if constexpr (kDK) gst.store(base + C::OFF_G);
    if constexpr (!C::kBf16) {
      if constexpr (kDK) qtst.store(base + C::OFF_QT);
      if constexpr (kDV) gtst.store(base + C::OFF_GT);
    }
    if (threadIdx.x < C::BMS) {
      ld0[(b * C::LW + 0) * C::BMS + threadIdx.x] = l2_valid ? l2_reg : INFINITY;
      ld0[(b * C::LW + 1) * C::BMS + threadIdx.x] = dl_reg;
      if constexpr (NODES)
        ld0[(b * C::LW + 2) * C::BMS + threadIdx.x] = __builtin_bit_cast(float, qk_reg);
    }
  };

  Cursor cur{e0, hk * rep, 0};
  if (n_steps > 0) {
    issue(0, cur, int(entry(e0) & 0x3fffffffu));
    if constexpr (C::kDma) {
#pragma unroll
      for (int j = 0; j < 2 * NT_LOADS; ++j) dma_part(j);
    } else {
      commit(0);
    }
  }
  {  // K and V stay in registers; their loads overlap the first stage's
    const int64_t off = (kvrow * hkv + hk) * D + 8 * half;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      kf[s] = kvvalid ? frag_load(Kg + off + 16 * s) : frag_zero<T>();
      if constexpr (kDK) vf[s] = kvvalid ? frag_load(Vg + off + 16 * s) : frag_zero<T>();
    }
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      mark_ready(kf[s]);
      if constexpr (kDK) mark_ready(vf[s]);
    }
    if constexpr (NODES) {
      mark_ready(klo);
      mark_ready(kw);
    } else {
      mark_ready(reach);
    }
  }
  if constexpr (!C::kDma) __syncthreads();

  for (int n = 0; n < n_steps; ++n) {
    const int b = kSingle ? 0 : n & 1;
    if constexpr (C::kDma) {
      // this wave's loads of stage n are in; after the barrier everyone's are, and
      // every wave is done with stage n - 1, which the next issue overwrites
      wait_vmcnt<0>();
      __syncthreads();
    }
    const uint32_t ent = entry(cur.e);
    const bool partial = (ent >> 30) == 1;
    const int q0i = int(ent & 0x3fffffffu) * kTileM + cur.sub * C::BMS;
    const Cursor nxt = advance(cur);
    if (n + 1 < n_steps) {
      if (nxt.e - e0 - wbase >= 64) {  // next window (a vector load; rare)
        window_load(nxt.e - e0);
        mark_ready(*reinterpret_cast<int32_t*>(&wreg));
      }
      // one buffer: the next sub-step is staged after this one's math
      if constexpr (!kSingle) issue(n + 1, nxt, int(entry(nxt.e) & 0x3fffffffu));
    } else if constexpr (C::kDma) {
      st_next = smem_u + ((n + 1) & 1) * C::STAGE_BYTES;  // idle buffer, zero-byte loads
      rq = dma_rsrc(Qg, 0);
      rg = rq;
    }

    const char* st = smem + b * C::STAGE_BYTES;  // DMA stage
    const T* Qs = buf0 + b * C::BUF_ELEMS;       // register-path buffer
    const T* Gs = Qs + C::OFF_G;
    const T* Qt = Qs + C::OFF_QT;
    const T* Gt = Qs + C::OFF_GT;
    const float* Ls = C::kDma ? reinterpret_cast<const float*>(st + 2 * C::TILE_BYTES)
                              : ld0 + (b * C::LW + 0) * C::BMS;
    const float* Dsh = Ls + C::BMS;
    const int32_t* Qk = reinterpret_cast<const int32_t*>(Ls + 2 * C::BMS);  // node form

    {
      const int qd0 = q0i - kvrow_i;  // q - kv at the sub-step's first row
#pragma unroll
      for (int qb = 0; qb < C::BMS / 32; ++qb) {
        f32x16 sacc = zero16(), pacc = zero16();
        const T* qr = Qs + (32 * qb + l32) * C::NS + 8 * half;
        const T* gr = Gs + (32 * qb + l32) * C::NS + 8 * half;
        // the rows' LSE (log2 units) and D, read before the products so that their
        // latency passes under them
        f32x4 l2v[4], dlv[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int ql = 32 * qb + g * 8 + half * 4;
          l2v[g] = *reinterpret_cast<const f32x4*>(Ls + ql);
          if constexpr (kDK) dlv[g] = *reinterpret_cast<const f32x4*>(Dsh + ql);
        }
        if constexpr (C::kDma) {
          // Q and dO fragments read PF reduction steps ahead of their MFMAs
          constexpr int NS = D / 16, PF = 3;
          Frag<T> qq[PF], gq[PF];
          constexpr int RD = kDK ? 2 : 1;  // fragment reads per reduction step
#pragma unroll
          for (int s = 0; s < PF - 1; ++s) {
            qq[s] = frag_load_swz<D / 8>(st, 32 * qb + l32, half + 2 * s);
            if constexpr (kDK)
              gq[s] = frag_load_swz<D / 8>(st + C::TILE_BYTES, 32 * qb + l32, half + 2 * s);
          }
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            if (s + PF - 1 < NS) {
              const int sl = (s + PF - 1) % PF, c = half + 2 * (s + PF - 1);
              qq[sl] = frag_load_swz<D / 8>(st, 32 * qb + l32, c);
              if constexpr (kDK) gq[sl] = frag_load_swz<D / 8>(st + C::TILE_BYTES, 32 * qb + l32, c);
            }
            mma(sacc, qq[s % PF], kf[s]);
            if constexpr (kDK) mma(pacc, gq[s % PF], vf[s]);
            if (qb == 0) {  // the next stage's tile loads, spread over these steps
#pragma unroll
              for (int j = 0; j < 2 * NT_LOADS; ++j)
                if ((j * NS) / (2 * NT_LOADS) == s) dma_part(j);
            }
          }
          __builtin_amdgcn_sched_group_barrier(0x100, kDK ? 8 : 4, 1);  // LSE / D
          __builtin_amdgcn_sched_group_barrier(0x100, RD * (PF - 1), 1);
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            if (s + PF - 1 < NS) __builtin_amdgcn_sched_group_barrier(0x100, RD, 1);
            __builtin_amdgcn_sched_group_barrier(0x008, RD, 1);
          }
        } else {
#pragma unroll
          for (int s = 0; s < D / 16; ++s) {
            mma(sacc, frag_load(qr + 16 * s), kf[s]);
            if constexpr (kDK) mma(pacc, frag_load(gr + 16 * s), vf[s]);
          }
        }
        float pv[16], ds[16];
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int u = 0; u < 4; ++u)
            pv[4 * g + u] = __builtin_amdgcn_exp2f(fmaf(sacc[4 * g + u], c, -l2v[g][u]));
        if (NODES && partial) {  // uniform branch; node form
          const bool nc = p.causal == 0;
          int4 qkv[4];  // the rows' node numbers
#pragma unroll
          for (int g = 0; g < 4; ++g)
            qkv[g] = *reinterpret_cast<const int4*>(Qk + 32 * qb + g * 8 + half * 4);
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int kq[4] = {qkv[g].x, qkv[g].y, qkv[g].z, qkv[g].w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const int ii = 4 * g + u;
              const bool keep = ((qd0 + 32 * qb + acc_row(ii, half) >= 0) | nc) &
                                (uint32_t(kq[u] - klo) < uint32_t(kw));
              pv[ii] = keep ? pv[ii] : 0.f;
            }
          }
        } else if (partial) {  // uniform branch; full tiles skip the mask
#pragma unroll
          for (int ii = 0; ii < 16; ++ii)
            pv[ii] = visible_u(qd0 + 32 * qb + acc_row(ii, half), reach) ? pv[ii] : 0.f;
        }
        if constexpr (kDK) {
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int u = 0; u < 4; ++u) ds[4 * g + u] = pv[4 * g + u] * (pacc[4 * g + u] - dlv[g][u]);
        }
        if constexpr (C::kDma) {
          // dV += dO^T P and dK += Q^T dS over these 32 queries (two 16-query
          // fragments t): P and dS rounded to bf16, the (t, db) transposed reads
          // PF products ahead of their MFMAs; then, where split_wanted, the
          // residuals in a second pass
          constexpr int ND = D / 32, NI = 2 * ND, PF = 3;
          constexpr int TR = 2 * ((kDV ? 1 : 0) + (kDK ? 1 : 0));  // reads per product
          constexpr int MF = (kDV ? 1 : 0) + (kDK ? 1 : 0);        // MFMAs per product
          Frag<T> pf[2], sf[2];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            if constexpr (kDV) pf[t] = frag_from<T>(pv + 8 * t);
            if constexpr (kDK) sf[t] = frag_from<T>(ds + 8 * t);
          }
          const char* gst = st + C::TILE_BYTES;
          Frag<T> ga[PF], qa[PF];
          auto tr_load = [&](int i, int sl) {
            if constexpr (kDV)
              ga[sl] = frag_load_tr_swz<D / 8>(gst, 32 * qb + 16 * (i / ND), 32 * (i % ND));
            if constexpr (kDK)
              qa[sl] = frag_load_tr_swz<D / 8>(st, 32 * qb + 16 * (i / ND), 32 * (i % ND));
          };
#pragma unroll
          for (int i = 0; i < PF - 1; ++i) tr_load(i, i);
#pragma unroll
          for (int i = 0; i < NI; ++i) {
            if (i + PF - 1 < NI) tr_load(i + PF - 1, (i + PF - 1) % PF);
            if constexpr (kDV) mma(adv[i % ND], ga[i % PF], pf[i / ND]);
            if constexpr (kDK) mma(adk[i % ND], qa[i % PF], sf[i / ND]);
          }
          __builtin_amdgcn_sched_group_barrier(0x100, TR * (PF - 1), 2);
#pragma unroll
          for (int i = 0; i < NI; ++i) {
            if (i + PF - 1 < NI) __builtin_amdgcn_sched_group_barrier(0x100, TR, 2);
            __builtin_amdgcn_sched_group_barrier(0x008, MF, 2);
          }
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            if (split_wanted<T, MODE, kDV, kDK>(pv + 8 * t, ds + 8 * t)) {
#pragma unroll
              for (int db = 0; db < ND; ++db) {
                if constexpr (kDV)
                  mma(adv[db], frag_load_tr_swz<D / 8>(gst, 32 * qb + 16 * t, 32 * db),
                      frag_residual(pv + 8 * t, pf[t]));
                if constexpr (kDK)
                  mma(adk[db], frag_load_tr_swz<D / 8>(st, 32 * qb + 16 * t, 32 * db),
                      frag_residual(ds + 8 * t, sf[t]));
              }
            }
          }
        } else {
          // fp32: dV += dO^T P and dK += Q^T dS over these 32 queries (two 16-query
          // fragments t).  The products go into fresh blocks that are then added to the
          // accumulators: a key seen by ~10^3 rows would otherwise take ~10^3 MFMA
          // steps in one chain, each rounding at the magnitude of the running sum; per
          // 32 queries the sum rounds there once.
          Frag<T> pf[2], sf[2];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            if constexpr (kDV) pf[t] = frag_from<T>(pv + 8 * t);
            if constexpr (kDK) sf[t] = frag_from<T>(ds + 8 * t);
          }
#pragma unroll
          for (int db = 0; db < DC / 32; ++db) {
            f32x16 pvp = zero16(), pkp = zero16();
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              const int col0 = 32 * qb + 16 * t + 8 * half;
              if constexpr (kDV) mma(pvp, frag_load(Gt + (32 * db + l32) * C::TS + col0), pf[t]);
              if constexpr (kDK) mma(pkp, frag_load(Qt + (32 * db + l32) * C::TS + col0), sf[t]);
            }
            if constexpr (kDV) adv[db] += pvp;
            if constexpr (kDK) adk[db] += pkp;
            // one column block's partial sums at a time (registers)
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    }
    if constexpr (kSingle) {  // every wave is done with the buffer: stage the next step
      if (n + 1 < n_steps) {
        __syncthreads();
        issue(n + 1, nxt, int(entry(nxt.e) & 0x3fffffffu));
        commit(0);
      }
      __syncthreads();
    } else if constexpr (!C::kDma) {
      if (n + 1 < n_steps) commit(b ^ 1);
      __syncthreads();
    }
    cur = nxt;
  }
  if constexpr (C::kDma) wait_vmcnt<0>();  // no load into LDS outlives the work-group

  if (kvvalid) {
    G* dkp = static_cast<G*>(p.dk) + (kvrow * hkv + hk) * D + c0;
    G* dvp = static_cast<G*>(p.dv) + (kvrow * hkv + hk) * D + c0;
    const float sc = p.scale;
#pragma unroll
    for (int db = 0; db < DC / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * db + g * 8 + half * 4;
        if constexpr (kDK)
          vec4_store(dkp + d, vec4_from(adk[db][4 * g] * sc, adk[db][4 * g + 1] * sc,
                                        adk[db][4 * g + 2] * sc, adk[db][4 * g + 3] * sc,
                                        static_cast<G*>(nullptr)));
        if constexpr (kDV)
          vec4_store(dvp + d, vec4_from(adv[db][4 * g], adv[db][4 * g + 1], adv[db][4 * g + 2],
                                        adv[db][4 * g + 3], static_cast<G*>(nullptr)));
      }
  }
}

// ---------------------------------------------------------------------------
// dq: the forward's walk over the CSR list with K and V staged row-major in a
// double-buffered LDS pipeline; Q and dO stay in registers.  bf16 takes K^T for
// dQ^T += K^T dS^T from the LDS transpose read of the K tile; fp32 stages K^T, in one
// buffer where two would not fit (d = 256), and then for the launch's column slice
// of dQ only (CS slices, columns c0 .. c0 + D / CS - 1).
// ---------------------------------------------------------------------------
template <typename T, int D, bool NODES, int CS = 1>
struct DqCfg {
  static constexpr bool kBf16 = std::is_same<T, bf16_t>::value;
  static constexpr int NW = 4;
  static constexpr int NT = NW * 64;
  static constexpr int BM = 32 * NW;
  static_assert(BM == kTileM, "q-tile must match the map");
  static constexpr int EB = int(sizeof(T));
  // keys per sub-step (one LDS stage, one barrier): bf16 stages 64 keys up to d = 128
  // and runs the math in blocks of 32 keys (the dQ products of a block right after its
  // dS, so two waves fit on a SIMD); fp32 and bf16 d = 256 stage 32 where 64 would not
  // fit in registers or LDS
  static constexpr int BN = kBf16 ? (D <= 128 ? 64 : 32) : (D * EB > 256 ? 32 : 64);
  static constexpr int NSUB = kTileN / BN;
  static constexpr int NS = D + (kBf16 ? 32 : 16) / EB;  // see DkdvCfg::NS
  static constexpr int TS = BN + 16 / EB;
  static constexpr int DC = D / CS;  // dQ columns per launch
  static constexpr int N_ELEMS = BN * NS;
  static constexpr int T_ELEMS = kBf16 ? 0 : DC * TS;
  static constexpr int BUF_ELEMS = 2 * N_ELEMS + T_ELEMS;
  // bf16: K | V | mask words (end[], or lo[] | w[]) stages filled by direct-to-LDS
  // loads into swizzled tiles (as the forward); fp32: through registers
  static constexpr bool kDma = kBf16;
  static constexpr int MW = NODES ? 2 : 1;
  static constexpr int TILE_BYTES = BN * D * 2;
  static constexpr int STAGE_BYTES = 2 * TILE_BYTES + MW * 256;
  static constexpr int NBUF = 2 * BUF_ELEMS * EB + 2 * MW * BN * 4 <= kLdsMax ? 2 : 1;
  static constexpr int LDS_BYTES = kDma ? 2 * STAGE_BYTES : NBUF * BUF_ELEMS * EB + 2 * MW * BN * 4;
  static constexpr int WAVES_PER_EU = (kBf16 && D <= 128) ? 2 : 1;
  static_assert(CS == 1 || !kDma, "column slices exist on the register path only");
  static_assert(LDS_BYTES <= kLdsMax, "LDS");
};

// PRE: the kernel also does the preparation of its rows (bwd_pre_kernel's work): it
// holds dO for exactly its (row, head) pairs, so it loads O beside it, forms D and
// LSE in log2 units in registers and writes them to the workspace for the dK/dV
// kernel, which then runs after it.
template <typename T, typename G, int D, int MODE, bool PRE, bool NODES, int CS = 1>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(DqCfg<T, D, NODES, CS>::WAVES_PER_EU)))
void dq_kernel(BwdParams p) {
  using C = DqCfg<T, D, NODES, CS>;
  constexpr int DC = C::DC;
  constexpr bool kSingle = !C::kDma && C::NBUF == 1;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS_BYTES];
  T* const buf0 = reinterpret_cast<T*>(smem);
  int32_t* const es0 = reinterpret_cast<int32_t*>(smem + C::NBUF * C::BUF_ELEMS * C::EB);

  const int64_t w_id = xcd_remap(blockIdx.x, p.chunk);
  if (w_id >= p.n_work) return;
  const int64_t ntok = p.T;
  const int hq = p.hq, hkv = p.hkv, rep = hq / hkv;
  const int h = int(w_id % hq);
  const int qt = p.qorder[w_id / hq];
  const int hk = h / rep;

  const int lane = threadIdx.x & 63, wave = wave_id();
  const int half = lane >> 5, l32 = lane & 31;
  const int64_t qrow = int64_t(qt) * C::BM + 32 * wave + l32;
  const int wave_last = qt * C::BM + 32 * wave + 31;  // this wave's last row
  const bool qvalid = qrow < ntok;
  const int qrow_i = int(qrow);

  const T* Qg = static_cast<const T*>(p.q);
  const T* Gg = static_cast<const T*>(p.dout);
  const T* Kg = static_cast<const T*>(p.k);
  const T* Vg = static_cast<const T*>(p.v);

  Frag<T> qf[D / 16], gf[D / 16];  // loaded below, once the first tile's loads are in flight
  float l2 = INFINITY, dl = 0.f;
  f32x16 adq[DC / 32];
#pragma unroll
  for (int db = 0; db < DC / 32; ++db) adq[db] = zero16();
  const int c0 = CS > 1 ? p.c0 : 0;
  const float c = p.c;
  const int64_t ldk = int64_t(hkv) * D;
  const int64_t koff = int64_t(hk) * D;

  const int e0 = p.row_ptr[qt], e1 = p.row_ptr[qt + 1];
  int n_steps = (e1 - e0) * C::NSUB;
  if (e1 > e0) {
    const int64_t left = ntok - int64_t(p.col[e1 - 1]) * kTileN;
    if (left < kTileN) n_steps -= C::NSUB - int((left + C::BN - 1) / C::BN);
  }

  // CSR entries (kv-tile index | kind << 30) of a 64-entry window in one register,
  // read with readlane (see the forward kernel)
  int wbase = 0;
  uint32_t wreg = 0;
  auto window_load = [&](int base) {
    wbase = base;
    const int e = e0 + base + lane;
    wreg = e < e1 ? uint32_t(p.col[e]) | (uint32_t(p.kind[e]) << 30) : 0u;
  };
  auto entry = [&](int n) {
    return uint32_t(__builtin_amdgcn_readlane(int(wreg), n / C::NSUB - wbase));
  };
  window_load(0);
  mark_ready(*reinterpret_cast<int32_t*>(&wreg));

  RowStage<T, C::BN, D, C::NS, C::NT> kst, vst;
  using TStage = TransStage<T, C::BN, DC, C::TS, C::NT>;
  typename std::conditional<C::kBf16, int, TStage>::type ktst;
  DmaTile<C::BN, D, C::NT> dt;
  const int pitch = int(ldk) * 2;
  if constexpr (C::kDma) dt.init(pitch);
  int32_t e_reg = 0, kv_reg = 0, w_reg = 0;
  int32_t qkey = 0;  // node form: this row's node number (0: a pad or past T)
  const int32_t* const ev = NODES ? p.nlo : p.end;

  auto issue = [&](int n, int col_n) {
    const int64_t kv0 = int64_t(col_n) * kTileN + (n % C::NSUB) * C::BN;
    const int nvalid = ntok - kv0 < C::BN ? int(ntok - kv0) : C::BN;
    if constexpr (C::kDma) {  // straight into LDS stage n & 1: K | V | mask words
      const uint32_t st = lds_addr_u(smem) + (n & 1) * C::STAGE_BYTES;
      dt.load(Kg + kv0 * ldk + koff, nvalid, pitch, st);
      dt.load(Vg + kv0 * ldk + koff, nvalid, pitch, st + C::TILE_BYTES);
      if (wave == 0 && lane < C::BN)  // keys past the end read end = 0 (or w = 0): never visible
        dma_load4(dma_rsrc(ev + kv0, nvalid * 4), lane * 4, st + 2 * C::TILE_BYTES);
      if constexpr (NODES)
        if (wave == 1 && lane < C::BN)
          dma_load4(dma_rsrc(p.nw + kv0, nvalid * 4), lane * 4,
                    st + 2 * C::TILE_BYTES + C::BN * 4);
    } else {
      {  // every lane loads; a key past the end reads end = 0 and gets reach 0
        const int r = int(threadIdx.x) & (C::BN - 1);
        e_reg = int32_t(buf_load4(buf_rsrc(ev + kv0, nvalid * 4), r * 4));
        if constexpr (NODES) w_reg = int32_t(buf_load4(buf_rsrc(p.nw + kv0, nvalid * 4), r * 4));
        kv_reg = r < nvalid ? int32_t(kv0 + r) : 0;
      }
      kst.load(Kg + kv0 * ldk + koff, ldk, nvalid);
      vst.load(Vg + kv0 * ldk + koff, ldk, nvalid);
      if constexpr (!C::kBf16) ktst.load(Kg + kv0 * ldk + koff + c0, ldk, nvalid);
    }
  };
  auto commit = [&](int b) {  // register path
    T* base = buf0 + b * C::BUF_ELEMS;
    kst.store(base);
    vst.store(base + C::N_ELEMS);
    if constexpr (!C::kBf16) ktst.store(base + 2 * C::N_ELEMS);
    if (threadIdx.x < C::BN) {
      if constexpr (NODES) {  // lo | w
        es0[b * 2 * C::BN + threadIdx.x] = e_reg;
        es0[b * 2 * C::BN + C::BN + threadIdx.x] = w_reg;
      } else {
        es0[b * C::BN + threadIdx.x] = e_reg - kv_reg;  // reach
      }
    }
  };

  if (n_steps > 0) {
    issue(0, int(entry(0) & 0x3fffffffu));
    if constexpr (!C::kDma) commit(0);
  }
  {  // Q and dO stay in registers; their loads overlap the first tile's
    const int64_t off = (qrow * hq + h) * D + 8 * half;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      qf[s] = qvalid ? frag_load(Qg + off + 16 * s) : frag_zero<T>();
      gf[s] = qvalid ? frag_load(Gg + off + 16 * s) : frag_zero<T>();
    }
    if constexpr (PRE) {
      // D = sum_d dO * O over the row (each lane half holds half of it) and LSE in
      // log2 units (+inf on rows that saw no key, so their probabilities are 0)
      const T* Og = static_cast<const T*>(p.o);
      float lse = -INFINITY, part = 0.f;
      if (qvalid) {
        lse = p.lse[int64_t(h) * ntok + qrow];
#pragma unroll
        for (int s = 0; s < D / 16; ++s) part += frag_dot(frag_load(Og + off + 16 * s), gf[s]);
      }
      dl = part + __shfl_xor(part, 32);
      l2 = lse == -INFINITY ? INFINITY : lse * kLog2e;
      if (qvalid && half == 0) {
        p.Dl[int64_t(h) * ntok + qrow] = dl;
        p.L2[int64_t(h) * ntok + qrow] = l2;
      }
    } else if (qvalid) {
      l2 = p.L2[int64_t(h) * ntok + qrow];
      dl = p.Dl[int64_t(h) * ntok + qrow];
    }
    if constexpr (NODES) qkey = qvalid ? p.nkey[qrow] : 0;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      mark_ready(qf[s]);
      mark_ready(gf[s]);
    }
    mark_ready(l2);
    mark_ready(dl);
    if constexpr (NODES) mark_ready(qkey);
  }
  if constexpr (!C::kDma) __syncthreads();

  for (int n = 0; n < n_steps; ++n) {
    const int b = kSingle ? 0 : n & 1;
    if constexpr (C::kDma) {  // see the forward kernel
      wait_vmcnt<0>();
      __syncthreads();
    }
    const uint32_t ent = entry(n);
    const bool partial = (ent >> 30) == 1;
    const int kv0i = int(ent & 0x3fffffffu) * kTileN + (n % C::NSUB) * C::BN;
    if (n + 1 < n_steps) {
      if ((n + 1) / C::NSUB - wbase >= 64) {  // next window (a vector load; rare)
        window_load((n + 1) / C::NSUB);
        mark_ready(*reinterpret_cast<int32_t*>(&wreg));
      }
      // one buffer: the next sub-step is staged after this one's math
      if constexpr (!kSingle) issue(n + 1, int(entry(n + 1) & 0x3fffffffu));
    }

    const char* st = smem + b * C::STAGE_BYTES;  // DMA stage
    const T* Ks = buf0 + b * C::BUF_ELEMS;       // register-path buffer
    const T* Vs = Ks + C::N_ELEMS;
    const T* Kt = Ks + 2 * C::N_ELEMS;
    const int32_t* Es = C::kDma ? reinterpret_cast<const int32_t*>(st + 2 * C::TILE_BYTES)
                                : es0 + b * C::MW * C::BN;

    // keys of a partial tile all after this wave's rows: no kept pair (kv <= q is
    // part of every causal mask), nothing to add to dQ (the DMA path decides per block
    // of 32 keys)
    if (C::kDma || !(partial && p.causal && kv0i > wave_last)) {
      const int qd = qrow_i - kv0i;
      float ds[C::kDma ? 1 : C::BN / 32][16];
#pragma unroll
      for (int kb = 0; kb < C::BN / 32; ++kb) {
        if (C::kDma && partial && p.causal && kv0i + 32 * kb > wave_last) continue;
        f32x16 sacc = zero16(), pacc = zero16();
        if constexpr (C::kDma) {
          // K and V fragments read PF reduction steps ahead of their MFMAs
          constexpr int NS = D / 16, PF = 3;
          Frag<T> kq[PF], vq[PF];
#pragma unroll
          for (int s = 0; s < PF - 1; ++s) {
            kq[s] = frag_load_swz<D / 8>(st, 32 * kb + l32, half + 2 * s);
            vq[s] = frag_load_swz<D / 8>(st + C::TILE_BYTES, 32 * kb + l32, half + 2 * s);
          }
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            if (s + PF - 1 < NS) {
              const int sl = (s + PF - 1) % PF, cc = half + 2 * (s + PF - 1);
              kq[sl] = frag_load_swz<D / 8>(st, 32 * kb + l32, cc);
              vq[sl] = frag_load_swz<D / 8>(st + C::TILE_BYTES, 32 * kb + l32, cc);
            }
            mma(sacc, kq[s % PF], qf[s]);
            mma(pacc, vq[s % PF], gf[s]);
          }
          __builtin_amdgcn_sched_group_barrier(0x100, 2 * (PF - 1), 1);
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            if (s + PF - 1 < NS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
          }
        } else {
          const T* kr = Ks + (32 * kb + l32) * C::NS + 8 * half;
          const T* vr = Vs + (32 * kb + l32) * C::NS + 8 * half;
#pragma unroll
          for (int s = 0; s < D / 16; ++s) {
            mma(sacc, frag_load(kr + 16 * s), qf[s]);
            mma(pacc, frag_load(vr + 16 * s), gf[s]);
          }
        }
        float pv[16];
#pragma unroll
        for (int ii = 0; ii < 16; ++ii) pv[ii] = __builtin_amdgcn_exp2f(fmaf(sacc[ii], c, -l2));
        if (NODES && partial) {  // uniform branch; node form
          const bool nc = p.causal == 0;
          int4 los[4], ws[4];
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            los[g] = *reinterpret_cast<const int4*>(Es + 32 * kb + g * 8 + half * 4);
            ws[g] = *reinterpret_cast<const int4*>(Es + C::BN + 32 * kb + g * 8 + half * 4);
          }
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int kvl = 32 * kb + g * 8 + half * 4;
            const int lv[4] = {los[g].x, los[g].y, los[g].z, los[g].w};
            const int wv[4] = {ws[g].x, ws[g].y, ws[g].z, ws[g].w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const bool keep =
                  ((kvl + u <= qd) | nc) & (uint32_t(qkey - lv[u]) < uint32_t(wv[u]));
              pv[4 * g + u] = keep ? pv[4 * g + u] : 0.f;
            }
          }
        } else if (partial) {  // uniform branch; full tiles skip the mask
          // this lane's end[] (or reach) values first, their LDS reads in flight
          // together; the two tests combined without a short circuit, so no test
          // turns into a branch around a read
          int4 evs[4];
#pragma unroll
          for (int g = 0; g < 4; ++g)
            evs[g] = *reinterpret_cast<const int4*>(Es + 32 * kb + g * 8 + half * 4);
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int kvl = 32 * kb + g * 8 + half * 4;
            const int rv[4] = {evs[g].x, evs[g].y, evs[g].z, evs[g].w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              bool keep;
              if constexpr (C::kDma)  // raw end[]: kv <= q < end
                keep = (kvl + u <= qd) & (qrow_i < rv[u]);
              else  // reach = end - kv
                keep = visible_u(qd - kvl - u, rv[u]);
              pv[4 * g + u] = keep ? pv[4 * g + u] : 0.f;
            }
          }
        }
        float* const dsk = ds[C::kDma ? 0 : kb];
#pragma unroll
        for (int ii = 0; ii < 16; ++ii) dsk[ii] = pv[ii] * (pacc[ii] - dl);
        if constexpr (C::kDma) {
          // dQ^T += K^T dS^T over this block's 32 keys (16-key fragments t): dS rounded,
          // the (t, db) transposed K reads PF products ahead of their MFMAs; then, where
          // split_wanted, the residuals
          constexpr int ND = D / 32, NI = 2 * ND, PF = 3;
          Frag<T> sf[2];
#pragma unroll
          for (int t = 0; t < 2; ++t) sf[t] = frag_from<T>(dsk + 8 * t);
          Frag<T> ka[PF];
#pragma unroll
          for (int i = 0; i < PF - 1; ++i)
            ka[i] = frag_load_tr_swz<D / 8>(st, 32 * kb + 16 * (i / ND), 32 * (i % ND));
#pragma unroll
          for (int i = 0; i < NI; ++i) {
            if (i + PF - 1 < NI) {
              const int j = i + PF - 1;
              ka[j % PF] = frag_load_tr_swz<D / 8>(st, 32 * kb + 16 * (j / ND), 32 * (j % ND));
            }
            mma(adq[i % ND], ka[i % PF], sf[i / ND]);
          }
          __builtin_amdgcn_sched_group_barrier(0x100, 2 * (PF - 1), 2);
#pragma unroll
          for (int i = 0; i < NI; ++i) {
            if (i + PF - 1 < NI) __builtin_amdgcn_sched_group_barrier(0x100, 2, 2);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 2);
          }
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            if (split_wanted<T, MODE, false>(nullptr, dsk + 8 * t)) {
              const Frag<T> sl = frag_residual(dsk + 8 * t, sf[t]);
#pragma unroll
              for (int db = 0; db < ND; ++db)
                mma(adq[db], frag_load_tr_swz<D / 8>(st, 32 * kb + 16 * t, 32 * db), sl);
            }
          }
        }
      }
      if constexpr (!C::kDma) {
        // fp32: dQ^T += K^T dS^T over these BN keys, into a fresh block that is then
        // added to dQ (one chain over every key of a long list would round at the
        // magnitude of the running sum on each of its steps)
#pragma unroll
        for (int db = 0; db < DC / 32; ++db) {
          f32x16 part = zero16();
#pragma unroll
          for (int t = 0; t < C::BN / 16; ++t)
            mma(part, frag_load(Kt + (32 * db + l32) * C::TS + 16 * t + 8 * half),
                frag_from<T>(&ds[t >> 1][(t & 1) * 8]));
          adq[db] += part;
          __builtin_amdgcn_sched_barrier(0);  // one partial block at a time (registers)
        }
      }
    }
    if constexpr (kSingle) {  // every wave is done with the buffer: stage the next step
      if (n + 1 < n_steps) {
        __syncthreads();
        issue(n + 1, int(entry(n + 1) & 0x3fffffffu));
        commit(0);
      }
      __syncthreads();
    } else if constexpr (!C::kDma) {
      if (n + 1 < n_steps) commit(b ^ 1);
      __syncthreads();
    }
  }
  if constexpr (C::kDma) wait_vmcnt<0>();  // no load into LDS outlives the work-group

  if (qvalid) {
    G* dqp = static_cast<G*>(p.dq) + (qrow * hq + h) * D + c0;
    const float sc = p.scale;
#pragma unroll
    for (int db = 0; db < DC / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * db + g * 8 + half * 4;
        vec4_store(dqp + d, vec4_from(adq[db][4 * g] * sc, adq[db][4 * g + 1] * sc,
                                      adq[db][4 * g + 2] * sc, adq[db][4 * g + 3] * sc,
                                      static_cast<G*>(nullptr)));
      }
  }
}

size_t ws_align(size_t x) { return (x + 255) / 256 * 256; }

template <typename T, typename G, int D, int MODE, bool NODES>
hipError_t launch_bwd_t(const psa_tile_map& map, const AttnShape& s, const void* q,
                        const void* k, const void* v, const void* o, const float* lse,
                        const void* dout, void* dq, void* dk, void* dv, void* workspace,
                        int stages, hipStream_t stream) {
  BwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.dout = dout;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  const size_t plane = ws_align(size_t(s.T) * s.hq * sizeof(float));
  p.Dl = static_cast<float*>(workspace);
  p.L2 = reinterpret_cast<float*>(static_cast<char*>(workspace) + plane);
  p.end = map.end;
  p.nkey = map.nkey;
  p.nlo = map.nlo;
  p.nw = map.nw;
  p.causal = map.causal;
  p.row_ptr = map.row_ptr;
  p.col = map.col;
  p.kind = map.kind;
  p.col_ptr = map.col_ptr;
  p.row = map.row;
  p.kind_csc = map.kind_csc;
  p.qorder = map.qorder;
  p.korder = map.korder;
  p.T = s.T;
  p.hq = s.hq;
  p.hkv = s.hkv;
  p.scale = s.scale;
  p.c = s.scale * kLog2e;
  p.c0 = 0;
  const int rep = s.hq / s.hkv;
  // fp32 at d >= 128: dV and dK in separate passes (room for the per-sub-step partial
  // sums of fp32), and at d = 256 each of them, and dQ, in two launches of half the
  // columns
  constexpr bool kF32 = std::is_same<T, float>::value;
  constexpr int CS = kF32 && D > 128 ? 2 : 1;
  constexpr bool kTwoPass = D > 128 || (kF32 && D >= 128);

  // PREPARE together with DQ: the dQ kernel does the preparation of its rows and
  // runs first; dK/dV then reads what it wrote.
  const bool fused = (stages & PSA_STAGE_PREPARE) && (stages & PSA_STAGE_DQ);
  auto launch_dq = [&](auto pre_t) {
    constexpr bool PRE = decltype(pre_t)::value;
    p.n_work = map.nq * s.hq;
    p.chunk = rep * 2;
    const int64_t per = 8 * int64_t(p.chunk);
    const int64_t grid = (p.n_work + per - 1) / per * per;
    p.c0 = 0;
    hipLaunchKernelGGL((dq_kernel<T, G, D, MODE, PRE, NODES, CS>), dim3(unsigned(grid)),
                       dim3(256), 0, stream, p);
    // the other column slices read the D and LSE rows the first one prepared
    for (int c = 1; c < CS; ++c) {
      p.c0 = c * (D / CS);
      hipLaunchKernelGGL((dq_kernel<T, G, D, MODE, false, NODES, CS>), dim3(unsigned(grid)),
                         dim3(256), 0, stream, p);
    }
    p.c0 = 0;
  };
  if (fused) {
    launch_dq(std::true_type{});
  } else if (stages & PSA_STAGE_PREPARE) {
    const int64_t rows = s.T * s.hq;
    hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3(unsigned((rows + 15) / 16)), dim3(256), 0,
                       stream, p);
  }
  if (stages & PSA_STAGE_DKDV) {
    p.n_work = map.nk * s.hkv;
    p.chunk = 2;
    const int64_t per = 8 * int64_t(p.chunk);
    const int64_t grid = (p.n_work + per - 1) / per * per;
    if constexpr (kTwoPass) {  // dV and dK in two passes (see dkdv_kernel)
      for (int c = 0; c < CS; ++c) {  // each in column slices (fp32, d = 256)
        p.c0 = c * (D / CS);
        hipLaunchKernelGGL((dkdv_kernel<T, G, D, MODE, 1, NODES, CS>), dim3(unsigned(grid)),
                           dim3(256), 0, stream, p);
      }
      for (int c = 0; c < CS; ++c) {
        p.c0 = c * (D / CS);
        hipLaunchKernelGGL((dkdv_kernel<T, G, D, MODE, 2, NODES, CS>), dim3(unsigned(grid)),
                           dim3(256), 0, stream, p);
      }
      p.c0 = 0;
    } else {
      hipLaunchKernelGGL((dkdv_kernel<T, G, D, MODE, 0, NODES>), dim3(unsigned(grid)),
                         dim3(256), 0, stream, p);
    }
  }
  if ((stages & PSA_STAGE_DQ) && !fused) launch_dq(std::false_type{});
  return hipGetLastError();
}

}  // namespace
}  // namespace psa

bool bwd_supported(psa_dtype dt, int32_t d) {
  return dt != PSA_FP8_E4M3 && fwd_supported(dt, d);
}

size_t bwd_workspace_bytes(const AttnShape& s) {
  return 2 * psa::ws_align(size_t(s.T) * s.hq * sizeof(float));
}

// The backward's workspace (D and LSE in log2 units, [hq, T] fp32 each) for callers
// that cannot allocate: a file-scope device array, of which each GPU the library runs
// on holds its own copy until the process ends.  In host code its name is only a
// stand-in; the device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) float scratch[kBwdScratchBytes / sizeof(float)];

hipError_t bwd_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* per_device[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!per_device[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    per_device[dev] = p;
  }
  *ptr = per_device[dev];
  return hipSuccess;
}

hipError_t launch_bwd(const psa_tile_map& map, psa_dtype dt, psa_dtype gdt, const AttnShape& s,
                      const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dout, void* dq, void* dk, void* dv,
                      void* workspace, int stages, bool split, hipStream_t stream) {
  using psa::bf16_t;
#define PSA_BWD(T, G, D, MODE)                                                            \
  return map.form == kFormNodes                                                            \
             ? psa::launch_bwd_t<T, G, D, MODE, true>(map, s, q, k, v, o, lse, dout, dq, dk, \
                                                      dv, workspace, stages, stream)       \
             : psa::launch_bwd_t<T, G, D, MODE, false>(map, s, q, k, v, o, lse, dout, dq, dk, \
                                                       dv, workspace, stages, stream)
#define PSA_BWD_BF16(G, D)                          \
  if (split) PSA_BWD(bf16_t, G, D, psa::kSplitAll); \
  PSA_BWD(bf16_t, G, D, psa::kSplitAdaptive)
  if (dt == PSA_BF16 && gdt == PSA_FP32) {
    switch (s.d) {
      case 64: PSA_BWD_BF16(float, 64);
      case 128: PSA_BWD_BF16(float, 128);
      case 256: PSA_BWD_BF16(float, 256);
    }
  } else if (dt == PSA_BF16 && gdt == PSA_BF16) {
    switch (s.d) {
      case 64: PSA_BWD_BF16(bf16_t, 64);
      case 128: PSA_BWD_BF16(bf16_t, 128);
      case 256: PSA_BWD_BF16(bf16_t, 256);
    }
  } else if (dt == PSA_FP32 && gdt == PSA_FP32) {  // fp32 products: nothing to split
    switch (s.d) {
      case 64: PSA_BWD(float, float, 64, psa::kSplitAdaptive);
      case 128: PSA_BWD(float, float, 128, psa::kSplitAdaptive);
      case 256: PSA_BWD(float, float, 256, psa::kSplitAdaptive);
    }
  }
#undef PSA_BWD_BF16
#undef PSA_BWD
  return hipErrorInvalidValue;
}
