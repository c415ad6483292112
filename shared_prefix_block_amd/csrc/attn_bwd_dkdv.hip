// dK and dV of the backward: one work-group per (kv-tile of 128 keys, kv head), see
// attn_bwd.hip for the whole backward.
//
// Like the other attention units, this one is compiled with MFMA results in VGPRs
// (-mllvm -amdgpu-mfma-vgpr-form, set by the build), and the kernel pins its K and V
// fragments in AGPRs: the per-step S and dP products then land where the softmax
// gradient reads them, instead of being copied out of AGPRs one register at a time
// (64 copies per 64-row sub-step at d = 128), and bf16 at d = 64 fits two waves per
// SIMD.
//
// Source of the gradient formulas: the analytic softmax-attention backward
// (FlashAttention-2); the mask, layout and GQA conventions are the forward's
// (unsloth "prefix_grouper_kernel.py", _make_mask_mod, flex_shared_prefix_attention).
#include <hip/hip_runtime.h>

#include <cmath>
#include <type_traits>

#include "attn_bwd.h"

namespace psa {
namespace {

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
  // bf16: Q | dO | L2 | -D (| node numbers) stages filled by direct-to-LDS loads into
  // swizzled, unpadded tiles (as the forward's K and V); fp32: through registers.
  static constexpr bool kDma = kBf16;
  static constexpr int LW = NODES ? 3 : 2;  // per-row words: L2, -D (, key)
  static constexpr int TILE_BYTES = BMS * D * 2;
  // DMA path: one 64-word slot per per-row array (a wave's dword load fills 64 lanes)
  // and a spare slot for the waves that load none of them; register path: BMS words
  static constexpr int RS = kDma ? 64 : BMS;
  static constexpr int STAGE_BYTES = 2 * TILE_BYTES + (LW + 1) * 64 * 4;
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
  // more = false: no next step; the loads then cover 0 bytes and write zeros into the
  // idle stage
  auto issue = [&](int n, const Cursor& u, int q_tile, bool more) {
    const int h = u.h, sub = u.sub;
    if constexpr (C::kDma) {  // into LDS stage n & 1: Q | dO | L2 | -D
      // Branch-free, so that its scalar work shares a block with the MFMAs that follow
      // and runs under them; 32-bit rows (T < 2^31) and 32 x 32 -> 64-bit products (a
      // 64-bit multiply is five scalar instructions, and the one wave of a SIMD issues
      // every one of them)
      const int q0 = q_tile * kTileM + sub * C::BMS;
      const int nvalid = more ? min(int(ntok) - q0, C::BMS) : 0;
      const uint64_t off = uint64_t(uint32_t(q0)) * uint32_t(pitch) + uint32_t(h * (2 * D));
      const uint64_t at = (uint64_t(uint32_t(h)) * uint32_t(ntok) + uint32_t(q0)) * 4u;
      const uint32_t st = smem_u + (n & 1) * C::STAGE_BYTES;
      st_next = st;
      rq = dma_rsrc(reinterpret_cast<const char*>(Qg) + off, nvalid * pitch);
      rg = dma_rsrc(reinterpret_cast<const char*>(Gg) + off, nvalid * pitch);
      // the rows' L2, -D (node form: and node numbers): wave w < LW loads array w into
      // slot w, the other waves load L2 again into the spare slot.  Rows past T (and
      // lanes past BMS) read 0: they sit in a partial tile and are masked (node 0 is
      // never visible).
      const char* ws = reinterpret_cast<const char*>(wave == 1 ? p.nD : p.L2) + at;
      if constexpr (NODES)
        if (wave == 2) ws = reinterpret_cast<const char*>(p.nkey) + uint64_t(uint32_t(q0)) * 4u;
      const int slot = wave < C::LW ? wave : C::LW;
      dma_load4(dma_rsrc(ws, nvalid * 4), lane * 4, st + 2 * C::TILE_BYTES + slot * 256);
    } else {
      const int64_t q0 = int64_t(q_tile) * kTileM + sub * C::BMS;
      const int nvalid = ntok - q0 < C::BMS ? int(ntok - q0) : C::BMS;
      const T* qp = Qg + q0 * ldq + int64_t(h) * D;
      const T* gp = Gg + q0 * ldq + int64_t(h) * D;
      const int64_t at = int64_t(h) * ntok + q0;
      {  // the per-row values first, loaded by every lane; rows past the end read 0
        const int rr = int(threadIdx.x) & (C::BMS - 1);
        l2_reg = __builtin_bit_cast(float, buf_load4(buf_rsrc(p.L2 + at, nvalid * 4), rr * 4));
        dl_reg = __builtin_bit_cast(float, buf_load4(buf_rsrc(p.nD + at, nvalid * 4), rr * 4));
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
    issue(0, cur, int(entry(e0) & 0x3fffffffu), true);
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
      if constexpr (C::kBf16) {  // K and V in AGPRs, where MFMAs read them (see above)
        asm volatile("" : "+a"(kf[s].v));
        if constexpr (kDK) asm volatile("" : "+a"(vf[s].v));
      } else {
        mark_ready(kf[s]);
        if constexpr (kDK) mark_ready(vf[s]);
      }
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
    const bool more = n + 1 < n_steps;
    if (more && nxt.e - e0 - wbase >= 64) {  // next window (a vector load; rare)
      window_load(nxt.e - e0);
      mark_ready(*reinterpret_cast<int32_t*>(&wreg));
    }
    if constexpr (C::kDma) {
      issue(n + 1, nxt, int(entry(more ? nxt.e : cur.e) & 0x3fffffffu), more);
    } else if (more) {
      // one buffer: the next sub-step is staged after this one's math
      if constexpr (!kSingle) issue(n + 1, nxt, int(entry(nxt.e) & 0x3fffffffu), true);
    }

    const char* st = smem + b * C::STAGE_BYTES;  // DMA stage
    const T* Qs = buf0 + b * C::BUF_ELEMS;       // register-path buffer
    const T* Gs = Qs + C::OFF_G;
    const T* Qt = Qs + C::OFF_QT;
    const T* Gt = Qs + C::OFF_GT;
    const float* Ls = C::kDma ? reinterpret_cast<const float*>(st + 2 * C::TILE_BYTES)
                              : ld0 + (b * C::LW + 0) * C::BMS;
    const float* Dsh = Ls + C::RS;
    const int32_t* Qk = reinterpret_cast<const int32_t*>(Ls + 2 * C::RS);  // node form

    {
      const int qd0 = q0i - kvrow_i;  // q - kv at the sub-step's first row
#pragma unroll
      for (int qb = 0; qb < C::BMS / 32; ++qb) {
        f32x16 sacc = zero16(), pacc = zero16();
        const T* qr = Qs + (32 * qb + l32) * C::NS + 8 * half;
        const T* gr = Gs + (32 * qb + l32) * C::NS + 8 * half;
        // the rows' LSE (log2 units) and -D, read before the products so that their
        // latency passes under them
        f32x4 l2v[4], dlv[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int ql = 32 * qb + g * 8 + half * 4;
          l2v[g] = *reinterpret_cast<const f32x4*>(Ls + ql);
          if constexpr (kDK) dlv[g] = *reinterpret_cast<const f32x4*>(Dsh + ql);
        }
        // bf16: the dP sums start at the rows' -D, so dP - D comes out of the MFMAs
        // (16 subtractions fewer per block); fp32 subtracts after its own products
        if constexpr (C::kDma && kDK) {
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int u = 0; u < 4; ++u) pacc[4 * g + u] = dlv[g][u];
        }
        if constexpr (C::kDma) {
          // Q and dO fragments read PF - 1 reduction steps ahead of their MFMAs (one:
          // two and three measured 0-3 % slower, the LDS pipe being shared by the
          // four waves)
          constexpr int NS = D / 16, PF = 2;
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
            for (int u = 0; u < 4; ++u)
              ds[4 * g + u] = C::kDma ? pv[4 * g + u] * pacc[4 * g + u]
                                      : pv[4 * g + u] * (pacc[4 * g + u] + dlv[g][u]);
        }
        if constexpr (C::kDma) {
          // dV += dO^T P and dK += Q^T dS over these 32 queries (two 16-query
          // fragments t): P and dS rounded to bf16, the (t, db) transposed reads
          // PF - 1 products ahead of their MFMAs; then, where split_wanted, the
          // residuals in a second pass
          constexpr int ND = D / 32, NI = 2 * ND, PF = 2;
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
        issue(n + 1, nxt, int(entry(nxt.e) & 0x3fffffffu), true);
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

}  // namespace

template <typename T, typename G, int D, int MODE, bool NODES>
hipError_t launch_dkdv_t(BwdParams p, int64_t n_ktiles, hipStream_t stream) {
  // fp32 at d >= 128: dV and dK in separate passes (room for the per-sub-step partial
  // sums of fp32), and at d = 256 each of them in two launches of half the columns
  constexpr bool kF32 = std::is_same<T, float>::value;
  constexpr int CS = kF32 && D > 128 ? 2 : 1;
  constexpr bool kTwoPass = D > 128 || (kF32 && D >= 128);
  p.n_work = n_ktiles * p.hkv;
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
  } else {
    p.c0 = 0;
    hipLaunchKernelGGL((dkdv_kernel<T, G, D, MODE, 0, NODES>), dim3(unsigned(grid)),
                       dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

// the variants the dispatch in attn_bwd.hip instantiates
#define PSA_DKDV(T, G, D, MODE)                                                          \
  template hipError_t launch_dkdv_t<T, G, D, MODE, true>(BwdParams, int64_t, hipStream_t); \
  template hipError_t launch_dkdv_t<T, G, D, MODE, false>(BwdParams, int64_t, hipStream_t);
#define PSA_DKDV_D(T, G, MODE) PSA_DKDV(T, G, 64, MODE) PSA_DKDV(T, G, 128, MODE) PSA_DKDV(T, G, 256, MODE)
PSA_DKDV_D(bf16_t, float, kSplitAdaptive)
PSA_DKDV_D(bf16_t, float, kSplitAll)
PSA_DKDV_D(bf16_t, bf16_t, kSplitAdaptive)
PSA_DKDV_D(bf16_t, bf16_t, kSplitAll)
PSA_DKDV_D(float, float, kSplitAdaptive)
#undef PSA_DKDV_D
#undef PSA_DKDV

}  // namespace psa
