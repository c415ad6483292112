// Backward kernels (FlashAttention-2 style gradients of the block-sparse forward).
//
//   bwd_pre : nD[h, q] = -sum_d dO[q, h, d] * O[q, h, d];  L2[h, q] = LSE * log2(e)
//             (+inf on rows that saw no key, so their probabilities come out 0).
//   dkdv    : (attn_bwd_dkdv.hip) one work-group per (kv-tile of 128 keys, kv head).  K and V stay in
//             registers; the CSC list of the kv-tile's non-empty q-tiles is walked for
//             every q head of the GQA group, so dK and dV are summed over the group
//             inside the work-group (no atomics, no repeated K/V).  Per q sub-step:
//             S = Q K^T and dP = dO V^T (Q, dO from LDS), P = exp2(S c - L2), masked on
//             partial tiles, dS = P (dP + nD), dV^T += dO^T P, dK^T += Q^T dS.
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

#include "attn_bwd.h"

namespace psa {
namespace {

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
    p.nD[int64_t(h) * p.T + q] = -acc;
    const float lse = p.lse[int64_t(h) * p.T + q];
    p.L2[int64_t(h) * p.T + q] = lse == -INFINITY ? INFINITY : lse * kLog2e;
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
    if constexpr (C::kDma) {  // straight into LDS stage n & 1: K | V | mask words
      // 32-bit rows (T < 2^31) and one 32 x 32 -> 64-bit product for the tile's byte
      // offset (a 64-bit multiply is five scalar instructions)
      const int kv0 = col_n * kTileN + (n % C::NSUB) * C::BN;
      const int nvalid = min(int(ntok) - kv0, C::BN);
      const uint64_t off = uint64_t(uint32_t(kv0)) * uint32_t(pitch) + uint32_t(hk * (2 * D));
      const uint32_t st = lds_addr_u(smem) + (n & 1) * C::STAGE_BYTES;
      dt.load(reinterpret_cast<const char*>(Kg) + off, nvalid, pitch, st);
      dt.load(reinterpret_cast<const char*>(Vg) + off, nvalid, pitch, st + C::TILE_BYTES);
      if (wave == 0 && lane < C::BN)  // keys past the end read end = 0 (or w = 0): never visible
        dma_load4(dma_rsrc(ev + kv0, nvalid * 4), lane * 4, st + 2 * C::TILE_BYTES);
      if constexpr (NODES)
        if (wave == 1 && lane < C::BN)
          dma_load4(dma_rsrc(p.nw + kv0, nvalid * 4), lane * 4,
                    st + 2 * C::TILE_BYTES + C::BN * 4);
    } else {
      const int64_t kv0 = int64_t(col_n) * kTileN + (n % C::NSUB) * C::BN;
      const int nvalid = ntok - kv0 < C::BN ? int(ntok - kv0) : C::BN;
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
        p.nD[int64_t(h) * ntok + qrow] = -dl;
        p.L2[int64_t(h) * ntok + qrow] = l2;
      }
    } else if (qvalid) {
      l2 = p.L2[int64_t(h) * ntok + qrow];
      dl = -p.nD[int64_t(h) * ntok + qrow];
    }
    if constexpr (NODES) qkey = qvalid ? p.nkey[qrow] : 0;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      if constexpr (C::kBf16 && D == 256) {  // in AGPRs, where the MFMAs read them
        asm volatile("" : "+a"(qf[s].v), "+a"(gf[s].v));
      } else {
        mark_ready(qf[s]);
        mark_ready(gf[s]);
      }
    }
    mark_ready(l2);
    mark_ready(dl);
    if constexpr (NODES) mark_ready(qkey);
  }
  if constexpr (!C::kDma) __syncthreads();
  // bf16: the dP sums start at -D (all 16 elements of a lane are its row's), so dP - D
  // comes out of the MFMAs
  f32x16 nd16;
#pragma unroll
  for (int i = 0; i < 16; ++i) nd16[i] = -dl;

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
        f32x16 sacc = zero16(), pacc = C::kDma ? nd16 : zero16();
        if constexpr (C::kDma) {
          // K and V fragments read PF - 1 reduction steps ahead of their MFMAs (one:
          // two measured ~1 % slower)
          constexpr int NS = D / 16, PF = 2;
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
        for (int ii = 0; ii < 16; ++ii) dsk[ii] = C::kDma ? pv[ii] * pacc[ii] : pv[ii] * (pacc[ii] - dl);
        if constexpr (C::kDma) {
          // dQ^T += K^T dS^T over this block's 32 keys (16-key fragments t): dS rounded,
          // the (t, db) transposed K reads PF - 1 products ahead of their MFMAs; then, where
          // split_wanted, the residuals
          constexpr int ND = D / 32, NI = 2 * ND, PF = 2;
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
  p.nD = static_cast<float*>(workspace);
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
  // fp32 at d = 256: dQ in two launches of half the columns (and dK, dV likewise, in
  // their own passes: launch_dkdv_t)
  constexpr bool kF32 = std::is_same<T, float>::value;
  constexpr int CS = kF32 && D > 128 ? 2 : 1;

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
    const hipError_t e = launch_dkdv_t<T, G, D, MODE, NODES>(p, map.nk, stream);
    if (e != hipSuccess) return e;
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
