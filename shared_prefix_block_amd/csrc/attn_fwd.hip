// Forward kernel: block-sparse masked softmax attention with an online softmax.
//
// One work-group = one q-tile of 128 rows (4 waves x 32 rows) for one q head.  It
// walks the q-tile's CSR list of non-empty kv-tiles (ascending, so for a completion
// row the prompt run comes first and its own completion run after it) in sub-steps
// of BN keys.  The K and V tiles of a sub-step live in one of two LDS buffers; the
// global reads of the next sub-step are issued into registers before the current
// one is computed and written to the other buffer after it, so each sub-step needs
// one barrier and its loads overlap the math.  Per sub-step and wave:
//   S^T = K Q^T on MFMA (Q stays in registers);
//   the mask, as a select, on partial tiles only: kv <= q < end[kv] (interval form)
//   or kv <= q with q's node in kv's subtree (node form, any layout);
//   the online softmax in the exp2 domain (log2(e) folded into the scale); the
//   running max is raised only when a row's max grows by more than 2^8 (the
//   result is the same: m cancels between O and l; it only bounds P by 2^8), so
//   the O rescale is skipped on almost every sub-step;
//   O^T += V^T P^T on MFMA with P from registers.  bf16 V stays row-major in LDS and
//   its transposed fragments come from the LDS transpose read; fp32 V is staged
//   transposed.
// The epilogue writes O = O / l and LSE = ln 2 * (m + log2 l); rows that saw no key
// get O = 0 and LSE = -inf.
//
// Sources: unsloth "prefix_grouper_kernel.py" (module docstring: masked blocks are
// skipped, realising the P + G*R saving; the comment on the flash block sizes: a
// completion row's two disjoint key runs go through one online softmax;
// flex_shared_prefix_attention: layout, GQA, default scale).
#include <hip/hip_runtime.h>

#include <cmath>
#include <type_traits>

#include "attn_common.h"
#include "psa_internal.h"

namespace psa {
namespace {

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* end;   // interval form
  const int32_t* nkey;  // node form
  const int32_t* nlo;
  const int32_t* nw;
  int32_t causal;  // node form: 0 drops the kv <= q conjunct
  const int32_t* row_ptr;
  const int32_t* col;
  const uint8_t* kind;
  const int32_t* qorder;
  int64_t T;
  int32_t hq, hkv;
  float c;  // scale * log2(e)
  int64_t n_work;
  int32_t chunk;
};

constexpr float kRescaleSlack = 8.0f;  // log2 units: P stays below 2^8

template <typename T, int D, bool NODES>
struct FwdCfg {
  static constexpr bool kBf16 = std::is_same<T, bf16_t>::value;
  // fp8 inputs: the scores on the fp8 MFMA; V is widened to bf16 on its way to LDS
  // (exactly) and the PV product, the softmax and O are those of the bf16 path
  static constexpr bool kFp8 = std::is_same<T, fp8_t>::value;
  using PT = typename std::conditional<kFp8, bf16_t, T>::type;  // P, V tile, O type
  static constexpr int NW = 4;
  static constexpr int NT = NW * 64;
  static constexpr int BM = 32 * NW;
  static_assert(BM == kTileM, "q-tile must match the map");
  static constexpr int EB = int(sizeof(T));
  static constexpr int BN = (!kBf16 && !kFp8 && D * EB > 256) ? 32 : 64;  // keys per sub-step
  static constexpr int NSUB = kTileN / BN;
  static constexpr int KS = D + 16 / EB;                  // K row stride (elements)
  static constexpr int VS = kBf16 ? D + 32 / EB : BN + 16 / EB;  // V (row-major) or V^T
  static constexpr int K_ELEMS = BN * KS;
  static constexpr int V_ELEMS = kBf16 ? BN * VS : D * VS;
  static constexpr int BUF_ELEMS = K_ELEMS + V_ELEMS;
  // bf16 tiles come in by direct-to-LDS loads into swizzled, unpadded tiles (two
  // stages of K | V | mask words); fp32 tiles go through registers into padded tiles.
  // Mask words per key: end[] (interval form) or lo[] | w[] (node form).
  // fp8: K by direct-to-LDS loads (rows of D bytes), V through registers (widened).
  static constexpr bool kDma = kBf16 || kFp8;
  static constexpr int MW = NODES ? 2 : 1;
  static constexpr int KT_BYTES = BN * D * EB;  // K tile (row-major, swizzled)
  static constexpr int VT_BYTES = BN * D * 2;   // V tile (bf16, row-major, swizzled)
  static constexpr int STAGE_BYTES = KT_BYTES + VT_BYTES + MW * BN * 4;
  static constexpr int LDS_BYTES = kDma ? 2 * STAGE_BYTES : 2 * BUF_ELEMS * EB + 2 * MW * BN * 4;
  static constexpr int WAVES_PER_EU = ((kBf16 || kFp8) && D <= 128) ? 2 : 1;
};

template <typename T, int D, bool NODES>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(FwdCfg<T, D, NODES>::WAVES_PER_EU))) void fwd_kernel(FwdParams p) {
  using C = FwdCfg<T, D, NODES>;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS_BYTES];
  T* const buf0 = reinterpret_cast<T*>(smem);
  int32_t* const es0 = reinterpret_cast<int32_t*>(smem + 2 * C::BUF_ELEMS * C::EB);

  const int64_t w_id = xcd_remap(blockIdx.x, p.chunk);
  if (w_id >= p.n_work) return;
  const int64_t ntok = p.T;
  const int hq = p.hq, hkv = p.hkv, rep = hq / hkv;
  const int h = int(w_id % hq);
  const int qt = p.qorder[w_id / hq];
  const int hk = h / rep;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int64_t qrow = int64_t(qt) * C::BM + 32 * wave + l32;
  const int wave_last = qt * C::BM + 32 * wave + 31;  // this wave's last row
  const bool qvalid = qrow < ntok;
  const int qrow_i = int(qrow);

  const T* Q = static_cast<const T*>(p.q);
  const T* K = static_cast<const T*>(p.k);
  const T* V = static_cast<const T*>(p.v);

  using PT = typename C::PT;
  constexpr int NQF = C::kFp8 ? D / 64 : D / 16;  // Q fragments (reduction steps of S)
  Frag<T> qf[NQF];  // loaded below, once the first tile's loads are in flight
  // d = 256 (bf16, e4m3): Q is pinned in AGPRs, where the MFMAs read it, and this unit
  // is compiled with MFMA results in VGPRs: S lands where the softmax reads it, instead
  // of the compiler keeping S and O in AGPRs and moving them (456 register moves per
  // sub-step at d = 256 before)
  constexpr bool kQInAgpr = (C::kBf16 || C::kFp8) && D == 256;

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = zero16();
  float m = -INFINITY, l = 0.f;
  const float c = p.c;
  const int64_t ldk = int64_t(hkv) * D;
  const int64_t koff = int64_t(hk) * D;

  // Sub-steps of the CSR list: every kv-tile gives NSUB of them, except a tile that
  // crosses T (always the last of the list) which stops at T.
  const int e0 = p.row_ptr[qt], e1 = p.row_ptr[qt + 1];
  int n_steps = (e1 - e0) * C::NSUB;
  if (e1 > e0) {
    const int64_t last0 = int64_t(p.col[e1 - 1]) * kTileN;
    const int64_t left = ntok - last0;
    if (left < kTileN) n_steps -= C::NSUB - int((left + C::BN - 1) / C::BN);
  }

  // CSR entries (kv-tile index | kind << 30) of a 64-entry window in one register,
  // lane i holding entry wbase + i; the loop reads them with readlane, so it issues
  // no scalar loads and the wait counts below see only the tile loads.
  int wbase = 0;
  uint32_t wreg = 0;
  auto window_load = [&](int base) {
    wbase = base;
    const int e = e0 + base + lane;
    wreg = e < e1 ? uint32_t(p.col[e]) | (uint32_t(p.kind[e]) << 30) : 0u;
  };
  auto entry = [&](int n) {  // packed entry of sub-step n (inside the window)
    return uint32_t(__builtin_amdgcn_readlane(int(wreg), n / C::NSUB - wbase));
  };
  window_load(0);
  mark_ready(*reinterpret_cast<int32_t*>(&wreg));

  // register-path staging (fp32 only; the DMA paths never touch it)
  using RT = typename std::conditional<C::kDma, float, T>::type;
  RowStage<RT, C::BN, D, C::KS, C::NT> kst;
  using VStage = typename std::conditional<C::kBf16, RowStage<RT, C::BN, D, C::VS, C::NT>,
                                           TransStage<RT, C::BN, D, C::VS, C::NT>>::type;
  VStage vst;
  DmaTile<C::BN, C::kFp8 ? D / 2 : D, C::NT> dt;  // K (and bf16 V) tile loads
  const int pitch = int(ldk) * C::EB;
  if constexpr (C::kDma) dt.init(pitch);
  // fp8: this thread's 16-byte chunks of the next V tile, widened at commit_v
  constexpr int NVC = C::kFp8 ? C::BN * (D / 16) / C::NT : 1;
  u32x4 vreg[NVC];
  int32_t e_reg = 0, kv_reg = 0, w_reg = 0;
  int32_t qkey = 0;  // node form: this row's node number (0: a pad or past T)
  const int32_t* const ev = NODES ? p.nlo : p.end;

  // DMA path: a stage's K and V tile loads are not issued in one burst (the wave
  // would stall on the memory-request queue) but one per reduction step of the
  // current sub-step's S product, where the MFMAs hide their issue cost.  Without a
  // next sub-step the descriptors cover 0 bytes and the loads only write zeros into
  // the idle buffer.
  constexpr int NL = DmaTile<C::BN, C::kFp8 ? D / 2 : D, C::NT>::N;  // loads per tile, wave
  constexpr int NDMA = C::kFp8 ? NL : 2 * NL;  // K and (bf16) V tile loads per stage
  DmaRsrc rk{}, rvv{};
  const uint32_t smem_u = lds_addr_u(smem);
  uint32_t st_next = smem_u;  // LDS address of the stage being filled
  auto dma_part = [&](int j) {
    if constexpr (C::kDma) {
      const int w = wave_id();  // wave-uniform: the LDS address stays scalar
      if (j < NL)
        dma_load16(rk, dt.voff[j], st_next + (j * (C::NT / 64) + w) * 1024);
      else
        dma_load16(rvv, dt.voff[j - NL],
                   st_next + C::KT_BYTES + ((j - NL) * (C::NT / 64) + w) * 1024);
    }
  };

  auto issue = [&](int n, int col_n) {  // global reads of sub-step n
    if constexpr (C::kDma) {  // straight into LDS stage n & 1: K | V | mask words
      static_assert(C::BN == 64, "one end[] value per lane");
      // 32-bit rows (T < 2^31) and one 32 x 32 -> 64-bit product for the tile's byte
      // offset (a 64-bit multiply is five scalar instructions)
      const int kv0 = col_n * kTileN + (n % C::NSUB) * C::BN;
      const int nvalid = min(int(ntok) - kv0, C::BN);
      const uint64_t off = uint64_t(uint32_t(kv0)) * uint32_t(pitch) + uint32_t(hk * D * C::EB);
      st_next = smem_u + (n & 1) * C::STAGE_BYTES;
      rk = dma_rsrc(reinterpret_cast<const char*>(K) + off, nvalid * pitch);
      if constexpr (C::kFp8) {  // V into registers (rows past the end read 0)
        const auto rs = buf_rsrc(reinterpret_cast<const char*>(V) + off, nvalid * pitch);
#pragma unroll
        for (int it = 0; it < NVC; ++it) {
          const int cidx = it * C::NT + int(threadIdx.x);
          vreg[it] = buf_load16(rs, (cidx / (D / 16)) * pitch + (cidx % (D / 16)) * 16);
        }
      } else {
        rvv = dma_rsrc(reinterpret_cast<const char*>(V) + off, nvalid * pitch);
      }
      const uint32_t mw = st_next + C::KT_BYTES + C::VT_BYTES;
      if (wave == 0)  // keys past the end read end = 0 (or w = 0): never visible
        dma_load4(dma_rsrc(ev + kv0, nvalid * 4), lane * 4, mw);
      if constexpr (NODES)
        if (wave == 1) dma_load4(dma_rsrc(p.nw + kv0, nvalid * 4), lane * 4, mw + C::BN * 4);
    } else {  // into registers; commit() stores them
      const int64_t kv0 = int64_t(col_n) * kTileN + (n % C::NSUB) * C::BN;
      const int nvalid = ntok - kv0 < C::BN ? int(ntok - kv0) : C::BN;
      // mask words first: the loads retire in order, so waiting for them at commit
      // does not wait for the K/V reads issued after them
      const int r = int(threadIdx.x) & (C::BN - 1);
      e_reg = int32_t(buf_load4(buf_rsrc(ev + kv0, nvalid * 4), r * 4));
      if constexpr (NODES) w_reg = int32_t(buf_load4(buf_rsrc(p.nw + kv0, nvalid * 4), r * 4));
      kv_reg = r < nvalid ? int32_t(kv0 + r) : 0;
      kst.load(reinterpret_cast<const RT*>(K) + kv0 * ldk + koff, ldk, nvalid);
      vst.load(reinterpret_cast<const RT*>(V) + kv0 * ldk + koff, ldk, nvalid);
    }
  };
  auto commit = [&](int b) {  // registers -> LDS buffer b (register path)
    T* kb = buf0 + b * C::BUF_ELEMS;
    kst.store(reinterpret_cast<RT*>(kb));
    vst.store(reinterpret_cast<RT*>(kb + C::K_ELEMS));
    if (threadIdx.x < C::BN) {
      if constexpr (NODES) {  // lo | w
        es0[b * 2 * C::BN + threadIdx.x] = e_reg;
        es0[b * 2 * C::BN + C::BN + threadIdx.x] = w_reg;
      } else {
        es0[b * C::BN + threadIdx.x] = e_reg - kv_reg;  // reach
      }
    }
  };

  // fp8: the staged V chunks of the next sub-step, widened to bf16 into buffer b
  auto commit_v = [&](int b) {
    if constexpr (C::kFp8) {
      char* vt = smem + b * C::STAGE_BYTES + C::KT_BYTES;
#pragma unroll
      for (int it = 0; it < NVC; ++it) {
        const int cidx = it * C::NT + int(threadIdx.x);
        const int r = cidx / (D / 16), cc = cidx % (D / 16);
        uint32_t w[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) fp8x4_to_bf16(vreg[it][j], w[2 * j], w[2 * j + 1]);
        *reinterpret_cast<u32x4*>(vt + swz_off<D / 8>(r, 2 * cc)) = u32x4{w[0], w[1], w[2], w[3]};
        *reinterpret_cast<u32x4*>(vt + swz_off<D / 8>(r, 2 * cc + 1)) =
            u32x4{w[4], w[5], w[6], w[7]};
      }
    }
  };

  if (n_steps > 0) {
    issue(0, int(entry(0) & 0x3fffffffu));
    if constexpr (C::kDma) {
#pragma unroll
      for (int j = 0; j < NDMA; ++j) dma_part(j);
      commit_v(0);
    } else {
      commit(0);
    }
  }
  {  // Q stays in registers; its loads overlap the first tile's
    if constexpr (C::kFp8) {  // lane half h: bytes 64 s + 32 h .. +32 of the row
      const char* qp = reinterpret_cast<const char*>(Q + (qrow * hq + h) * D) + 32 * half;
#pragma unroll
      for (int s = 0; s < NQF; ++s) {
        u32x4 a = u32x4{0u, 0u, 0u, 0u}, bb = a;
        if (qvalid) {
          a = *reinterpret_cast<const u32x4*>(qp + 64 * s);
          bb = *reinterpret_cast<const u32x4*>(qp + 64 * s + 16);
        }
        qf[s].v = i32x8{int(a[0]), int(a[1]), int(a[2]), int(a[3]),
                        int(bb[0]), int(bb[1]), int(bb[2]), int(bb[3])};
      }
    } else {
      const T* qp = Q + (qrow * hq + h) * D + 8 * half;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) qf[s] = qvalid ? frag_load(qp + 16 * s) : frag_zero<T>();
    }
    if constexpr (NODES) qkey = qvalid ? p.nkey[qrow] : 0;
#pragma unroll
    for (int s = 0; s < NQF; ++s) {
      if constexpr (kQInAgpr)  // see kQInAgpr
        asm volatile("" : "+a"(qf[s].v));
      else
        mark_ready(qf[s]);
    }
    if constexpr (NODES) mark_ready(qkey);
  }
  if constexpr (!C::kDma) __syncthreads();

  for (int n = 0; n < n_steps; ++n) {
    const int b = n & 1;
    if constexpr (C::kDma) {
      // this wave's loads of stage n are in; after the barrier everyone's are, and
      // every wave is done reading stage n - 1, which the next issue overwrites
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
      issue(n + 1, int(entry(n + 1) & 0x3fffffffu));
    } else if constexpr (C::kDma) {
      st_next = smem_u + ((n + 1) & 1) * C::STAGE_BYTES;  // idle buffer, zero-byte loads
      rk = dma_rsrc(K, 0);
      rvv = rk;
    }

    const char* st = smem + b * C::STAGE_BYTES;  // DMA stage
    const T* Ks = buf0 + b * C::BUF_ELEMS;       // register-path buffer
    const T* Vs = Ks + C::K_ELEMS;
    const int32_t* Es = C::kDma ? reinterpret_cast<const int32_t*>(st + C::KT_BYTES + C::VT_BYTES)
                                : es0 + b * C::MW * C::BN;

    // a partial tile's sub-step whose keys all come after this wave's rows holds no
    // kept pair (kv <= q is part of every causal mask): the wave skips its products
    // and softmax update (both would leave its state as it is); the next stage's tile
    // loads still go out
    if (partial && p.causal && kv0i > wave_last) {
      if constexpr (C::kDma) {
#pragma unroll
        for (int j = 0; j < NDMA; ++j) dma_part(j);
      }
    } else {
      // S^T = K Q^T for BN keys x 32 queries (this wave)
      // (the BN/32 accumulation chains are interleaved so that consecutive MFMAs do
      // not wait on each other's results)
      float sv[C::BN / 32][16];
      {
        f32x16 acc_s[C::BN / 32];
#pragma unroll
        for (int kb = 0; kb < C::BN / 32; ++kb) acc_s[kb] = zero16();
        const T* kr = Ks + l32 * C::KS + 8 * half;
        if constexpr (C::kFp8) {
          // every K fragment of the sub-step first (two 16-byte chunks of a row per
          // lane: bytes 64 s + 32 h .. +32), then the MFMAs over 64 reduction indices
          constexpr int NS = D / 64, NK = C::BN / 32;
          Frag<fp8_t> kq[NS][NK];
#pragma unroll
          for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int kb = 0; kb < NK; ++kb) {
              const u32x4 a = frag_load_swz<D / 16>(st, 32 * kb + l32, 4 * s + 2 * half).v;
              const u32x4 bb = frag_load_swz<D / 16>(st, 32 * kb + l32, 4 * s + 2 * half + 1).v;
              kq[s][kb].v = i32x8{int(a[0]), int(a[1]), int(a[2]), int(a[3]),
                                  int(bb[0]), int(bb[1]), int(bb[2]), int(bb[3])};
            }
#pragma unroll
          for (int s = 0; s < NS; ++s) {
#pragma unroll
            for (int kb = 0; kb < NK; ++kb) mma(acc_s[kb], kq[s][kb], qf[s]);
            // the next stage's K tile loads, spread over these steps
#pragma unroll
            for (int j = 0; j < NDMA; ++j)
              if ((j * NS) / NDMA == s) dma_part(j);
          }
        } else if constexpr (C::kDma) {
          // K fragments read PF reduction steps ahead of their MFMAs, so that LDS
          // latency overlaps the MFMAs in flight
          constexpr int NS = D / 16, NK = C::BN / 32, PF = 3;
          Frag<T> kq[PF][NK];
#pragma unroll
          for (int s = 0; s < PF - 1; ++s)
#pragma unroll
            for (int kb = 0; kb < NK; ++kb)
              kq[s][kb] = frag_load_swz<D / 8>(st, 32 * kb + l32, half + 2 * s);
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            if (s + PF - 1 < NS) {
#pragma unroll
              for (int kb = 0; kb < NK; ++kb)
                kq[(s + PF - 1) % PF][kb] =
                    frag_load_swz<D / 8>(st, 32 * kb + l32, half + 2 * (s + PF - 1));
            }
#pragma unroll
            for (int kb = 0; kb < NK; ++kb) mma(acc_s[kb], kq[s % PF][kb], qf[s]);
            // the next stage's tile loads, spread over these steps
#pragma unroll
            for (int j = 0; j < 2 * NL; ++j)
              if ((j * NS) / (2 * NL) == s) dma_part(j);
          }
          // keep that order: the first PF-1 steps' reads, then per step the reads
          // PF-1 steps ahead followed by this step's MFMAs
          __builtin_amdgcn_sched_group_barrier(0x100, (PF - 1) * NK, 0);
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            if (s + PF - 1 < NS) __builtin_amdgcn_sched_group_barrier(0x100, NK, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, NK, 0);
          }
        } else {
#pragma unroll
          for (int s = 0; s < D / 16; ++s)
#pragma unroll
            for (int kb = 0; kb < C::BN / 32; ++kb)
              mma(acc_s[kb], frag_load(kr + 32 * kb * C::KS + 16 * s), qf[s]);
        }
#pragma unroll
        for (int kb = 0; kb < C::BN / 32; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) sv[kb][i] = acc_s[kb][i];
      }
      if (NODES && partial) {  // uniform branch; node form
        const int qd = qrow_i - kv0i;
        const bool nc = p.causal == 0;
#pragma unroll
        for (int kb = 0; kb < C::BN / 32; ++kb) {
          int4 los[4], ws[4];  // this lane's keys' lo and w, read together
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
              sv[kb][4 * g + u] = keep ? sv[kb][4 * g + u] : -INFINITY;
            }
          }
        }
      } else if (partial) {  // uniform branch; full tiles skip the mask
        const int qd = qrow_i - kv0i;  // q - kv for the sub-step's first key
        // all of this lane's end[] (or reach) values first, so that their LDS reads
        // are in flight together
        int4 evs[C::BN / 32][4];
#pragma unroll
        for (int kb = 0; kb < C::BN / 32; ++kb)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            evs[kb][g] = *reinterpret_cast<const int4*>(Es + 32 * kb + g * 8 + half * 4);
#pragma unroll
        for (int kb = 0; kb < C::BN / 32; ++kb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int kvl = 32 * kb + g * 8 + half * 4;
            const int4 ev = evs[kb][g];
            const int rv[4] = {ev.x, ev.y, ev.z, ev.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              bool keep;
              if constexpr (C::kDma)  // raw end[]: kv <= q < end
                keep = (kvl + u <= qd) & (qrow_i < rv[u]);
              else  // reach = end - kv
                keep = visible_u(qd - kvl - u, rv[u]);
              sv[kb][4 * g + u] = keep ? sv[kb][4 * g + u] : -INFINITY;
            }
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < C::BN / 32; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sv[kb][i]);
      mx = max_halves(mx) * c;
      // raise the running max only when it grows by more than the slack
      const bool grow = mx > m + kRescaleSlack || (m == -INFINITY && mx > -INFINITY);
      if (__ballot(grow)) {  // wave-uniform branch
        const float m_new = grow ? mx : m;
        const float alpha = grow ? __builtin_amdgcn_exp2f(m - m_new) : 1.f;  // 0 if m = -inf
        m = m_new;
        l *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) acc[db] *= alpha;
      }
      const float m_use = m == -INFINITY ? 0.f : m;
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < C::BN / 32; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(sv[kb][i], c, -m_use));
          sv[kb][i] = pv;
          rs += pv;
        }
      l += rs;

      // O^T += V^T P^T, 16 keys per step
      if constexpr (C::kDma && D > 128) {
        // P fragments first; the (t, db) transposed V reads PF products ahead of
        // their MFMAs, so that LDS latency overlaps the MFMAs in flight (at d = 128
        // the compiler's own order of the reads is faster, at d = 256 this one)
        constexpr int NT16 = C::BN / 16, ND = D / 32, NI = NT16 * ND, PF = 3;
        Frag<PT> pfr[NT16];
#pragma unroll
        for (int t = 0; t < NT16; ++t) pfr[t] = frag_from<PT>(&sv[t >> 1][(t & 1) * 8]);
        const char* vst = st + C::KT_BYTES;
        Frag<PT> va[PF];
#pragma unroll
        for (int i = 0; i < PF - 1; ++i)
          va[i] = frag_load_tr_swz<D / 8>(vst, 16 * (i / ND), 32 * (i % ND));
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          if (i + PF - 1 < NI) {
            const int j = i + PF - 1;
            va[j % PF] = frag_load_tr_swz<D / 8>(vst, 16 * (j / ND), 32 * (j % ND));
          }
          mma(acc[i % ND], va[i % PF], pfr[i / ND]);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * (PF - 1), 3);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          if (i + PF - 1 < NI) __builtin_amdgcn_sched_group_barrier(0x100, 2, 3);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 3);
        }
      } else if constexpr (C::kDma) {
#pragma unroll
        for (int t = 0; t < C::BN / 16; ++t) {
          const Frag<PT> pf = frag_from<PT>(&sv[t >> 1][(t & 1) * 8]);
#pragma unroll
          for (int db = 0; db < D / 32; ++db)
            mma(acc[db], frag_load_tr_swz<D / 8>(st + C::KT_BYTES, 16 * t, 32 * db), pf);
        }
      } else {
        // fp32: the sub-step's product goes into a fresh block and is added to O
        // afterwards.  One accumulator chain over every key of a long list would round
        // at the magnitude of the running sum on each of its ~keys/2 steps; per-sub-step
        // partial sums round there once per sub-step.
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          f32x16 part = zero16();
#pragma unroll
          for (int t = 0; t < C::BN / 16; ++t)
            mma(part, frag_load(Vs + (32 * db + l32) * C::VS + 16 * t + 8 * half),
                frag_from<PT>(&sv[t >> 1][(t & 1) * 8]));
          acc[db] += part;
        }
      }
    }

    if constexpr (C::kFp8) {  // the next sub-step's V, widened (the barrier at the top
      if (n + 1 < n_steps) commit_v(b ^ 1);  // of the next step publishes it)
    }
    if constexpr (!C::kDma) {
      if (n + 1 < n_steps) commit(b ^ 1);
      __syncthreads();
    }
  }

  if constexpr (C::kDma) wait_vmcnt<0>();  // no load into LDS outlives the work-group
  const float lt = l + __shfl_xor(l, 32);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (qvalid) {
    PT* op = static_cast<PT*>(p.o) + (qrow * hq + h) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * db + g * 8 + half * 4;
        vec4_store(op + d, vec4_from(acc[db][4 * g] * inv, acc[db][4 * g + 1] * inv,
                                     acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv,
                                     static_cast<PT*>(nullptr)));
      }
    if (half == 0 && p.lse)  // no LSE store for a forward without gradient
      p.lse[int64_t(h) * ntok + qrow] =
          lt > 0.f ? (m + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
  }
}

template <typename T, int D>
hipError_t launch_fwd_t(const psa_tile_map& map, const AttnShape& s, const void* q,
                        const void* k, const void* v, void* o, float* lse,
                        hipStream_t stream) {
  FwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.end = map.end;
  p.nkey = map.nkey;
  p.nlo = map.nlo;
  p.nw = map.nw;
  p.causal = map.causal;
  p.row_ptr = map.row_ptr;
  p.col = map.col;
  p.kind = map.kind;
  p.qorder = map.qorder;
  p.T = s.T;
  p.hq = s.hq;
  p.hkv = s.hkv;
  p.c = s.scale * kLog2e;
  p.n_work = map.nq * s.hq;
  const int rep = s.hq / s.hkv;
  p.chunk = rep * 2;
  const int64_t per = 8 * int64_t(p.chunk);
  const int64_t grid = (p.n_work + per - 1) / per * per;
  if (map.form == kFormNodes)
    hipLaunchKernelGGL((fwd_kernel<T, D, true>), dim3(unsigned(grid)), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((fwd_kernel<T, D, false>), dim3(unsigned(grid)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace
}  // namespace psa

bool fwd_supported(psa_dtype dt, int32_t d) {
  if (dt == PSA_BF16 || dt == PSA_FP8_E4M3) return d == 64 || d == 128 || d == 256;
  if (dt == PSA_FP32) return d == 64 || d == 128 || d == 256;
  return false;
}

hipError_t launch_fwd(const psa_tile_map& map, psa_dtype dt, const AttnShape& s,
                      const void* q, const void* k, const void* v, void* o, float* lse,
                      hipStream_t stream) {
  using psa::bf16_t;
  using psa::fp8_t;
  if (dt == PSA_BF16) {
    switch (s.d) {
      case 64: return psa::launch_fwd_t<bf16_t, 64>(map, s, q, k, v, o, lse, stream);
      case 128: return psa::launch_fwd_t<bf16_t, 128>(map, s, q, k, v, o, lse, stream);
      case 256: return psa::launch_fwd_t<bf16_t, 256>(map, s, q, k, v, o, lse, stream);
    }
  } else if (dt == PSA_FP8_E4M3) {
    switch (s.d) {
      case 64: return psa::launch_fwd_t<fp8_t, 64>(map, s, q, k, v, o, lse, stream);
      case 128: return psa::launch_fwd_t<fp8_t, 128>(map, s, q, k, v, o, lse, stream);
      case 256: return psa::launch_fwd_t<fp8_t, 256>(map, s, q, k, v, o, lse, stream);
    }
  } else {
    switch (s.d) {
      case 64: return psa::launch_fwd_t<float, 64>(map, s, q, k, v, o, lse, stream);
      case 128: return psa::launch_fwd_t<float, 128>(map, s, q, k, v, o, lse, stream);
      case 256: return psa::launch_fwd_t<float, 256>(map, s, q, k, v, o, lse, stream);
    }
  }
  return hipErrorInvalidValue;
}
