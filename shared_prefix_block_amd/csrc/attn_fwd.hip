// Forward kernel: block-sparse masked softmax attention with an online softmax.
//
// One work-group = one q-tile of 128 rows (4 waves x 32 rows) for one q head.  It
// walks the q-tile's CSR list of non-empty kv-tiles (ascending, so for a completion
// row the prompt run comes first and its own completion run after it) in sub-steps
// of BN keys: K (row-major) and V (transposed, rows permuted) are staged in LDS,
// S^T = K Q^T runs on MFMA with Q held in registers, the per-element mask
// kv <= q < end[kv] is applied only on partial tiles, the running max / sum are
// updated (exp2 with log2(e) folded into the scale), and O^T += V^T P^T runs on MFMA
// with P taken from registers.  The epilogue divides by the row sum and writes
// O and LSE = ln 2 * (m + log2 l); rows that saw no key get O = 0, LSE = -inf.
//
// Sources: unsloth "prefix_grouper_kernel.py" (module docstring: masked blocks are
// skipped and the P + G*R saving is realised; the comment on the flash block sizes:
// the two disjoint key runs of a completion row go through one online softmax;
// flex_shared_prefix_attention: layout, GQA, default scale).
#include <hip/hip_runtime.h>

#include <cmath>

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
  const int32_t* end;
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

template <typename T, int D>
struct FwdCfg {
  static constexpr int NW = 4;
  static constexpr int NT = NW * 64;
  static constexpr int BM = 32 * NW;
  static_assert(BM == kTileM, "q-tile must match the map");
  static constexpr int BN = (D * int(sizeof(T)) > 256) ? 32 : 64;  // keys per sub-step
  static constexpr int EB = int(sizeof(T));
  static constexpr int KS = D + 16 / EB;   // K tile row stride (elements)
  static constexpr int VS = BN + 16 / EB;  // V^T tile row stride (elements)
  static constexpr int K_ELEMS = BN * KS;
  static constexpr int V_ELEMS = D * VS;
  static constexpr int LDS_BYTES = (K_ELEMS + V_ELEMS) * EB + BN * 4;
};

template <typename T, int D>
__global__ __launch_bounds__(256) void fwd_kernel(FwdParams p) {
  using C = FwdCfg<T, D>;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS_BYTES];
  T* Ks = reinterpret_cast<T*>(smem);
  T* Vt = Ks + C::K_ELEMS;
  int32_t* Es = reinterpret_cast<int32_t*>(Vt + C::V_ELEMS);

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
  const bool qvalid = qrow < ntok;
  const int qrow_i = int(qrow);

  const T* Q = static_cast<const T*>(p.q);
  const T* K = static_cast<const T*>(p.k);
  const T* V = static_cast<const T*>(p.v);

  Frag<T> qf[D / 16];
  {
    const T* qp = Q + (qrow * hq + h) * D + 8 * half;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qf[s] = qvalid ? frag_load(qp + 16 * s) : frag_zero<T>();
  }

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = zero16();
  float m = -INFINITY, l = 0.f;
  const float c = p.c;
  const int64_t ldk = int64_t(hkv) * D;

  const int e0 = p.row_ptr[qt], e1 = p.row_ptr[qt + 1];
  for (int e = e0; e < e1; ++e) {
    const int j = p.col[e];
    const bool partial = p.kind[e] == 1;
    for (int sub = 0; sub < kTileN / C::BN; ++sub) {
      const int64_t kv0 = int64_t(j) * kTileN + sub * C::BN;
      if (kv0 >= ntok) break;
      const int nvalid = ntok - kv0 < C::BN ? int(ntok - kv0) : C::BN;
      const int kv0i = int(kv0);
      __syncthreads();
      const T* kp = K + kv0 * ldk + int64_t(hk) * D;
      const T* vp = V + kv0 * ldk + int64_t(hk) * D;
      stage_rows<T, C::BN, D, C::KS, C::NT>(Ks, kp, ldk, nvalid);
      stage_rows_t<T, C::BN, D, C::VS, C::NT>(Vt, vp, ldk, nvalid);
      if (partial && threadIdx.x < C::BN) {
        const int r = threadIdx.x;
        Es[r] = r < nvalid ? p.end[kv0 + r] : int32_t(kv0 + r);
      }
      __syncthreads();

      // S^T = K Q^T for BN keys x 32 queries (this wave)
      float sv[C::BN / 32][16];
#pragma unroll
      for (int kb = 0; kb < C::BN / 32; ++kb) {
        f32x16 acc_s = zero16();
        const T* kr = Ks + (32 * kb + l32) * C::KS + 8 * half;
#pragma unroll
        for (int s = 0; s < D / 16; ++s) mma(acc_s, frag_load(kr + 16 * s), qf[s]);
#pragma unroll
        for (int i = 0; i < 16; ++i) sv[kb][i] = acc_s[i];
      }
      if (partial) {  // uniform branch; the mask itself is a select, no divergence
#pragma unroll
        for (int kb = 0; kb < C::BN / 32; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int kvl = 32 * kb + acc_row(i, half);
            sv[kb][i] = visible(kv0i + kvl, qrow_i, Es[kvl]) ? sv[kb][i] : -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < C::BN / 32; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sv[kb][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m, mx * c);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m - m_use);
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) acc[db] *= alpha;
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
#pragma unroll
      for (int t = 0; t < C::BN / 16; ++t) {
        float pv[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) pv[jj] = sv[t >> 1][(t & 1) * 8 + jj];
        const Frag<T> pf = frag_from<T>(pv);
        const T* vr = Vt + l32 * C::VS + 16 * t + 8 * half;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) mma(acc[db], frag_load(vr + 32 * db * C::VS), pf);
      }
    }
  }

  const float lt = l + __shfl_xor(l, 32);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (qvalid) {
    T* op = static_cast<T*>(p.o) + (qrow * hq + h) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * db + g * 8 + half * 4;
        vec4_store(op + d, vec4_from(acc[db][4 * g] * inv, acc[db][4 * g + 1] * inv,
                                     acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv,
                                     static_cast<T*>(nullptr)));
      }
    if (half == 0)
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
  hipLaunchKernelGGL((fwd_kernel<T, D>), dim3(unsigned(grid)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace
}  // namespace psa

bool fwd_supported(psa_dtype dt, int32_t d) {
  if (dt == PSA_BF16) return d == 64 || d == 128 || d == 256;
  if (dt == PSA_FP32) return d == 64 || d == 128;
  return false;
}

hipError_t launch_fwd(const psa_tile_map& map, psa_dtype dt, const AttnShape& s,
                      const void* q, const void* k, const void* v, void* o, float* lse,
                      hipStream_t stream) {
  using psa::bf16_t;
  if (dt == PSA_BF16) {
    switch (s.d) {
      case 64: return psa::launch_fwd_t<bf16_t, 64>(map, s, q, k, v, o, lse, stream);
      case 128: return psa::launch_fwd_t<bf16_t, 128>(map, s, q, k, v, o, lse, stream);
      case 256: return psa::launch_fwd_t<bf16_t, 256>(map, s, q, k, v, o, lse, stream);
    }
  } else {
    switch (s.d) {
      case 64: return psa::launch_fwd_t<float, 64>(map, s, q, k, v, o, lse, stream);
      case 128: return psa::launch_fwd_t<float, 128>(map, s, q, k, v, o, lse, stream);
    }
  }
  return hipErrorInvalidValue;
}
