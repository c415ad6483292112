// Building blocks shared by the forward and backward attention kernels (gfx950).
//
// Matrix work uses the CDNA 32x32 MFMA shapes: v_mfma_f32_32x32x16_bf16 for bf16
// inputs and v_mfma_f32_32x32x2_f32 for fp32 inputs, both accumulating in fp32.
// A "fragment" is the 8 consecutive reduction-index values one lane feeds to a
// 32x32 product over 16 reduction indices: lane l (row or column l % 32, half
// h = l / 32) holds reduction indices 8h .. 8h+7.  For bf16 that is one MFMA; for
// fp32 it is 8 MFMAs of 2 reduction indices each (lane half h supplies index j of
// its 8 in MFMA j), which sums the same 16 products in another order.
//
// Accumulator layout of a 32x32 block (the same for both MFMAs): lane l holds
// column l % 32 and rows (i / 4) * 8 + (l / 32) * 4 + (i % 4) for i = 0 .. 15.
//
// Scores are formed with the key index as the row (S^T = K Q^T), so each lane owns
// one query column and the row-wise softmax needs only in-lane work plus one
// exchange between lane halves.  The probabilities then feed the second product
// straight from registers as its B operand; the reduction index (keys) of that
// operand follows the accumulator's row order, so the tiles used as the A operand
// are stored transposed in LDS with rows permuted to match: within every 16 rows,
// groups of 4 rows (g = 0..3) sit at slots 0, 2, 1, 3.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace psa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

struct bf16_t {  // raw bfloat16 storage
  uint16_t bits;
};
struct fp8_t {  // raw fp8 storage, OCP e4m3 (the forward's scores take it)
  uint8_t bits;
};
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kLdsMax = 160 * 1024;  // LDS bytes a work-group may take on gfx950
constexpr float kLn2 = 0.6931471805599453f;

// The wave's index in its work-group, as a wave-uniform (scalar) value: addresses and
// branches derived from it then stay in scalar registers.  (The backward kernels and
// DmaTile::load take it; in the forward it measured slower: the compiler schedules
// that loop differently.)
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
}

// ---------------------------------------------------------------------------
// fragments
// ---------------------------------------------------------------------------
template <typename T>
struct Frag;
template <>
struct Frag<bf16_t> {
  u32x4 v;
};
template <>
struct Frag<float> {
  f32x4 lo, hi;
};
// fp8: the 32 consecutive reduction-index values one lane feeds to a 32x32 product over
// 64 reduction indices (lane half h holds indices 32h .. 32h+31 of both operands; any
// assignment the two operands share gives the same sum, and a probe of the MFMA with
// small integers confirmed this one exactly).
template <>
struct Frag<fp8_t> {
  i32x8 v;
};

template <typename T>
__device__ __forceinline__ Frag<T> frag_zero();
template <>
__device__ __forceinline__ Frag<bf16_t> frag_zero<bf16_t>() {
  Frag<bf16_t> f;
  f.v = u32x4{0u, 0u, 0u, 0u};
  return f;
}
template <>
__device__ __forceinline__ Frag<float> frag_zero<float>() {
  Frag<float> f;
  f.lo = f32x4{0.f, 0.f, 0.f, 0.f};
  f.hi = f.lo;
  return f;
}

// 8 consecutive elements (16-byte aligned for bf16, 32-byte for fp32).
__device__ __forceinline__ Frag<bf16_t> frag_load(const bf16_t* p) {
  Frag<bf16_t> f;
  f.v = *reinterpret_cast<const u32x4*>(p);
  return f;
}
__device__ __forceinline__ Frag<float> frag_load(const float* p) {
  Frag<float> f;
  f.lo = *reinterpret_cast<const f32x4*>(p);
  f.hi = *reinterpret_cast<const f32x4*>(p + 4);
  return f;
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> one packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// Fragment from 8 fp32 values (probabilities or score gradients).
template <typename T>
__device__ __forceinline__ Frag<T> frag_from(const float* x);
template <>
__device__ __forceinline__ Frag<bf16_t> frag_from<bf16_t>(const float* x) {
  Frag<bf16_t> f;
  f.v = u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
              pack_bf16x2(x[6], x[7])};
  return f;
}
template <>
__device__ __forceinline__ Frag<float> frag_from<float>(const float* x) {
  Frag<float> f;
  f.lo = f32x4{x[0], x[1], x[2], x[3]};
  f.hi = f32x4{x[4], x[5], x[6], x[7]};
  return f;
}

// Residual of a rounded fragment: with hi = frag_from(x) (x rounded to bf16), returns
// lo = bf16(x - hi).  x - hi is exact in fp32, so hi + lo carries x to about 2^-17
// relative instead of 2^-9, and a product with hi followed by one with lo (exact
// bf16 x bf16 products, fp32 sums) is that much closer to the fp32 product.  The
// backward uses it for P and dS where they are large.
__device__ __forceinline__ Frag<bf16_t> frag_residual(const float* x, const Frag<bf16_t>& hi) {
  Frag<bf16_t> lo;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float h0 = __builtin_bit_cast(float, hi.v[j] << 16);          // element 2j
    const float h1 = __builtin_bit_cast(float, hi.v[j] & 0xffff0000u);  // element 2j+1
    lo.v[j] = pack_bf16x2(x[2 * j] - h0, x[2 * j + 1] - h1);
  }
  return lo;
}
// fp32 fragments hold x exactly: the residual is 0 (the kernels never ask for it; it
// keeps the shared code well-formed for both types).
__device__ __forceinline__ Frag<float> frag_residual(const float*, const Frag<float>&) {
  Frag<float> lo;
  lo.lo = f32x4{0.f, 0.f, 0.f, 0.f};
  lo.hi = lo.lo;
  return lo;
}

__device__ __forceinline__ void mma(f32x16& c, const Frag<bf16_t>& a, const Frag<bf16_t>& b) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a.v),
                                              __builtin_bit_cast(bf16x8, b.v), c, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x16& c, const Frag<float>& a, const Frag<float>& b) {
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[0], b.lo[0], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[1], b.lo[1], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[2], b.lo[2], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[3], b.lo[3], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi[0], b.hi[0], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi[1], b.hi[1], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi[2], b.hi[2], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi[3], b.hi[3], c, 0, 0, 0);
}

// OCP e4m3 x e4m3 on the 32x32x64 scaled MFMA with unit scales (exponent 127).  Its
// products are exact; a probe found its sums within ~1e-4 relative of fp32 sums when
// the terms span many binades.
__device__ __forceinline__ void mma(f32x16& c, const Frag<fp8_t>& a, const Frag<fp8_t>& b) {
  c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a.v, b.v, c, 0, 0, 0, 127, 0, 127);
}

// Four OCP e4m3 bytes of w -> two packed bf16 pairs (exact: every e4m3 value is a bf16
// value, and the fp32 conversion's low half is zero).
__device__ __forceinline__ void fp8x4_to_bf16(uint32_t w, uint32_t& lo, uint32_t& hi) {
  const uint32_t a = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_f32_fp8(int(w), 0));
  const uint32_t b = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_f32_fp8(int(w), 1));
  const uint32_t c = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_f32_fp8(int(w), 2));
  const uint32_t d = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_f32_fp8(int(w), 3));
  lo = (a >> 16) | (b & 0xffff0000u);
  hi = (c >> 16) | (d & 0xffff0000u);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Maximum of x over lanes l and l ^ 32 (the two halves of a wave) in VALU, without an
// LDS round trip.  v_permlane32_swap a, b exchanges the upper half of a with the lower
// half of b; from two copies of x it leaves (x_lo, x_lo) in a and (x_hi, x_hi) in b, and
// their elementwise max is max(x_l, x_(l^32)) in every lane.  It is written as inline
// assembly because the compiler's model of the intrinsic folds the two results of a
// swap of one value into one.  The s_nop gives the two wait states a permlane needs
// after a VALU write of its operands.
__device__ __forceinline__ float max_halves(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}

// The mask in interval form: key kv is visible to row q iff kv <= q < end[kv], i.e.
// (unsigned)(q - kv) < reach[kv] with reach = end - kv >= 0 (0 for a pad: never
// visible).  One compare, used as a select (no short-circuit branch).
__device__ __forceinline__ bool visible_u(int q_minus_kv, int reach) {
  return uint32_t(q_minus_kv) < uint32_t(reach);
}

// Tile kind of list entry e (0 empty, 1 partial, 2 full) read as part of an aligned
// dword: a wave-uniform 4-byte load goes through the scalar unit, so testing it never
// waits on the vector loads in flight (a byte load would be a vector load).
__device__ __forceinline__ int tile_kind(const uint8_t* kinds, int e) {
  const uint32_t w = reinterpret_cast<const uint32_t*>(kinds)[e >> 2];
  return int((w >> (8 * (e & 3))) & 0xffu);
}
// The same in two halves, for reading a sub-step ahead: the dword holding entry e,
// and the kind extracted from it when it is needed.
__device__ __forceinline__ uint32_t tile_kind_word(const uint8_t* kinds, int e) {
  return reinterpret_cast<const uint32_t*>(kinds)[e >> 2];
}
__device__ __forceinline__ int kind_from_word(uint32_t w, int e) {
  return int((w >> (8 * (e & 3))) & 0xffu);
}

// Row (within a 32x32 accumulator block) of element i for lane half h.
__device__ __forceinline__ int acc_row(int i, int half) { return (i >> 2) * 8 + half * 4 + (i & 3); }

// Position of row r inside a transposed, row-permuted tile (see the file comment).
__device__ __forceinline__ int perm_pos(int r) {
  const int g = (r >> 2) & 3;
  return (r & ~15) + (((g & 1) << 1) | (g >> 1)) * 4 + (r & 3);
}

// Sum of the 8 elementwise products of two fragments, in fp32.
__device__ __forceinline__ float frag_dot(const Frag<bf16_t>& a, const Frag<bf16_t>& b) {
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    acc = fmaf(__builtin_bit_cast(float, a.v[j] << 16), __builtin_bit_cast(float, b.v[j] << 16), acc);
    acc = fmaf(__builtin_bit_cast(float, a.v[j] & 0xffff0000u),
               __builtin_bit_cast(float, b.v[j] & 0xffff0000u), acc);
  }
  return acc;
}
__device__ __forceinline__ float frag_dot(const Frag<float>& a, const Frag<float>& b) {
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) acc = fmaf(a.lo[j], b.lo[j], fmaf(a.hi[j], b.hi[j], acc));
  return acc;
}

// ---------------------------------------------------------------------------
// 4-element vectors for stores and the transposing stage
// ---------------------------------------------------------------------------
template <typename T>
struct Vec4;
template <>
struct Vec4<bf16_t> {
  u32x2 v;
};
template <>
struct Vec4<float> {
  f32x4 v;
};

// ---------------------------------------------------------------------------
// Buffer loads. A raw (stride 0) buffer resource spans `bytes` bytes from `base`;
// a load at an offset at or past that returns zeros. Built per tile over its valid
// rows, it zero-fills the rows past the end of the sequence without a branch, and
// the per-lane offsets stay loop-invariant 32-bit registers (no 64-bit address
// arithmetic per load). Word 3 selects 32-bit data format, as gfx9 raw buffers use.
constexpr int kBufWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), short(0), bytes, kBufWord3);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

// Make the wait-count pass wait here for the loads that produced a value. A loop
// keeps its operand fragments in registers; without this the pass, which merges all
// paths into the loop header, leaves their loads pending there and makes the loop's
// first MFMA wait for the tile prefetch issued just before it as well. The empty asm
// passes the value through; it is not volatile and touches no memory, so uniform
// loads in the loop still go through the scalar unit.
__device__ __forceinline__ void mark_ready(u32x4& v) { asm("" : "+v"(v)); }
__device__ __forceinline__ void mark_ready(f32x4& v) { asm("" : "+v"(v)); }
__device__ __forceinline__ void mark_ready(float& v) { asm("" : "+v"(v)); }
__device__ __forceinline__ void mark_ready(int32_t& v) { asm("" : "+v"(v)); }
__device__ __forceinline__ void mark_ready(Frag<bf16_t>& f) { mark_ready(f.v); }
__device__ __forceinline__ void mark_ready(Frag<fp8_t>& f) { asm("" : "+v"(f.v)); }
__device__ __forceinline__ void mark_ready(Frag<float>& f) {
  mark_ready(f.lo);
  mark_ready(f.hi);
}

__device__ __forceinline__ Vec4<bf16_t> vec4_load(const bf16_t* p) {
  Vec4<bf16_t> r;
  r.v = *reinterpret_cast<const u32x2*>(p);
  return r;
}
__device__ __forceinline__ Vec4<float> vec4_load(const float* p) {
  Vec4<float> r;
  r.v = *reinterpret_cast<const f32x4*>(p);
  return r;
}
__device__ __forceinline__ void vec4_bload(Vec4<bf16_t>& v, __amdgpu_buffer_rsrc_t r, int off) {
  v.v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ void vec4_bload(Vec4<float>& v, __amdgpu_buffer_rsrc_t r, int off) {
  v.v = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
template <typename T>
__device__ __forceinline__ Vec4<T> vec4_zero();
template <>
__device__ __forceinline__ Vec4<bf16_t> vec4_zero<bf16_t>() {
  Vec4<bf16_t> r;
  r.v = u32x2{0u, 0u};
  return r;
}
template <>
__device__ __forceinline__ Vec4<float> vec4_zero<float>() {
  Vec4<float> r;
  r.v = f32x4{0.f, 0.f, 0.f, 0.f};
  return r;
}
__device__ __forceinline__ void vec4_store(bf16_t* p, const Vec4<bf16_t>& x) {
  *reinterpret_cast<u32x2*>(p) = x.v;
}
__device__ __forceinline__ void vec4_store(float* p, const Vec4<float>& x) {
  *reinterpret_cast<f32x4*>(p) = x.v;
}
__device__ __forceinline__ Vec4<bf16_t> vec4_from(float a, float b, float c, float d,
                                                  bf16_t*) {
  Vec4<bf16_t> r;
  r.v = u32x2{pack_bf16x2(a, b), pack_bf16x2(c, d)};
  return r;
}
__device__ __forceinline__ Vec4<float> vec4_from(float a, float b, float c, float d, float*) {
  Vec4<float> r;
  r.v = f32x4{a, b, c, d};
  return r;
}

// 4x4 transpose: in r[k] = row k (4 columns); out c[j] = column j (4 rows).
__device__ __forceinline__ void transpose4(const Vec4<bf16_t>* r, Vec4<bf16_t>* c) {
  // element (k, j) is 16-bit half (j & 1) of word (j >> 1) of r[k]
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int w = j >> 1, sh = (j & 1) * 16;
    uint32_t e0 = (r[0].v[w] >> sh) & 0xffffu, e1 = (r[1].v[w] >> sh) & 0xffffu;
    uint32_t e2 = (r[2].v[w] >> sh) & 0xffffu, e3 = (r[3].v[w] >> sh) & 0xffffu;
    c[j].v = u32x2{e0 | (e1 << 16), e2 | (e3 << 16)};
  }
}
__device__ __forceinline__ void transpose4(const Vec4<float>* r, Vec4<float>* c) {
#pragma unroll
  for (int j = 0; j < 4; ++j) c[j].v = f32x4{r[0].v[j], r[1].v[j], r[2].v[j], r[3].v[j]};
}

__device__ __forceinline__ float to_f32(bf16_t x) {
  return __builtin_bit_cast(float, uint32_t(x.bits) << 16);
}
__device__ __forceinline__ float to_f32(float x) { return x; }

// ---------------------------------------------------------------------------
// Global -> LDS staging of one tile of `R` rows x `D` columns of a [T, heads, D]
// tensor (row stride `ld` elements); rows at or past `nvalid` are zero-filled.
// ---------------------------------------------------------------------------
// Row-major copy: dst[r * S + c].
template <typename T, int R, int D, int S, int NT>
__device__ __forceinline__ void stage_rows(T* dst, const T* src, int64_t ld, int nvalid) {
  constexpr int E = 16 / int(sizeof(T));  // elements per 16-byte chunk
  constexpr int CPR = D / E;              // chunks per row
  constexpr int CHUNKS = R * CPR;
  static_assert(CHUNKS % NT == 0, "tile must split evenly over the threads");
#pragma unroll
  for (int it = 0; it < CHUNKS / NT; ++it) {
    const int c = it * NT + int(threadIdx.x);
    const int r = c / CPR, cc = (c % CPR) * E;
    u32x4 val = u32x4{0u, 0u, 0u, 0u};
    if (r < nvalid) val = *reinterpret_cast<const u32x4*>(src + int64_t(r) * ld + cc);
    *reinterpret_cast<u32x4*>(dst + r * S + cc) = val;
  }
}

// Transposed, row-permuted copy: dst[c * S + perm_pos(r)].  Each thread moves 4x4
// blocks: 4 row loads (consecutive threads read consecutive columns of a row), an
// in-register transpose, 4 stores of 4 permuted-row values each.
template <typename T, int R, int D, int S, int NT>
__device__ __forceinline__ void stage_rows_t(T* dst, const T* src, int64_t ld, int nvalid) {
  constexpr int CG = D / 4;  // column groups
  constexpr int BLOCKS = (R / 4) * CG;
  static_assert(BLOCKS % NT == 0, "tile must split evenly over the threads");
#pragma unroll
  for (int it = 0; it < BLOCKS / NT; ++it) {
    const int b = it * NT + int(threadIdx.x);
    const int r0 = (b / CG) * 4, c0 = (b % CG) * 4;
    Vec4<T> rows[4], cols[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      rows[k] = (r0 + k < nvalid) ? vec4_load(src + int64_t(r0 + k) * ld + c0) : vec4_zero<T>();
    transpose4(rows, cols);
    const int pos = perm_pos(r0);
#pragma unroll
    for (int j = 0; j < 4; ++j) vec4_store(dst + (c0 + j) * S + pos, cols[j]);
  }
}

// ---------------------------------------------------------------------------
// Software-pipelined staging: load() issues the global reads of a tile into
// registers, store() writes them to LDS later, so the reads of tile i+1 are in
// flight while tile i is being computed.
// ---------------------------------------------------------------------------
// Row-major: dst[r * S + c], 16 bytes per lane per chunk, consecutive lanes read
// consecutive 16-byte pieces of a row.
template <typename T, int R, int D, int S, int NT>
struct RowStage {
  static constexpr int E = 16 / int(sizeof(T));
  static constexpr int CPR = D / E;
  static constexpr int N = R * CPR / NT;
  static_assert((R * CPR) % NT == 0, "tile must split evenly over the threads");
  u32x4 r[N];
  // rows >= nvalid read as zeros; nvalid * ld * sizeof(T) must fit in an int
  __device__ __forceinline__ void load(const T* src, int64_t ld, int nvalid) {
    const int pitch = int(ld) * int(sizeof(T));
    const auto rs = buf_rsrc(src, nvalid * pitch);
#pragma unroll
    for (int it = 0; it < N; ++it) {
      const int c = it * NT + int(threadIdx.x);
      const int row = c / CPR, cc = (c % CPR) * E;
      r[it] = buf_load16(rs, row * pitch + cc * int(sizeof(T)));
    }
  }
  __device__ __forceinline__ void store(T* dst) const {
#pragma unroll
    for (int it = 0; it < N; ++it) {
      const int c = it * NT + int(threadIdx.x);
      const int row = c / CPR, cc = (c % CPR) * E;
      *reinterpret_cast<u32x4*>(dst + row * S + cc) = r[it];
    }
  }
};

// ---------------------------------------------------------------------------
// Swizzled bf16 tiles filled by direct-to-LDS buffer loads.
//
// A tile of R rows x D bf16 is stored row-major without padding; the 16-byte chunk c
// of row r sits at chunk slot c ^ swz(r).  The swizzle spreads the rows that one
// LDS pass serves over distinct bank groups, both for fragment reads along a row
// (ds_read_b128: 16 consecutive rows, one chunk each) and for transposed reads
// (ds_read_b64_tr_b16: 4 consecutive rows, 4 consecutive chunks each), which row
// padding would otherwise do.
// The tile is written by buffer_load_dwordx4 ... lds: each lane of a wave fetches
// 16 bytes from global memory and the hardware stores lane i at LDS base + 16 i, so
// lane i is given the global chunk whose swizzled slot is i.  Rows past `nvalid`
// are outside the buffer resource and come in as zeros.  The loads bypass the
// registers; the caller waits for them (vmcnt) before the barrier that publishes
// the tile.
// ---------------------------------------------------------------------------
// The chunk permutation of row r stays inside the row (values below NC).  Rows of 4
// chunks (64 bytes: e4m3 at d = 64) put 4 rows in one 256-byte bank sweep, so rows
// r and r + 4 differ by r >> 2 alone.
template <int NC>
__device__ __forceinline__ int swz(int r) {
  static_assert(NC == 4 || NC == 8 || NC == 16 || NC == 32, "chunks per row");
  if constexpr (NC == 4) return (r >> 2) & 3;
  return NC >= 16 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ lds_void* to_lds(void* p) { return (lds_void*)p; }

// Direct-to-LDS buffer loads, written as inline assembly: the compiler's wait-count
// pass does not model them, so it cannot add conservative vmcnt waits in front of
// unrelated LDS reads (it does so for the transposed reads, which carry no memory
// operand).  The caller waits for them with wait_vmcnt before the barrier that
// publishes the data; other vector loads only ever wait longer because of them.
// The descriptor and the LDS address are made wave-uniform explicitly (SGPR operands).
struct DmaRsrc {
  u32x4 d;
};
__device__ __forceinline__ DmaRsrc dma_rsrc(const void* base, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  DmaRsrc r;
  r.d = u32x4{uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(a))),
              uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(a >> 32) & 0xffffu)),
              uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(bytes))), uint32_t(kBufWord3)};
  return r;
}
// LDS byte address of a pointer into the work-group's shared memory, wave-uniform.
// Kernels take it once for their shared array and form stage addresses from it with
// scalar arithmetic: converting a generic pointer per load costs vector instructions
// (a 64-bit add, two readfirstlanes and a null check) on every load.
__device__ __forceinline__ uint32_t lds_addr_u(void* p) {
  return uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(reinterpret_cast<uintptr_t>(to_lds(p)))));
}
// 16 bytes per lane from byte offset voff of the buffer; lane i lands at LDS address
// lds + 16 i (lds wave-uniform).
__device__ __forceinline__ void dma_load16(const DmaRsrc& r, int voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(r.d), "s"(lds)
               : "memory");
}
// 4 bytes per lane; lane i lands at lds + 4 i.
__device__ __forceinline__ void dma_load4(const DmaRsrc& r, int voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(r.d), "s"(lds)
               : "memory");
}

template <int R, int D, int NT>
struct DmaTile {
  static constexpr int NC = D / 8;  // 16-byte chunks per row
  static constexpr int NW = NT / 64;
  static constexpr int N = R * NC / NT;  // wave loads per tile
  static constexpr int BYTES = R * D * 2;
  static_assert((R * NC) % NT == 0, "tile must split evenly over the waves");
  int voff[N];  // global byte offset (relative to the tile's first row) of each load
  __device__ __forceinline__ void init(int pitch_bytes) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int k = (j * NW + w) * 64 + lane;  // chunk slot this lane fills
      const int r = k / NC, c = (k % NC) ^ swz<NC>(r);
      voff[j] = r * pitch_bytes + c * 16;
    }
  }
  // Enqueue the loads of rows [0, nvalid) of the tile at `src` into LDS address `dst`.
  __device__ __forceinline__ void load(const void* src, int nvalid, int pitch_bytes,
                                       uint32_t dst) const {
    const DmaRsrc rs = dma_rsrc(src, nvalid * pitch_bytes);
    const int w = wave_id();
#pragma unroll
    for (int j = 0; j < N; ++j) dma_load16(rs, voff[j], dst + (j * NW + w) * 1024);
  }
};

// Byte offset of (row r, 16-byte chunk c) inside a swizzled tile with NC chunks a row.
template <int NC>
__device__ __forceinline__ int swz_off(int r, int c) {
  return r * NC * 16 + ((c ^ swz<NC>(r)) << 4);
}

// frag_load from a swizzled tile: 8 bf16 at row r, chunk c.
template <int NC>
__device__ __forceinline__ Frag<bf16_t> frag_load_swz(const char* tile, int r, int c) {
  Frag<bf16_t> f;
  f.v = *reinterpret_cast<const u32x4*>(tile + swz_off<NC>(r, c));
  return f;
}

// frag_load_tr (same lane mapping) from a swizzled tile; col0 is a multiple of 32.
template <int NC>
__device__ __forceinline__ Frag<bf16_t> frag_load_tr_swz(const char* tile, int row0, int col0) {
  const int lane = threadIdx.x & 63;
  const int s16 = lane & 15, g16 = lane >> 4, h = lane >> 5;
  const int row = row0 + 4 * h + (s16 >> 2);
  const int chunk = (col0 >> 3) + (g16 & 1) * 2 + ((s16 & 3) >> 1);
  const int byte = (s16 & 1) * 8;
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const lds_i16x4* p0 = (const lds_i16x4*)(tile + swz_off<NC>(row, chunk) + byte);
  const lds_i16x4* p1 = (const lds_i16x4*)(tile + swz_off<NC>(row + 8, chunk) + byte);
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<lds_i16x4*>(p0));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<lds_i16x4*>(p1));
  const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
  Frag<bf16_t> f;
  f.v = u32x4{ua[0], ua[1], ub[0], ub[1]};
  return f;
}

// s_waitcnt vmcnt(n), leaving the other counters alone (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Transposed + row-permuted (see stage_rows_t), for operands whose element type has
// no LDS transpose read (fp32).
template <typename T, int R, int D, int S, int NT>
struct TransStage {
  static constexpr int CG = D / 4;
  static constexpr int N = (R / 4) * CG / NT;
  static_assert(((R / 4) * CG) % NT == 0, "tile must split evenly over the threads");
  Vec4<T> rows[N][4];
  // rows >= nvalid read as zeros; nvalid * ld * sizeof(T) must fit in an int
  __device__ __forceinline__ void load(const T* src, int64_t ld, int nvalid) {
    const int pitch = int(ld) * int(sizeof(T));
    const auto rs = buf_rsrc(src, nvalid * pitch);
#pragma unroll
    for (int it = 0; it < N; ++it) {
      const int b = it * NT + int(threadIdx.x);
      const int r0 = (b / CG) * 4, c0 = (b % CG) * 4;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        vec4_bload(rows[it][k], rs, (r0 + k) * pitch + c0 * int(sizeof(T)));
    }
  }
  __device__ __forceinline__ void store(T* dst) const {
#pragma unroll
    for (int it = 0; it < N; ++it) {
      const int b = it * NT + int(threadIdx.x);
      const int r0 = (b / CG) * 4, c0 = (b % CG) * 4;
      Vec4<T> cols[4];
      transpose4(rows[it], cols);
      const int pos = perm_pos(r0);
#pragma unroll
      for (int j = 0; j < 4; ++j) vec4_store(dst + (c0 + j) * S + pos, cols[j]);
    }
  }
};

// A-operand fragment of a product whose reduction index runs over the ROWS of a
// row-major bf16 LDS tile (row stride S elements): lane l gets column
// col0 + (l % 32) and the 8 rows row0 + {4h .. 4h+3, 8+4h .. 8+4h+3}, h = l / 32,
// which is the row order of the accumulator-derived B operand.  Two
// ds_read_b64_tr_b16: within each 16-lane group, lane s addresses row (s / 4) and
// columns 4 (s % 4) .. +3 of a 4-row x 16-column block, and the hardware hands lane
// i the 4 rows of column i.
__device__ __forceinline__ Frag<bf16_t> frag_load_tr(const bf16_t* tile, int S, int row0,
                                                     int col0) {
  const int lane = threadIdx.x & 63;
  const int s16 = lane & 15, g16 = lane >> 4, h = lane >> 5;
  const int row = row0 + 4 * h + (s16 >> 2);
  const int col = col0 + (g16 & 1) * 16 + (s16 & 3) * 4;
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const lds_i16x4* p0 = (const lds_i16x4*)(tile + row * S + col);
  const lds_i16x4* p1 = (const lds_i16x4*)(tile + (row + 8) * S + col);
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<lds_i16x4*>(p0));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<lds_i16x4*>(p1));
  const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
  Frag<bf16_t> f;
  f.v = u32x4{ua[0], ua[1], ub[0], ub[1]};
  return f;
}

// blockIdx -> work item so that runs of `chunk` consecutive items land on one XCD
// (work-groups are dealt to the 8 XCDs round-robin).  `grid` is a multiple of 8*chunk.
__device__ __forceinline__ int64_t xcd_remap(int64_t bid, int64_t chunk) {
  const int64_t xcd = bid & 7, slot = bid >> 3;
  return ((slot / chunk) * 8 + xcd) * chunk + slot % chunk;
}

}  // namespace psa
