// Shared device helpers for the gfx950 kernels of the hybrid GDN + sink/SWA
// layer: bf16 conversion, MFMA operand fragments and wave reductions.
//
// MFMA used everywhere: v_mfma_f32_16x16x32_bf16 (CDNA4).  For one 16x16
// output tile D = A(16x32) * B(32x16) + C, lane l (0..63), g = l / 16:
//   A fragment: A[l % 16][kset(g)]   (8 bf16)
//   B fragment: B[kset(g)][l % 16]   (8 bf16)
//   C/D:        D[4g + i][l % 16], i = 0..3 (4 fp32)
// The reduction index set kset(g) only has to be the same for A and B, so a
// kernel may choose it per product.  Two choices are used:
//   "linear":  kset(g) = {8g .. 8g+7}
//   "acc":     kset(g) = {4g .. 4g+3} U {16+4g .. 16+4g+3}
// The "acc" set is what a lane holds when two vertically stacked output tiles
// are read as one operand, so an fp32 accumulator X can feed the next MFMA
// without leaving registers, either as the B operand of (.)X or as the A
// operand of X^T(.).
//
// LDS tiles store their reduction dimension in "acc order": inside each
// 32-wide block, logical index c = 16h + 4g + i sits at position 8g + 4h + i.
// The "acc" set of lane group g is then the 8 contiguous positions 8g..8g+7,
// so every operand read from LDS is one 16-byte access, and any product
// whose two LDS operands share that order reduces over the same indices.
//
// fp32 inputs use a split-bf16 product: x = hi + lo with hi = bf16(x),
// lo = bf16(x - hi), and a*b ~ hi*hi + hi*lo + lo*hi (relative error about
// 2^-16), keeping one code path and one operand layout for both precisions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// logical index -> position in acc order, and back
__host__ __device__ __forceinline__ constexpr int acc_pos(int c) {
  return (c & ~31) | ((c & 12) << 1) | ((c & 16) >> 2) | (c & 3);
}
__host__ __device__ __forceinline__ constexpr int acc_idx(int p) {
  return (p & ~31) | ((p & 4) << 2) | ((p & 24) >> 1) | (p & 3);
}
static_assert(acc_pos(0) == 0 && acc_pos(4) == 8 && acc_pos(16) == 4 && acc_pos(20) == 12 &&
              acc_pos(31) == 31 && acc_pos(45) == 57, "acc order");
static_assert(acc_idx(acc_pos(7)) == 7 && acc_idx(acc_pos(29)) == 29 && acc_idx(acc_pos(63)) == 63,
              "acc order inverse");

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return static_cast<float>(x); }

template <class T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return static_cast<bf16>(x); }

// ---------------------------------------------------------------- fragments

template <class Tl> struct Frag;
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<float> { bf16x8 hi, lo; };

__device__ __forceinline__ f32x4 mfma(const Frag<bf16>& a, const Frag<bf16>& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma(const Frag<float>& a, const Frag<float>& b, f32x4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.hi, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.lo, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, c, 0, 0, 0);
  return c;
}

template <class Tl> __device__ __forceinline__ Frag<Tl> frag_from8(const float (&x)[8]);
template <> __device__ __forceinline__ Frag<bf16> frag_from8<bf16>(const float (&x)[8]) {
  Frag<bf16> f;
#pragma unroll
  for (int i = 0; i < 8; ++i) f.v[i] = static_cast<bf16>(x[i]);
  return f;
}
template <> __device__ __forceinline__ Frag<float> frag_from8<float>(const float (&x)[8]) {
  Frag<float> f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    bf16 h = static_cast<bf16>(x[i]);
    f.hi[i] = h;
    f.lo[i] = static_cast<bf16>(x[i] - static_cast<float>(h));
  }
  return f;
}

// Operand from two stacked accumulator tiles (the "acc" reduction set),
// each value multiplied by s0 (first tile) / s1 (second tile) per slot.
template <class Tl>
__device__ __forceinline__ Frag<Tl> frag_from_acc(const f32x4& a, const f32x4& b) {
  float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return frag_from8<Tl>(x);
}
template <class Tl>
__device__ __forceinline__ Frag<Tl> frag_from_acc_scaled(const f32x4& a, const f32x4& b,
                                                         const f32x4& sa, const f32x4& sb) {
  float x[8] = {a[0] * sa[0], a[1] * sa[1], a[2] * sa[2], a[3] * sa[3],
                b[0] * sb[0], b[1] * sb[1], b[2] * sb[2], b[3] * sb[3]};
  return frag_from8<Tl>(x);
}

// 8 contiguous LDS elements ("linear" set); p must be 16-byte aligned.
__device__ __forceinline__ Frag<bf16> lds_frag8(const bf16* p) {
  Frag<bf16> f;
  f.v = *reinterpret_cast<const bf16x8*>(p);
  return f;
}
__device__ __forceinline__ Frag<float> lds_frag8(const float* p) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return frag_from8<float>(x);
}
// 4 + 4 LDS elements (the "acc" set): p0[0..3] and p1[0..3].
__device__ __forceinline__ Frag<bf16> lds_frag44(const bf16* p0, const bf16* p1) {
  bf16x4 a = *reinterpret_cast<const bf16x4*>(p0);
  bf16x4 b = *reinterpret_cast<const bf16x4*>(p1);
  Frag<bf16> f;
  f.v = bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return f;
}
__device__ __forceinline__ Frag<float> lds_frag44(const float* p0, const float* p1) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p0);
  f32x4 b = *reinterpret_cast<const f32x4*>(p1);
  float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return frag_from8<float>(x);
}

// 8 contiguous LDS elements, each multiplied by s[0..7] (fp32, 16-byte
// aligned) before the fragment is formed.
__device__ __forceinline__ Frag<bf16> lds_frag8_scaled(const bf16* p, const float* s) {
  const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
  const f32x4 s0 = *reinterpret_cast<const f32x4*>(s);
  const f32x4 s1 = *reinterpret_cast<const f32x4*>(s + 4);
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = static_cast<float>(v[i]) * s0[i];
    x[4 + i] = static_cast<float>(v[4 + i]) * s1[i];
  }
  return frag_from8<bf16>(x);
}
__device__ __forceinline__ Frag<float> lds_frag8_scaled(const float* p, const float* s) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  const f32x4 s0 = *reinterpret_cast<const f32x4*>(s);
  const f32x4 s1 = *reinterpret_cast<const f32x4*>(s + 4);
  float x[8] = {a[0] * s0[0], a[1] * s0[1], a[2] * s0[2], a[3] * s0[3],
                b[0] * s1[0], b[1] * s1[1], b[2] * s1[2], b[3] * s1[3]};
  return frag_from8<float>(x);
}
// 8 contiguous LDS elements; elements 0..3 multiplied by s0[0..3] and 4..7
// by s1[0..3] (fp32, 16-byte aligned) before the fragment is formed.
__device__ __forceinline__ Frag<bf16> lds_frag8_scaled(const bf16* p, const float* s0p, const float* s1p) {
  const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
  const f32x4 s0 = *reinterpret_cast<const f32x4*>(s0p);
  const f32x4 s1 = *reinterpret_cast<const f32x4*>(s1p);
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = static_cast<float>(v[i]) * s0[i];
    x[4 + i] = static_cast<float>(v[4 + i]) * s1[i];
  }
  return frag_from8<bf16>(x);
}
__device__ __forceinline__ Frag<float> lds_frag8_scaled(const float* p, const float* s0p, const float* s1p) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  const f32x4 s0 = *reinterpret_cast<const f32x4*>(s0p);
  const f32x4 s1 = *reinterpret_cast<const f32x4*>(s1p);
  float x[8] = {a[0] * s0[0], a[1] * s0[1], a[2] * s0[2], a[3] * s0[3],
                b[0] * s1[0], b[1] * s1[1], b[2] * s1[2], b[3] * s1[3]};
  return frag_from8<float>(x);
}

// 8 contiguous global elements converted to a fragment (q rows etc.).
__device__ __forceinline__ Frag<bf16> gbl_frag8(const bf16* p) {
  Frag<bf16> f;
  f.v = *reinterpret_cast<const bf16x8*>(p);
  return f;
}
__device__ __forceinline__ Frag<float> gbl_frag8(const float* p) { return lds_frag8(p); }

template <class Tl> __device__ __forceinline__ Frag<Tl> zero_frag();
template <> __device__ __forceinline__ Frag<bf16> zero_frag<bf16>() {
  Frag<bf16> f;
#pragma unroll
  for (int i = 0; i < 8; ++i) f.v[i] = static_cast<bf16>(0.0f);
  return f;
}
template <> __device__ __forceinline__ Frag<float> zero_frag<float>() {
  Frag<float> f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    f.hi[i] = static_cast<bf16>(0.0f);
    f.lo[i] = static_cast<bf16>(0.0f);
  }
  return f;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ------------------------------------------------------- global vector I/O
// 16-byte chunks of a row of element type T (8 bf16 or 4 fp32).

template <class T> struct Vec16;
template <> struct Vec16<bf16> { typedef bf16x8 type; static constexpr int n = 8; };
template <> struct Vec16<float> { typedef f32x4 type; static constexpr int n = 4; };

// Store 4 consecutive values (from an fp32 accumulator) as T.
__device__ __forceinline__ void store4(float* p, const f32x4& x) { *reinterpret_cast<f32x4*>(p) = x; }
__device__ __forceinline__ void store4(bf16* p, const f32x4& x) {
  *reinterpret_cast<bf16x4*>(p) = bf16x4{static_cast<bf16>(x[0]), static_cast<bf16>(x[1]),
                                         static_cast<bf16>(x[2]), static_cast<bf16>(x[3])};
}
__device__ __forceinline__ f32x4 load4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f32x4 load4(const bf16* p) {
  bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  return f32x4{static_cast<float>(v[0]), static_cast<float>(v[1]), static_cast<float>(v[2]),
               static_cast<float>(v[3])};
}

// Transposed staging: w[j] holds one dword (EPD = 4 / sizeof(T) elements) of
// row j of a row-major tile, for N consecutive rows.  Store element e of
// every dword contiguously at dst (one column of the transposed tile), as
// whole 8- or 16-byte writes.
template <class T, int N>
__device__ __forceinline__ void store_column(T* dst, const uint32_t (&w)[N], int e) {
  if constexpr (sizeof(T) == 2) {
    uint32_t packed[N / 2];
#pragma unroll
    for (int m = 0; m < N / 2; ++m) {
      const uint32_t lo = (w[2 * m] >> (16 * e)) & 0xFFFFu;
      const uint32_t hi = (w[2 * m + 1] >> (16 * e)) & 0xFFFFu;
      packed[m] = lo | (hi << 16);
    }
    if constexpr (N % 8 == 0) {
#pragma unroll
      for (int m = 0; m < N / 8; ++m)
        *reinterpret_cast<uint4*>(dst + 8 * m) =
            uint4{packed[4 * m], packed[4 * m + 1], packed[4 * m + 2], packed[4 * m + 3]};
    } else {
      static_assert(N == 4, "column length");
      *reinterpret_cast<uint2*>(dst) = uint2{packed[0], packed[1]};
    }
  } else {
    static_assert(N % 4 == 0, "column length");
#pragma unroll
    for (int m = 0; m < N / 4; ++m)
      *reinterpret_cast<uint4*>(dst + 4 * m) = uint4{w[4 * m], w[4 * m + 1], w[4 * m + 2], w[4 * m + 3]};
  }
}

// Same, for a tile whose reduction dimension is kept in acc order: the N
// logical rows key0 .. key0+N-1 (key0 a multiple of 4) are written as runs
// of 4, each contiguous at position acc_pos(key0 + 4m) of the column.
template <class T, int N>
__device__ __forceinline__ void store_column_acc(T* col, int key0, const uint32_t (&w)[N], int e) {
  static_assert(N % 4 == 0, "column length");
#pragma unroll
  for (int m = 0; m < N / 4; ++m) {
    T* dst = col + acc_pos(key0 + 4 * m);
    if constexpr (sizeof(T) == 2) {
      uint32_t p0 = ((w[4 * m] >> (16 * e)) & 0xFFFFu) | (((w[4 * m + 1] >> (16 * e)) & 0xFFFFu) << 16);
      uint32_t p1 = ((w[4 * m + 2] >> (16 * e)) & 0xFFFFu) | (((w[4 * m + 3] >> (16 * e)) & 0xFFFFu) << 16);
      *reinterpret_cast<uint2*>(dst) = uint2{p0, p1};
    } else {
      *reinterpret_cast<uint4*>(dst) = uint4{w[4 * m], w[4 * m + 1], w[4 * m + 2], w[4 * m + 3]};
    }
  }
}

// ------------------------------------------------------------ barriers

// Workgroup barrier for LDS hazards only.  __syncthreads() also fences global
// memory, which on gfx9 waits for every outstanding global load (vmcnt(0))
// and so turns register prefetches of the next tile into stalls.  Here each
// wave waits for its own LDS operations (lgkmcnt(0); encoding keeps vmcnt
// and expcnt at their maxima) and then meets the others at s_barrier; the
// empty asm statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ------------------------------------------------------ workgroup mapping

// Workgroup ids are handed to the 8 XCDs round-robin, so ids id, id + 8,
// id + 16, ... run on one XCD and share its L2.  For launches over `units`
// work units of G members each that read common data (the query heads of one
// KV head), this maps a 1-D id so that the G members of a unit are
// consecutive on one XCD.  Launch 8 * G * ceil(units / 8) workgroups; ids
// that map past the last unit return false.
__device__ __forceinline__ bool xcd_grouped(int id, int G, int units, int& unit, int& member) {
  const int x = id & 7;
  const int s = id >> 3;
  member = s % G;
  unit = (s / G) * 8 + x;
  return unit < units;
}
__host__ __forceinline__ unsigned xcd_grouped_grid(long long units, int G) {
  return (unsigned)(8LL * G * ((units + 7) / 8));
}

// ------------------------------------------------------------ wave helpers

// Wave index inside the workgroup as a scalar (wave-uniform) value, so that
// branches and loops on it compile to scalar control flow.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

__device__ __forceinline__ float shfl_xor(float x, int m) { return __shfl_xor(x, m, 64); }

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += shfl_xor(x, m);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, shfl_xor(x, m));
  return x;
}

}  // namespace gdn
