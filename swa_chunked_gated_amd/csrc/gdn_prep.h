// Chunk preparation of the chunked gated delta rule: the per-chunk work that
// does not depend on the recurrent state, as a device function that one wave
// runs for one (chunk, head, sequence).  Used by the preparation kernel
// (gdn_prep.hip) and by the fused preparation + scan kernel
// (gdn_scan_full.hip).
//
// Method (page "The Key to Going Linear: Analysis-Driven Transformer
// Linearization", section 线性注意力替换机制): GDN update
// S_i = a_i (I - b_i k_i k_i^T) S_{i-1} + b_i k_i v_i^T.  Unrolled over a chunk
// of stream tokens with g = inclusive cumsum of log2 a inside the chunk and
// gamma = 2^g, the chunk is exact with
//   L_rs = b_r (gamma_r / gamma_s) k_r.k_s  (s < r),   Tm = (I + L)^-1,
//   U = Tm diag(b) V - Tm diag(b gamma) K S0,  ...
// so Tm diag(b) and Tm diag(b gamma) (and g, gamma) are all the scan needs
// from here.
//
// K K^T on MFMA; the unit lower-triangular inverse as 16x16 diagonal blocks
// by forward substitution in fp32 plus the off-diagonal blocks by block
// recursion on fp32 MFMA (16x16x4, exact fp32 products).  Outputs per chunk
// (workspace, element type T): TB = Tm diag(b) and TBG = Tm diag(b gamma) as
// 64 rows of 64, each row's columns stored in acc order (the order the scan's
// LDS tiles use), and fp32 g[64], gamma[64]; the full preparation writes
// -Wm, the decayed K^T and the decayed causal scores A instead of TBG.

#pragma once

#include "common.h"

namespace gdn {
namespace prep {

constexpr int kC = 64;          // chunk length
constexpr int kSL = 68;         // fp32 stride of the 64x64 solve buffer

// Layouts of the fp32 solve buffer, by 16-row block rows R = 0..3.  Square:
// the whole 64 x 64 matrix, row stride kSL.  Packed: only the blocks on and
// below the diagonal, block row R holding 16 (R + 1) columns at row stride
// 16 (R + 1) + 4 (each stride spreads a 16-lane column read over distinct
// banks): 11 KiB instead of 17, so that more preparation waves fit a
// compute unit.
struct SquareL {
  static constexpr int size = kC * kSL;
  __host__ __device__ static constexpr int stride(int) { return kSL; }
  __host__ __device__ static constexpr int row0(int R) { return 16 * R * kSL; }
};
struct PackedL {
  static constexpr int size = 16 * (20 + 36 + 52 + 68);
  __host__ __device__ static constexpr int stride(int R) { return 16 * (R + 1) + 4; }
  __host__ __device__ static constexpr int row0(int R) {
    return R == 0 ? 0 : R == 1 ? 16 * 20 : R == 2 ? 16 * (20 + 36) : 16 * (20 + 36 + 52);
  }
};
// block (R, C) of the solve buffer; element (r, s) of the matrix
template <class LL>
__device__ __forceinline__ float* lblk(float* Lf, int R, int C) { return Lf + LL::row0(R) + 16 * C; }
template <class LL>
__device__ __forceinline__ int lidx(int r, int s) { return LL::row0(r >> 4) + (r & 15) * LL::stride(r >> 4) + s; }

// Orders this wave's LDS accesses: every earlier LDS operation has completed
// before any later one is issued (no workgroup barrier).
__device__ __forceinline__ void wave_lds_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  asm volatile("" ::: "memory");
}

// Global stores of the preparation's results, at element offset `off` from
// a wave-uniform base.  DEV: device-scope stores (cache policy sc1, through
// a buffer resource on the base: written through to memory and visible to
// every compute unit once complete), so that a consumer in the same kernel
// can read the tiles coherently; else plain stores.
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kCpolSc1 = 16;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dev_rsrc(void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7fffffff, 0x00020000);
}
template <bool DEV, class T, class V>
__device__ __forceinline__ void put16(T* base, int off, const V& x) {      // one 16-byte piece
  static_assert(sizeof(V) == 16, "16 bytes");
  if constexpr (DEV) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), dev_rsrc(base),
                                           off * (int)sizeof(T), 0, kCpolSc1);
  } else {
    *reinterpret_cast<V*>(base + off) = x;
  }
}
template <bool DEV, class T>
__device__ __forceinline__ void put4v(T* base, int off, const f32x4& x) {  // 4 values as T
  if constexpr (DEV) {
    static_assert(sizeof(T) == 2, "device-scope stores for bf16 tiles only");
    const bf16x4 y = bf16x4{static_cast<bf16>(x[0]), static_cast<bf16>(x[1]), static_cast<bf16>(x[2]),
                            static_cast<bf16>(x[3])};
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, y), dev_rsrc(base), off * 2, 0, kCpolSc1);
  } else {
    store4(base + off, x);
  }
}
// Eight values as T (x then y), stored nontemporally: the light
// preparation's tiles stream out and are read back by the next launch, long
// after L2 would have dropped them, so they should not take L2 lines from
// the K rows that the other query heads of the chunk are about to read.
template <class T>
__device__ __forceinline__ void put8nt(T* base, int off, const f32x4& x, const f32x4& y) {
  if constexpr (sizeof(T) == 2) {
    const bf16x8 v = bf16x8{static_cast<bf16>(x[0]), static_cast<bf16>(x[1]), static_cast<bf16>(x[2]),
                            static_cast<bf16>(x[3]), static_cast<bf16>(y[0]), static_cast<bf16>(y[1]),
                            static_cast<bf16>(y[2]), static_cast<bf16>(y[3])};
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4*>(base + off));
  } else {
    __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(base + off));
    __builtin_nontemporal_store(y, reinterpret_cast<f32x4*>(base + off + 4));
  }
}
template <bool DEV>
__device__ __forceinline__ void put1f(float* base, int off, float x) {
  if constexpr (DEV) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, x), dev_rsrc(base), off * 4, 0,
                                          kCpolSc1);
  } else {
    base[off] = x;
  }
}

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// C += A(16x16) B(16x16), both fp32 row-major in LDS (row strides SA, SB).
template <int SA, int SB>
__device__ __forceinline__ f32x4 mm16(const float* A, const float* B, f32x4 c, int l16, int lg) {
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) c = mfma4(A[l16 * SA + 4 * kk + lg], B[(4 * kk + lg) * SB + l16], c);
  return c;
}
// C += A(16x16, LDS, row stride SA) Y(16x16, accumulator registers of this wave).
template <int SA>
__device__ __forceinline__ f32x4 mm16_acc(const float* A, const f32x4& Y, f32x4 c, int l16, int lg) {
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) c = mfma4(A[l16 * SA + 4 * lg + kk], Y[kk], c);
  return c;
}
template <int S>
__device__ __forceinline__ void st16(float* blk, const f32x4& x, int l16, int lg) {
#pragma unroll
  for (int i = 0; i < 4; ++i) blk[(4 * lg + i) * S + l16] = x[i];
}

// Inclusive prefix sum over the 64 lanes of a wave: DPP row shifts inside
// each row of 16 lanes, then the row totals (read as scalars) added on.
__device__ __forceinline__ float wave_prefix_sum(float x, int lane) {
  // row_shr:s (dpp control 0x110 + s); lanes with lane % 16 < s receive 0
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xF, 0xF, true));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 15));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 31));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 47));
  const int row = lane >> 4;
  float off = 0.f;
  if (row >= 1) off = r0;
  if (row >= 2) off = off + r1;
  if (row >= 3) off = off + r2;
  return x + off;
}

// (I + L)^-1 in place for the strictly lower 64 x 64 L in Lf (fp32, layout
// LL, unit diagonal implied, zero on and above the diagonal of the diagonal
// blocks), by one wave: 16x16 diagonal blocks by forward substitution (lane
// = block x column j; row r of the block's inverse column is e_j[r] -
// sum_{s<r} L[r][s] x[s], with L's rows read as 16-byte pieces), then the
// off-diagonal blocks by block recursion on fp32 MFMA (exact fp32 products).
// A wave's LDS operations complete in program order; wave_lds_fence marks
// the phases.
template <class LL>
__device__ __forceinline__ void unit_lower_inverse_wave(float* Lf, int lane) {
  const int l16 = lane & 15;
  const int lg = lane >> 4;
  constexpr int S0 = LL::stride(0), S1 = LL::stride(1), S2 = LL::stride(2), S3 = LL::stride(3);
  {
    const int blk = lane >> 4;
    const int j = l16;
    const int SB = LL::stride(blk);
    float* Lb = Lf + LL::row0(blk) + 16 * blk;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float lr[16];
#pragma unroll
      for (int q4 = 0; q4 < (r + 3) / 4; ++q4) {
        const f32x4 t = *reinterpret_cast<const f32x4*>(&Lb[r * SB + 4 * q4]);
#pragma unroll
        for (int e = 0; e < 4; ++e) lr[4 * q4 + e] = t[e];
      }
      float acc = r == j ? 1.f : 0.f;
#pragma unroll
      for (int s2 = 0; s2 < r; ++s2) acc -= lr[s2] * x[s2];
      x[r] = acc;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) Lb[r * SB + j] = x[r];
  }
  wave_lds_fence();
  // level 1: X10 = -X11 L10 X00, X32 = -X33 L32 X22
  {
    const f32x4 y0 = mm16<S1, S0>(lblk<LL>(Lf, 1, 0), lblk<LL>(Lf, 0, 0), zero4(), l16, lg);
    const f32x4 x10 = -mm16_acc<S1>(lblk<LL>(Lf, 1, 1), y0, zero4(), l16, lg);
    const f32x4 y1 = mm16<S3, S2>(lblk<LL>(Lf, 3, 2), lblk<LL>(Lf, 2, 2), zero4(), l16, lg);
    const f32x4 x32 = -mm16_acc<S3>(lblk<LL>(Lf, 3, 3), y1, zero4(), l16, lg);
    st16<S1>(lblk<LL>(Lf, 1, 0), x10, l16, lg);
    st16<S3>(lblk<LL>(Lf, 3, 2), x32, l16, lg);
  }
  wave_lds_fence();
  // level 2: bottom-left 32x32 block = -X_BR (L_BL X_TL); every product is
  // read before any of the four 16x16 blocks is overwritten.  Block (R, C),
  // R = 2, 3, C = 0, 1: first Y = sum_{K = C..1} L(R, K) X(K, C), then
  // -sum_{K = 2..R} X(R, K) Y(K, C).
  f32x4 y[4];
  y[0] = mm16<S2, S0>(lblk<LL>(Lf, 2, 0), lblk<LL>(Lf, 0, 0), zero4(), l16, lg);
  y[0] = mm16<S2, S1>(lblk<LL>(Lf, 2, 1), lblk<LL>(Lf, 1, 0), y[0], l16, lg);
  y[1] = mm16<S2, S1>(lblk<LL>(Lf, 2, 1), lblk<LL>(Lf, 1, 1), zero4(), l16, lg);
  y[2] = mm16<S3, S0>(lblk<LL>(Lf, 3, 0), lblk<LL>(Lf, 0, 0), zero4(), l16, lg);
  y[2] = mm16<S3, S1>(lblk<LL>(Lf, 3, 1), lblk<LL>(Lf, 1, 0), y[2], l16, lg);
  y[3] = mm16<S3, S1>(lblk<LL>(Lf, 3, 1), lblk<LL>(Lf, 1, 1), zero4(), l16, lg);
  wave_lds_fence();
  st16<S2>(lblk<LL>(Lf, 2, 0), y[0], l16, lg);
  st16<S2>(lblk<LL>(Lf, 2, 1), y[1], l16, lg);
  st16<S3>(lblk<LL>(Lf, 3, 0), y[2], l16, lg);
  st16<S3>(lblk<LL>(Lf, 3, 1), y[3], l16, lg);
  wave_lds_fence();
  y[0] = mm16<S2, S2>(lblk<LL>(Lf, 2, 2), lblk<LL>(Lf, 2, 0), zero4(), l16, lg);
  y[1] = mm16<S2, S2>(lblk<LL>(Lf, 2, 2), lblk<LL>(Lf, 2, 1), zero4(), l16, lg);
  y[2] = mm16<S3, S2>(lblk<LL>(Lf, 3, 2), lblk<LL>(Lf, 2, 0), zero4(), l16, lg);
  y[2] = mm16<S3, S3>(lblk<LL>(Lf, 3, 3), lblk<LL>(Lf, 3, 0), y[2], l16, lg);
  y[3] = mm16<S3, S2>(lblk<LL>(Lf, 3, 2), lblk<LL>(Lf, 2, 1), zero4(), l16, lg);
  y[3] = mm16<S3, S3>(lblk<LL>(Lf, 3, 3), lblk<LL>(Lf, 3, 1), y[3], l16, lg);
  wave_lds_fence();
  st16<S2>(lblk<LL>(Lf, 2, 0), -y[0], l16, lg);
  st16<S2>(lblk<LL>(Lf, 2, 1), -y[1], l16, lg);
  st16<S3>(lblk<LL>(Lf, 3, 0), -y[2], l16, lg);
  st16<S3>(lblk<LL>(Lf, 3, 1), -y[3], l16, lg);
  wave_lds_fence();
}

template <class T, int D, bool FULL>
struct PrepSmem {
  static constexpr int PAD = 16 / sizeof(T);
  static constexpr int SC = kC + PAD;       // [*][64] rows
  // full preparation: K^T (tokens in acc order); the scores A, whose area then
  // holds TB = Tm diag(b) once A is written out; TBG = Tm diag(b gamma) and
  // then the chunk's V rows reuse the solve buffer
  static constexpr int oKT = 0;
  static constexpr int oA = oKT + (FULL ? D * SC : 0);
  static constexpr int nT = oA + (FULL ? kC * SC : 0);
  static constexpr int SV = D + PAD;                        // V rows, in the solve buffer
  static_assert(!FULL || (kC * SV * (int)sizeof(T) <= 4 * kC * kSL && SC * (int)sizeof(T) <= 4 * kSL),
                "TBG rows and V rows fit the solve buffer");
  static constexpr int bytesT = (nT * (int)sizeof(T) + 15) / 16 * 16;
  using LL = typename std::conditional<FULL, SquareL, PackedL>::type;
  static constexpr int nL = LL::size;                       // solve buffer
  static constexpr int bytes = bytesT + 4 * (nL + 4 * kC);  // + g, gamma, b, K^T factors
};

// One (chunk c, query head h, sequence bi) by one wave, in the LDS at
// smem_raw (PrepSmem bytes, 16-byte aligned, private to the wave): every
// operand fragment of K K^T (and Q K^T) is loaded straight from global memory
// into registers, so the only LDS a chunk needs is the 64 x 64 fp32 solve
// buffer (plus, for the full preparation, K^T, TBG and A staging).  No
// workgroup barrier: the wave's own LDS operations complete in program order.
// TM (light preparation only): also write Tm itself, [64][64] in natural
// column order, to wtm (the backward pass needs Tm^T products).
// SH = 4 (light preparation only): the four waves of the workgroup take four
// query heads of one KV head and the same chunk, whose K K^T they share:
// smem_raw is then the workgroup's LDS, one PrepSmem slice per wave in wave
// order, wv this wave's index; each wave forms a quarter of the ten 16x16
// blocks of K K^T on and below the diagonal (loading only the K rows those
// blocks need) and writes them, scaled by each head's gates, into every
// wave's solve buffer, between two workgroup barriers.
template <class T, int D, bool FULL, bool DEV = false, bool TM = false, int SH = 1>
__device__ __forceinline__ void gdn_prep_chunk(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ a, const float* __restrict__ b, T* __restrict__ wtb,
    T* __restrict__ wwm, T* __restrict__ wktg, T* __restrict__ wa,
    float* __restrict__ wut, float* __restrict__ wg, int T_, int H, int Hkv, int n_sink, int window,
    int nch, int c, int h, int bi, unsigned char* smem_raw, T* __restrict__ wtm = nullptr,
    int wv = 0) {
  static_assert(!(TM && FULL), "Tm is written by the light preparation");
  static_assert(SH == 1 || (SH == 4 && !FULL), "shared K K^T: light preparation, four heads");
  using SM = PrepSmem<T, D, FULL>;
  unsigned char* const wg_raw = smem_raw;      // SH = 4: the workgroup's slices
  if constexpr (SH > 1) smem_raw += wv * SM::bytes;
  using LL = typename SM::LL;
  constexpr int EPC = 16 / (int)sizeof(T);     // elements per 16-byte piece
  constexpr int QV = 8 / EPC;                  // 16-byte pieces per fragment
  constexpr int KS = D / 32;                   // 32-wide k-steps over d
  constexpr int SC = SM::SC;
  typedef typename Vec16<T>::type V16;

  T* sT = reinterpret_cast<T*>(smem_raw);
  T* KTs = sT + SM::oKT;
  T* As = sT + SM::oA;
  T* TBs = As;                                 // after A is written out
  float* Lf = reinterpret_cast<float*>(smem_raw + SM::bytesT);
  T* TBGs = reinterpret_cast<T*>(Lf);          // row r written after Lf row r is read
  float* lgs = Lf + SM::nL;
  float* gam = lgs + kC;
  float* bet = gam + kC;
  float* fac = bet + kC;                       // 2^{g_C - g} in acc position order

  const int g = h / (H / Hkv);
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15;
  const int lg = lane >> 4;
  const int iend = T_ - window;                // stream tokens are [n_sink, iend)
  const int i0 = n_sink + c * kC;
  const size_t ci = ((size_t)bi * H + h) * nch + c;
  const T* kbase = k + ((size_t)(bi * T_ + i0) * Hkv + g) * D;
  const T* qbase = q + ((size_t)(bi * T_ + i0 + window) * H + h) * D;

  // ---- this chunk's gates first (a = 1, b = 0 past the stream end).  Every
  // load is unconditional (rows past the stream read its last row), so the
  // memory counters the compiler waits on stay exact and the gate math
  // waits for the gates only.
  const int tok = i0 + lane;
  const size_t tokc = (size_t)(bi * T_ + min(tok, iend - 1)) * H + h;
  const float ar = a[tokc];
  const float br0 = b[tokc];
  asm volatile("" ::: "memory");   // the gates' loads go out first

  // ---- operand pieces: lane holds rows 16 mt + l16, dims 32 p + 8 lg .. +7
  // (SH = 4: slot sl holds row block kblk(sl) of this wave's blocks; waves 0
  // and 1 form blocks (m, m), (m+1, m), (m+1, m+1) of m = 2 wv from row blocks
  // m, m+1, waves 2 and 3 blocks (wv, 0), (wv, 1) from row blocks 0, 1, wv)
  constexpr int NKB = SH > 1 ? 3 : 4;
  auto kblk = [&](int sl) { return SH == 1 ? sl : wv == 1 ? 2 + sl : sl < 2 ? sl : wv; };
  V16 kr[NKB][KS][QV];
  V16 qr[FULL ? 4 : 1][FULL ? KS : 1][QV];
  const bool whole = i0 + kC <= iend;          // uniform: no row past the stream
#pragma unroll
  for (int mt = 0; mt < NKB; ++mt) {
    if (SH > 1 && mt == 2 && wv < 2) break;
    const int r = min(16 * kblk(mt) + l16, iend - 1 - i0);
#pragma unroll
    for (int p = 0; p < KS; ++p)
#pragma unroll
      for (int u = 0; u < QV; ++u) {
        const int col = 32 * p + 8 * lg + u * EPC;
        kr[mt][p][u] = *reinterpret_cast<const V16*>(kbase + (size_t)r * Hkv * D + col);
        if constexpr (FULL) qr[mt][p][u] = *reinterpret_cast<const V16*>(qbase + (size_t)r * H * D + col);
      }
  }
  // Rows past the stream keep their duplicated values: with a = 1 and b = 0
  // there, they add nothing.  Their L rows are b_r (...) = 0, so their TB
  // (and TBG) rows and columns are zero, which zeroes their Wm and U rows and
  // the products of their K^T columns; their query rows are never stored.
  const float av = tok < iend ? ar : 1.f;
  const float bv = tok < iend ? br0 : 0.f;
  (void)whole;
  auto frag_of = [&](const V16 (&pc)[QV]) {
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = to_f32(pc[i / EPC][i % EPC]);
    return frag_from8<T>(x);
  };

  // ---- zero the solve buffer (and the score tile, whose strictly upper
  // 16x16 tiles stay zero); gates: g = inclusive cumsum of log2 a, gamma =
  // 2^g, b
  if constexpr (FULL) {
#pragma unroll
    for (int i = lane; i < SM::nL / 4; i += 64) reinterpret_cast<f32x4*>(Lf)[i] = zero4();
#pragma unroll
    for (int i = lane; i < kC * SC / EPC; i += 64) {
      V16 z;
#pragma unroll
      for (int e = 0; e < EPC; ++e) z[e] = from_f32<T>(0.f);
      reinterpret_cast<V16*>(As)[i] = z;
    }
  }
  {
    const float x = wave_prefix_sum(__builtin_amdgcn_logf(av), lane);
    lgs[lane] = x;
    gam[lane] = __builtin_amdgcn_exp2f(x);
    bet[lane] = bv;
  }
  wave_lds_fence();
  if (FULL) fac[lane] = __builtin_amdgcn_exp2f(fminf(lgs[kC - 1] - lgs[acc_idx(lane)], 0.f));

  // ---- L = strictly lower (b_r 2^{g_r - g_s} k_r.k_s); full: also
  // A = [s <= r] 2^{g_r - g_s} q_r.k_s
  if constexpr (SH > 1) {
    __syncthreads();                           // every head's gates are in LDS
    // block (mt, nt) of K K^T, scaled by the gates of each head of the
    // workgroup into that head's solve buffer
    auto emit = [&](int mt, int nt, const f32x4& acc) {
      const int r0 = 16 * mt + 4 * lg;
      const int s = 16 * nt + l16;
#pragma unroll
      for (int hh = 0; hh < SH; ++hh) {
        float* Lh = reinterpret_cast<float*>(wg_raw + hh * SM::bytes + SM::bytesT);
        const float* lh = Lh + SM::nL;         // that head's g, then gamma, then b
        const f32x4 lr = *reinterpret_cast<const f32x4*>(&lh[r0]);
        const f32x4 br = *reinterpret_cast<const f32x4*>(&lh[2 * kC + r0]);
        const float ls = lh[s];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = r0 + i;
          const float dec = __builtin_amdgcn_exp2f(fminf(lr[i] - ls, 0.f));
          Lh[lidx<LL>(r, s)] = s < r ? br[i] * dec * acc[i] : 0.f;
        }
      }
    };
    auto kkt = [&](int sm, int sn) {
      f32x4 acc = zero4();
#pragma unroll
      for (int p = 0; p < KS; ++p) acc = mfma(frag_of(kr[sm][p]), frag_of(kr[sn][p]), acc);
      return acc;
    };
    if (wv < 2) {
      const int m = 2 * wv;
      const f32x4 t00 = kkt(0, 0), t10 = kkt(1, 0), t11 = kkt(1, 1);
      emit(m, m, t00);
      emit(m + 1, m, t10);
      emit(m + 1, m + 1, t11);
    } else {
      const f32x4 t0 = kkt(2, 0), t1 = kkt(2, 1);
      emit(wv, 0, t0);
      emit(wv, 1, t1);
    }
    __syncthreads();                           // every block of this head's L is in LDS
  }
#pragma unroll
  for (int mt = 0; mt < (SH > 1 ? 0 : 4); ++mt) {
    const int r0 = 16 * mt + 4 * lg;
    const f32x4 lr = *reinterpret_cast<const f32x4*>(&lgs[r0]);
    const f32x4 br = *reinterpret_cast<const f32x4*>(&bet[r0]);
#pragma unroll
    for (int nt = 0; nt <= mt; ++nt) {
      const int s = 16 * nt + l16;
      const float ls = lgs[s];
      f32x4 acc = zero4(), accq = zero4();
#pragma unroll
      for (int p = 0; p < KS; ++p) {
        const Frag<T> kb = frag_of(kr[nt][p]);
        acc = mfma(frag_of(kr[mt][p]), kb, acc);
        if constexpr (FULL) accq = mfma(frag_of(qr[mt][p]), kb, accq);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = r0 + i;
        const float dec = __builtin_amdgcn_exp2f(fminf(lr[i] - ls, 0.f));
        Lf[lidx<LL>(r, s)] = s < r ? br[i] * dec * acc[i] : 0.f;
        if constexpr (FULL) As[r * SC + acc_pos(s)] = from_f32<T>(s <= r ? dec * accq[i] : 0.f);
      }
    }
  }
  if constexpr (FULL) {
    // K^T (tokens in acc order) from the row pieces
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int p = 0; p < KS; ++p)
#pragma unroll
        for (int i = 0; i < 8; ++i)
          KTs[(32 * p + 8 * lg + i) * SC + acc_pos(16 * mt + l16)] = kr[mt][p][i / EPC][i % EPC];
  }
  wave_lds_fence();
  if constexpr (FULL) {
    // ---- A [64][64] out now, so that its area can take TB
    T* aa = wa + ci * (kC * kC);
#pragma unroll
    for (int i = lane; i < kC * (kC / EPC); i += 64) {
      const int r = i / (kC / EPC);
      const int pc = (i % (kC / EPC)) * EPC;
      put16<DEV>(aa, r * kC + pc, *reinterpret_cast<const V16*>(&As[r * SC + pc]));
    }
  }
  unit_lower_inverse_wave<LL>(Lf, lane);

  // full preparation: the chunk's V rows (zero past the stream end), loaded
  // now and staged once the solve buffer is free
  constexpr int NPV = FULL ? kC * D / EPC / 64 : 1;
  V16 vr[NPV];
  if constexpr (FULL) {
#pragma unroll
    for (int n = 0; n < NPV; ++n) {
      const int j = lane + 64 * n;
      const int r = j / (D / EPC);
      if (whole || i0 + r < iend) {
        vr[n] = *reinterpret_cast<const V16*>(v + ((size_t)(bi * T_ + i0 + r) * Hkv + g) * D + (j % (D / EPC)) * EPC);
      } else {
#pragma unroll
        for (int e = 0; e < EPC; ++e) vr[n][e] = from_f32<T>(0.f);
      }
    }
  }

  // ---- TB = Tm diag(b) (and, for the full preparation, TBG = Tm diag(b
  // gamma)): row r, columns s0..s0+3 at positions acc_pos(s0)..+3 of the row;
  // the full preparation keeps both in LDS, the light one writes TB (the scan
  // scales it by gamma where it needs TBG)
  T* tb = wtb + ci * (kC * kC);
  if constexpr (FULL) {
#pragma unroll 4
    for (int i = lane; i < kC * kC / 4; i += 64) {
      const int r = i >> 4;
      const int s0 = (i & 15) * 4;
      const f32x4 tm = *reinterpret_cast<const f32x4*>(&Lf[lidx<LL>(r, s0)]);
      const f32x4 bb = *reinterpret_cast<const f32x4*>(&bet[s0]);
      const f32x4 gg = *reinterpret_cast<const f32x4*>(&gam[s0]);
      const f32x4 x = tm * bb;
      store4(&TBs[r * SC + acc_pos(s0)], x);
      store4(&TBGs[r * SC + acc_pos(s0)], x * gg);
    }
  } else {
    // lane: the 8 positions 8 q .. 8 q + 7 (q = lane % 8) of rows 8 it +
    // lane / 8 in acc order, which hold columns c0 .. c0 + 3 and c0 + 16 ..
    // c0 + 19 (c0 = 32 (q / 4) + 4 (q % 4)): one 16-byte store per row.
    // Every row's block row R = it / 2 is known at compile time, and the
    // reads (all issued before the stores) stay inside the packed buffer: a
    // column block above the diagonal reads some other row's values, which
    // the select zeroes.
    static_assert(!DEV, "the light preparation's tiles are read by later launches");
    const int q8 = lane & 7;
    const int c0 = 32 * (q8 >> 2) + 4 * (q8 & 3);
    const int r8 = lane >> 3;
    const f32x4 b0 = *reinterpret_cast<const f32x4*>(&bet[c0]);
    const f32x4 b1 = *reinterpret_cast<const f32x4*>(&bet[c0 + 16]);
    f32x4 t0[8], t1[8];
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const float* row = &Lf[LL::row0(it >> 1) + (8 * (it & 1) + r8) * LL::stride(it >> 1)];
      t0[it] = *reinterpret_cast<const f32x4*>(row + c0);
      t1[it] = *reinterpret_cast<const f32x4*>(row + c0 + 16);
    }
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int R = it >> 1;
      const int r = 8 * it + r8;
      const f32x4 x0 = (c0 >> 4) <= R ? t0[it] * b0 : zero4();
      const f32x4 x1 = ((c0 + 16) >> 4) <= R ? t1[it] * b1 : zero4();
      put8nt(tb, r * kC + 8 * q8, x0, x1);
      if constexpr (TM) {
        put4v<DEV>(wtm + ci * (kC * kC), r * kC + c0, (c0 >> 4) <= R ? t0[it] : zero4());
        put4v<DEV>(wtm + ci * (kC * kC), r * kC + c0 + 16, ((c0 + 16) >> 4) <= R ? t1[it] : zero4());
      }
    }
  }
  put1f<DEV>(wg + ci * (2 * kC), lane, lgs[lane]);
  put1f<DEV>(wg + ci * (2 * kC), kC + lane, gam[lane]);
  if constexpr (FULL) {
    wave_lds_fence();
    // ---- -Wm = -(TBG K): per 16-row dk tile, Wm^T = K^T TBG^T on MFMA,
    // written as [token][dk]
    T* wm = wwm + ci * (kC * D);
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt) {
      Frag<T> kf[2];
#pragma unroll
      for (int p = 0; p < 2; ++p) kf[p] = lds_frag8(&KTs[(16 * mt + l16) * SC + 32 * p + 8 * lg]);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        f32x4 acc = zero4();
#pragma unroll
        for (int p = 0; p < 2; ++p) acc = mfma(kf[p], lds_frag8(&TBGs[(16 * nt + l16) * SC + 32 * p + 8 * lg]), acc);
        put4v<DEV>(wm, (16 * nt + l16) * D + 16 * mt + 4 * lg, -acc);
      }
    }
    // ---- K^T 2^{g_C - g} [D][64] (row r holds d_k index acc_pos(r), the
    // state row order of the scan's accumulators), 16-byte pieces
    T* ktg = wktg + ci * (D * kC);
#pragma unroll 4
    for (int i = lane; i < D * (kC / EPC); i += 64) {
      const int r = i / (kC / EPC);
      const int pc = (i % (kC / EPC)) * EPC;
      const V16 x = *reinterpret_cast<const V16*>(&KTs[acc_pos(r) * SC + pc]);
      V16 y;
#pragma unroll
      for (int e = 0; e < EPC; ++e) y[e] = from_f32<T>(to_f32(x[e]) * fac[pc + e]);
      put16<DEV>(ktg, r * kC + pc, y);
    }
    // ---- Ut = TB V [64][D] in fp32, written transposed as [D][64] (the
    // scan reads each column's 4 consecutive tokens as one 16-byte piece):
    // V rows staged in the solve buffer (TBG is no longer needed), V operands gathered
    // column-wise (slot j of lane group lg is token 32 p + 16 (j / 4) + 4 lg + j % 4)
    T* Vs = reinterpret_cast<T*>(Lf);
#pragma unroll
    for (int n = 0; n < NPV; ++n) {
      const int j = lane + 64 * n;
      *reinterpret_cast<V16*>(&Vs[(j / (D / EPC)) * SM::SV + (j % (D / EPC)) * EPC]) = vr[n];
    }
    wave_lds_fence();
    Frag<T> tf[4][2];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int p = 0; p < 2; ++p) tf[rt][p] = lds_frag8(&TBs[(16 * rt + l16) * SC + 32 * p + 8 * lg]);
    float* ut = wut + ci * (D * kC);
#pragma unroll 2
    for (int ct = 0; ct < D / 16; ++ct) {
      Frag<T> vf[2];
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        float x[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
          x[jj] = to_f32(Vs[(32 * p + 16 * (jj / 4) + 4 * lg + jj % 4) * SM::SV + 16 * ct + l16]);
        vf[p] = frag_from8<T>(x);
      }
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        f32x4 acc = zero4();
#pragma unroll
        for (int p = 0; p < 2; ++p) acc = mfma(tf[rt][p], vf[p], acc);
        put16<DEV>(ut, (16 * ct + l16) * kC + 16 * rt + 4 * lg, acc);
      }
    }
  }
}

}  // namespace prep
}  // namespace gdn
