// Q/K/V structural preparation on gfx950: RoPE -> causal depthwise short
// convolution -> L2 normalisation, fused in one pass per tensor.
//
// Method (page "The Key to Going Linear: Analysis-Driven Transformer
// Linearization", section 实践建议 item 3): a kernel-size-8 short convolution
// on the Q/K/V projections, placed after RoPE and before the L2
// normalisation.  Conventions where the page is silent: causal, depthwise,
// zero history, no bias, no activation, tap w[c, ks-1] multiplies the current
// token; rotate-half RoPE with inv_freq_j = theta^(-2j/d) at position pos0 + t
// on q and k; L2 norm x / sqrt(sum x^2 + 1e-6) on q and k.
//
// Work split (prefill): one launch for q, k and v; a lane owns 16 bytes of
// channels of one head, a wave the heads of one 64-token tile, and the tile
// re-reads a 7-token causal halo (details at the prefill kernel below).  The
// rotation angle is set in fp64 at the tile start and then advanced one
// token at a time by a fixed complex rotation (error grows ~1e-7 per token).
//
// Decode (one new token per sequence) keeps a short history per sequence;
// see the decode section below.

#include <math.h>

#include "common.h"
#include "launch.h"

namespace gdn {
namespace {

// Sum over the N (32 or 64) lanes holding one head, in registers: within
// each row of 16 lanes by DPP (lane ^ 1, lane ^ 2, then the half-row and row
// mirrors, each step adding the other half of the group so far), then across
// rows with the row-swap permutes.  Every lane of the group ends with the sum.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int N>
__device__ __forceinline__ float head_sum(float x) {
  static_assert(N == 32 || N == 64, "a head spans half or all of the wave");
  x += dpp_f<0xB1>(x);    // quad_perm [1, 0, 3, 2]
  x += dpp_f<0x4E>(x);    // quad_perm [2, 3, 0, 1]
  x += dpp_f<0x141>(x);   // row_half_mirror
  x += dpp_f<0x140>(x);   // row_mirror
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  if constexpr (N == 64) {
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(b[0]) + __uint_as_float(b[1]);
  }
  return x;
}

constexpr int kMaxKs = 8;

// ----------------------------------------------------------------- prefill
//
// One launch for q, k and v.  A lane owns V = 4 consecutive channels of one
// head (one 8-byte load and store per token for bf16, 16 bytes for fp32), so
// LPH = D / 4 lanes hold a head and a wave covers HW = 64 / LPH heads: a
// token's loads are 512 contiguous bytes at d = 128 in bf16.  Four channels
// keep the 8-tap window and the taps at 64 VGPRs, so several waves share a
// SIMD and hide each other's loads.  Inside each row of 16 lanes, lanes 0-7
// hold channels of the head's first half and lanes 8-15 the matching
// channels of its second half, so the RoPE partner of channel c (c +- D/2) is
// always 8 lanes away in the same row and its raw input words come over by
// one DPP move; the rotation, the window over time and the per-head norm stay
// in registers.  A wave walks kTT tokens; the kWT
// waves of a workgroup take consecutive tiles of the same heads, and
// workgroups are laid out so that the spans of one head group follow each
// other on one XCD: the 7-token causal halo a tile re-reads was fetched into
// that XCD's L2 by the tile before it.
constexpr int kTT = 64;      // tokens per wave
constexpr int kWT = 4;       // waves (consecutive tiles) per workgroup
constexpr int kLB = 8;       // tokens whose loads are issued together

template <class T, int D>
struct ConvGeom {
  static constexpr int V = 4;                      // channels per lane
  static constexpr int LPH = D / V;                // lanes per head
  static constexpr int HW = 64 / LPH;              // heads per wave
  static constexpr int NWD = V * (int)sizeof(T) / 4;   // 32-bit words per lane and token
};

// The 32-bit word held by lane ^ 8: the RoPE partner (row_ror:8 inside each
// row of 16 lanes).
__device__ __forceinline__ uint32_t partner(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false);
}

// Sum over the N lanes of one head (every lane of the group gets the sum).
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 16 || N == 32, "a head spans 16 or 32 lanes");
  x += dpp_f<0xB1>(x);    // quad_perm [1, 0, 3, 2]
  x += dpp_f<0x4E>(x);    // quad_perm [2, 3, 0, 1]
  x += dpp_f<0x141>(x);   // row_half_mirror
  x += dpp_f<0x140>(x);   // row_mirror
  if constexpr (N == 32) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  }
  return x;
}

// A lane's token: NWD raw 32-bit words <-> V fp32 values.
template <class T> struct Raw;
// Loads and stores are nontemporal: apart from a tile's 7-token halo, each
// input and output byte is touched once.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
template <> struct Raw<bf16> {
  typedef uint2 type;
  __device__ static uint2 load(const uint2* p) {
    const unsigned long long v = __builtin_nontemporal_load(reinterpret_cast<const unsigned long long*>(p));
    return uint2{(uint32_t)v, (uint32_t)(v >> 32)};
  }
  __device__ static void store(uint2* p, const uint2& v) {
    __builtin_nontemporal_store((unsigned long long)v.x | ((unsigned long long)v.y << 32),
                                reinterpret_cast<unsigned long long*>(p));
  }
  __device__ static void words(const uint2& r, uint32_t (&w)[2]) { w[0] = r.x; w[1] = r.y; }
  __device__ static void unpack(const uint32_t (&w)[2], float (&f)[4]) {
    f[0] = __uint_as_float(w[0] << 16);
    f[1] = __uint_as_float(w[0] & 0xFFFF0000u);
    f[2] = __uint_as_float(w[1] << 16);
    f[3] = __uint_as_float(w[1] & 0xFFFF0000u);
  }
  __device__ static uint2 pack(const float (&f)[4]) {
    const bf16x4 b{static_cast<bf16>(f[0]), static_cast<bf16>(f[1]), static_cast<bf16>(f[2]),
                   static_cast<bf16>(f[3])};
    return *reinterpret_cast<const uint2*>(&b);
  }
};
template <> struct Raw<float> {
  typedef uint4 type;
  __device__ static uint4 load(const uint4* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return uint4{v[0], v[1], v[2], v[3]};
  }
  __device__ static void store(uint4* p, const uint4& v) {
    __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(p));
  }
  __device__ static void words(const uint4& r, uint32_t (&w)[4]) { w[0] = r.x; w[1] = r.y; w[2] = r.z; w[3] = r.w; }
  __device__ static void unpack(const uint32_t (&w)[4], float (&f)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
  }
  __device__ static uint4 pack(const float (&f)[4]) {
    return uint4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3])};
  }
};

// One tile: tokens [t0, min(t0 + kTT, T)) of the heads of head group hg.
template <class T, int D, bool ROPE, bool NORM>
__device__ __forceinline__ void conv_tile(const T* __restrict__ x, const float* __restrict__ w,
                                          T* __restrict__ y, int T_, int nh, int ks, float theta,
                                          int pos0, int bi, int hg, int t0) {
  using G = ConvGeom<T, D>;
  using R = Raw<T>;
  using RT = typename R::type;
  constexpr int V = G::V;
  constexpr int LPH = G::LPH;
  constexpr int NWD = G::NWD;
  constexpr int NH = kMaxKs - 1;    // most halo tokens
  const int lane = threadIdx.x & 63;
  const int h = hg * G::HW + lane / LPH;
  if (h >= nh || t0 >= T_) return;  // whole head groups leave together
  // first channel of the lane in its head: row r of 16 lanes, position p
  const int lh = lane % LPH;
  const int cb = ((lh >> 4) * 8 + (lh & 7)) * V + ((lh & 8) ? D / 2 : 0);
  const size_t ch = (size_t)h * D + cb;
  const int t1 = min(t0 + kTT, T_);
  const int ts = max(0, t0 - (ks - 1));   // first halo token
  const size_t row = (size_t)nh * D;
  const size_t rs = row / V;              // row stride in lane units
  const RT* xb = reinterpret_cast<const RT*>(x + (size_t)bi * T_ * row + ch);
  RT* yb = reinterpret_cast<RT*>(y + (size_t)bi * T_ * row + ch);

  // taps: wt[jj][e] multiplies channel cb + e of the input jj tokens back
  float wt[kMaxKs][V];
  if (ks == kMaxKs) {
    const f32x4* wp = reinterpret_cast<const f32x4*>(w + ch * kMaxKs);
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const f32x4 lo = wp[2 * e];
      const f32x4 hi = wp[2 * e + 1];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        wt[kMaxKs - 1 - i][e] = lo[i];
        wt[kMaxKs - 5 - i][e] = hi[i];
      }
    }
  } else {
#pragma unroll
    for (int jj = 0; jj < kMaxKs; ++jj)
#pragma unroll
      for (int e = 0; e < V; ++e) wt[jj][e] = jj < ks ? w[(ch + e) * ks + ks - 1 - jj] : 0.f;
  }
  float win[kMaxKs][V];
#pragma unroll
  for (int jj = 0; jj < kMaxKs; ++jj)
#pragma unroll
    for (int e = 0; e < V; ++e) win[jj][e] = 0.f;

  // RoPE: channel c < D/2 becomes x_c cos - x_{c+D/2} sin, channel c >= D/2
  // becomes x_c cos + x_{c-D/2} sin, at frequency j = c mod D/2; the sign sits
  // in sn and sf.  The angle at the first halo token comes from fp64 (reduced
  // to [-pi, pi] before the fp32 sincos) and then advances one token at a
  // time by the fixed rotation (cf, sf).
  float cs[V], sn[V], cf[V], sf[V];
  if constexpr (ROPE) {
    const int j0 = cb % (D / 2);
    const float sg = (lh & 8) ? 1.f : -1.f;
    const double lt = log((double)theta);
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const double f = exp(-(2.0 * (j0 + e) / D) * lt);
      const double ang = (double)(pos0 + ts) * f;
      const double twopi = 6.283185307179586476925;
      const float red = (float)(ang - twopi * rint(ang / twopi));
      float c0, s0, c1, s1;
      sincosf(red, &s0, &c0);
      sincosf((float)f, &s1, &c1);
      cs[e] = c0;
      sn[e] = sg * s0;
      cf[e] = c1;
      sf[e] = sg * s1;
    }
  }

  // one token into the window (RoPE at the running angle, then the shift)
  auto push = [&](const RT& raw) {
    uint32_t wd[NWD];
    R::words(raw, wd);
    float xv[V];
    R::unpack(wd, xv);
    if constexpr (ROPE) {
      uint32_t pw[NWD];
#pragma unroll
      for (int i = 0; i < NWD; ++i) pw[i] = partner(wd[i]);
      float pv[V];
      R::unpack(pw, pv);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        xv[e] = xv[e] * cs[e] + pv[e] * sn[e];
        const float cn = cs[e] * cf[e] - sn[e] * sf[e];
        sn[e] = sn[e] * cf[e] + cs[e] * sf[e];
        cs[e] = cn;
      }
    }
#pragma unroll
    for (int jj = kMaxKs - 1; jj > 0; --jj)
#pragma unroll
      for (int e = 0; e < V; ++e) win[jj][e] = win[jj - 1][e];
#pragma unroll
    for (int e = 0; e < V; ++e) win[0][e] = xv[e];
  };
  // the convolution at the newest token (and the per-head norm), stored
  auto emit = [&](int t) {
    float yv[V];
#pragma unroll
    for (int e = 0; e < V; ++e) {
      float acc = 0.f;
#pragma unroll
      for (int jj = 0; jj < kMaxKs; ++jj) acc += wt[jj][e] * win[jj][e];
      yv[e] = acc;
    }
    if constexpr (NORM) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < V; ++e) ss += yv[e] * yv[e];
      const float inv = __builtin_amdgcn_rsqf(group_sum<LPH>(ss) + 1e-6f);
#pragma unroll
      for (int e = 0; e < V; ++e) yv[e] *= inv;
    }
    R::store(&yb[(size_t)t * rs], R::pack(yv));
  };

  // halo tokens ts .. t0-1 and the first block are loaded together; loads
  // are clamped into [ts, t1) (the extra values are never pushed)
  RT hr[NH];
#pragma unroll
  for (int u = 0; u < NH; ++u) hr[u] = R::load(&xb[(size_t)min(ts + u, t1 - 1) * rs]);
  RT xr[kLB];
#pragma unroll
  for (int u = 0; u < kLB; ++u) xr[u] = R::load(&xb[(size_t)min(t0 + u, t1 - 1) * rs]);
#pragma unroll
  for (int u = 0; u < NH; ++u)
    if (u < t0 - ts) push(hr[u]);
  // full blocks with straight-line bodies (every token stored), so that the
  // tokens' head reductions overlap; the next block's loads are issued
  // before the current block is computed
  int t = t0;
  for (; t + kLB <= t1; t += kLB) {
    RT xn[kLB];
    const bool more = t + kLB < t1;
    if (more) {
#pragma unroll
      for (int u = 0; u < kLB; ++u) xn[u] = R::load(&xb[(size_t)min(t + kLB + u, t1 - 1) * rs]);
    }
#pragma unroll
    for (int u = 0; u < kLB; ++u) {
      push(xr[u]);
      emit(t + u);
    }
    if (more) {
#pragma unroll
      for (int u = 0; u < kLB; ++u) xr[u] = xn[u];
    }
  }
  // ragged end of the sequence (xr holds the block at t): token by token
  if (t < t1) {
#pragma unroll
    for (int u = 0; u < kLB; ++u) {
      if (t + u < t1) {
        push(xr[u]);
        emit(t + u);
      }
    }
  }
}

// The three tensors of a prefill call; units[i] counts (sequence, head group)
// pairs of tensor i.
struct ConvPrefillSet {
  const void* x[3];
  const float* w[3];
  void* y[3];
  int nh[3];
  int units[3];
};

template <class T, int D, bool ROPE, bool NORM>
__global__ __launch_bounds__(64 * kWT) void shortconv_kernel(ConvPrefillSet set, int T_, int ks, float theta,
                                                             int pos0, int spans, int units) {
  using G = ConvGeom<T, D>;
  int unit, span;
  if (!xcd_grouped(blockIdx.x, spans, units, unit, span)) return;
  int ti = 0;
  while (ti < 2 && unit >= set.units[ti]) unit -= set.units[ti++];
  const int groups = (set.nh[ti] + G::HW - 1) / G::HW;
  const int bi = unit / groups;
  const int hg = unit % groups;
  const int t0 = (span * kWT + wave_id()) * kTT;
  const T* x = static_cast<const T*>(set.x[ti]);
  T* y = static_cast<T*>(set.y[ti]);
  if (ti < 2)
    conv_tile<T, D, ROPE, NORM>(x, set.w[ti], y, T_, set.nh[ti], ks, theta, pos0, bi, hg, t0);
  else
    conv_tile<T, D, false, false>(x, set.w[ti], y, T_, set.nh[ti], ks, theta, pos0, bi, hg, t0);
}

template <class T, int D>
hipError_t launch_all(const ShortConvArgs& p, hipStream_t s) {
  using G = ConvGeom<T, D>;
  const int rope = p.flags & 1;
  const int norm = (p.flags >> 1) & 1;
  ConvPrefillSet set;
  const void* xs[3] = {p.q, p.k, p.v};
  const float* ws[3] = {p.wq, p.wk, p.wv};
  void* ys[3] = {p.q_out, p.k_out, p.v_out};
  const int nhs[3] = {p.H, p.Hkv, p.Hkv};
  long long units = 0;
  for (int i = 0; i < 3; ++i) {
    set.x[i] = xs[i];
    set.w[i] = ws[i];
    set.y[i] = ys[i];
    set.nh[i] = nhs[i];
    const long long u = (long long)p.B * ((nhs[i] + G::HW - 1) / G::HW);
    if (u > INT32_MAX) return hipErrorInvalidValue;
    set.units[i] = (int)u;
    units += u;
  }
  const long long spans = ((long long)p.T + kWT * kTT - 1) / (kWT * kTT);
  const long long grid = 8LL * spans * ((units + 7) / 8);
  if (units == 0 || spans == 0) return hipSuccess;
  if (grid * 64 * kWT > INT32_MAX) return hipErrorInvalidValue;
#define GDN_SC_LAUNCH(R, N)                                                                          \
  hipLaunchKernelGGL((shortconv_kernel<T, D, R, N>), dim3((unsigned)grid), dim3(64 * kWT), 0, s, set, p.T, \
                     p.ksize, p.rope_theta, p.pos0, (int)spans, (int)units)
  if (rope) {
    if (norm) GDN_SC_LAUNCH(true, true); else GDN_SC_LAUNCH(true, false);
  } else {
    if (norm) GDN_SC_LAUNCH(false, true); else GDN_SC_LAUNCH(false, false);
  }
#undef GDN_SC_LAUNCH
  return hipGetLastError();
}

// ------------------------------------------------------------------ decode
//
// Decode keeps, per sequence and tensor, the inputs of the last ks - 1 tokens
// after RoPE and before the convolution (fp32, so a decode step convolves the
// same values the prefill kernel keeps in registers); token i sits at ring
// index i mod (ks - 1) of hist [B][ks-1][channels].

// RoPE factors of pair j at absolute position `apos`: the angle in fp64,
// reduced to [-pi, pi] before the fp32 cos / sin.
template <int D>
__device__ __forceinline__ void rope_cs(int j, long long apos, float theta, float& cs, float& sn) {
  const double f = exp(-(2.0 * j / D) * log((double)theta));
  const double ang = (double)apos * f;
  const double twopi = 6.283185307179586476925;
  const double red = ang - twopi * rint(ang / twopi);
  cs = (float)cos(red);
  sn = (float)sin(red);
}

// The three tensors of one call (q, k, v), selected by blockIdx.z.
struct ConvTensor {
  const void* x;      // raw inputs
  const float* w;     // [nh * D, ks]
  float* hist;        // [B][ks-1][nh * D]
  void* y;            // decode outputs
  int nh, rope, norm;
};
struct ConvSet {
  ConvTensor t[3];
};

// One decode step: one wave per (sequence, 64 / (D/2) heads), lane j owning
// the RoPE pair (j, j + D/2) of its head as in the prefill kernel.  Each
// thread reads and then rewrites only its own two channels of the history.
template <class T, int D>
__global__ __launch_bounds__(256) void shortconv_decode_kernel(ConvSet set, const int* __restrict__ pos,
                                                               int ks, float theta, int pos0) {
  constexpr int LPH = D / 2;
  constexpr int HW = 64 / LPH;
  const ConvTensor tt = set.t[blockIdx.z];
  const int lane = threadIdx.x & 63;
  const int h = (blockIdx.x * 4 + (threadIdx.x >> 6)) * HW + lane / LPH;
  if (h >= tt.nh) return;              // whole head groups leave together
  const int j = lane % LPH;
  const int bi = blockIdx.y;
  const int t = pos[bi];
  if (t < 0) return;                   // outside the contract (pos >= 0)
  const int C = tt.nh * D;
  const int c1 = h * D + j;
  const int c2 = c1 + LPH;
  const T* x = reinterpret_cast<const T*>(tt.x) + (size_t)bi * C;
  float x1 = to_f32(x[c1]);
  float x2 = to_f32(x[c2]);
  if (tt.rope) {
    float cs, sn;
    rope_cs<D>(j, (long long)pos0 + t, theta, cs, sn);
    const float r1 = x1 * cs - x2 * sn;
    const float r2 = x2 * cs + x1 * sn;
    x1 = r1;
    x2 = r2;
  }
  const float* w = tt.w;
  float y1 = w[(size_t)c1 * ks + ks - 1] * x1;
  float y2 = w[(size_t)c2 * ks + ks - 1] * x2;
  if (ks > 1) {
    const int m = ks - 1;
    float* hb = tt.hist + (size_t)bi * m * C;
    for (int jj = 1; jj < ks; ++jj) {
      if (t - jj < 0) break;           // zero history before the sequence start
      const float* hr = hb + (size_t)((t - jj) % m) * C;
      y1 += w[(size_t)c1 * ks + ks - 1 - jj] * hr[c1];
      y2 += w[(size_t)c2 * ks + ks - 1 - jj] * hr[c2];
    }
    float* hw = hb + (size_t)(t % m) * C;   // token t - ks + 1 leaves the ring
    hw[c1] = x1;
    hw[c2] = x2;
  }
  if (tt.norm) {
    const float ss = head_sum<LPH>(y1 * y1 + y2 * y2);
    const float inv = 1.0f / sqrtf(ss + 1e-6f);
    y1 *= inv;
    y2 *= inv;
  }
  T* y = reinterpret_cast<T*>(tt.y) + (size_t)bi * C;
  y[c1] = from_f32<T>(y1);
  y[c2] = from_f32<T>(y2);
}

// History after a prefill of T_ tokens: ring slot r holds token
// i = T_ - 1 - ((T_ - 1 - r) mod (ks - 1)), rotated at position pos0 + i, or
// zero when i < 0.  One thread per (pair, head); grid x = 3 * pair blocks
// (the tensor is blockIdx.x mod 3), y = ring slot, z = sequence.
template <class T, int D>
__global__ __launch_bounds__(256) void shortconv_history_kernel(ConvSet set, int T_, int ks, float theta,
                                                                int pos0) {
  constexpr int LPH = D / 2;
  const ConvTensor tt = set.t[blockIdx.x % 3];
  const int idx = (blockIdx.x / 3) * 256 + threadIdx.x;
  if (idx >= tt.nh * LPH) return;
  const int h = idx / LPH;
  const int j = idx % LPH;
  const int r = blockIdx.y;
  const int bi = blockIdx.z;
  const int m = ks - 1;
  const int C = tt.nh * D;
  const int c1 = h * D + j;
  const int c2 = c1 + LPH;
  const int i = T_ - 1 - (((T_ - 1 - r) % m) + m) % m;
  float x1 = 0.f, x2 = 0.f;
  if (i >= 0) {
    const T* x = reinterpret_cast<const T*>(tt.x) + ((size_t)bi * T_ + i) * C;
    x1 = to_f32(x[c1]);
    x2 = to_f32(x[c2]);
    if (tt.rope) {
      float cs, sn;
      rope_cs<D>(j, (long long)pos0 + i, theta, cs, sn);
      const float r1 = x1 * cs - x2 * sn;
      const float r2 = x2 * cs + x1 * sn;
      x1 = r1;
      x2 = r2;
    }
  }
  float* hr = tt.hist + ((size_t)bi * m + r) * C;
  hr[c1] = x1;
  hr[c2] = x2;
}

ConvSet conv_set(const ShortConvArgs& p, float* const hist[3]) {
  const int rope = p.flags & 1;
  const int norm = (p.flags >> 1) & 1;
  ConvSet set;
  set.t[0] = ConvTensor{p.q, p.wq, hist[0], p.q_out, p.H, rope, norm};
  set.t[1] = ConvTensor{p.k, p.wk, hist[1], p.k_out, p.Hkv, rope, norm};
  set.t[2] = ConvTensor{p.v, p.wv, hist[2], p.v_out, p.Hkv, 0, 0};
  return set;
}

template <class T, int D>
hipError_t launch_decode_t(const ShortConvArgs& p, float* const hist[3], const int* pos, hipStream_t s) {
  constexpr int HW = 128 / D;
  const int units = (p.H + HW - 1) / HW;   // q has the most heads
  const dim3 grid((units + 3) / 4, p.B, 3);
  hipLaunchKernelGGL((shortconv_decode_kernel<T, D>), grid, dim3(256), 0, s, conv_set(p, hist), pos,
                     p.ksize, p.rope_theta, p.pos0);
  return hipGetLastError();
}

template <class T, int D>
hipError_t launch_history_t(const ShortConvArgs& p, float* const hist[3], hipStream_t s) {
  const int pairs = p.H * (D / 2);   // q has the most heads
  const dim3 grid(3 * ((pairs + 255) / 256), p.ksize - 1, p.B);
  hipLaunchKernelGGL((shortconv_history_kernel<T, D>), grid, dim3(256), 0, s, conv_set(p, hist), p.T,
                     p.ksize, p.rope_theta, p.pos0);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_shortconv_decode(const ShortConvArgs& p, float* const hist[3], const int* pos,
                                   hipStream_t s) {
  if (p.bf16) return p.D == 64 ? launch_decode_t<bf16, 64>(p, hist, pos, s) : launch_decode_t<bf16, 128>(p, hist, pos, s);
  return p.D == 64 ? launch_decode_t<float, 64>(p, hist, pos, s) : launch_decode_t<float, 128>(p, hist, pos, s);
}

hipError_t launch_shortconv_history(const ShortConvArgs& p, float* const hist[3], hipStream_t s) {
  if (p.bf16) return p.D == 64 ? launch_history_t<bf16, 64>(p, hist, s) : launch_history_t<bf16, 128>(p, hist, s);
  return p.D == 64 ? launch_history_t<float, 64>(p, hist, s) : launch_history_t<float, 128>(p, hist, s);
}

hipError_t launch_shortconv(const ShortConvArgs& p, hipStream_t s) {
  if (p.bf16) return p.D == 64 ? launch_all<bf16, 64>(p, s) : launch_all<bf16, 128>(p, s);
  return p.D == 64 ? launch_all<float, 64>(p, s) : launch_all<float, 128>(p, s);
}

}  // namespace gdn
