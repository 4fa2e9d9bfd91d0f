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
// Work split: one wave per (sequence, head, 64-token tile); consecutive
// workgroups take consecutive heads of the same tile.  Lane j owns the
// RoPE pair (j, j + d/2) of its head, so rotation, the 8-tap sliding window
// over time and the per-head norm (a register-only reduction over the head's
// lanes) never leave registers; the tile re-reads a 7-token causal halo.  The rotation
// angle is set in fp64 at the tile start and then advanced one token at a
// time by a fixed complex rotation (error grows ~1e-7 per token).
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

constexpr int kTT = 64;      // tokens per wave
constexpr int kMaxKs = 8;
constexpr int kLB = 16;      // tokens whose loads are issued together

template <class T, int D, bool ROPE, bool NORM>
__global__ __launch_bounds__(256) void shortconv_kernel(const T* __restrict__ x, const float* __restrict__ w,
                                                        T* __restrict__ y, int T_, int nh, int ks,
                                                        float theta, int pos0) {
  constexpr int LPH = D / 2;        // lanes per head
  constexpr int HW = 64 / LPH;      // heads per wave
  constexpr int NH = kMaxKs - 1;    // most halo tokens
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int unit = blockIdx.x * 4 + wv;
  const int h = unit * HW + lane / LPH;
  if (h >= nh) return;              // whole head groups leave together
  const int j = lane % LPH;
  const int bi = blockIdx.z;
  const int t0 = blockIdx.y * kTT;
  const int t1 = min(t0 + kTT, T_);
  const int c1 = h * D + j;
  const int c2 = c1 + LPH;

  float w1[kMaxKs], w2[kMaxKs];     // w?[jj] multiplies the input jj tokens back
#pragma unroll
  for (int jj = 0; jj < kMaxKs; ++jj) {
    w1[jj] = jj < ks ? w[(size_t)c1 * ks + ks - 1 - jj] : 0.f;
    w2[jj] = jj < ks ? w[(size_t)c2 * ks + ks - 1 - jj] : 0.f;
  }
  float win1[kMaxKs], win2[kMaxKs];
#pragma unroll
  for (int jj = 0; jj < kMaxKs; ++jj) {
    win1[jj] = 0.f;
    win2[jj] = 0.f;
  }

  const int ts = max(0, t0 - (ks - 1));   // first halo token
  float cs = 1.f, sn = 0.f, cf = 1.f, sf = 0.f;
  if constexpr (ROPE) {
    const double f = exp(-(2.0 * j / D) * log((double)theta));
    const double ang = (double)(pos0 + ts) * f;
    const double twopi = 6.283185307179586476925;
    const double red = ang - twopi * rint(ang / twopi);
    cs = (float)cos(red);
    sn = (float)sin(red);
    cf = (float)cos(f);
    sf = (float)sin(f);
  }

  const size_t row = (size_t)nh * D;
  const T* xb = x + (size_t)bi * T_ * row;
  T* yb = y + (size_t)bi * T_ * row;
  // one token into the window: RoPE at the running angle, then the shift
  auto push = [&](float x1, float x2) {
    if constexpr (ROPE) {
      const float r1 = x1 * cs - x2 * sn;
      const float r2 = x2 * cs + x1 * sn;
      x1 = r1;
      x2 = r2;
      const float cn = cs * cf - sn * sf;
      sn = sn * cf + cs * sf;
      cs = cn;
    }
#pragma unroll
    for (int jj = kMaxKs - 1; jj > 0; --jj) {
      win1[jj] = win1[jj - 1];
      win2[jj] = win2[jj - 1];
    }
    win1[0] = x1;
    win2[0] = x2;
  };
  // the convolution at the newest token (and the per-head norm), stored
  auto emit = [&](int t) {
    float y1 = 0.f, y2 = 0.f;
#pragma unroll
    for (int jj = 0; jj < kMaxKs; ++jj) {
      y1 += w1[jj] * win1[jj];
      y2 += w2[jj] * win2[jj];
    }
    if constexpr (NORM) {
      const float ss = head_sum<LPH>(y1 * y1 + y2 * y2);
      const float inv = 1.0f / sqrtf(ss + 1e-6f);
      y1 *= inv;
      y2 *= inv;
    }
    yb[(size_t)t * row + c1] = from_f32<T>(y1);
    yb[(size_t)t * row + c2] = from_f32<T>(y2);
  };

  // halo tokens ts .. t0-1 and the first block are loaded together; loads
  // are clamped into [ts, t1) (the extra values are never pushed)
  T hr1[NH], hr2[NH];
#pragma unroll
  for (int u = 0; u < NH; ++u) {
    const size_t tt = (size_t)min(ts + u, t1 - 1);
    hr1[u] = xb[tt * row + c1];
    hr2[u] = xb[tt * row + c2];
  }
  // the tile's tokens in blocks of kLB with straight-line bodies (every
  // token of a full block is stored), so that the tokens' reductions overlap;
  // the loads of a block are issued together
  int t = t0;
  T xr1[kLB], xr2[kLB];
  auto load_block = [&](int tb) {
#pragma unroll
    for (int u = 0; u < kLB; ++u) {
      const size_t tt = (size_t)min(tb + u, t1 - 1);
      xr1[u] = xb[tt * row + c1];
      xr2[u] = xb[tt * row + c2];
    }
  };
  load_block(t0);
#pragma unroll
  for (int u = 0; u < NH; ++u)
    if (u < t0 - ts) push(to_f32(hr1[u]), to_f32(hr2[u]));
  for (; t + kLB <= t1; t += kLB) {
    if (t > t0) load_block(t);
#pragma unroll
    for (int u = 0; u < kLB; ++u) {
      push(to_f32(xr1[u]), to_f32(xr2[u]));
      emit(t + u);
    }
  }
  // ragged end of the sequence: the remaining tokens one by one
  if (t < t1) {
    if (t > t0) load_block(t);
#pragma unroll
    for (int u = 0; u < kLB; ++u) {
      if (t + u < t1) {
        push(to_f32(xr1[u]), to_f32(xr2[u]));
        emit(t + u);
      }
    }
  }
}

template <class T, int D>
hipError_t launch_one(const void* x, const float* w, void* y, const ShortConvArgs& p, int nh,
                      int rope, int norm, hipStream_t s) {
  constexpr int HW = 128 / D;
  const int units = (nh + HW - 1) / HW;
  // head groups vary fastest, so the workgroups in flight cover whole token
  // rows (every head of the same 64 tokens) rather than one head's column
  const dim3 grid((units + 3) / 4, (p.T + kTT - 1) / kTT, p.B);
#define GDN_SC_LAUNCH(R, N)                                                                        \
  hipLaunchKernelGGL((shortconv_kernel<T, D, R, N>), grid, dim3(256), 0, s, (const T*)x, w, (T*)y, p.T, \
                     nh, p.ksize, p.rope_theta, p.pos0)
  if (rope) {
    if (norm) GDN_SC_LAUNCH(true, true); else GDN_SC_LAUNCH(true, false);
  } else {
    if (norm) GDN_SC_LAUNCH(false, true); else GDN_SC_LAUNCH(false, false);
  }
#undef GDN_SC_LAUNCH
  return hipGetLastError();
}

template <class T, int D>
hipError_t launch_all(const ShortConvArgs& p, hipStream_t s) {
  const int rope = p.flags & 1;
  const int norm = (p.flags >> 1) & 1;
  hipError_t e = launch_one<T, D>(p.q, p.wq, p.q_out, p, p.H, rope, norm, s);
  if (e != hipSuccess) return e;
  e = launch_one<T, D>(p.k, p.wk, p.k_out, p, p.Hkv, rope, norm, s);
  if (e != hipSuccess) return e;
  return launch_one<T, D>(p.v, p.wv, p.v_out, p, p.Hkv, 0, 0, s);
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
