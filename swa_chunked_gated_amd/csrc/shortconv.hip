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
// Work split: one wave per (sequence, head, 64-token tile).  Lane j owns the
// RoPE pair (j, j + d/2) of its head, so rotation, the 8-tap sliding window
// over time and the per-head norm (a butterfly over the head's lanes) never
// leave registers; the tile re-reads a 7-token causal halo.  The rotation
// angle is set in fp64 at the tile start and then advanced one token at a
// time by a fixed complex rotation (error grows ~1e-7 per token).

#include <math.h>

#include "common.h"
#include "launch.h"

namespace gdn {
namespace {

constexpr int kTT = 64;      // tokens per wave
constexpr int kMaxKs = 8;

template <class T, int D>
__global__ __launch_bounds__(256) void shortconv_kernel(const T* __restrict__ x, const float* __restrict__ w,
                                                        T* __restrict__ y, int T_, int nh, int ks,
                                                        float theta, int pos0, int rope, int norm) {
  constexpr int LPH = D / 2;        // lanes per head
  constexpr int HW = 64 / LPH;      // heads per wave
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int unit = blockIdx.y * 4 + wv;
  const int h = unit * HW + lane / LPH;
  if (h >= nh) return;              // whole head groups leave together
  const int j = lane % LPH;
  const int bi = blockIdx.z;
  const int t0 = blockIdx.x * kTT;
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

  const int ts = max(0, t0 - (ks - 1));
  float cs = 1.f, sn = 0.f, cf = 1.f, sf = 0.f;
  if (rope) {
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
  for (int t = ts; t < t1; ++t) {
    float x1 = to_f32(xb[(size_t)t * row + c1]);
    float x2 = to_f32(xb[(size_t)t * row + c2]);
    if (rope) {
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
    if (t < t0) continue;
    float y1 = 0.f, y2 = 0.f;
#pragma unroll
    for (int jj = 0; jj < kMaxKs; ++jj) {
      y1 += w1[jj] * win1[jj];
      y2 += w2[jj] * win2[jj];
    }
    if (norm) {
      float ss = y1 * y1 + y2 * y2;
#pragma unroll
      for (int m = 1; m < LPH; m <<= 1) ss += shfl_xor(ss, m);
      const float inv = 1.0f / sqrtf(ss + 1e-6f);
      y1 *= inv;
      y2 *= inv;
    }
    yb[(size_t)t * row + c1] = from_f32<T>(y1);
    yb[(size_t)t * row + c2] = from_f32<T>(y2);
  }
}

template <class T, int D>
hipError_t launch_one(const void* x, const float* w, void* y, const ShortConvArgs& p, int nh,
                      int rope, int norm, hipStream_t s) {
  constexpr int HW = 128 / D;
  const int units = (nh + HW - 1) / HW;
  const dim3 grid((p.T + kTT - 1) / kTT, (units + 3) / 4, p.B);
  hipLaunchKernelGGL((shortconv_kernel<T, D>), grid, dim3(256), 0, s, (const T*)x, w, (T*)y, p.T,
                     nh, p.ksize, p.rope_theta, p.pos0, rope, norm);
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

}  // namespace

hipError_t launch_shortconv(const ShortConvArgs& p, hipStream_t s) {
  if (p.bf16) return p.D == 64 ? launch_all<bf16, 64>(p, s) : launch_all<bf16, 128>(p, s);
  return p.D == 64 ? launch_all<float, 64>(p, s) : launch_all<float, 128>(p, s);
}

}  // namespace gdn
