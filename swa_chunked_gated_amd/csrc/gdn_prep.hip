// Chunk preparation for the chunked gated delta rule (prefill): the part of
// each 64-token chunk's work that does not depend on the recurrent state, done
// for every chunk at once so that the sequential scan over chunks only keeps
// the state-dependent products.
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
// One workgroup of 4 waves per (chunk, query head, sequence).  K K^T on MFMA;
// the unit lower-triangular inverse as 16x16 diagonal blocks by forward
// substitution in fp32 plus the off-diagonal blocks by block recursion on
// fp32 MFMA (16x16x4, exact fp32 products).  Outputs per chunk (workspace,
// element type T): TB = Tm diag(b) and TBG = Tm diag(b gamma) as 64 rows of
// 64, each row's columns stored in acc order (the order the scan's LDS tiles
// use, so the scan copies them with 16-byte moves), and fp32 g[64], gamma[64].

#include "common.h"
#include "launch.h"

namespace gdn {
namespace {

constexpr int kC = 64;          // chunk length
constexpr int kSL = 68;         // fp32 stride of the 64x64 solve buffer
// the 10 lower-triangular 16x16 tiles (row, col) of a 64x64 matrix
__constant__ const int kPrepTileM[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
__constant__ const int kPrepTileN[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// C += A(16x16) B(16x16), both fp32 row-major in LDS.
__device__ __forceinline__ f32x4 mm16(const float* A, const float* B, f32x4 c, int l16, int lg) {
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) c = mfma4(A[l16 * kSL + 4 * kk + lg], B[(4 * kk + lg) * kSL + l16], c);
  return c;
}
// C += A(16x16, LDS) Y(16x16, accumulator registers of this wave).
__device__ __forceinline__ f32x4 mm16_acc(const float* A, const f32x4& Y, f32x4 c, int l16, int lg) {
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) c = mfma4(A[l16 * kSL + 4 * lg + kk], Y[kk], c);
  return c;
}
__device__ __forceinline__ void st16(float* blk, const f32x4& x, int l16, int lg) {
#pragma unroll
  for (int i = 0; i < 4; ++i) blk[(4 * lg + i) * kSL + l16] = x[i];
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

template <class T, int D>
__global__ __launch_bounds__(256) void gdn_prep_kernel(
    const T* __restrict__ k, const float* __restrict__ a, const float* __restrict__ b,
    T* __restrict__ wtb, T* __restrict__ wtbg, float* __restrict__ wg, int T_, int H, int Hkv,
    int n_sink, int window, int nch) {
  constexpr int NTH = 256;
  constexpr int EPC = 16 / (int)sizeof(T);     // elements per 16-byte chunk
  constexpr int SK = D + EPC;                  // Ks row stride (one chunk of padding)
  constexpr int CH = D / EPC;                  // chunks per K row
  constexpr int NPK = kC * CH / NTH;
  static_assert(kC * CH % NTH == 0, "K staging");
  typedef typename Vec16<T>::type V16;

  __shared__ __attribute__((aligned(16))) T Ks[kC * SK];
  __shared__ __attribute__((aligned(16))) float Lf[kC * kSL];
  __shared__ __attribute__((aligned(16))) float lgs[kC];
  __shared__ __attribute__((aligned(16))) float gam[kC];
  __shared__ __attribute__((aligned(16))) float bet[kC];

  const int c = blockIdx.x;
  const int h = blockIdx.y;
  const int bi = blockIdx.z;
  const int g = h / (H / Hkv);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = wave_id();
  const int l16 = lane & 15;
  const int lg = lane >> 4;
  const int iend = T_ - window;                // stream tokens are [n_sink, iend)
  const int i0 = n_sink + c * kC;
  const size_t ci = ((size_t)bi * H + h) * nch + c;

  // K rows of the chunk (zero past the stream end), natural column order:
  // K K^T reads both operands from the same rows, so any order is consistent
#pragma unroll
  for (int j = 0; j < NPK; ++j) {
    const int idx = tid + j * NTH;
    const int r = idx / CH;
    const int cc = (idx % CH) * EPC;
    V16 x;
    if (i0 + r < iend) {
      x = *reinterpret_cast<const V16*>(k + ((size_t)(bi * T_ + i0 + r) * Hkv + g) * D + cc);
    } else {
#pragma unroll
      for (int e = 0; e < EPC; ++e) x[e] = from_f32<T>(0.f);
    }
    *reinterpret_cast<V16*>(&Ks[r * SK + cc]) = x;
  }
  for (int i = tid; i < kC * kSL; i += NTH) Lf[i] = 0.f;
  // gates: g = inclusive cumsum of log2 a (a = 1 past the stream end), b
  if (tid < 64) {
    const int tok = i0 + lane;
    const float av = tok < iend ? a[(size_t)(bi * T_ + tok) * H + h] : 1.f;
    const float x = wave_prefix_sum(__builtin_amdgcn_logf(av), lane);
    lgs[lane] = x;
    gam[lane] = __builtin_amdgcn_exp2f(x);
  } else if (tid < 128) {
    const int tok = i0 + lane;
    bet[lane] = tok < iend ? b[(size_t)(bi * T_ + tok) * H + h] : 0.f;
  }
  __syncthreads();

  // ---- L = strictly lower (b_r 2^{g_r - g_s} k_r.k_s) on the 10 lower tiles
  for (int job = wv; job < 10; job += 4) {
    const int mt = kPrepTileM[job];
    const int nt = kPrepTileN[job];
    const int r0 = 16 * mt + 4 * lg;
    const int s = 16 * nt + l16;
    const f32x4 lr = *reinterpret_cast<const f32x4*>(&lgs[r0]);
    const f32x4 br = *reinterpret_cast<const f32x4*>(&bet[r0]);
    const float ls = lgs[s];
    Frag<T> xa[D / 32], xb[D / 32];
#pragma unroll
    for (int p = 0; p < D / 32; ++p) {
      xa[p] = lds_frag8(&Ks[(16 * mt + l16) * SK + 32 * p + 8 * lg]);
      xb[p] = lds_frag8(&Ks[(16 * nt + l16) * SK + 32 * p + 8 * lg]);
    }
    f32x4 acc = zero4();
#pragma unroll
    for (int p = 0; p < D / 32; ++p) acc = mfma(xa[p], xb[p], acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = r0 + i;
      const float dec = __builtin_amdgcn_exp2f(fminf(lr[i] - ls, 0.f));
      Lf[r * kSL + s] = s < r ? br[i] * dec * acc[i] : 0.f;
    }
  }
  __syncthreads();
  // ---- diagonal 16x16 blocks of (I + L)^-1 by forward substitution
  if (wv == 0) {
    const int blk = lane >> 4;
    const int j = l16;
    float* Lb = Lf + 16 * blk * kSL + 16 * blk;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float acc = r == j ? 1.f : 0.f;
#pragma unroll
      for (int s2 = 0; s2 < r; ++s2) acc -= Lb[r * kSL + s2] * x[s2];
      x[r] = acc;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) Lb[r * kSL + j] = x[r];
  }
  __syncthreads();
  // ---- level 1: X10 = -X11 L10 X00, X32 = -X33 L32 X22
  if (wv < 2) {
    const int o0 = wv == 0 ? 0 : 32;
    const float* L10 = Lf + (o0 + 16) * kSL + o0;
    const float* X00 = Lf + o0 * kSL + o0;
    const float* X11 = Lf + (o0 + 16) * kSL + o0 + 16;
    f32x4 y = mm16(L10, X00, zero4(), l16, lg);
    f32x4 xo = -mm16_acc(X11, y, zero4(), l16, lg);
    st16(Lf + (o0 + 16) * kSL + o0, xo, l16, lg);
  }
  __syncthreads();
  // ---- level 2: bottom-left 32x32 block = -X_BR (L_BL X_TL), one wave per 16x16 block
  {
    const int br = 32 + 16 * ((wv >> 1) & 1);   // block row
    const int bc = 16 * (wv & 1);               // block column
    f32x4 y = zero4();
    for (int kb = bc; kb < 32; kb += 16) y = mm16(Lf + br * kSL + kb, Lf + kb * kSL + bc, y, l16, lg);
    __syncthreads();
    st16(Lf + br * kSL + bc, y, l16, lg);
    __syncthreads();
    f32x4 xo = zero4();
    for (int kb = 32; kb <= br; kb += 16) xo = mm16(Lf + br * kSL + kb, Lf + kb * kSL + bc, xo, l16, lg);
    __syncthreads();
    st16(Lf + br * kSL + bc, -xo, l16, lg);
    __syncthreads();
  }
  // ---- TB = Tm diag(b), TBG = Tm diag(b gamma): row r, columns s0..s0+3 at
  // positions acc_pos(s0)..+3 of the row
  T* tb = wtb + ci * (kC * kC);
  T* tbg = wtbg + ci * (kC * kC);
  for (int i = tid; i < kC * kC / 4; i += NTH) {
    const int r = i >> 4;
    const int s0 = (i & 15) * 4;
    const f32x4 tm = *reinterpret_cast<const f32x4*>(&Lf[r * kSL + s0]);
    const f32x4 bb = *reinterpret_cast<const f32x4*>(&bet[s0]);
    const f32x4 gg = *reinterpret_cast<const f32x4*>(&gam[s0]);
    const f32x4 x = tm * bb;
    store4(tb + r * kC + acc_pos(s0), x);
    store4(tbg + r * kC + acc_pos(s0), x * gg);
  }
  if (tid < 64) wg[ci * (2 * kC) + tid] = lgs[tid];
  else if (tid < 128) wg[ci * (2 * kC) + tid] = gam[tid - 64];
}

template <class T, int D>
hipError_t launch_prep_t(const PrefillArgs& p, int nch, hipStream_t s) {
  const GdnWorkspace w = gdn_workspace_layout(p.workspace, p.B, p.H, nch, sizeof(T));
  hipLaunchKernelGGL((gdn_prep_kernel<T, D>), dim3(nch, p.H, p.B), dim3(256), 0, s, (const T*)p.k,
                     p.a, p.b, (T*)w.tb, (T*)w.tbg, w.g, p.T, p.H, p.Hkv, p.n_sink, p.window, nch);
  return hipGetLastError();
}

}  // namespace

GdnWorkspace gdn_workspace_layout(void* base, int B, int H, int nch, size_t elt) {
  GdnWorkspace w;
  const size_t n = (size_t)B * H * nch;
  unsigned char* p = static_cast<unsigned char*>(base);
  w.tb = p;
  w.tbg = p + n * kC * kC * elt;
  w.g = reinterpret_cast<float*>(p + 2 * n * kC * kC * elt);
  w.bytes = 2 * n * kC * kC * elt + n * 2 * kC * sizeof(float);
  return w;
}

hipError_t launch_gdn_prep(const PrefillArgs& p, int nch, hipStream_t s) {
  if (p.bf16) return p.D == 64 ? launch_prep_t<bf16, 64>(p, nch, s) : launch_prep_t<bf16, 128>(p, nch, s);
  return p.D == 64 ? launch_prep_t<float, 64>(p, nch, s) : launch_prep_t<float, 128>(p, nch, s);
}

}  // namespace gdn
