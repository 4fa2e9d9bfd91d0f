// Softmax branch of the hybrid layer over sinks + sliding window (prefill),
// flash-style, for gfx950.
//
// Method (page "The Key to Going Linear: Analysis-Driven Transformer
// Linearization", section 填补近似缺口的实用设计): query t attends with
// softmax to A(t) = { i <= t : i < n_sink or i > t - window }: the sink tokens
// keep full attention and the window holds the most recent tokens, the
// current one included.  Logits are q.k / sqrt(d) (section 从 softmax 到
// delta 规则的一阶近似, Lemma 1).
//
// Work split: one workgroup per (sequence, group of query heads sharing one
// KV head, tile of QT query rows); each wave owns 32 query rows of one head.
// Keys are visited in two phases, the sinks [0, n_sink) and then the window
// [max(n_sink, t0 - window + 1), t_end), so a key in both ranges is counted
// once.  64-key blocks of K (row-major) and V (transposed) are staged in LDS
// once and shared by every head of the group.
//
// The product is computed transposed, S^T = K Q^T, so each lane's
// accumulator column is one query: the running max and sum stay per lane
// (plus one butterfly over the 4 lane groups), and the probabilities feed
// O^T += V^T P^T straight from registers (the "acc" reduction set).
// Exponentials use exp2 with log2(e) folded into the scale.  A 16-key tile
// that no query of the wave can see is skipped.
//
// Epilogue: o = O / l, plus the value o already holds on rows t >= add_from
// (the linear branch, or the caller's values when accumulating), cast to the
// output type.

#include "common.h"
#include "launch.h"

namespace gdn {
namespace {

constexpr int kNQ = 2;    // 16-query tiles per wave

// Keys per LDS block: 64 for bf16, 32 for fp32 (keeps the register prefetch
// of a block small).
template <class T> struct KeyBlock { static constexpr int n = sizeof(T) == 2 ? 64 : 32; };

template <class T, int D, int NW>
__global__ __launch_bounds__(64 * NW) void swa_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                      const T* __restrict__ v, T* __restrict__ o,
                                                      int T_, int H, int Hkv, int HPW, int QT,
                                                      int n_sink, int window, int add_from) {
  constexpr int KB = KeyBlock<T>::n;
  constexpr int NTH = 64 * NW;
  constexpr int PAD = 16 / sizeof(T);
  constexpr int SK = D + PAD;      // Ks row stride
  constexpr int SV = KB + PAD;     // VTs row stride
  // staging: each thread owns one dword column of KPT consecutive keys
  constexpr int EPD = 4 / sizeof(T);
  constexpr int DPR = D / EPD;
  constexpr int KPT = KB * DPR / NTH;
  static_assert(NTH % DPR == 0 && KPT >= 4 && KPT % 4 == 0, "staging shape");
  __shared__ __attribute__((aligned(16))) T Ks[2][KB * SK];
  __shared__ __attribute__((aligned(16))) T VTs[2][D * SV];

  const int tile = blockIdx.x;
  const int hgrp = blockIdx.y;
  const int bi = blockIdx.z;
  const int G = H / Hkv;
  const int h0 = hgrp * HPW;
  const int g = h0 / G;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = wave_id();
  const int l16 = lane & 15;
  const int lg = lane >> 4;
  const int NWQ = QT / (16 * kNQ);
  const int h = h0 + wv / NWQ;
  const int t0 = tile * QT;
  const int qb = t0 + (wv % NWQ) * 16 * kNQ;      // first query row of this wave
  const int t_end = min(t0 + QT, T_);
  const float scale = kLog2e / sqrtf((float)D);
  const int sdc = tid % DPR;                       // staging dword column
  const int sk0 = (tid / DPR) * KPT;               // staging first key of the block

  // query fragments (B operand of S^T = K Q^T, "linear" set over d)
  Frag<T> qf[kNQ][D / 32];
#pragma unroll
  for (int nq = 0; nq < kNQ; ++nq) {
    const int t = qb + 16 * nq + l16;
#pragma unroll
    for (int p = 0; p < D / 32; ++p) {
      if (t < T_)
        qf[nq][p] = gbl_frag8(q + ((size_t)(bi * T_ + t) * H + h) * D + 32 * p + 8 * lg);
      else
        qf[nq][p] = zero_frag<T>();
    }
  }

  f32x4 oacc[D / 16][kNQ];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
    for (int nq = 0; nq < kNQ; ++nq) oacc[dt][nq] = zero4();
  float mrun[kNQ], lrun[kNQ];
#pragma unroll
  for (int nq = 0; nq < kNQ; ++nq) {
    mrun[nq] = -INFINITY;
    lrun[nq] = 0.f;
  }

  const int sink_end = min(n_sink, t_end);
  const int win_lo = max(n_sink, t0 - window + 1);
  const int nb_sink = (sink_end + KB - 1) / KB;
  const int nb_win = t_end > win_lo ? (t_end - win_lo + KB - 1) / KB : 0;
  const int nb = nb_sink + nb_win;
  const int qlast = qb + 16 * kNQ - 1;

  // ---- register prefetch of a key block and its commit to an LDS buffer
  uint32_t pk[KPT], pv[KPT];
  const size_t kvstride = (size_t)Hkv * D;
  auto prefetch = [&](int blk) {
    const bool sinkph = blk < nb_sink;
    const int kb0 = sinkph ? blk * KB : win_lo + (blk - nb_sink) * KB;
    const int kend = sinkph ? sink_end : t_end;
    const size_t off = ((size_t)(bi * T_ + kb0 + sk0) * Hkv + g) * D + sdc * EPD;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const bool ok = kb0 + sk0 + j < kend;
      pk[j] = ok ? *reinterpret_cast<const uint32_t*>(k + off + j * kvstride) : 0u;
      pv[j] = ok ? *reinterpret_cast<const uint32_t*>(v + off + j * kvstride) : 0u;
    }
  };
  auto commit = [&](int buf) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) *reinterpret_cast<uint32_t*>(&Ks[buf][(sk0 + j) * SK + sdc * EPD]) = pk[j];
#pragma unroll
    for (int e = 0; e < EPD; ++e) store_column<T, KPT>(&VTs[buf][(sdc * EPD + e) * SV + sk0], pv, e);
  };

  if (nb > 0) {
    prefetch(0);
    commit(0);
  }
  lds_barrier();

  for (int blk = 0; blk < nb; ++blk) {
    const int buf = blk & 1;
    const bool sinkph = blk < nb_sink;
    const int kb0 = sinkph ? blk * KB : win_lo + (blk - nb_sink) * KB;
    const int kend = sinkph ? sink_end : t_end;
    if (blk + 1 < nb) prefetch(blk + 1);
    const T* Kb = Ks[buf];
    const T* Vb = VTs[buf];

    // ---- S^T tiles for this wave (tiles no query of the wave sees are skipped)
    bool tile_on[KB / 16];
    f32x4 sacc[KB / 16][kNQ];
#pragma unroll
    for (int kt = 0; kt < KB / 16; ++kt) {
      const int k0 = kb0 + 16 * kt;
      bool on = k0 < kend && k0 <= qlast && qb < T_;
      if (!sinkph) on = on && (k0 + 15 > qb - window);
      tile_on[kt] = on;
#pragma unroll
      for (int nq = 0; nq < kNQ; ++nq) sacc[kt][nq] = zero4();
      if (on) {
        Frag<T> af[D / 32];
#pragma unroll
        for (int p = 0; p < D / 32; ++p) af[p] = lds_frag8(&Kb[(16 * kt + l16) * SK + 32 * p + 8 * lg]);
#pragma unroll
        for (int p = 0; p < D / 32; ++p)
#pragma unroll
          for (int nq = 0; nq < kNQ; ++nq) sacc[kt][nq] = mfma(af[p], qf[nq][p], sacc[kt][nq]);
      }
    }

    // ---- mask, online softmax (per lane = per query, 4 lane groups)
#pragma unroll
    for (int nq = 0; nq < kNQ; ++nq) {
      const int t = qb + 16 * nq + l16;
      float mloc = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < KB / 16; ++kt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kb0 + 16 * kt + 4 * lg + i;
          bool valid = tile_on[kt] && key < kend && key <= t && t < T_;
          if (!sinkph) valid = valid && key > t - window;
          const float sc = valid ? sacc[kt][nq][i] * scale : -INFINITY;
          sacc[kt][nq][i] = sc;
          mloc = fmaxf(mloc, sc);
        }
      }
      mloc = fmaxf(mloc, shfl_xor(mloc, 16));
      mloc = fmaxf(mloc, shfl_xor(mloc, 32));
      const float mnew = fmaxf(mrun[nq], mloc);
      const float alpha = mnew == -INFINITY ? 1.f : exp2f(mrun[nq] - mnew);
      float psum = 0.f;
#pragma unroll
      for (int kt = 0; kt < KB / 16; ++kt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float sc = sacc[kt][nq][i];
          const float pr = sc == -INFINITY ? 0.f : exp2f(sc - mnew);
          sacc[kt][nq][i] = pr;
          psum += pr;
        }
      }
      mrun[nq] = mnew;
      lrun[nq] = lrun[nq] * alpha + psum;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) oacc[dt][nq] *= alpha;
    }

    // ---- O^T += V^T P^T
#pragma unroll
    for (int pp = 0; pp < KB / 32; ++pp) {
      if (!(tile_on[2 * pp] || tile_on[2 * pp + 1])) continue;
      Frag<T> pf[kNQ];
#pragma unroll
      for (int nq = 0; nq < kNQ; ++nq) pf[nq] = frag_from_acc<T>(sacc[2 * pp][nq], sacc[2 * pp + 1][nq]);
      Frag<T> vf[D / 16];
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        const T* vrow = &Vb[(16 * dt + l16) * SV + 32 * pp + 4 * lg];
        vf[dt] = lds_frag44(vrow, vrow + 16);
      }
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
        for (int nq = 0; nq < kNQ; ++nq) oacc[dt][nq] = mfma(vf[dt], pf[nq], oacc[dt][nq]);
    }

    if (blk + 1 < nb) commit(buf ^ 1);
    lds_barrier();
  }

  // ---- epilogue
#pragma unroll
  for (int nq = 0; nq < kNQ; ++nq) {
    float l = lrun[nq];
    l += shfl_xor(l, 16);
    l += shfl_xor(l, 32);
    const int t = qb + 16 * nq + l16;
    if (t >= T_) continue;
    const float inv = 1.0f / l;
    T* orow = o + ((size_t)(bi * T_ + t) * H + h) * D;
    const bool addl = t >= add_from;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      f32x4 val = oacc[dt][nq] * inv;
      const int d0 = 16 * dt + 4 * lg;
      if (addl) val += load4(orow + d0);
      store4(orow + d0, val);
    }
  }
}

template <class T>
__global__ void zero_head_rows_kernel(T* __restrict__ o, int T_, int H, int D, int N) {
  const int rows = min(N, T_);
  const size_t per_seq = (size_t)rows * H * D;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int bi = blockIdx.y;
  if (idx < per_seq) o[(size_t)bi * T_ * H * D + idx] = from_f32<T>(0.f);
}

template <class T, int D>
hipError_t launch_swa_t(const PrefillArgs& p, int add_from, hipStream_t s) {
  // heads per workgroup: the largest power of two (<= 8) dividing G
  const int G = p.H / p.Hkv;
  int HPW = 1;
  while (HPW < 8 && G % (2 * HPW) == 0) HPW *= 2;
  const int QT = HPW <= 4 ? 64 : 32;
  const int waves = HPW * (QT / (16 * kNQ));
  const dim3 grid((p.T + QT - 1) / QT, p.H / HPW, p.B);
#define GDN_SWA_LAUNCH(NWV)                                                                         \
  hipLaunchKernelGGL((swa_kernel<T, D, NWV>), grid, dim3(64 * NWV), 0, s, (const T*)p.q,           \
                     (const T*)p.k, (const T*)p.v, (T*)p.o, p.T, p.H, p.Hkv, HPW, QT, p.n_sink,    \
                     p.window, add_from)
  if (waves == 2) GDN_SWA_LAUNCH(2);
  else if (waves == 4) GDN_SWA_LAUNCH(4);
  else GDN_SWA_LAUNCH(8);
#undef GDN_SWA_LAUNCH
  return hipGetLastError();
}

}  // namespace

hipError_t launch_swa_prefill(const PrefillArgs& p, int add_from, hipStream_t s) {
  if (p.bf16) return p.D == 64 ? launch_swa_t<bf16, 64>(p, add_from, s) : launch_swa_t<bf16, 128>(p, add_from, s);
  return p.D == 64 ? launch_swa_t<float, 64>(p, add_from, s) : launch_swa_t<float, 128>(p, add_from, s);
}

hipError_t launch_zero_head_rows(const PrefillArgs& p, hipStream_t s) {
  const int N = p.n_sink + p.window;
  const size_t per_seq = (size_t)std::min(N, p.T) * p.H * p.D;
  if (per_seq == 0) return hipSuccess;
  const dim3 grid((unsigned)((per_seq + 255) / 256), p.B);
  if (p.bf16)
    hipLaunchKernelGGL(zero_head_rows_kernel<bf16>, grid, dim3(256), 0, s, (bf16*)p.o, p.T, p.H, p.D, N);
  else
    hipLaunchKernelGGL(zero_head_rows_kernel<float>, grid, dim3(256), 0, s, (float*)p.o, p.T, p.H, p.D, N);
  return hipGetLastError();
}

}  // namespace gdn
