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
// Work split: one workgroup per (sequence, up to 4 query heads sharing one
// KV head, run of TPW consecutive tiles of QT query rows); each wave owns 32
// query rows of one head.  The next key block is fetched into registers
// while the current one is used from LDS (two LDS buffers), across tiles.
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
__global__ __launch_bounds__(64 * NW, 2) void swa_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                      const T* __restrict__ v, T* __restrict__ o,
                                                      int T_, int H, int Hkv, int HPW, int QT, int TPW,
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
  const int tile0 = blockIdx.x * TPW;                 // first query tile of this workgroup
  const int ntile = min(TPW, (T_ + QT - 1) / QT - tile0);
  const float scale = kLog2e / sqrtf((float)D);
  const int sdc = tid % DPR;                       // staging dword column
  const int sk0 = (tid / DPR) * KPT;               // staging first key of the block

  // Key blocks of query tile t0: sinks [0, min(n_sink, t_end)) then the
  // window [max(n_sink, t0 - window + 1), t_end), KB keys per block.
  struct Blk { int kb0, kend, sink; };
  auto tile_blocks = [&](int t0, int& nbs, int& nbw, int& sink_end, int& win_lo, int& t_end) {
    t_end = min(t0 + QT, T_);
    sink_end = min(n_sink, t_end);
    win_lo = max(n_sink, t0 - window + 1);
    nbs = (sink_end + KB - 1) / KB;
    nbw = t_end > win_lo ? (t_end - win_lo + KB - 1) / KB : 0;
  };
  // flat block index over the workgroup's tiles -> block description
  auto block_at = [&](int flat, Blk& bl) -> bool {
    for (int ti = 0; ti < ntile; ++ti) {
      int nbs, nbw, se, wl, te;
      tile_blocks((tile0 + ti) * QT, nbs, nbw, se, wl, te);
      if (flat < nbs + nbw) {
        const bool sk = flat < nbs;
        bl.kb0 = sk ? flat * KB : wl + (flat - nbs) * KB;
        bl.kend = sk ? se : te;
        bl.sink = sk;
        return true;
      }
      flat -= nbs + nbw;
    }
    return false;
  };

  // ---- register prefetch of a key block and its commit to an LDS buffer
  uint32_t pk[KPT], pv[KPT];
  const size_t kvstride = (size_t)Hkv * D;
  // a thread stages KPT consecutive keys of one dword column; the transposed
  // V tile keeps its key dimension in acc order (written in runs of 4 keys)
  auto prefetch = [&](const Blk& bl) {
    const size_t off = ((size_t)(bi * T_ + bl.kb0 + sk0) * Hkv + g) * D + sdc * EPD;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const bool ok = bl.kb0 + sk0 + j < bl.kend;
      pk[j] = ok ? *reinterpret_cast<const uint32_t*>(k + off + j * kvstride) : 0u;
      pv[j] = ok ? *reinterpret_cast<const uint32_t*>(v + off + j * kvstride) : 0u;
    }
  };
  auto commit = [&](int buf) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) *reinterpret_cast<uint32_t*>(&Ks[buf][(sk0 + j) * SK + sdc * EPD]) = pk[j];
#pragma unroll
    for (int e = 0; e < EPD; ++e) store_column_acc<T, KPT>(&VTs[buf][(sdc * EPD + e) * SV], sk0, pv, e);
  };

  int flat = 0;   // running block counter (selects the LDS buffer)
  {
    Blk b0;
    if (block_at(0, b0)) {
      prefetch(b0);
      commit(0);
    }
  }
  lds_barrier();

  for (int ti = 0; ti < ntile; ++ti) {
    const int t0 = (tile0 + ti) * QT;
    const int qb = t0 + (wv % NWQ) * 16 * kNQ;      // first query row of this wave
    const int qlast = qb + 16 * kNQ - 1;
    int nbs, nbw, sink_end, win_lo, t_end;
    tile_blocks(t0, nbs, nbw, sink_end, win_lo, t_end);

    // query fragments (B operand of S^T = K Q^T, "linear" set over d),
    // pre-multiplied by log2(e) / sqrt(d) so the scores come out of the MFMA
    // already in exp2 units
    Frag<T> qf[kNQ][D / 32];
#pragma unroll
    for (int nq = 0; nq < kNQ; ++nq) {
      const int t = qb + 16 * nq + l16;
#pragma unroll
      for (int p = 0; p < D / 32; ++p) {
        float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (t < T_) {
          const T* qp = q + ((size_t)(bi * T_ + t) * H + h) * D + 32 * p + 8 * lg;
          const f32x4 a = load4(qp);
          const f32x4 b = load4(qp + 4);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            x[i] = a[i] * scale;
            x[4 + i] = b[i] * scale;
          }
        }
        qf[nq][p] = frag_from8<T>(x);
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

    for (int blk = 0; blk < nbs + nbw; ++blk, ++flat) {
      const int buf = flat & 1;
      const bool sinkph = blk < nbs;
      const int kb0 = sinkph ? blk * KB : win_lo + (blk - nbs) * KB;
      const int kend = sinkph ? sink_end : t_end;
      Blk nx;
      const bool has_next = block_at(flat + 1, nx);
      if (has_next) prefetch(nx);
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

      // ---- mask, online softmax (per lane = per query, 4 lane groups).
      // A 16x16 tile whose keys are all visible to all its queries skips the
      // per-element mask.  The running max is only moved (and O rescaled)
      // when a block raises it by more than 8 in log2 units, which keeps
      // every exponent <= 2^8 while sparing most rescales.
#pragma unroll
      for (int nq = 0; nq < kNQ; ++nq) {
        const int q0 = qb + 16 * nq;
        const int t = q0 + l16;
        float mloc = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < KB / 16; ++kt) {
          const int k0 = kb0 + 16 * kt;
          const bool full = tile_on[kt] && k0 + 15 < kend && k0 + 15 <= q0 && q0 + 15 < T_ &&
                            (sinkph || k0 > q0 + 15 - window);
          if (full) {
#pragma unroll
            for (int i = 0; i < 4; ++i) mloc = fmaxf(mloc, sacc[kt][nq][i]);
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int key = k0 + 4 * lg + i;
              bool valid = tile_on[kt] && key < kend && key <= t && t < T_;
              if (!sinkph) valid = valid && key > t - window;
              const float sc = valid ? sacc[kt][nq][i] : -INFINITY;
              sacc[kt][nq][i] = sc;
              mloc = fmaxf(mloc, sc);
            }
          }
        }
        mloc = fmaxf(mloc, shfl_xor(mloc, 16));
        mloc = fmaxf(mloc, shfl_xor(mloc, 32));
        float mref = mrun[nq];
        if (__any(mloc > mref + 8.f)) {   // some query of the wave needs a new reference
          const float mnew = fmaxf(mref, mloc);
          const float alpha = mnew == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(mref - mnew);
          lrun[nq] *= alpha;
#pragma unroll
          for (int dt = 0; dt < D / 16; ++dt) oacc[dt][nq] *= alpha;
          mref = mnew;
          mrun[nq] = mnew;
        }
        // a lane that has seen no key yet only holds -inf scores: any finite
        // reference sends them to exp2(-inf) = 0
        const float mexp = mref == -INFINITY ? 0.f : mref;
        float psum = 0.f;
#pragma unroll
        for (int kt = 0; kt < KB / 16; ++kt) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float pr = __builtin_amdgcn_exp2f(sacc[kt][nq][i] - mexp);
            sacc[kt][nq][i] = pr;
            psum += pr;
          }
        }
        lrun[nq] += psum;
      }

      // ---- O^T += V^T P^T
#pragma unroll
      for (int pp = 0; pp < KB / 32; ++pp) {
        if (!(tile_on[2 * pp] || tile_on[2 * pp + 1])) continue;
        Frag<T> pf[kNQ];
#pragma unroll
        for (int nq = 0; nq < kNQ; ++nq) pf[nq] = frag_from_acc<T>(sacc[2 * pp][nq], sacc[2 * pp + 1][nq]);
        // V fragments in two halves to bound the live registers
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          Frag<T> vf[D / 32];
#pragma unroll
          for (int dd = 0; dd < D / 32; ++dd)
            vf[dd] = lds_frag8(&Vb[(16 * (hf * D / 32 + dd) + l16) * SV + 32 * pp + 8 * lg]);
#pragma unroll
          for (int dd = 0; dd < D / 32; ++dd)
#pragma unroll
            for (int nq = 0; nq < kNQ; ++nq)
              oacc[hf * D / 32 + dd][nq] = mfma(vf[dd], pf[nq], oacc[hf * D / 32 + dd][nq]);
        }
      }

      if (has_next) commit(buf ^ 1);
      lds_barrier();
    }

    // ---- epilogue of this query tile
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
  // heads per workgroup: the largest power of two (<= 4) dividing G; one
  // wave per head and 32 query rows (two waves when a group has one head),
  // so two 4-wave workgroups fit on a CU.  Each workgroup walks TPW
  // consecutive query tiles with one continuous K/V prefetch pipeline.
  const int G = p.H / p.Hkv;
  int HPW = 1;
  while (HPW < 4 && G % (2 * HPW) == 0) HPW *= 2;
  const int QT = HPW == 1 ? 64 : 32;
  const int waves = HPW * (QT / (16 * kNQ));
  const int ntiles = (p.T + QT - 1) / QT;
  const int groups = p.H / HPW;
  // keep at least ~4 workgroups per CU of work before batching tiles
  int TPW = 1;
  while (TPW < 8 && (size_t)((ntiles + 2 * TPW - 1) / (2 * TPW)) * groups * p.B >= 2048) TPW *= 2;
  const dim3 grid((ntiles + TPW - 1) / TPW, groups, p.B);
#define GDN_SWA_LAUNCH(NWV)                                                                         \
  hipLaunchKernelGGL((swa_kernel<T, D, NWV>), grid, dim3(64 * NWV), 0, s, (const T*)p.q,           \
                     (const T*)p.k, (const T*)p.v, (T*)p.o, p.T, p.H, p.Hkv, HPW, QT, TPW,         \
                     p.n_sink, p.window, add_from)
  if (waves == 2) GDN_SWA_LAUNCH(2);
  else GDN_SWA_LAUNCH(4);
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
