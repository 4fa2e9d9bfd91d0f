// Softmax branch of the hybrid layer over sinks + sliding window (prefill):
// the per-workgroup tile routine, used by the softmax kernel (swa.hip) and,
// linked to the chunked scan, by the fused prefill kernel (gdn_scan_full.hip).
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
// (16-byte loads; unguarded when the block is whole) while the current one
// is used from LDS (two LDS buffers), across tiles.
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
// Epilogue: o = w_swa O / l, plus the value o already holds on rows
// t >= add_from (the linear branch, or the caller's values when
// accumulating), cast to the output type.  w_swa weighs the softmax branch
// (inference-time hybridisation; 1 for the plain sum).

#pragma once

#include <type_traits>

#include "common.h"

namespace gdn {
namespace swa {


constexpr int kNQ = 2;    // 16-query tiles per wave
// A linked tile with at most this many key blocks fetches them all at once
// (one memory latency for the tile instead of one per block).
constexpr int kDeepBlocks = 3;

// Max over lanes l, l^16, l^32, l^48 (the four lane groups holding one
// query's scores), with the row-swap permutes: VALU only, no LDS round trip.
// Every lane of the group ends with the same value.
__device__ __forceinline__ float max_lane_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
// max of three floats in one instruction (the scores are never NaN, so the
// NaN-quieting that fmaxf needs in IEEE mode is left out)
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Keys per LDS block: 64 for bf16, 32 for fp32 (keeps the register prefetch
// of a block small).
template <class T> struct KeyBlock { static constexpr int n = sizeof(T) == 2 ? 64 : 32; };

// Waits until *f == epoch (read at device scope); later loads of the wave
// are issued only after that (in-order issue; the asm keeps the compiler from
// moving them above the loop).  SLEEP (units of 64 clocks) spaces the polls,
// so that many waiting waves do not load the memory system.  Bounded: after
// `ticks` of the 100 MHz real-time counter it gives up and returns false, so
// a missing producer can never hang the GPU; the caller then poisons what it
// computes from the data it waited for (NaN), so a give-up is never silent.
template <int SLEEP = 1>
__device__ __forceinline__ bool wait_ready(const uint64_t* f, uint64_t epoch, uint64_t ticks) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();          // 100 MHz
  bool ok = true;
  while (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != epoch) {
    __builtin_amdgcn_s_sleep(SLEEP);
    if (__builtin_amdgcn_s_memrealtime() - t0 > ticks) {
      ok = false;
      break;
    }
  }
  asm volatile("" ::: "memory");
  return ok;
}

// Waits until the n (<= 64) consecutive flags f[0..n) all equal epoch: lane
// i reads flag i, every poll reads them all at once.  Bounded like
// wait_ready; the result is the same in every lane.
template <int SLEEP = 1>
__device__ __forceinline__ bool wait_ready_span(const uint64_t* f, int n, uint64_t epoch, int lane,
                                                uint64_t ticks) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  const bool mine = lane < n;
  bool done = false;
  while (true) {
    const bool ok = !mine || __hip_atomic_load(f + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == epoch;
    if (__all(ok)) {
      done = true;
      break;
    }
    __builtin_amdgcn_s_sleep(SLEEP);
    if (__builtin_amdgcn_s_memrealtime() - t0 > ticks) break;
  }
  asm volatile("" ::: "memory");
  return done;
}

// LDS of swa_tiles: two K blocks (row-major) then two V^T blocks.
template <class T, int D>
struct SwaSmem {
  static constexpr int KB = KeyBlock<T>::n;
  static constexpr int SK = D + 16 / (int)sizeof(T);
  static constexpr int SV = KB + 16 / (int)sizeof(T);
  static constexpr int nK = KB * SK;
  static constexpr int nV = D * SV;
  static constexpr int bytes = (2 * nK + 2 * nV) * (int)sizeof(T);
  // linked tiles of few blocks: every block staged at once, K then V^T per block
  static constexpr int deep_bytes = kDeepBlocks * (nK + nV) * (int)sizeof(T);
  // resident key blocks: three window blocks (a ring) and the sink block
  static constexpr int ring_bytes = 4 * (nK + nV) * (int)sizeof(T);
};

// The query tiles bx * TPW .. of (sequence bi, query heads hgrp * HPW ..
// + HPW - 1) by one workgroup of NW waves (every wave of the workgroup calls
// it: it uses workgroup barriers), staging through `lds` (SwaSmem bytes).
// LINKED: o's rows >= add_from hold the linear branch written by the chunked
// scan running in the same kernel; before reading them a wave waits for the
// done flags of the scan chunks (64 rows from add_from each) that cover its
// rows, nflag flags per (sequence, head, chunk), and reads them at device
// scope.
// RING (not linked; QT = KB, n_sink <= KB, window <= 2 KB + 1; SwaSmem
// ring_bytes of LDS): key blocks are aligned to multiples of KB and stay
// resident while the workgroup walks its consecutive tiles.  A tile's window
// spans at most three such blocks, held in slots (block index mod 3); the
// sink keys sit in a fourth slot staged once.  Each tile stages only the one
// block the next tile adds, into the slot of the block it no longer needs.
template <class T, int D, int NW, bool LINKED, bool RING = false>
__device__ __forceinline__ void swa_tiles(const T* __restrict__ q, const T* __restrict__ k,
                                          const T* __restrict__ v, T* __restrict__ o, int T_, int H,
                                          int Hkv, int HPW, int QT, int TPW, int n_sink, int window,
                                          int add_from, int bx, int hgrp, int bi, T* lds,
                                          const uint64_t* done, uint64_t epoch, int nch, int nflag,
                                          float w_swa, uint64_t wait_ticks = 0) {
  constexpr int KB = KeyBlock<T>::n;
  constexpr int NTH = 64 * NW;
  constexpr int PAD = 16 / sizeof(T);
  constexpr int SK = D + PAD;      // Ks row stride
  constexpr int SV = KB + PAD;     // VTs row stride
  // staging in 16-byte chunks: K row-major, one chunk per task; V as pieces
  // of 4 consecutive keys x one chunk, transposed in registers into runs of
  // 4 keys (contiguous in acc order) of EPC dims
  constexpr int EPC = 16 / sizeof(T);
  constexpr int CH = D / EPC;                      // chunks per row
  constexpr int NPK = KB * CH / NTH;               // K chunks per thread
  constexpr int NVP = (KB / 4) * CH;               // V pieces per block
  constexpr int NPV = (NVP + NTH - 1) / NTH;       // V pieces per thread
  static_assert(KB * CH % NTH == 0 && NPK >= 1, "staging shape");
  static_assert(!(LINKED && RING), "resident blocks are for the unlinked kernel");
  typedef typename Vec16<T>::type V16;
  auto Ks = [&](int buf) { return lds + buf * (KB * SK); };
  auto VTs = [&](int buf) { return lds + 2 * (KB * SK) + buf * (D * SV); };

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
  const int tile0 = bx * TPW;                         // first query tile of this workgroup
  const int ntile = min(TPW, (T_ + QT - 1) / QT - tile0);
  const float scale = kLog2e / sqrtf((float)D);

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
  // RING: tile t0's sink block (if any) and its window blocks blo..bhi
  // (KB-aligned; empty when bhi < blo)
  auto ring_range = [&](int t0, int& nbs, int& blo, int& bhi, int& sink_end, int& t_end) {
    t_end = min(t0 + QT, T_);
    sink_end = min(n_sink, t_end);
    nbs = sink_end > 0 ? 1 : 0;
    const int lo = max(n_sink, t0 - window + 1);
    blo = lo / KB;
    bhi = t_end > lo ? (t_end - 1) / KB : blo - 1;
  };
  // block blk of the workgroup's tile ti -> block description (every tile
  // has at least one block)
  auto block_of = [&](int ti, int blk, Blk& bl) {
    int nbs, nbw, se, wl, te;
    tile_blocks((tile0 + ti) * QT, nbs, nbw, se, wl, te);
    const bool sk = blk < nbs;
    bl.kb0 = sk ? blk * KB : wl + (blk - nbs) * KB;
    bl.kend = sk ? se : te;
    bl.sink = sk;
  };

  // query fragments (B operand of S^T = K Q^T, "linear" set over d) of tile
  // ti: 16-byte loads, then converted and pre-multiplied by log2(e) / sqrt(d)
  // so the scores come out of the MFMA already in exp2 units
  constexpr int QV = 8 / EPC;                      // 16-byte pieces per fragment
  typedef V16 QRaw[QV];
  auto load_q = [&](int ti, QRaw (&qr)[kNQ][D / 32]) {
    const int qb = (tile0 + ti) * QT + (wv % NWQ) * 16 * kNQ;
#pragma unroll
    for (int nq = 0; nq < kNQ; ++nq) {
      const int t = qb + 16 * nq + l16;
#pragma unroll
      for (int p = 0; p < D / 32; ++p) {
#pragma unroll
        for (int u = 0; u < QV; ++u) {
          if (t < T_) {
            qr[nq][p][u] = *reinterpret_cast<const V16*>(q + ((size_t)(bi * T_ + t) * H + h) * D + 32 * p +
                                                         8 * lg + u * EPC);
          } else {
#pragma unroll
            for (int i = 0; i < EPC; ++i) qr[nq][p][u][i] = from_f32<T>(0.f);
          }
        }
      }
    }
  };

  // ---- register prefetch of a key block and its commit to an LDS buffer.
  // Every lane always loads (rows past the block's last key read that key
  // again, so no address leaves the tensor); the rows past it are zeroed at
  // commit.  One unconditional load sequence keeps the prefetch asynchronous:
  // the loads are waited for only when the block is committed.
  typedef V16 PK[NPK];
  typedef V16 PV[NPV][4];
  constexpr int NSET = LINKED ? kDeepBlocks : 1;   // register sets
  PK pks[NSET];
  PV pvs[NSET];
  int nks[NSET];                                   // keys of each prefetched block that exist
  const size_t kvstride = (size_t)Hkv * D;
  auto prefetch = [&](const Blk& bl, PK& pk, PV& pv, int& pf_nkey) {
    const size_t off = ((size_t)(bi * T_ + bl.kb0) * Hkv + g) * D;
    const T* kp = k + off;
    const T* vp = v + off;
    pf_nkey = bl.kend - bl.kb0;
    const int last = pf_nkey - 1;
#pragma unroll
    for (int j = 0; j < NPK; ++j) {
      const int i = tid + j * NTH;
      pk[j] = *reinterpret_cast<const V16*>(kp + min(i / CH, last) * kvstride + (i % CH) * EPC);
    }
#pragma unroll
    for (int j = 0; j < NPV; ++j) {
      const int i = tid + j * NTH;
      if (NVP % NTH == 0 || i < NVP) {
        const int key0 = 4 * (i % (KB / 4));
        const T* src = vp + (i / (KB / 4)) * EPC;
#pragma unroll
        for (int x = 0; x < 4; ++x) pv[j][x] = *reinterpret_cast<const V16*>(src + min(key0 + x, last) * kvstride);
      }
    }
  };
  auto commit = [&](T* Kd, T* Vd, const PK& pk, const PV& pv, int pf_nkey) {
    const bool whole = pf_nkey >= KB;              // uniform
    V16 z;
#pragma unroll
    for (int x = 0; x < EPC; ++x) z[x] = from_f32<T>(0.f);
#pragma unroll
    for (int j = 0; j < NPK; ++j) {
      const int i = tid + j * NTH;
      *reinterpret_cast<V16*>(&Kd[(i / CH) * SK + (i % CH) * EPC]) = whole || i / CH < pf_nkey ? pk[j] : z;
    }
#pragma unroll
    for (int j = 0; j < NPV; ++j) {
      const int i = tid + j * NTH;
      if (NVP % NTH == 0 || i < NVP) {
        const int key0 = 4 * (i % (KB / 4));
        V16 pvv[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) pvv[x] = whole || key0 + x < pf_nkey ? pv[j][x] : z;
        T* col = &Vd[(i / (KB / 4)) * EPC * SV + acc_pos(key0)];
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          if constexpr (sizeof(T) == 2) {
            *reinterpret_cast<bf16x4*>(col + e * SV) = bf16x4{pvv[0][e], pvv[1][e], pvv[2][e], pvv[3][e]};
          } else {
            *reinterpret_cast<f32x4*>(col + e * SV) = f32x4{pvv[0][e], pvv[1][e], pvv[2][e], pvv[3][e]};
          }
        }
      }
    }
  };

  Frag<T> ones;
  {
    float x1[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
    ones = frag_from8<T>(x1);
  }
  // Deep staging (linked, one tile of at most kDeepBlocks blocks): the
  // loads of every block and of the queries are issued together, then every
  // block is committed to its own LDS area.  Otherwise blocks go through two
  // LDS buffers, the next one prefetched into registers while the current
  // one is used.
  auto DKs = [&](int blk) { return lds + blk * (KB * SK + D * SV); };
  auto DVTs = [&](int blk) { return DKs(blk) + KB * SK; };
  bool deep = false;
  QRaw qraw[kNQ][D / 32];
  if constexpr (LINKED) {
    if (ntile == 1) {
      int nbs, nbw, se, wl, te;
      tile_blocks(tile0 * QT, nbs, nbw, se, wl, te);
      const int nblk = nbs + nbw;
      if (nblk <= kDeepBlocks) {
        deep = true;
#pragma unroll
        for (int b2 = 0; b2 < kDeepBlocks; ++b2)
          if (b2 < nblk) {
            Blk bl;
            block_of(0, b2, bl);
            prefetch(bl, pks[b2], pvs[b2], nks[b2]);
          }
        load_q(0, qraw);
#pragma unroll
        for (int b2 = 0; b2 < kDeepBlocks; ++b2)
          if (b2 < nblk) commit(DKs(b2), DVTs(b2), pks[b2], pvs[b2], nks[b2]);
      }
    }
  }
  int flat = 0;   // running block counter (selects the LDS buffer)
  if constexpr (RING) {
    // the first tile's blocks: the sinks into slot 3, window block b into
    // slot b mod 3 (each staged whole, up to the sequence end)
    if (ntile > 0) {
      int nbs0, blo0, bhi0, se0, te0;
      ring_range(tile0 * QT, nbs0, blo0, bhi0, se0, te0);
      if (nbs0) {
        const Blk bl{0, min(n_sink, T_), 1};
        prefetch(bl, pks[0], pvs[0], nks[0]);
        commit(DKs(3), DVTs(3), pks[0], pvs[0], nks[0]);
      }
      for (int b2 = blo0; b2 <= bhi0; ++b2) {
        const Blk bl{b2 * KB, min(b2 * KB + KB, T_), 0};
        prefetch(bl, pks[0], pvs[0], nks[0]);
        commit(DKs(b2 % 3), DVTs(b2 % 3), pks[0], pvs[0], nks[0]);
      }
    }
  } else if (!deep && ntile > 0) {
    Blk b0;
    block_of(0, 0, b0);
    prefetch(b0, pks[0], pvs[0], nks[0]);
    commit(Ks(0), VTs(0), pks[0], pvs[0], nks[0]);
  }
  lds_barrier();

  for (int ti = 0; ti < ntile; ++ti) {
    const int t0 = (tile0 + ti) * QT;
    const int qb = t0 + (wv % NWQ) * 16 * kNQ;      // first query row of this wave
    const int qlast = qb + 16 * kNQ - 1;
    int nbs, nbw, sink_end, win_lo, t_end;
    int blo = 0, nb = 0;            // RING: first window block; block staged for the next tile
    bool newblk = false;
    if constexpr (RING) {
      int bhi;
      ring_range(t0, nbs, blo, bhi, sink_end, t_end);
      nbw = bhi - blo + 1;
      win_lo = 0;
      if (ti + 1 < ntile) {
        int nbs2, blo2, bhi2, se2, te2;
        ring_range(t0 + QT, nbs2, blo2, bhi2, se2, te2);
        nb = bhi2;
        newblk = bhi2 > bhi;
        if (newblk) {
          const Blk bl{nb * KB, min(nb * KB + KB, T_), 0};
          prefetch(bl, pks[0], pvs[0], nks[0]);
        }
      }
    } else {
      tile_blocks(t0, nbs, nbw, sink_end, win_lo, t_end);
    }
    const int nblk = nbs + nbw;

    if (!deep) load_q(ti, qraw);
    Frag<T> qf[kNQ][D / 32];
#pragma unroll
    for (int nq = 0; nq < kNQ; ++nq)
#pragma unroll
      for (int p = 0; p < D / 32; ++p) {
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = to_f32(qraw[nq][p][i / EPC][i % EPC]) * scale;
        qf[nq][p] = frag_from8<T>(x);
      }


    f32x4 oacc[D / 16][kNQ];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
      for (int nq = 0; nq < kNQ; ++nq) oacc[dt][nq] = zero4();
    // running max (reference) per query and the row sums, the latter as an
    // MFMA accumulator: a 16-row "ones" tile times P^T gives sum_k p in every
    // row, so l is summed from the same rounded p that multiply V
    float mrun[kNQ];
    f32x4 lacc[kNQ];
#pragma unroll
    for (int nq = 0; nq < kNQ; ++nq) {
      mrun[nq] = -INFINITY;
      lacc[nq] = zero4();
    }

    for (int blk = 0; blk < nblk; ++blk, ++flat) {
      const int buf = flat & 1;
      const bool sinkph = blk < nbs;
      const int kb0 = RING ? (sinkph ? 0 : (blo + blk - nbs) * KB)
                           : (sinkph ? blk * KB : win_lo + (blk - nbs) * KB);
      const int kend = sinkph ? sink_end : t_end;
      const bool last = blk + 1 == nblk;
      const bool has_next = !last || ti + 1 < ntile;
      if (!RING && !deep && has_next) {
        Blk nx;
        block_of(last ? ti + 1 : ti, last ? 0 : blk + 1, nx);
        prefetch(nx, pks[0], pvs[0], nks[0]);
      }
      const int slot = sinkph ? 3 : (blo + blk - nbs) % 3;   // RING
      const T* Kb = RING ? DKs(slot) : deep ? DKs(blk) : Ks(buf);
      const T* Vb = RING ? DVTs(slot) : deep ? DVTs(blk) : VTs(buf);

      // ---- S^T tiles for this wave, computed relative to the running max:
      // the accumulators start at -mbase, so the MFMAs return s - mbase
      // (tiles no query of the wave sees are skipped; which ones is a scalar
      // bit mask)
      int onmask = 0;
#pragma unroll
      for (int kt = 0; kt < KB / 16; ++kt) {
        const int k0 = kb0 + 16 * kt;
        bool on = k0 < kend && k0 <= qlast && qb < T_;
        if (!sinkph) on = on && (k0 + 15 > qb - window) && (!RING || k0 + 15 >= n_sink);
        onmask |= on ? 1 << kt : 0;
      }
      onmask = __builtin_amdgcn_readfirstlane(onmask);
      float mbase[kNQ];
      f32x4 negm[kNQ];
#pragma unroll
      for (int nq = 0; nq < kNQ; ++nq) {
        mbase[nq] = mrun[nq] == -INFINITY ? 0.f : mrun[nq];
        negm[nq] = f32x4{-mbase[nq], -mbase[nq], -mbase[nq], -mbase[nq]};
      }
      f32x4 sacc[KB / 16][kNQ];
#pragma unroll
      for (int kt = 0; kt < KB / 16; ++kt) {
#pragma unroll
        for (int nq = 0; nq < kNQ; ++nq) sacc[kt][nq] = negm[nq];
        if ((onmask >> kt) & 1) {
          Frag<T> af[D / 32];
#pragma unroll
          for (int p = 0; p < D / 32; ++p) af[p] = lds_frag8(&Kb[(16 * kt + l16) * SK + 32 * p + 8 * lg]);
#pragma unroll
          for (int p = 0; p < D / 32; ++p)
#pragma unroll
            for (int nq = 0; nq < kNQ; ++nq) sacc[kt][nq] = mfma(af[p], qf[nq][p], sacc[kt][nq]);
        }
      }

      // ---- mask and block max per query (per lane; 4 lane groups share a
      // query).  A tile whose keys are all visible to all its queries skips
      // the per-element mask.  Window phase: a key is visible iff
      // 0 <= t - key < window (a key past the tile end is later than every
      // real query of it); sink phase: iff key <= t and key < kend.
      float mloc[kNQ];
      auto mask_and_max = [&](auto sink_tag) {
        constexpr bool SINK = decltype(sink_tag)::value;
#pragma unroll
        for (int nq = 0; nq < kNQ; ++nq) {
          const int q0 = qb + 16 * nq;
          const int t = q0 + l16;
          float m = -INFINITY;
#pragma unroll
          for (int kt = 0; kt < KB / 16; ++kt) {
            if (!((onmask >> kt) & 1)) continue;
            const int k0 = kb0 + 16 * kt;
            // (RING window blocks may start below n_sink: those keys belong
            // to the sink phase)
            const bool full = SINK ? (k0 + 15 <= q0 && k0 + 15 < kend)
                                   : (k0 + 15 <= q0 && k0 > q0 + 15 - window && (!RING || k0 >= n_sink));
            if (!full) {
              const int key0 = k0 + 4 * lg;
              const int d0 = t - key0;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const bool valid = SINK ? ((d0 - i >= 0) & (key0 + i < kend))
                                        : ((unsigned)(d0 - i) < (unsigned)window) & (!RING || key0 + i >= n_sink);
                sacc[kt][nq][i] = valid ? sacc[kt][nq][i] : -INFINITY;
              }
            }
            m = max3f(m, max3f(sacc[kt][nq][0], sacc[kt][nq][1], sacc[kt][nq][2]), sacc[kt][nq][3]);
          }
          mloc[nq] = m;
        }
      };
      if (sinkph) mask_and_max(std::true_type{});
      else mask_and_max(std::false_type{});

      // ---- lazy rescale: the running max only moves (and O is rescaled)
      // when the block raises it by more than 8 in log2 units, which keeps
      // every exponent <= 2^8 while sparing most rescales.  Scores are held
      // relative to mbase (the running max, or 0 before any key); a move
      // shifts them to the new reference.
#pragma unroll
      for (int nq = 0; nq < kNQ; ++nq) {
        const float mblk = mbase[nq] + max_lane_groups(mloc[nq]);
        const float mref = mrun[nq];
        if (__any(mblk > mref + 8.f)) {   // some query of the wave needs a new reference
          const float mnew = fmaxf(mref, mblk);
          const float alpha = mnew == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(mref - mnew);
          lacc[nq] *= alpha;
#pragma unroll
          for (int dt = 0; dt < D / 16; ++dt) oacc[dt][nq] *= alpha;
          mrun[nq] = mnew;
          // a lane that has seen no key yet keeps reference 0: its scores
          // are all -inf and give p = 0 whatever the shift
          const float shift = (mnew == -INFINITY ? 0.f : mnew) - mbase[nq];
#pragma unroll
          for (int kt = 0; kt < KB / 16; ++kt) sacc[kt][nq] -= shift;
        }
      }

      // ---- p = exp2(s - m), row sums, O^T += V^T P^T, 32 keys at a time
#pragma unroll
      for (int pp = 0; pp < KB / 32; ++pp) {
        const bool on0 = (onmask >> (2 * pp)) & 1;
        const bool on1 = (onmask >> (2 * pp + 1)) & 1;
        if (!(on0 || on1)) continue;
        Frag<T> pf[kNQ];
#pragma unroll
        for (int nq = 0; nq < kNQ; ++nq) {
          f32x4 p0 = zero4(), p1 = zero4();
          if (on0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) p0[i] = __builtin_amdgcn_exp2f(sacc[2 * pp][nq][i]);
          }
          if (on1) {
#pragma unroll
            for (int i = 0; i < 4; ++i) p1[i] = __builtin_amdgcn_exp2f(sacc[2 * pp + 1][nq][i]);
          }
          pf[nq] = frag_from_acc<T>(p0, p1);
          lacc[nq] = mfma(ones, pf[nq], lacc[nq]);
        }
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

      if (!deep && !RING) {
        if (has_next) commit(Ks(buf ^ 1), VTs(buf ^ 1), pks[0], pvs[0], nks[0]);
        lds_barrier();
      }
    }

    // ---- epilogue of this query tile
    bool linked_ok = true;   // LINKED: the scan published every row this wave adds onto
    if constexpr (LINKED) {
      // the done flags of the scan chunks covering this wave's rows are
      // consecutive: one flag per lane, polled together
      const int r_lo = max(qb, add_from);
      const int r_hi = min(qlast, T_ - 1);
      if (r_lo <= r_hi) {
        const int c_lo = (r_lo - add_from) / 64;
        const int nf = ((r_hi - add_from) / 64 - c_lo + 1) * nflag;
        const uint64_t* f0 = done + ((size_t)(bi * H + h) * nch + c_lo) * nflag;
        for (int s0 = 0; s0 < nf && linked_ok; s0 += 64)
          linked_ok = wait_ready_span<32>(f0 + s0, min(64, nf - s0), epoch, lane, wait_ticks);
      }
    }
    // what o holds on rows >= add_from, read before any row is written: every
    // load is issued unconditionally (rows past the sequence read its last
    // row) and the values are selected afterwards, so the loads overlap
    typedef typename std::conditional<sizeof(T) == 2, bf16x4, f32x4>::type Raw4;
    Raw4 raw[kNQ][D / 16];
#pragma unroll
    for (int nq = 0; nq < kNQ; ++nq) {
      const int tr = min(qb + 16 * nq + l16, T_ - 1);
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        const int d0 = 16 * dt + 4 * lg;
        if constexpr (LINKED) {
          // wave-uniform base, device-scope read of the scan's output
          static_assert(sizeof(T) == 2, "linked tiles are bf16");
          typedef unsigned int u2 __attribute__((ext_vector_type(2)));
          const T* obase = o + ((size_t)(bi * T_ + qb) * H + h) * D;
          raw[nq][dt] = __builtin_bit_cast(
              Raw4, __builtin_amdgcn_raw_buffer_load_b64(
                        __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(obase), 0, 0x7fffffff, 0x00020000),
                        ((tr - qb) * H * D + d0) * 2, 0, 16));
        } else {
          raw[nq][dt] = *reinterpret_cast<const Raw4*>(o + ((size_t)(bi * T_ + tr) * H + h) * D + d0);
        }
      }
    }
#pragma unroll
    for (int nq = 0; nq < kNQ; ++nq) {
      const float l = lacc[nq][0];
      const int t = qb + 16 * nq + l16;
      if (t >= T_) continue;
      const float inv = w_swa / l;
      T* orow = o + ((size_t)(bi * T_ + t) * H + h) * D;
      const bool addl = t >= add_from;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        f32x4 val = oacc[dt][nq] * inv;
        if (addl) val += f32x4{static_cast<float>(raw[nq][dt][0]), static_cast<float>(raw[nq][dt][1]),
                               static_cast<float>(raw[nq][dt][2]), static_cast<float>(raw[nq][dt][3])};
        // a row whose linear part was never published is poisoned, not guessed
        if (LINKED && addl && !linked_ok) val = f32x4{__builtin_nanf(""), __builtin_nanf(""),
                                                      __builtin_nanf(""), __builtin_nanf("")};
        store4(orow + 16 * dt + 4 * lg, val);
      }
    }
    if constexpr (RING) {
      // the next tile's new block replaces the one only this tile needed
      if (newblk) {
        lds_barrier();
        commit(DKs(nb % 3), DVTs(nb % 3), pks[0], pvs[0], nks[0]);
        lds_barrier();
      }
    }
  }
}

}  // namespace swa
}  // namespace gdn
