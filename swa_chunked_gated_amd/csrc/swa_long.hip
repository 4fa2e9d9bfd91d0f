// Softmax branch of the hybrid layer for long budgets (bf16, d = 128):
// sinks + a sliding window of hundreds of tokens, on gfx950.
//
// Method (page "The Key to Going Linear: Analysis-Driven Transformer
// Linearization", section 填补近似缺口的实用设计; budget 896 in section 实验):
// query t attends with softmax to A(t) = { i <= t : i < n_sink or
// i > t - window } with logits q.k / sqrt(d) (section 从 softmax 到 delta
// 规则的一阶近似, Lemma 1).  The arithmetic is that of the general tile
// routine (swa_tile.h): S^T = K Q^T per 16-key tile with q pre-scaled by
// log2(e) / sqrt(d), an online softmax in the exp2 domain with lazy rescaling,
// row sums on the matrix cores against a ones operand, O^T += V^T P^T, and
// o = w_swa O / l plus what o holds on rows t >= add_from.
//
// What changes for long budgets is the movement of K and V.  A query tile
// walks 15-16 blocks of 64 keys at budget 896, so staging cost and latency
// are paid on every block.  Here blocks reach LDS by direct loads
// (global_load_lds, no registers, no conversion work), three blocks ahead,
// into a ring of four slots, and V is read back transposed by the gfx950
// transposing LDS reads; a block step is one wait, one barrier and the
// block's direct loads, then only MFMAs, the softmax arithmetic and LDS
// reads.
//
// Work split: one 8-wave workgroup per (sequence, HPW query heads of one KV
// head, run of consecutive query tiles); wave w owns 32 query rows of head
// h0 + w / NSUB (NSUB = 8 / HPW row groups per tile, QT = 32 NSUB rows).
// Every K/V block staged serves all eight waves.  Runs of one head group
// follow each other on one XCD, so the blocks that consecutive tiles share
// are met again in that XCD's L2.

#include <algorithm>
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "swa_tile.h"

namespace gdn {
namespace {

constexpr int lD = 128;                          // head dimension
constexpr int lKB = 64;                          // keys per block
constexpr int lS = 144;                          // LDS row stride (elements): 288 bytes
constexpr int lTile = lKB * lS * 2;              // bytes of one K or V block
constexpr int lSlot = 2 * lTile;                 // K then V
constexpr int lPieces = lTile / 1024;            // 1 KB direct loads per K or V block
constexpr int lTPW = 8;                          // most query tiles per workgroup
static_assert(lTile % 1024 == 0, "whole 1 KB direct loads");
// W waves per workgroup, a ring of NS slots (NS - 1 blocks ahead)
template <int W, int NS>
struct LongCfg {
  static constexpr int dma = (2 * lPieces + W - 1) / W;   // direct loads per wave and block
  static constexpr int lds = NS * lSlot;
  static_assert(lds <= 160 * 1024, "LDS of one workgroup");
};

// One direct load: 16 bytes per lane from sbase + voff (a wave-uniform base
// in SGPRs, a 32-bit lane offset) into LDS at lds + 16 lane (1 KB per wave).
// Written as asm so that the compiler, which cannot tell which LDS bytes it
// writes, does not wait for it before LDS reads; the kernel waits itself
// (vmcnt) before the barrier that hands a slot to its readers.  It has no
// register result; m0 holds the wave-uniform LDS address.
__device__ __forceinline__ void dma_lds16(const void* sbase, unsigned voff, const void* lds) {
  const unsigned la = __builtin_amdgcn_readfirstlane(
      (unsigned)(size_t)(const __attribute__((address_space(3))) void*)lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(la), "v"(voff), "s"(sbase)
               : "memory", "m0");
}

// s_waitcnt vmcnt(n) (n < 64: bits 3:0 and 15:14), leaving the other
// counters alone
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
  asm volatile("" ::: "memory");
}

typedef __attribute__((address_space(3))) bf16x4* lds4_ptr;

// max of two scores in one instruction (scores are never NaN, so the
// NaN-quieting that fmaxf needs in IEEE mode is left out)
__device__ __forceinline__ float max2(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
// max over lanes l, l^16, l^32, l^48 (the four lane groups holding one
// query's scores) with the row-swap permutes
__device__ __forceinline__ float max_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = max2(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max2(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// ADD: some rows add what o holds (rows t >= add_from < T); without it the
// kernel keeps no registers for them.
template <int W, int NS, int HPW, bool ADD>
__global__ __launch_bounds__(64 * W, 8 / W) void swa_long_kernel(const bf16* __restrict__ q,
                                                              const bf16* __restrict__ k,
                                                              const bf16* __restrict__ v, bf16* __restrict__ o,
                                                              int T_, int H, int Hkv, int n_sink, int window,
                                                              int add_from, float w_swa, int tpw, int nruns,
                                                              int units) {
  constexpr int NSUB = W / HPW;
  constexpr int lWaves = W;
  constexpr int lSlots = NS;
  constexpr int lDmaPerWave = LongCfg<W, NS>::dma;
  constexpr int QT = 32 * NSUB;
  constexpr int kNQ = 2;                         // 16-query tiles per wave
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];

  const int groups = H / HPW;
  int unit, run;
  if (!xcd_grouped(blockIdx.x, nruns, units, unit, run)) return;
  const int bi = unit / groups;
  const int h0 = (unit % groups) * HPW;
  const int gk = h0 / (H / Hkv);
  const int ntiles_seq = (T_ + QT - 1) / QT;
  const int tile0 = run * tpw;
  const int ntile = min(tpw, ntiles_seq - tile0);
  if (ntile <= 0) return;                        // whole workgroup

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = wave_id();
  const int g = lane >> 4;
  const int j = lane & 15;
  const int h = h0 + wv / NSUB;
  const int sub = wv % NSUB;
  const size_t kvrow = (size_t)Hkv * lD;
  const bf16* kb = k + ((size_t)bi * T_ * Hkv + gk) * lD;
  const bf16* vb = v + ((size_t)bi * T_ * Hkv + gk) * lD;
  const float scale = kLog2e / sqrtf((float)lD);

  // Key blocks of the tile at t0: the sinks [0, sink_end) in blocks of 64,
  // then the window [win_lo, t_end).  Block b -> first key, keys present,
  // and whether it is a sink block.
  auto nblocks = [&](int t0) {
    const int t_end = min(t0 + QT, T_);
    const int sink_end = min(n_sink, t_end);
    const int win_lo = max(n_sink, t0 - window + 1);
    const int nbs = (sink_end + lKB - 1) / lKB;
    const int nbw = t_end > win_lo ? (t_end - win_lo + lKB - 1) / lKB : 0;
    return nbs + nbw;
  };
  auto block_of = [&](int t0, int b, int& kb0, int& kend, bool& sink) {
    const int t_end = min(t0 + QT, T_);
    const int sink_end = min(n_sink, t_end);
    const int win_lo = max(n_sink, t0 - window + 1);
    const int nbs = (sink_end + lKB - 1) / lKB;
    sink = b < nbs;
    kb0 = sink ? b * lKB : win_lo + (b - nbs) * lKB;
    kend = sink ? min(kb0 + lKB, sink_end) : min(kb0 + lKB, t_end);
  };

  // this wave's direct loads of a block into slot sl: pieces wv + 8 m of the
  // 36 (K pieces 0..17, then V); a lane whose 16 bytes fall in a row's
  // padding, and rows past the block's last key, load that row's first
  // piece or the last key's row again (never used: padding is not read and
  // keys past the block are masked and meet p = 0).  Lane offsets of a whole
  // block are fixed; a partial block clamps the rows.
  // Per piece m of this wave: its source (K or V of the KV head), its LDS
  // offset in a slot and its lane's byte offset from the block's first row
  // (a block's rows start kb0 * kvrow elements in; sequences of at most
  // 2 GiB of K per batch row keep every offset in 32 bits).
  // piece m of this wave: the row (bits 0-7) and byte column (bits 8-17)
  // of the lane's 16 bytes; padding lanes load the row's first piece again
  int pinfo[lDmaPerWave];
#pragma unroll
  for (int m = 0; m < lDmaPerWave; ++m) {
    const int i = min(wv + lWaves * m, 2 * lPieces - 1);
    const int n = i >= lPieces ? i - lPieces : i;
    const int off = 1024 * n + 16 * lane;
    const int pc = (off % (lS * 2)) >> 4;
    pinfo[m] = off / (lS * 2) | (pc < lD / 8 ? 16 * pc : 0) << 8;
  }
  // (wave-uniform) source and LDS offset of piece m
  auto psrc = [&](int m) { return min(wv + lWaves * m, 2 * lPieces - 1) >= lPieces ? vb : kb; };
  auto plds = [&](int m) {
    const int i = min(wv + lWaves * m, 2 * lPieces - 1);
    return i >= lPieces ? lTile + 1024 * (i - lPieces) : 1024 * i;
  };
  // a block's rows start kb0 * kvrow elements in (K or V of one batch row
  // within 2 GiB keeps the offsets in 32 bits); rows past the block's last
  // key load that key's row again
  auto issue = [&](int kb0, int nkey, int sl) {
    const unsigned char* base = smem_raw + sl * lSlot;
    const unsigned boff = (unsigned)kb0 * (unsigned)kvrow * 2u;
#pragma unroll
    for (int m = 0; m < lDmaPerWave; ++m) {
      const int row = min(pinfo[m] & 0xFF, nkey - 1);
      dma_lds16(psrc(m), boff + (unsigned)(row * (int)kvrow * 2 + (pinfo[m] >> 8)), base + plds(m));
    }
  };

  // issue cursor over the flat sequence of (tile, block) of this workgroup
  int c_ti = 0, c_b = 0, c_nb = nblocks(tile0 * QT), c_flat = 0;
  int nflat = 0;
  for (int ti = 0; ti < ntile; ++ti) nflat += nblocks((tile0 + ti) * QT);
  auto issue_next = [&]() {
    if (c_flat >= nflat) return;
    int kb0, kend;
    bool sk;
    block_of((tile0 + c_ti) * QT, c_b, kb0, kend, sk);
    issue(kb0, kend - kb0, c_flat % lSlots);
    ++c_flat;
    if (++c_b == c_nb) {
      c_b = 0;
      ++c_ti;
      if (c_ti < ntile) c_nb = nblocks((tile0 + c_ti) * QT);
    }
  };

  // query fragments of tile ti (B operand of S^T = K Q^T, "linear" set over
  // d), pre-multiplied by log2(e) / sqrt(d); rows past the sequence read its
  // last row and are zeroed
  typedef bf16x8 QRaw[kNQ][lD / 32];
  auto load_q = [&](int ti, QRaw& qr) {
    const int qb = (tile0 + ti) * QT + 32 * sub;
#pragma unroll
    for (int nq = 0; nq < kNQ; ++nq) {
      const int t = min(qb + 16 * nq + j, T_ - 1);
      const bf16* src = q + ((size_t)(bi * T_ + t) * H + h) * lD + 8 * g;
#pragma unroll
      for (int p = 0; p < lD / 32; ++p) qr[nq][p] = *reinterpret_cast<const bf16x8*>(src + 32 * p);
    }
  };
  Frag<bf16> qf[kNQ][lD / 32];
  auto set_q = [&](int ti, const QRaw& qr) {
    const int qb = (tile0 + ti) * QT + 32 * sub;
#pragma unroll
    for (int nq = 0; nq < kNQ; ++nq) {
      const bool in = qb + 16 * nq + j < T_;
#pragma unroll
      for (int p = 0; p < lD / 32; ++p) {
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = in ? static_cast<float>(qr[nq][p][i]) * scale : 0.f;
        qf[nq][p] = frag_from8<bf16>(x);
      }
    }
  };

  Frag<bf16> ones;
  {
    float x1[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
    ones = frag_from8<bf16>(x1);
  }

  {
    QRaw qr;
    load_q(0, qr);
    set_q(0, qr);
  }
#pragma unroll
  for (int i = 0; i < lSlots - 1; ++i) issue_next();

  // lane parts of the LDS read addresses (elements): K rows j (16-byte
  // reads at d 32 p + 8 g), V rows 4 g + j / 4 (transposing reads of the
  // d columns 16 dt + 4 (j % 4) ..)
  const int kofs = j * lS + 8 * g;
  const int vofs = (4 * g + (j >> 2)) * lS + 4 * (j & 3);

  int flat = 0;
  for (int ti = 0; ti < ntile; ++ti) {
    const int t0 = (tile0 + ti) * QT;
    const int qb = t0 + 32 * sub;                 // first query row of this wave
    const int qlast = qb + 32 - 1;
    const int nblk = nblocks(t0);

    f32x4 oacc[lD / 16][kNQ];
#pragma unroll
    for (int dt = 0; dt < lD / 16; ++dt)
#pragma unroll
      for (int nq = 0; nq < kNQ; ++nq) oacc[dt][nq] = zero4();
    float mrun[kNQ];
    f32x4 lacc[kNQ];
#pragma unroll
    for (int nq = 0; nq < kNQ; ++nq) {
      mrun[nq] = -INFINITY;
      lacc[nq] = zero4();
    }
    typedef bf16x4 ORaw[kNQ][lD / 16];
    ORaw oraw;
    const bool addl = ADD && qlast >= add_from && qb < T_;   // some row of the wave adds what o holds

    for (int b = 0; b < nblk; ++b, ++flat) {
      // block flat has landed once at most the blocks issued after it are
      // outstanding (loads complete in order)
      const int newer = c_flat - 1 - flat;
      static_assert(NS == 2 || NS == 4, "ring of two or four slots");
      if (NS == 4 && newer >= 2) wait_vm<(NS - 2) * lDmaPerWave>();
      else if (NS == 4 && newer == 1) wait_vm<lDmaPerWave>();
      else wait_vm<0>();
      lds_barrier();                               // every wave's part is in; slot flat - 1 is free
      issue_next();
      const bool last = b + 1 == nblk;

      int kb0, kend;
      bool sinkph;
      block_of(t0, b, kb0, kend, sinkph);
      const bf16* Kb = reinterpret_cast<const bf16*>(smem_raw + (flat % lSlots) * lSlot);
      const bf16* Vb = Kb + lTile / 2;
      QRaw qnext;
      const bool more = last && ti + 1 < ntile;

      // Tiles of 16 keys that no query of the wave sees are skipped (a
      // scalar bit mask); their scores are -inf.  A block whose keys every
      // query of the wave sees (the bulk of a long budget: kb0 + 63 <= qb,
      // causal for the first query, and kb0 > qlast - window, in the last
      // query's window) needs no mask; otherwise the mask is applied per
      // element in tiles that some query sees partly.
      const bool interior = !sinkph && kend - kb0 == lKB && kb0 + lKB - 1 <= qb && kb0 > qlast - window;
      int onmask = 0xF;
      if (!interior) {
        onmask = 0;
#pragma unroll
        for (int kt = 0; kt < lKB / 16; ++kt) {
          const int k0 = kb0 + 16 * kt;
          bool on = k0 < kend && k0 <= qlast && qb < T_;
          if (!sinkph) on = on && k0 + 15 > qb - window;
          onmask |= on ? 1 << kt : 0;
        }
        onmask = __builtin_amdgcn_readfirstlane(onmask);
      }
      // accumulators start at -mbase (the MFMAs return s - mbase) or, for
      // keys a query does not see, at -inf (so they stay -inf)
      // (window: 0 <= t - key < window; sinks: key <= t and key < kend)
      float mbase[kNQ];
      f32x4 sacc[lKB / 16][kNQ];
#pragma unroll
      for (int nq = 0; nq < kNQ; ++nq) mbase[nq] = mrun[nq] == -INFINITY ? 0.f : mrun[nq];
#pragma unroll
      for (int kt = 0; kt < lKB / 16; ++kt)
#pragma unroll
        for (int nq = 0; nq < kNQ; ++nq) sacc[kt][nq] = f32x4{-mbase[nq], -mbase[nq], -mbase[nq], -mbase[nq]};
      if (!interior) {
        const int jg = j - 4 * g;                  // t - key = (q0 - k0) + jg - i
#pragma unroll
        for (int kt = 0; kt < lKB / 16; ++kt) {
          const int k0 = kb0 + 16 * kt;
          const bool on = (onmask >> kt) & 1;
#pragma unroll
          for (int nq = 0; nq < kNQ; ++nq) {
            const int q0 = qb + 16 * nq;
            const int d0 = q0 - k0 + jg;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const bool valid = on && (sinkph ? ((d0 - i >= 0) & (k0 + 4 * g + i < kend))
                                               : ((unsigned)(d0 - i) < (unsigned)window));
              sacc[kt][nq][i] = valid ? sacc[kt][nq][i] : -INFINITY;
            }
          }
        }
      }
      // the next tile's K fragments are read before this tile's MFMAs (a
      // skipped tile's are read too: in bounds, and the reads overlap); with
      // the registers the rows of o take (ADD), one tile at a time
      if constexpr (ADD) {
#pragma unroll
        for (int kt = 0; kt < lKB / 16; ++kt) {
          if ((onmask >> kt) & 1) {
            Frag<bf16> af[lD / 32];
#pragma unroll
            for (int p = 0; p < lD / 32; ++p) af[p] = lds_frag8(Kb + kofs + 16 * kt * lS + 32 * p);
#pragma unroll
            for (int p = 0; p < lD / 32; ++p)
#pragma unroll
              for (int nq = 0; nq < kNQ; ++nq) sacc[kt][nq] = mfma(af[p], qf[nq][p], sacc[kt][nq]);
          }
        }
      } else {
      Frag<bf16> afc[lD / 32], afn[lD / 32];
#pragma unroll
      for (int p = 0; p < lD / 32; ++p) afc[p] = lds_frag8(Kb + kofs + 32 * p);
#pragma unroll
      for (int kt = 0; kt < lKB / 16; ++kt) {
        if (kt + 1 < lKB / 16) {
#pragma unroll
          for (int p = 0; p < lD / 32; ++p) afn[p] = lds_frag8(Kb + kofs + 16 * (kt + 1) * lS + 32 * p);
        }
        __builtin_amdgcn_sched_barrier(0);
        if ((onmask >> kt) & 1) {
#pragma unroll
          for (int p = 0; p < lD / 32; ++p)
#pragma unroll
            for (int nq = 0; nq < kNQ; ++nq) sacc[kt][nq] = mfma(afc[p], qf[nq][p], sacc[kt][nq]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (kt + 1 < lKB / 16) {
#pragma unroll
          for (int p = 0; p < lD / 32; ++p) afc[p] = afn[p];
        }
      }
      }

      // the tile's last block: the next tile's queries (into the registers
      // of the fragments just used) and the rows of o to add onto, loaded
      // now so that they arrive during the rest of the block
      if (more) load_q(ti + 1, qnext);
      if (ADD && last && addl) {
#pragma unroll
        for (int nq = 0; nq < kNQ; ++nq) {
          const int tr = min(qb + 16 * nq + j, T_ - 1);
#pragma unroll
          for (int dt = 0; dt < lD / 16; ++dt)
            oraw[nq][dt] =
                *reinterpret_cast<const bf16x4*>(o + ((size_t)(bi * T_ + tr) * H + h) * lD + 16 * dt + 4 * g);
        }
      }

      // ---- block max per query (4 lane groups share a query; skipped tiles
      // hold -inf), then the lazy rescale: the reference moves only when a
      // block raises the max by more than 8 (log2 units), keeping every
      // exponent <= 2^8
      float mblk[kNQ];
#pragma unroll
      for (int nq = 0; nq < kNQ; ++nq) {
        float m = swa::max3f(sacc[0][nq][0], sacc[0][nq][1], sacc[0][nq][2]);
        m = swa::max3f(m, sacc[0][nq][3], sacc[1][nq][0]);
        m = swa::max3f(m, sacc[1][nq][1], sacc[1][nq][2]);
        m = swa::max3f(m, sacc[1][nq][3], sacc[2][nq][0]);
        m = swa::max3f(m, sacc[2][nq][1], sacc[2][nq][2]);
        m = swa::max3f(m, sacc[2][nq][3], sacc[3][nq][0]);
        m = swa::max3f(m, sacc[3][nq][1], sacc[3][nq][2]);
        m = max2(m, sacc[3][nq][3]);
        mblk[nq] = mbase[nq] + max_groups(m);
      }
      if (__builtin_expect(__any(mblk[0] > mrun[0] + 8.f || mblk[1] > mrun[1] + 8.f), 0)) {
        asm volatile("" ::: "memory");             // rare: keep it a branch, not predicated code
#pragma unroll
        for (int nq = 0; nq < kNQ; ++nq) {
          const float mref = mrun[nq];
          const float mnew = fmaxf(mref, mblk[nq]);
          const float alpha = mnew == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(mref - mnew);
          lacc[nq] *= alpha;
#pragma unroll
          for (int dt = 0; dt < lD / 16; ++dt) oacc[dt][nq] *= alpha;
          mrun[nq] = mnew;
          const float shift = (mnew == -INFINITY ? 0.f : mnew) - mbase[nq];
#pragma unroll
          for (int kt = 0; kt < lKB / 16; ++kt) sacc[kt][nq] -= shift;
        }
      }

      // ---- p = exp2(s - m) (0 for -inf), row sums, O^T += V^T P^T, 32 keys
      // at a time (pairs of tiles no query sees are skipped)
#pragma unroll
      for (int pp = 0; pp < lKB / 32; ++pp) {
        if (!((onmask >> (2 * pp)) & 3)) continue;
        Frag<bf16> pf[kNQ];
#pragma unroll
        for (int nq = 0; nq < kNQ; ++nq) {
          f32x4 p0, p1;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            p0[i] = __builtin_amdgcn_exp2f(sacc[2 * pp][nq][i]);
            p1[i] = __builtin_amdgcn_exp2f(sacc[2 * pp + 1][nq][i]);
          }
          pf[nq] = frag_from_acc<bf16>(p0, p1);
          lacc[nq] = mfma(ones, pf[nq], lacc[nq]);
        }
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          Frag<bf16> vf[lD / 32];
#pragma unroll
          for (int dd = 0; dd < lD / 32; ++dd) {
            const bf16* p = Vb + vofs + 32 * pp * lS + 16 * (hf * lD / 32 + dd);
            const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds4_ptr)(p));
            const bf16x4 c = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds4_ptr)(p + 16 * lS));
            vf[dd].v = __builtin_shufflevector(a, c, 0, 1, 2, 3, 4, 5, 6, 7);
          }
#pragma unroll
          for (int dd = 0; dd < lD / 32; ++dd)
#pragma unroll
            for (int nq = 0; nq < kNQ; ++nq)
              oacc[hf * lD / 32 + dd][nq] = mfma(vf[dd], pf[nq], oacc[hf * lD / 32 + dd][nq]);
        }
      }

      if (last) {
        // ---- epilogue of this query tile
#pragma unroll
        for (int nq = 0; nq < kNQ; ++nq) {
          const int t = qb + 16 * nq + j;
          if (t >= T_) continue;
          const float inv = w_swa / lacc[nq][0];
          bf16* orow = o + ((size_t)(bi * T_ + t) * H + h) * lD;
          const bool add = addl && t >= add_from;
#pragma unroll
          for (int dt = 0; dt < lD / 16; ++dt) {
            f32x4 val = oacc[dt][nq] * inv;
            if (ADD && add)
              val += f32x4{static_cast<float>(oraw[nq][dt][0]), static_cast<float>(oraw[nq][dt][1]),
                           static_cast<float>(oraw[nq][dt][2]), static_cast<float>(oraw[nq][dt][3])};
            store4(orow + 16 * dt + 4 * g, val);
          }
        }
        if (more) set_q(ti + 1, qnext);
      }
    }
  }
}

}  // namespace

bool swa_long_applies(const PrefillArgs& p) {
  // budgets whose query tiles walk many key blocks (the resident-block
  // kernel covers windows up to 129 keys); K and V of one batch row within
  // 2 GiB (32-bit lane offsets of the direct loads)
  return p.bf16 && p.D == lD && p.window >= 256 &&
         (long long)p.T * p.Hkv * lD * 2 < (1LL << 31);
}

hipError_t launch_swa_long(const PrefillArgs& p, int add_from, hipStream_t s) {
  // one 8-wave workgroup per compute unit with a four-slot ring
  constexpr int W = 8, NS = 4;
  constexpr int lds = LongCfg<W, NS>::lds;
  const int G = p.H / p.Hkv;
  int HPW = 1;
  while (HPW < W && G % (2 * HPW) == 0) HPW *= 2;
  const int QT = 32 * (W / HPW);
  const int ntiles = (p.T + QT - 1) / QT;
  const int tpw = std::min(lTPW, ntiles);
  const int nruns = (ntiles + tpw - 1) / tpw;
  const long long units = (long long)p.B * (p.H / HPW);
  const long long grid = xcd_grouped_grid(units, nruns);
  if (grid > INT32_MAX || units > INT32_MAX) return hipErrorInvalidValue;
#define GDN_LONG_LAUNCH(NH, AD)                                                                         \
  do {                                                                                                  \
    hipError_t e = hipFuncSetAttribute((const void*)swa_long_kernel<W, NS, NH, AD>,                     \
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);                \
    if (e != hipSuccess) return e;                                                                      \
    hipLaunchKernelGGL((swa_long_kernel<W, NS, NH, AD>), dim3((unsigned)grid), dim3(64 * W), lds, s,    \
                       (const bf16*)p.q, (const bf16*)p.k, (const bf16*)p.v, (bf16*)p.o, p.T, p.H,      \
                       p.Hkv, p.n_sink, p.window, add_from, p.w_swa, tpw, nruns, (int)units);           \
  } while (0)
  const bool add = add_from < p.T;
  switch (HPW) {
    case 8: if (add) GDN_LONG_LAUNCH(8, true); else GDN_LONG_LAUNCH(8, false); break;
    case 4: if (add) GDN_LONG_LAUNCH(4, true); else GDN_LONG_LAUNCH(4, false); break;
    case 2: if (add) GDN_LONG_LAUNCH(2, true); else GDN_LONG_LAUNCH(2, false); break;
    default: if (add) GDN_LONG_LAUNCH(1, true); else GDN_LONG_LAUNCH(1, false); break;
  }
#undef GDN_LONG_LAUNCH
  return hipGetLastError();
}

}  // namespace gdn
