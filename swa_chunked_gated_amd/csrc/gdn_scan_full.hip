// State scan of the chunked gated delta rule (prefill, bf16 I/O) for the case
// where the chunk preparation has already computed every state-independent
// chunk quantity: few (sequence, head) chains, so the scan alone cannot fill
// the GPU and its per-chunk latency is what counts.
//
// Method (page "The Key to Going Linear: Analysis-Driven Transformer
// Linearization"): section 线性注意力替换机制 gives the gated delta rule
// S_i = a_i (I - b_i k_i k_i^T) S_{i-1} + b_i k_i v_i^T; section
// 填补近似缺口的实用设计 has the recurrence cover only evicted tokens, read
// with lag `window`: o_lin[t] = S^(t-window)^T q_t.  Chunk form (64 stream
// tokens, incoming state S; derived by unrolling the recurrence):
//   U = Ut - Wm S,   O = diag(gamma) Q S + A U,   S <- gamma_C S + KTg U
// with Ut = Tm diag(b) V, Wm = Tm diag(b gamma) K, KTg = K^T diag(gamma_C /
// gamma) and A the decayed causal scores, all read from the preparation.
//
// Work split: one workgroup per (sequence, head, 16 * NW state columns) with
// NW compute waves and one loader wave.  Each compute wave owns 16 state
// columns as fp32 MFMA accumulators for the whole sequence; the accumulator
// row r of the state holds d_k index acc_pos(r), the order in which MFMA
// accumulators turn into operands, so that the query and -Wm tiles are read
// in their natural d_k order (the preparation writes KTg rows to match).  The
// loader wave streams chunk c+1's tiles (query rows, V rows, TB, -Wm, KTg, A,
// gates) from global memory straight into the second of two LDS buffers with
// global-to-LDS loads, while the compute waves run chunk c from the first
// buffer; one workgroup barrier per chunk hands the buffer over.  The compute
// waves issue no loads of their own, so their MFMA and LDS work never queues
// behind the vector-memory traffic of the next chunk.

#include <atomic>
#include <chrono>
#include <random>

#include "common.h"
#include "gdn_prep.h"
#include "launch.h"
#include "swa_tile.h"

namespace gdn {
namespace {

using swa::wait_ready;

constexpr int kC = 64;   // chunk length

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(1))) void* gbl_void_ptr;

// Lane L of the wave loads 16 (4) bytes at g into LDS at base + 16 L (4 L).
// dma16c / dma4c read at device scope (cache policy sc1): coherent with
// the device-scope stores of another compute unit in the same kernel (the
// preparation's tiles); dma16 is a plain load (the layer's inputs).
__device__ __forceinline__ void dma16(const void* g, void* base) {
  __builtin_amdgcn_global_load_lds((gbl_void_ptr)(void*)g, (lds_void_ptr)base, 16, 0, 0);
}
__device__ __forceinline__ void dma16c(const void* g, void* base) {
  __builtin_amdgcn_global_load_lds((gbl_void_ptr)(void*)g, (lds_void_ptr)base, 16, 0, 16);
}
__device__ __forceinline__ void dma4c(const void* g, void* base) {
  __builtin_amdgcn_global_load_lds((gbl_void_ptr)(void*)g, (lds_void_ptr)base, 4, 0, 16);
}

template <int D, int NW>
struct FullSmem {
  static constexpr int SK = D + 8;          // row stride of [64][D] tiles (elements)
  static constexpr int SC = kC + 8;         // row stride of [*][64] tiles
  static constexpr int DVS = 16 * NW;       // state columns per workgroup
  static constexpr int SU = kC + 4;         // fp32 row stride of Ut^T
  // one buffer: Q, -Wm, KTg, A (bf16), then Ut^T [DVS][SU], g (log2), gamma
  // [64 each] fp32
  static constexpr int oQ = 0;
  static constexpr int oWm = oQ + kC * SK;
  static constexpr int oKT = oWm + kC * SK;
  static constexpr int oA = oKT + D * SC;
  static constexpr int nT = oA + kC * SC;
  static constexpr int nU = DVS * SU;
  static constexpr int buf_bytes = nT * 2 + 4 * nU + 2 * kC * 4;
  static constexpr int bytes = 2 * buf_bytes;
  static_assert((nT * 2) % 16 == 0, "16-byte tiles");
};

// Preparation waves per preparation workgroup (each needs its own PrepSmem).
constexpr int kPrepWaves = 3;
// Query tiles per softmax workgroup (one continuous K/V prefetch pipeline).
constexpr int kSwaTiles = 1;
// Injected faults (set only by tests, see gdn_hybrid_set_test_faults): the
// preparation does not publish its ready flags / the scan does not publish
// its done flags, so that every wait on them runs into its time bound.
constexpr int kFaultNoReady = 1;
constexpr int kFaultNoDone = 2;

// Dynamic LDS of the fused kernel: the scan's two buffers, or the
// preparation waves' work areas, whichever is larger.
template <int D, int NW>
constexpr int fused_lds_bytes() {
  constexpr int scan = FullSmem<D, NW>::bytes;
  constexpr int prep = kPrepWaves * prep::PrepSmem<bf16, D, true>::bytes;
  return scan > prep ? scan : prep;
}

// Placement on the XCDs (workgroup i of a launch runs on XCD i % 8; each XCD
// has its own L2): chains (sequence, head) are spread over the XCDs so that a
// chain's preparation items and its scan workgroups share one XCD, and with
// kXcdByGroup the query heads of one KV head share it too (their preparation
// reads the same K and V rows).  A chain is named by its XCD x and its slot
// among that XCD's chains.
constexpr int kXcdNone = 0;
constexpr int kXcdByGroup = 1;     // B Hkv divisible by 8
constexpr int kXcdByChain = 2;     // B H divisible by 8
__device__ __forceinline__ int xcd_chain(int mode, int G, int x, int slot) {
  if (mode == kXcdByGroup) return ((slot / G) * 8 + x) * G + slot % G;
  return slot * 8 + x;
}

// Grid, in dispatch order: n_prep preparation workgroups, one scan workgroup
// per (sequence, head, column slice), then n_swa softmax workgroups.
//  * With n_prep = 0 the workspace is already complete (the preparation
//    kernel ran before) and the scan waits for nothing.  Otherwise
//    preparation waves take (chunk, head, sequence) items in chunk-major
//    order, write the chunk's tiles with device-scope stores (written through
//    to memory), wait for them to complete and publish
//    ready[(b H + h) nch + c] = epoch; the scan's loader waves wait for that
//    flag and then read the tiles with device-scope loads.
//  * With n_swa > 0 the softmax branch is part of the kernel: the scan stores
//    its rows at device scope and publishes them chunk by chunk (done flags);
//    a softmax workgroup computes its tile and, before adding onto rows that
//    hold the linear branch, waits for the flags of the chunks covering them.
// Every wait is on work of an earlier part of the grid, which is dispatched
// in full before the waiting workgroups (preparation workgroups wait for
// nothing, scan workgroups only for preparation), so the waits always end.
template <int D, int NW, int NL>
__global__ __launch_bounds__(64 * (NW + NL)) void gdn_scan_full_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ a, const float* __restrict__ b, bf16* __restrict__ w_wm,
    bf16* __restrict__ w_ktg, bf16* __restrict__ w_a, float* __restrict__ w_ut,
    float* __restrict__ w_g, uint64_t* __restrict__ ready, uint64_t epoch, int n_prep,
    uint64_t* __restrict__ done, int n_swa, bf16* __restrict__ o, float* __restrict__ state_out,
    int B, int T_, int H, int Hkv, int n_sink, int window, int flags, int xcd, float w_lin,
    float w_swa, uint64_t wait_ticks, int faults) {
  using SM = FullSmem<D, NW>;
  using PS = prep::PrepSmem<bf16, D, true>;
  static_assert(NL >= 1 && NL <= 4, "one to four loader waves");
  static_assert(PS::bytes % 16 == 0 && fused_lds_bytes<D, NW>() <= 160 * 1024, "LDS of one workgroup");
  static_assert(swa::SwaSmem<bf16, D>::deep_bytes <= fused_lds_bytes<D, NW>(), "softmax tiles' LDS");
  constexpr int SK = SM::SK;
  constexpr int SC = SM::SC;
  constexpr int DVS = SM::DVS;
  constexpr int MT = D / 16;             // 16-row tiles of the state
  constexpr int P = D / 8;               // 16-byte pieces of a D-wide row

  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  auto buf = [&](int b) { return reinterpret_cast<bf16*>(smem_raw + b * SM::buf_bytes); };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = wave_id();
  const int iend = T_ - window;          // stream tokens are [n_sink, iend)
  const int nch = iend > n_sink ? (iend - n_sink + kC - 1) / kC : 0;

  if ((int)blockIdx.x < n_prep) {
    // ======================= preparation workgroup
    if (wv >= kPrepWaves) return;
    const int BH = B * H;
    // items in chunk-major order; with an XCD placement, this workgroup's
    // XCD takes only the chains placed on it
    const int x = xcd ? ((int)blockIdx.x - n_prep % 8 + 8) % 8 : 0;
    const int per = xcd ? BH / 8 : BH;
    const int first = xcd ? ((int)blockIdx.x / 8) * kPrepWaves + wv : (int)blockIdx.x * kPrepWaves + wv;
    const int stride = xcd ? (n_prep / 8) * kPrepWaves : n_prep * kPrepWaves;
    for (int it = first; it < nch * per; it += stride) {
      const int c = it / per;
      const int bh = xcd ? xcd_chain(xcd, H / Hkv, x, it % per) : it % per;
      prep::gdn_prep_chunk<bf16, D, true, true>(q, k, v, a, b, nullptr, w_wm, w_ktg, w_a,
                                                w_ut, w_g, T_, H, Hkv, n_sink, window, nch, c,
                                                bh % H, bh / H, smem_raw + wv * PS::bytes);
      // every device-scope tile store of this wave has completed (vmcnt 0)
      // before the flag is stored
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0x0F70);
      asm volatile("" ::: "memory");
      if (lane == 0 && !(faults & kFaultNoReady))
        __hip_atomic_store(ready + (size_t)bh * nch + c, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }

  const int n_scan = B * H * (D / DVS);
  if ((int)blockIdx.x >= n_prep + n_scan) {
    // ======================= softmax workgroup: kSwaTiles consecutive tiles
    // of 64 query rows of the 4 query heads of a KV head (workgroups in row
    // order), adding onto the linear output once the scan has published it.
    // These come last in the grid and start as preparation workgroups finish.
    const int wg = blockIdx.x - n_prep - n_scan;
    const int groups = H / 4;
    const int bx = wg / (groups * B);
    const int rest = wg % (groups * B);
    swa::swa_tiles<bf16, D, NW + NL, true>(q, k, v, o, T_, H, Hkv, 4, 64, kSwaTiles, n_sink, window,
                                           n_sink + window, bx, rest % groups, rest / groups,
                                           reinterpret_cast<bf16*>(smem_raw), done, epoch, nch,
                                           (D / DVS) * NW, w_swa, wait_ticks);
    return;
  }

  const int sw = blockIdx.x - n_prep;
  const int sp = xcd ? (sw / 8) % (D / DVS) : sw % (D / DVS);   // column slice
  const int ch = xcd ? xcd_chain(xcd, H / Hkv, sw % 8, sw / 8 / (D / DVS)) : sw / (D / DVS);
  const int h = ch % H;
  const int bi = ch / H;
  const int g = h / (H / Hkv);
  const int l16 = lane & 15;
  const int lg = lane >> 4;
  const int c0 = sp * DVS;
  const size_t chain = (size_t)bi * H + h;
  // lost[b][l]: loader wave l gave up waiting for a chunk it staged into
  // buffer b (or an earlier one); the compute waves then poison the state
  __shared__ int lost[2][NL];

  if (wv >= NW) {
    // ======================= loader waves: tile t of a chunk is loaded by
    // loader kOwner[NL - 1][t] (tiles: Q, Ut^T, -Wm, KTg, A, gates)
    constexpr int kOwner[4][6] = {{0, 0, 0, 0, 0, 0},
                                  {0, 0, 1, 1, 0, 0},
                                  {0, 2, 1, 2, 0, 0},
                                  {0, 3, 1, 2, 3, 0}};
    const int ld = wv - NW;
    auto mine = [&](int t) { return kOwner[NL - 1][t] == ld; };
    // Every LDS image is whole 1 KiB blocks of 16-byte slots; slot s = 64 n +
    // lane of block n holds piece s % (P + 1) of row s / (P + 1) (the last
    // piece of a row is padding and repeats piece 0).  The per-lane byte
    // offsets of the source pieces are the same for every chunk, so they are
    // formed once here and each load is a uniform base plus a lane offset.
    constexpr int NQ = kC * (P + 1) / 64;            // blocks of the Q and -Wm images
    constexpr int NU = DVS * 17 / 64;                // blocks of the Ut^T image ([DVS][64] fp32)
    constexpr int NK = D * 9 / 64;                   // blocks of the KTg image ([D][64])
    constexpr int NS = kC * 9 / 64;                  // blocks of the A image
    static_assert((DVS * 17) % 64 == 0 && (D * 9) % 64 == 0, "whole 1 KiB blocks");
    const size_t qrow = (size_t)H * D * 2;           // bytes between query rows
    auto piece = [&](int n, int pp, int& r, int& p) {
      const int s = 64 * n + lane;
      r = s / (pp + 1);
      p = s % (pp + 1);
      if (p == pp) p = 0;
    };
    uint32_t oq[NQ], ow[NQ], ou[NU], ok[NK];
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
      int r, p;
      piece(n, P, r, p);
      oq[n] = (uint32_t)(r * qrow + p * 16);
      ow[n] = (uint32_t)((r * P + p) * 16);
    }
#pragma unroll
    for (int n = 0; n < NU; ++n) {
      int r, p;
      piece(n, 16, r, p);
      ou[n] = (uint32_t)(((c0 + r) * kC + 4 * p) * 4);    // column c0 + r of Ut^T
    }
#pragma unroll
    for (int n = 0; n < NK; ++n) {
      int r, p;
      piece(n, 8, r, p);
      ok[n] = (uint32_t)((r * 8 + p) * 16);
    }
    // ready flag of the next chunk to stage, read one chunk ahead so that its
    // latency hides behind the current chunk's loads
    uint64_t seen = 0;
    bool gave_up = false;    // sticky: once a wait gave up, later chunks are not waited for
    auto stage = [&](int c, int b) {
      bf16* B = buf(b);
      const int i0 = n_sink + c * kC;
      const int Cc = min(kC, iend - i0);
      const size_t ci = chain * nch + c;
      if (n_prep > 0) {
        if (!gave_up && seen != epoch) gave_up = !wait_ready(ready + ci, epoch, wait_ticks);
        asm volatile("" ::: "memory");
        seen = c + 1 < nch ? __hip_atomic_load(ready + ci + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
      }
      // query rows i0 + window + r; in a partial chunk the rows past the
      // stream repeat its last row (their outputs are never stored)
      const char* qb = reinterpret_cast<const char*>(q + ((size_t)(bi * T_ + i0 + window) * H + h) * D);
      if (mine(0)) {
        if (Cc == kC) {
#pragma unroll
          for (int n = 0; n < NQ; ++n) dma16(qb + oq[n], B + SM::oQ + 512 * n);
        } else {
#pragma unroll
          for (int n = 0; n < NQ; ++n) {
            int r, p;
            piece(n, P, r, p);
            dma16(qb + min(r, Cc - 1) * qrow + p * 16, B + SM::oQ + 512 * n);
          }
        }
      }
      if (mine(1)) {
        const char* ub = reinterpret_cast<const char*>(w_ut + ci * (D * kC));
        float* U = reinterpret_cast<float*>(B + SM::nT);
#pragma unroll
        for (int n = 0; n < NU; ++n) dma16c(ub + ou[n], U + 256 * n);
      }
      const char* wb = reinterpret_cast<const char*>(w_wm + ci * (kC * D));
      const char* kb = reinterpret_cast<const char*>(w_ktg + ci * (D * kC));
      const char* ab = reinterpret_cast<const char*>(w_a + ci * (kC * kC));
      if (mine(2)) {
#pragma unroll
        for (int n = 0; n < NQ; ++n) dma16c(wb + ow[n], B + SM::oWm + 512 * n);
      }
      if (mine(3)) {
#pragma unroll
        for (int n = 0; n < NK; ++n) dma16c(kb + ok[n], B + SM::oKT + 512 * n);
      }
      if (mine(4)) {
#pragma unroll
        for (int n = 0; n < NS; ++n) dma16c(ab + ok[n], B + SM::oA + 512 * n);
      }
      if (mine(5)) {
        float* gate = reinterpret_cast<float*>(B + SM::nT) + SM::nU;
        dma4c(w_g + ci * (2 * kC) + lane, gate);
        dma4c(w_g + ci * (2 * kC) + 64 + lane, gate + 64);
      }
      if (lane == 0) lost[b][ld] = gave_up ? 1 : 0;
      __builtin_amdgcn_s_waitcnt(0);   // this buffer is complete in LDS
    };
    if (nch > 0) stage(0, 0);
    for (int c = 0; c < nch; ++c) {
      lds_barrier();                   // buffer c & 1 is handed to the compute waves
      if (c + 1 < nch) stage(c + 1, (c + 1) & 1);
    }
    return;
  }

  // ======================= compute waves: state columns c0 + cw .. + 15
  const int cw = 16 * wv;
  f32x4 S[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) S[mt] = zero4();

  // linked softmax tiles read this wave's output rows of chunk c once
  // done[((b H + h) nch + c) (D / DVS) NW + sp NW + wave] = epoch; it is set
  // six chunks later, when the rows' device-scope stores have completed
  // (vmcnt counts this wave's stores in order: waiting until at most the
  // twenty row stores of the five previous chunks are outstanding)
  const size_t done0 = chain * nch * (D / DVS) * NW + sp * NW + wv;
  auto publish = [&](int c) {
    if (lane == 0 && !(faults & kFaultNoDone))
      __hip_atomic_store(done + done0 + (size_t)c * (D / DVS) * NW, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  for (int c = 0; c < nch; ++c) {
    lds_barrier();                     // chunk c's buffer is complete
    if (n_swa > 0 && c >= 6) {
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0x4F74);   // vmcnt(20)
      asm volatile("" ::: "memory");
      publish(c - 6);
    }
    bool stale = false;
#pragma unroll
    for (int l = 0; l < NL; ++l) stale |= lost[c & 1][l] != 0;
    if (stale) {
      // the chunk's tiles were not published in time: the state and every
      // output from this chunk on become NaN instead of silently wrong
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) S[mt] = f32x4{__builtin_nanf(""), __builtin_nanf(""),
                                                    __builtin_nanf(""), __builtin_nanf("")};
    }
    const bf16* B = buf(c & 1);
    const bf16* Qs = B + SM::oQ;
    const bf16* Wms = B + SM::oWm;
    const bf16* KTs = B + SM::oKT;
    const bf16* Aqs = B + SM::oA;
    const float* UTs = reinterpret_cast<const float*>(B + SM::nT);
    const float* gam = UTs + SM::nU + kC;
    const int i0 = n_sink + c * kC;
    const int Cc = min(kC, iend - i0);

    Frag<bf16> sf[D / 32];
#pragma unroll
    for (int p = 0; p < D / 32; ++p) sf[p] = frag_from_acc<bf16>(S[2 * p], S[2 * p + 1]);

    // O^T = S^T Q^T (operand slot j of lane group lg is d_k 32 p + 8 lg + j
    // on both sides)
    f32x4 ot[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) ot[rt] = zero4();
#pragma unroll
    for (int ph = 0; ph < D / 64; ++ph) {
      Frag<bf16> qf[4][2];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) qf[rt][pp] = lds_frag8(&Qs[(16 * rt + l16) * SK + 64 * ph + 32 * pp + 8 * lg]);
#pragma unroll
      for (int pp = 0; pp < 2; ++pp)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) ot[rt] = mfma(sf[2 * ph + pp], qf[rt][pp], ot[rt]);
    }

    // U = Ut - Wm S   (tokens x this wave's 16 columns): the accumulators
    // start from Ut (rows 16 mt + 4 lg .. +3 of column cw + l16)
    f32x4 U[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) U[mt] = *reinterpret_cast<const f32x4*>(&UTs[(cw + l16) * SM::SU + 16 * mt + 4 * lg]);
#pragma unroll
    for (int ph = 0; ph < D / 64; ++ph) {
      Frag<bf16> wf[4][2];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) wf[mt][pp] = lds_frag8(&Wms[(16 * mt + l16) * SK + 64 * ph + 32 * pp + 8 * lg]);
#pragma unroll
      for (int pp = 0; pp < 2; ++pp)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) U[mt] = mfma(wf[mt][pp], sf[2 * ph + pp], U[mt]);
    }

    // O^T: gamma of each query column on the S^T Q^T part, then + U^T A^T
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) ot[rt] *= gam[16 * rt + l16];
    Frag<bf16> uf[2];
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) uf[pp] = frag_from_acc<bf16>(U[2 * pp], U[2 * pp + 1]);
    {
      Frag<bf16> af[4][2];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) af[rt][pp] = lds_frag8(&Aqs[(16 * rt + l16) * SC + 32 * pp + 8 * lg]);
#pragma unroll
      for (int pp = 0; pp < 2; ++pp)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) ot[rt] = mfma(uf[pp], af[rt][pp], ot[rt]);
    }

    // S = gamma_C S + KTg U
    const float gC = gam[kC - 1];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) S[mt] *= gC;
#pragma unroll
    for (int m4 = 0; m4 < MT / 4; ++m4) {
      Frag<bf16> kf[4][2];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) kf[i][pp] = lds_frag8(&KTs[(16 * (4 * m4 + i) + l16) * SC + 32 * pp + 8 * lg]);
#pragma unroll
      for (int pp = 0; pp < 2; ++pp)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[4 * m4 + i] = mfma(kf[i][pp], uf[pp], S[4 * m4 + i]);
    }

    // store (or add) the chunk's linear output rows
    if (flags & 1) {
      const bool accumulate = (flags & 8) != 0;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const int r = 16 * rt + l16;
        if (r < Cc) {
          bf16* orow = o + ((size_t)(bi * T_ + i0 + r + window) * H + h) * D + c0 + cw + 4 * lg;
          f32x4 val = ot[rt] * w_lin;
          if (n_swa > 0) {
            // device-scope store (read by the linked softmax tiles)
            const bf16x4 y = bf16x4{static_cast<bf16>(val[0]), static_cast<bf16>(val[1]),
                                    static_cast<bf16>(val[2]), static_cast<bf16>(val[3])};
            bf16* obase = o + ((size_t)(bi * T_ + i0 + window) * H + h) * D + c0 + cw;
            typedef unsigned int u2 __attribute__((ext_vector_type(2)));
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u2, y),
                                                  __builtin_amdgcn_make_buffer_rsrc(obase, 0, 0x7fffffff, 0x00020000),
                                                  (r * H * D + 4 * lg) * 2, 0, prep::kCpolSc1);
          } else {
            if (accumulate) val += load4(orow);
            store4(orow, val);
          }
        }
      }
    }
  }

  if (n_swa > 0) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): every row store has completed
    asm volatile("" ::: "memory");
    for (int c = max(0, nch - 6); c < nch; ++c) publish(c);
  }

  // linear-only overwrite: rows t < n_sink + window carry no linear output
  constexpr int kThreads = 64 * NW;
  if ((flags & 1) && !(flags & 2) && !(flags & 8)) {
    const int rows = min(n_sink + window, T_);
    for (int i = tid; i < rows * (DVS / 4); i += kThreads) {
      const int t = i / (DVS / 4);
      const int cc = (i % (DVS / 4)) * 4;
      store4(o + ((size_t)(bi * T_ + t) * H + h) * D + c0 + cc, zero4());
    }
  }
  if (flags & 4) {
    float* Sg = state_out + chain * D * D;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) Sg[(size_t)acc_pos(16 * mt + 4 * lg + i) * D + c0 + cw + l16] = S[mt][i];
  }
}

// Per-call value of the ready flags: a process-wide counter from a random
// start, so flags left in a reused workspace (or in fresh memory) never match.
uint64_t next_epoch() {
  static std::atomic<uint64_t> counter{[] {
    std::random_device rd;
    const uint64_t t = (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count();
    return (((uint64_t)rd() << 32) ^ (uint64_t)rd() ^ (t * 0x9E3779B97F4A7C15ull)) | 1ull;
  }()};
  return counter.fetch_add(2, std::memory_order_relaxed);   // odd: never the zero of cleared memory
}

template <int D, int NW, int NL>
hipError_t launch_full_t(const PrefillArgs& p, int nch, hipStream_t s, bool* swa_done) {
  using SM = FullSmem<D, NW>;
  constexpr int lds = fused_lds_bytes<D, NW>();
  auto kern = gdn_scan_full_kernel<D, NW, NL>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  const GdnWorkspace w = gdn_workspace_layout(p.workspace, p.B, p.H, nch, D, sizeof(bf16), true);
  const int n_scan = p.B * p.H * (D / SM::DVS);
  // Overlap the preparation with the scan when the scan leaves at least half
  // of the compute units free: each scan workgroup fills a compute unit (LDS),
  // the preparation workgroups take the rest.
  int dev = 0, cus = 0;
  e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  int n_prep = (nch > 0 && 2 * n_scan <= cus) ? cus - n_scan : 0;
  if (nch > 0 && n_prep == 0) {
    e = launch_gdn_prep(p, nch, s);
    if (e != hipSuccess) return e;
  }
  const uint64_t epoch = n_prep > 0 ? next_epoch() : 0;
  const TestFaults tf = test_faults();
  // XCD placement (the preparation's share needs whole rounds of 8 workgroups)
  int xcd = kXcdNone;
  if (n_prep % 8 == 0 && (p.B * p.H) % 8 == 0) xcd = (p.B * p.Hkv) % 8 == 0 ? kXcdByGroup : kXcdByChain;
  // The softmax branch joins the kernel (its tiles run on the preparation
  // workgroups after their chunks, adding onto the scan's rows as they are
  // published) when both branches are asked for without accumulation and a
  // KV head serves a multiple of 4 query heads.  Without the linear branch
  // the scan writes no rows for the tiles to add onto, so the softmax branch
  // then runs as its own launch (which writes every row).
  const bool link = n_prep > 0 && (p.flags & 1) && (p.flags & 2) && !(p.flags & 8) &&
                    (p.H / p.Hkv) % 4 == 0;
  const int n_swa = link ? ((p.T + 63) / 64 + kSwaTiles - 1) / kSwaTiles * (p.H / 4) * p.B : 0;
  if (swa_done) *swa_done = link;
  hipLaunchKernelGGL(kern, dim3(n_prep + n_scan + n_swa), dim3(64 * (NW + NL)), lds, s,
                     (const bf16*)p.q, (const bf16*)p.k, (const bf16*)p.v, p.a, p.b, (bf16*)w.wm,
                     (bf16*)w.ktg, (bf16*)w.a, w.ut, w.g, w.ready, epoch, n_prep, w.done, n_swa,
                     (bf16*)p.o, p.state_out, p.B, p.T, p.H, p.Hkv, p.n_sink, p.window, p.flags, xcd,
                     p.w_lin, p.w_swa, tf.wait_ticks, tf.faults);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gdn_full(const PrefillArgs& p, int nch, hipStream_t s, bool* swa_done) {
  if (swa_done) *swa_done = false;
  if (!p.bf16 || p.gla) return hipErrorInvalidValue;
  if (p.D == 64) return launch_full_t<64, 4, 4>(p, nch, s, swa_done);
  if (p.D == 128) return launch_full_t<128, 4, 4>(p, nch, s, swa_done);
  return hipErrorInvalidValue;
}

}  // namespace gdn
