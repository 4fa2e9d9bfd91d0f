// Linear branch of the hybrid layer (prefill) on gfx950: chunked gated delta
// rule, and the chunked GLA variant.
//
// Method (page "The Key to Going Linear: Analysis-Driven Transformer
// Linearization"):
//  * section 线性注意力替换机制: GDN state update S_i = a_i (I - b_i k_i k_i^T)
//    S_{i-1} + b_i k_i v_i^T (scalar gate a_i per head); GLA update
//    S_i = Diag(alpha_i) S_{i-1} + k_i v_i^T.
//  * section 填补近似缺口的实用设计: the recurrence only covers tokens that
//    have left the sink + window budget, so query t reads the state after
//    token t - window: o_lin[t] = S^(t-window)^T q_t, for t >= n_sink + window.
//
// Chunk form (64 stream tokens, gates g = inclusive cumsum of log a inside
// the chunk, gamma = exp(g), incoming state S0; derived from the recurrence
// by unrolling it over the chunk):
//   L_rs = b_r gamma_r/gamma_s k_r.k_s (s < r),  Tm = (I + L)^-1
//   Wm = Tm diag(b gamma) K,  Ut = Tm diag(b) V,  U = Ut - Wm S0
//   O  = diag(gamma) Q S0 + (gamma_r/gamma_s [s <= r] o Q K^T) U
//   S  = gamma_C S0 + K^T diag(gamma_C / gamma) U
// where Q holds the lag-shifted queries (rows i + window).  GLA, with
// per-channel cumulative log-gates G:
//   A = [s <= r] o (Q e^G)(K e^-G)^T,  O = (Q e^G) S0 + A V,
//   S = e^{G_C} o_rows S0 + (K e^{G_C - G})^T V.
// The delta rule with that diagonal gate (mode 2) replaces V by
// U = TB V - Wm S0 (TB = (I + L)^-1 diag(b), Wm = TB (K e^G), both from its
// preparation): O = (Q e^G) S0 + A U, S = e^{G_C} o_rows S0 + (K e^{G_C - G})^T U.
//
// Work split: one workgroup per (sequence, query head, column slice of the
// state).  The state's d_v columns are independent in both updates, so each
// wave owns 16 columns of S as fp32 MFMA accumulators in registers for the
// whole sequence, and every S-dependent product of a chunk is wave-local.
// The chunk preparation kernels (gdn_prep.hip, gla_prep.hip) have already
// produced the triangular solve (TB = Tm diag(b)) and the gates (GDN) or
// every state-independent tile (GLA); the GDN chunk's Q K^T scores and
// Wm = Tm diag(b gamma) K are formed here on MFMA (TB scaled by gamma as its
// fragments are read) and shared through LDS.  (bf16 GDN with too few chains
// to fill the GPU runs gdn_scan_full.hip instead.)
// Chunk c+1's inputs are loaded into registers while chunk c is computed.
// Every LDS tile keeps its reduction dimension in acc order (see common.h),
// so all MFMA operand reads are single 16-byte LDS accesses.

#include <algorithm>

#include "common.h"
#include "launch.h"

namespace gdn {
namespace {

constexpr int kC = 64;          // chunk length
// the 10 lower-triangular 16x16 tiles (row, col) of a 64x64 matrix
__constant__ const int kTileM[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
__constant__ const int kTileN[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};

// MODE: 0 the gated delta rule, 1 GLA, 2 the delta rule with a diagonal
// gate (the per-channel-gate tiles of GLA, plus TB and Wm).
template <class T, int D, int NW, int DW, int MODE>
struct Smem {
  static constexpr bool GLA = MODE != 0;    // per-channel gate tiles from the workspace
  static constexpr bool DELTA = MODE != 1;  // U = TB V - Wm S
  static constexpr int PAD = 16 / sizeof(T);
  static constexpr int SK = D + PAD;        // stride of [64][D] arrays
  static constexpr int SC = kC + PAD;       // stride of [*][64] arrays
  static constexpr int DVS = NW * DW;       // state columns per workgroup
  static constexpr int nK = kC * SK;
  static constexpr int nKT = D * SC;
  static constexpr int nVT = DVS * SC;
  static constexpr int nA = kC * SC;
  // element offsets in units of T (GLA keeps only Q 2^G, K^T 2^{G_C-G}, V^T, A)
  static constexpr int oK = 0;
  static constexpr int oKT = oK + (GLA ? 0 : nK);
  static constexpr int oQ = oKT + nKT;
  static constexpr int oVT = oQ + nK;
  static constexpr int oAq = oVT + nVT;
  static constexpr int oWm = oAq + nA;
  static constexpr int oTB = oWm + (DELTA ? nK : 0);
  static constexpr int nT = oTB + (DELTA ? nA : 0);
  static constexpr int bytesT = ((nT * (int)sizeof(T)) + 15) / 16 * 16;
  // fp32 part: GDN g (log2), gamma [64 each]; GLA 2^{G_C} [D]
  static constexpr int nGate = GLA ? D : 2 * kC;
  static constexpr int bytes = bytesT + 4 * nGate;
};

template <class T, int D, int NW, int DW, int MODE>
__global__ __launch_bounds__(64 * NW) void linear_chunk_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ w0, const T* __restrict__ w1, const T* __restrict__ w2,
    const T* __restrict__ w3, const T* __restrict__ w4, const float* __restrict__ wf, T* __restrict__ o,
    float* __restrict__ state_out, int T_, int H, int Hkv, int n_sink, int window, int flags,
    float w_lin, T* __restrict__ ckpt) {
  // w_lin weighs the linear branch in o (1 for the plain sum).  ckpt (the
  // backward pass's forward sweep): the state entering each chunk, in T,
  // per (sequence, head, chunk) in tile order (16 x 16 tiles (row tile,
  // column tile); in a tile, lane 16 g + j holds rows 4 g .. 4 g + 3 of
  // column j).
  // chunk preparation results (workspace), per (sequence, head, chunk):
  //   GDN, light: w0 = Tm diag(b), wf = g (log2), gamma (w1 unused)
  //   GLA:        w0 = Q 2^G, w1 = (K 2^{G_C - G})^T, w2 = A, wf = 2^{G_C}
  //   diagonal-gate delta rule: as GLA, plus w3 = TB, w4 = -Wm
  using SM = Smem<T, D, NW, DW, MODE>;
  constexpr bool GLA = SM::GLA;
  constexpr bool DGD = MODE == 2;
  constexpr int kThreads = 64 * NW;
  constexpr int SK = SM::SK;
  constexpr int SC = SM::SC;
  constexpr int DVS = SM::DVS;
  constexpr int VEC = 16 / sizeof(T);
  constexpr int NT = DW / 16;          // 16-column tiles per wave
  constexpr int MT = D / 16;           // 16-row tiles of the state
  // K and V are fetched as dwords: each wave covers 64/NW tokens, each lane
  // one dword column of TPT consecutive tokens, so a thread can write whole
  // 16-byte runs of the transposed tiles K^T and V^T.
  constexpr int EPD = 4 / sizeof(T);              // elements per dword
  constexpr int TPW = kC / NW;                    // tokens per wave
  constexpr int DPR = D / EPD;                    // dwords per K row
  constexpr int TPT = TPW * DPR / 64;             // tokens per thread (K)
  constexpr int DPRV = DVS / EPD;                 // dwords per V-slice row
  constexpr int TPTV = TPW * DPRV / 64;           // tokens per thread (V)
  static_assert(MT % NW == 0 || NW % MT == 0, "wave split of the state rows");
  constexpr int NPQ = kC * D / VEC / kThreads;    // Q 16-byte pieces per thread
  constexpr int NPK = D * kC / VEC / kThreads;    // GLA: K^T pieces per thread
  constexpr int NPA = kC * kC / VEC / kThreads;   // GLA: A pieces per thread
  static_assert(!GLA || ((D * kC / VEC) % kThreads == 0 && NPA >= 1), "GLA staging");
  static_assert(DPR <= 64 && 64 % DPR == 0 && DPRV <= 64 && 64 % DPRV == 0, "row shape");
  static_assert(TPT % 8 == 0 && TPTV % 8 == 0 && NPQ >= 1, "tile shape");

  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  T* sT = reinterpret_cast<T*>(smem_raw);
  T* Ks = sT + SM::oK;
  T* KTs = sT + SM::oKT;
  T* Qs = sT + SM::oQ;
  T* VTs = sT + SM::oVT;
  T* Aqs = sT + SM::oAq;
  T* Wms = sT + SM::oWm;
  T* TBs = sT + SM::oTB;
  float* gate = reinterpret_cast<float*>(smem_raw + SM::bytesT);   // GDN: g[64], gam[64]; GLA: 2^{G_C}[D]

  // the G query heads of a KV head and their column slices run on one XCD,
  // so the K and V rows they all read come from HBM once per group
  constexpr int NSP = D / DVS;        // column slices per chain
  const int G = H / Hkv;
  int unit, member;
  if (!xcd_grouped(blockIdx.x, G * NSP, Hkv, unit, member)) return;
  const int sp = member % NSP;        // column slice
  const int g = unit;
  const int bi = blockIdx.y;
  const int h = g * G + member / NSP;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = wave_id();
  const int l16 = lane & 15;
  const int lg = lane >> 4;
  const int c0 = sp * DVS;            // first state column of this workgroup
  const int cw = DW * wv;             // first column of this wave inside the slice
  const int iend = T_ - window;       // stream tokens are [n_sink, iend)
  const int nch = iend > n_sink ? (iend - n_sink + kC - 1) / kC : 0;
  // dword staging coordinates
  const int kdc = lane % DPR;                       // K dword column
  const int kr0 = TPW * wv + TPT * (lane / DPR);    // first token row
  const int vdc = lane % DPRV;
  const int vr0 = TPW * wv + TPTV * (lane / DPRV);

  // zero the score tiles once: their strictly upper parts are never written
  for (int i = tid; i < SM::nA; i += kThreads) Aqs[i] = from_f32<T>(0.f);

  f32x4 S[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) S[mt][nt] = zero4();

  // ---------------- register prefetch of one chunk's inputs
  typedef typename Vec16<T>::type V16;
  // V (dword columns, both updates); GDN: K (dword columns), Q (16-byte row
  // pieces), TB and g, gamma from the workspace; GLA: Q 2^G, K^T 2^{G_C-G},
  // A and 2^{G_C} from the workspace
  uint32_t pk[GLA ? 1 : TPT], pv[TPTV];
  V16 pq[NPQ];
  constexpr int NPT = GLA ? 1 : kC * kC / VEC / kThreads;
  static_assert(GLA || (kC * kC / VEC) % kThreads == 0, "TB staging");
  V16 ptb[GLA ? NPK : NPT], ptbg[GLA ? NPA : 1];
  constexpr int NPT2 = kC * kC / VEC / kThreads;   // diagonal-gate delta: TB pieces
  V16 pt2[DGD ? NPT2 : 1], pwm[DGD ? NPQ : 1];
  f32x4 pgm = zero4();
  const size_t chain = (size_t)bi * H + h;

  const size_t kvstride = (size_t)Hkv * D;           // elements between tokens
  const size_t qstride = (size_t)H * D;
  auto prefetch = [&](int c) {
    const int i0 = n_sink + c * kC;
    const bool full = i0 + kC <= iend;               // uniform: no masking needed
    const T* vp = v + ((size_t)(bi * T_ + i0 + vr0) * Hkv + g) * D + c0 + vdc * EPD;
    if (full) {
#pragma unroll
      for (int j = 0; j < TPTV; ++j) pv[j] = *reinterpret_cast<const uint32_t*>(vp + j * kvstride);
    } else {
#pragma unroll
      for (int j = 0; j < TPTV; ++j)
        pv[j] = i0 + vr0 + j < iend ? *reinterpret_cast<const uint32_t*>(vp + j * kvstride) : 0u;
    }
    const size_t ci = chain * nch + c;
    if constexpr (GLA) {
      const V16* qg = reinterpret_cast<const V16*>(w0 + ci * (kC * D));
      const V16* ktg = reinterpret_cast<const V16*>(w1 + ci * (D * kC));
      const V16* aa = reinterpret_cast<const V16*>(w2 + ci * (kC * kC));
#pragma unroll
      for (int n = 0; n < NPQ; ++n) pq[n] = qg[tid + n * kThreads];
#pragma unroll
      for (int n = 0; n < NPK; ++n) ptb[n] = ktg[tid + n * kThreads];
#pragma unroll
      for (int n = 0; n < NPA; ++n) ptbg[n] = aa[tid + n * kThreads];
      if (tid < D / 4) pgm = reinterpret_cast<const f32x4*>(wf + ci * D)[tid];
      if constexpr (DGD) {
        const V16* tb = reinterpret_cast<const V16*>(w3 + ci * (kC * kC));
        const V16* wm = reinterpret_cast<const V16*>(w4 + ci * (kC * D));
#pragma unroll
        for (int n = 0; n < NPT2; ++n) pt2[n] = tb[tid + n * kThreads];
#pragma unroll
        for (int n = 0; n < NPQ; ++n) pwm[n] = wm[tid + n * kThreads];
      }
    } else {
      const T* kp = k + ((size_t)(bi * T_ + i0 + kr0) * Hkv + g) * D + kdc * EPD;
      if (full) {
#pragma unroll
        for (int j = 0; j < TPT; ++j) pk[j] = *reinterpret_cast<const uint32_t*>(kp + j * kvstride);
      } else {
#pragma unroll
        for (int j = 0; j < TPT; ++j)
          pk[j] = i0 + kr0 + j < iend ? *reinterpret_cast<const uint32_t*>(kp + j * kvstride) : 0u;
      }
      const T* qp = q + ((size_t)(bi * T_ + i0 + window) * H + h) * D;
#pragma unroll
      for (int n = 0; n < NPQ; ++n) {
        const int j = tid + n * kThreads;
        const int r = j / (D / VEC);
        const int cc = (j % (D / VEC)) * VEC;
        if (full || i0 + r < iend) {
          pq[n] = *reinterpret_cast<const V16*>(qp + r * qstride + cc);
        } else {
#pragma unroll
          for (int x = 0; x < VEC; ++x) pq[n][x] = from_f32<T>(0.f);
        }
      }
      const V16* tb = reinterpret_cast<const V16*>(w0 + ci * (kC * kC));
#pragma unroll
      for (int n = 0; n < NPT; ++n) ptb[n] = tb[tid + n * kThreads];
      if (tid < 2 * kC / 4) pgm = reinterpret_cast<const f32x4*>(wf + ci * (2 * kC))[tid];
    }
  };

  auto commit = [&]() {
    // V transposed (tokens in acc order, runs of 4)
#pragma unroll
    for (int e = 0; e < EPD; ++e) store_column_acc<T, TPTV>(&VTs[(vdc * EPD + e) * SC], vr0, pv, e);
    if constexpr (GLA) {
      // workspace tiles are already in the LDS orders: 16-byte copies
#pragma unroll
      for (int n = 0; n < NPQ; ++n) {
        const int j = tid + n * kThreads;
        *reinterpret_cast<V16*>(&Qs[(j / (D / VEC)) * SK + (j % (D / VEC)) * VEC]) = pq[n];
      }
#pragma unroll
      for (int n = 0; n < NPK; ++n) {
        const int j = tid + n * kThreads;
        *reinterpret_cast<V16*>(&KTs[(j / (kC / VEC)) * SC + (j % (kC / VEC)) * VEC]) = ptb[n];
      }
#pragma unroll
      for (int n = 0; n < NPA; ++n) {
        const int j = tid + n * kThreads;
        *reinterpret_cast<V16*>(&Aqs[(j / (kC / VEC)) * SC + (j % (kC / VEC)) * VEC]) = ptbg[n];
      }
      if (tid < D / 4) *reinterpret_cast<f32x4*>(&gate[4 * tid]) = pgm;
      if constexpr (DGD) {
#pragma unroll
        for (int n = 0; n < NPT2; ++n) {
          const int j = tid + n * kThreads;
          *reinterpret_cast<V16*>(&TBs[(j / (kC / VEC)) * SC + (j % (kC / VEC)) * VEC]) = pt2[n];
        }
#pragma unroll
        for (int n = 0; n < NPQ; ++n) {
          const int j = tid + n * kThreads;
          *reinterpret_cast<V16*>(&Wms[(j / (D / VEC)) * SK + (j % (D / VEC)) * VEC]) = pwm[n];
        }
      }
    } else {
      // K row-major (one dword per token, columns in acc order) and
      // transposed (tokens in acc order, runs of 4)
#pragma unroll
      for (int j = 0; j < TPT; ++j)
        *reinterpret_cast<uint32_t*>(&Ks[(kr0 + j) * SK + acc_pos(kdc * EPD)]) = pk[j];
#pragma unroll
      for (int e = 0; e < EPD; ++e) store_column_acc<T, TPT>(&KTs[(kdc * EPD + e) * SC], kr0, pk, e);
#pragma unroll
      for (int n = 0; n < NPQ; ++n) {
        const int j = tid + n * kThreads;
        const int r = j / (D / VEC);
        const int cc = (j % (D / VEC)) * VEC;
        // runs of 4 logical columns stay contiguous in acc order
#pragma unroll
        for (int m = 0; m < VEC / 4; ++m) {
          T* dst = &Qs[r * SK + acc_pos(cc + 4 * m)];
          if constexpr (sizeof(T) == 2) {
            *reinterpret_cast<bf16x4*>(dst) = bf16x4{pq[n][4 * m], pq[n][4 * m + 1], pq[n][4 * m + 2], pq[n][4 * m + 3]};
          } else {
            *reinterpret_cast<V16*>(dst) = pq[n];
          }
        }
      }
#pragma unroll
      for (int n = 0; n < NPT; ++n) {
        const int j = tid + n * kThreads;           // 16-byte piece of the 64 x 64 tile
        const int r = j / (kC / VEC);
        const int pc = (j % (kC / VEC)) * VEC;      // already in acc order
        *reinterpret_cast<V16*>(&TBs[r * SC + pc]) = ptb[n];
      }
      if (tid < 2 * kC / 4) *reinterpret_cast<f32x4*>(&gate[4 * tid]) = pgm;
    }
  };

  if (nch > 0) prefetch(0);

  for (int c = 0; c < nch; ++c) {
    const int i0 = n_sink + c * kC;
    const int Cc = min(kC, iend - i0);
    if (ckpt) {
      // tile order: 16 x 16 tiles (row tile, column tile), lane l of a tile
      // holding its 4 accumulator rows, so each lane stores 8 bytes per tile
      T* Sc = ckpt + (chain * nch + c) * (size_t)(D * D);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          T* dst = Sc + ((mt * (D / 16) + (c0 + cw) / 16 + nt) * 256 + 4 * lane);
          if constexpr (sizeof(T) == 2) {
            *reinterpret_cast<bf16x4*>(dst) = bf16x4{from_f32<T>(S[mt][nt][0]), from_f32<T>(S[mt][nt][1]),
                                                     from_f32<T>(S[mt][nt][2]), from_f32<T>(S[mt][nt][3])};
          } else {
            store4(dst, S[mt][nt]);
          }
        }
    }
    lds_barrier();          // previous chunk's LDS reads are done
    commit();
    lds_barrier();
    if (c + 1 < nch) prefetch(c + 1);

    if constexpr (MODE == 0) {
      const float* lgs = gate;
      // ---- Q K^T -> A (decayed, masked s <= r) on the 10 lower 16x16 tiles;
      // the rest of the chunk's state-independent work comes from the chunk
      // preparation (TB, g, gamma)
      for (int job = wv; job < 10; job += NW) {
        const int mt = kTileM[job];
        const int nt = kTileN[job];
        const int r0 = 16 * mt + 4 * lg;
        const int s = 16 * nt + l16;
        const f32x4 lr = *reinterpret_cast<const f32x4*>(&lgs[r0]);
        const float ls = lgs[s];
        Frag<T> xa[D / 32], xb[D / 32];
#pragma unroll
        for (int p = 0; p < D / 32; ++p) {
          xa[p] = lds_frag8(&Qs[(16 * mt + l16) * SK + 32 * p + 8 * lg]);
          xb[p] = lds_frag8(&Ks[(16 * nt + l16) * SK + 32 * p + 8 * lg]);
        }
        f32x4 acc = zero4();
#pragma unroll
        for (int p = 0; p < D / 32; ++p) acc = mfma(xa[p], xb[p], acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = r0 + i;
          const float dec = __builtin_amdgcn_exp2f(fminf(lr[i] - ls, 0.f));
          Aqs[r * SC + acc_pos(s)] = from_f32<T>(s <= r ? dec * acc[i] : 0.f);
        }
      }
      // ---- Wm^T = K^T (Tm diag(b gamma))^T, stored as -Wm [token][dk];
      // each wave owns MT/NW dk tiles and reuses the TBG fragments, formed
      // from TB: the 8 acc-order positions 32p + 8lg .. +7 of a row are
      // tokens 32p + 4lg + 0..3 and 32p + 16 + 4lg + 0..3, scaled by gamma
      if (wv < MT) {
        const float* gmv = lgs + kC;
        Frag<T> tbg[4][2];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
          for (int p = 0; p < 2; ++p)
            tbg[nt][p] = lds_frag8_scaled(&TBs[(16 * nt + l16) * SC + 32 * p + 8 * lg],
                                          gmv + 32 * p + 4 * lg, gmv + 32 * p + 16 + 4 * lg);
        constexpr int MPW = MT >= NW ? MT / NW : 1;
#pragma unroll
        for (int mi = 0; mi < MPW; ++mi) {
          const int mt = wv * MPW + mi;
          Frag<T> kf[2];
#pragma unroll
          for (int p = 0; p < 2; ++p) kf[p] = lds_frag8(&KTs[(16 * mt + l16) * SC + 32 * p + 8 * lg]);
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) {
            f32x4 acc = zero4();
#pragma unroll
            for (int p = 0; p < 2; ++p) acc = mfma(kf[p], tbg[nt][p], acc);
            store4(&Wms[(16 * nt + l16) * SK + acc_pos(16 * mt + 4 * lg)], -acc);
          }
        }
      }
      lds_barrier();
    }

    // ================= per-wave S-dependent products on columns [cw, cw+DW)
    // Each block below first loads all the LDS fragments it needs and then
    // issues its MFMAs into independent accumulators, so the LDS latency is
    // paid once per block rather than once per MFMA.
    Frag<T> sf[D / 32][NT];
#pragma unroll
    for (int p = 0; p < D / 32; ++p)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) sf[p][nt] = frag_from_acc<T>(S[2 * p][nt], S[2 * p + 1][nt]);

    f32x4 ot[NT][4];    // O^T tiles: [dv tile][query tile]
#pragma unroll
    for (int dt = 0; dt < NT; ++dt)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) ot[dt][rt] = zero4();
    // O^T = S^T Q^T (+ gate scaling) ..., two 32-wide k-steps per block
#pragma unroll
    for (int ph = 0; ph < D / 64; ++ph) {
      Frag<T> qf[4][2];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          qf[rt][pp] = lds_frag8(&Qs[(16 * rt + l16) * SK + 64 * ph + 32 * pp + 8 * lg]);
        }
#pragma unroll
      for (int pp = 0; pp < 2; ++pp)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
          for (int dt = 0; dt < NT; ++dt) ot[dt][rt] = mfma(sf[2 * ph + pp][dt], qf[rt][pp], ot[dt][rt]);
    }

    if constexpr (MODE == 1) {
      // ... + V^T A^T
      {
        Frag<T> vf[NT][2], af[4][2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
#pragma unroll
          for (int dt = 0; dt < NT; ++dt) vf[dt][p] = lds_frag8(&VTs[(cw + 16 * dt + l16) * SC + 32 * p + 8 * lg]);
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) af[rt][p] = lds_frag8(&Aqs[(16 * rt + l16) * SC + 32 * p + 8 * lg]);
        }
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int dt = 0; dt < NT; ++dt) ot[dt][rt] = mfma(vf[dt][p], af[rt][p], ot[dt][rt]);
      }
      // S = 2^{G_C} o_rows S + (K 2^{G_C - G})^T V
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const f32x4 dec = *reinterpret_cast<const f32x4*>(&gate[16 * mt + 4 * lg]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) S[mt][nt] *= dec;
      }
      Frag<T> vb[2][NT];
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) vb[p][nt] = lds_frag8(&VTs[(cw + 16 * nt + l16) * SC + 32 * p + 8 * lg]);
#pragma unroll
      for (int m4 = 0; m4 < MT / 4; ++m4) {
        Frag<T> kf[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int p = 0; p < 2; ++p) kf[i][p] = lds_frag8(&KTs[(16 * (4 * m4 + i) + l16) * SC + 32 * p + 8 * lg]);
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) S[4 * m4 + i][nt] = mfma(kf[i][p], vb[p][nt], S[4 * m4 + i][nt]);
      }
    } else {
      const float* gam = gate + kC;
      // U = Tm diag(b) V - Wm S   (tokens x columns); the same in both delta modes
      f32x4 U[4][NT];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) U[mt][nt] = zero4();
      {
        Frag<T> vf[2][NT], tf[4][2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) vf[p][nt] = lds_frag8(&VTs[(cw + 16 * nt + l16) * SC + 32 * p + 8 * lg]);
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) tf[mt][p] = lds_frag8(&TBs[(16 * mt + l16) * SC + 32 * p + 8 * lg]);
        }
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) U[mt][nt] = mfma(tf[mt][p], vf[p][nt], U[mt][nt]);
      }
#pragma unroll
      for (int ph = 0; ph < D / 64; ++ph) {
        Frag<T> wf[4][2];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int pp = 0; pp < 2; ++pp) {
            wf[mt][pp] = lds_frag8(&Wms[(16 * mt + l16) * SK + 64 * ph + 32 * pp + 8 * lg]);
          }
#pragma unroll
        for (int pp = 0; pp < 2; ++pp)
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) U[mt][nt] = mfma(wf[mt][pp], sf[2 * ph + pp][nt], U[mt][nt]);
      }
      // O^T: (scalar gate) scale the S^T Q^T part by gamma of each query
      // column, then + U^T A^T
      if constexpr (!DGD) {
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          const float gq = gam[16 * rt + l16];
#pragma unroll
          for (int dt = 0; dt < NT; ++dt) ot[dt][rt] *= gq;
        }
      }
      // U as operand: plain, and (scalar gate) scaled by gamma_C / gamma_s
      Frag<T> uf[2][NT], us[2][NT];
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        f32x4 s0, s1;
        if constexpr (!DGD) {
          const float lgC = gate[kC - 1];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            s0[i] = __builtin_amdgcn_exp2f(fminf(lgC - gate[32 * pp + 4 * lg + i], 0.f));
            s1[i] = __builtin_amdgcn_exp2f(fminf(lgC - gate[32 * pp + 16 + 4 * lg + i], 0.f));
          }
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          uf[pp][nt] = frag_from_acc<T>(U[2 * pp][nt], U[2 * pp + 1][nt]);
          us[pp][nt] = DGD ? uf[pp][nt] : frag_from_acc_scaled<T>(U[2 * pp][nt], U[2 * pp + 1][nt], s0, s1);
        }
      }
      {
        Frag<T> af[4][2];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
          for (int pp = 0; pp < 2; ++pp) {
            af[rt][pp] = lds_frag8(&Aqs[(16 * rt + l16) * SC + 32 * pp + 8 * lg]);
          }
#pragma unroll
        for (int pp = 0; pp < 2; ++pp)
#pragma unroll
          for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int dt = 0; dt < NT; ++dt) ot[dt][rt] = mfma(uf[pp][dt], af[rt][pp], ot[dt][rt]);
      }
      // S = gamma_C S + K^T diag(gamma_C / gamma) U; diagonal gate:
      // S = 2^{G_C} o_rows S + (K 2^{G_C - G})^T U
      if constexpr (DGD) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const f32x4 dec = *reinterpret_cast<const f32x4*>(&gate[16 * mt + 4 * lg]);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) S[mt][nt] *= dec;
        }
      } else {
        const float gC = gam[kC - 1];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) S[mt][nt] *= gC;
      }
#pragma unroll
      for (int m4 = 0; m4 < MT / 4; ++m4) {
        Frag<T> kf[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int pp = 0; pp < 2; ++pp) {
            kf[i][pp] = lds_frag8(&KTs[(16 * (4 * m4 + i) + l16) * SC + 32 * pp + 8 * lg]);
          }
#pragma unroll
        for (int pp = 0; pp < 2; ++pp)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
              S[4 * m4 + i][nt] = mfma(kf[i][pp], us[pp][nt], S[4 * m4 + i][nt]);
      }
    }

    // ---- store (or add) the chunk's linear output rows
    if (flags & 1) {
      const bool accumulate = (flags & 8) != 0;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const int r = 16 * rt + l16;
        if (r < Cc) {
          T* orow = o + ((size_t)(bi * T_ + i0 + r + window) * H + h) * D + c0 + cw;
#pragma unroll
          for (int dt = 0; dt < NT; ++dt) {
            f32x4 val = ot[dt][rt] * w_lin;
            if (accumulate) val += load4(orow + 16 * dt + 4 * lg);
            store4(orow + 16 * dt + 4 * lg, val);
          }
        }
      }
    }
  }

  // linear-only overwrite: rows t < n_sink + window carry no linear output
  if ((flags & 1) && !(flags & 2) && !(flags & 8)) {
    const int rows = min(n_sink + window, T_);
    for (int i = tid; i < rows * (DVS / 4); i += kThreads) {
      const int t = i / (DVS / 4);
      const int cc = (i % (DVS / 4)) * 4;
      store4(o + ((size_t)(bi * T_ + t) * H + h) * D + c0 + cc, zero4());
    }
  }

  if (flags & 4) {
    float* Sg = state_out + (size_t)(bi * H + h) * D * D;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          Sg[(size_t)(16 * mt + 4 * lg + i) * D + c0 + cw + 16 * nt + l16] = S[mt][nt][i];
  }
}

template <class T, int D, int NW, int DW, int MODE>
hipError_t launch_linear_t(const PrefillArgs& p, hipStream_t s) {
  using SM = Smem<T, D, NW, DW, MODE>;
  auto kern = linear_chunk_kernel<T, D, NW, DW, MODE>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, SM::bytes);
  if (e != hipSuccess) return e;
  // x: the (column slice, query head) members of each KV head, placed by
  // xcd_grouped (a multiple of 8 wide, so the XCD of a workgroup is x mod 8
  // in every row); y: the sequence
  const dim3 grid(xcd_grouped_grid(p.Hkv, (D / SM::DVS) * (p.H / p.Hkv)), p.B);
  const int nch = gdn_stream_chunks(p.T, p.n_sink, p.window);
  const T* w0;
  const T* w1;
  const T* w2 = nullptr;
  const T* w3 = nullptr;
  const T* w4 = nullptr;
  const float* wf;
  if (MODE != 0) {
    const GlaWorkspace w = gla_workspace_layout(p.workspace, p.B, p.H, nch, D, sizeof(T), MODE == 2);
    w0 = (const T*)w.qg;
    w1 = (const T*)w.ktg;
    w2 = (const T*)w.a;
    w3 = (const T*)w.tb;
    w4 = (const T*)w.wm;
    wf = w.egc;
  } else {
    const GdnWorkspace w = gdn_workspace_layout(p.workspace, p.B, p.H, nch, D, sizeof(T), false);
    w0 = (const T*)w.tb;
    w1 = nullptr;   // Tm diag(b gamma) is formed from TB and gamma
    wf = w.g;
  }
  hipLaunchKernelGGL(kern, grid, dim3(64 * NW), SM::bytes, s, (const T*)p.q, (const T*)p.k,
                     (const T*)p.v, w0, w1, w2, w3, w4, wf, (T*)p.o, p.state_out, p.T, p.H, p.Hkv,
                     p.n_sink, p.window, p.flags, p.w_lin, (T*)p.ckpt);
  return hipGetLastError();
}

template <class T, int D, int NW, int MODE>
hipError_t launch_linear_f(const PrefillArgs& p, hipStream_t s) {
  return launch_linear_t<T, D, NW, 16, MODE>(p, s);
}

// 16 state columns per wave.  d = 128: one workgroup of 8 waves per chain
// when there are enough chains to fill the GPU, else two workgroups of 4
// waves per chain.  d = 64: one workgroup of 4 waves.
template <class T, int MODE>
hipError_t launch_linear_d(const PrefillArgs& p, hipStream_t s) {
  if (p.D == 64) return launch_linear_f<T, 64, 4, MODE>(p, s);
  if ((size_t)p.B * p.H >= 256) return launch_linear_f<T, 128, 8, MODE>(p, s);
  return launch_linear_f<T, 128, 4, MODE>(p, s);
}

// bf16: d = 64 or 128; fp32: d = 64 only (its state tiles fit LDS only there)
template <class T, int MODE>
hipError_t launch_linear_dt(const PrefillArgs& p, hipStream_t s) {
  if constexpr (sizeof(T) == 2) return launch_linear_d<T, MODE>(p, s);
  else return launch_linear_f<T, 64, 4, MODE>(p, s);
}

template <class T>
hipError_t launch_linear_m(const PrefillArgs& p, hipStream_t s) {
  if (!p.gla) return launch_linear_dt<T, 0>(p, s);
  return p.dgd ? launch_linear_dt<T, 2>(p, s) : launch_linear_dt<T, 1>(p, s);
}

}  // namespace

hipError_t launch_linear_ckpt(const PrefillArgs& p, hipStream_t s) {
  if (!p.bf16 || p.gla || p.D != 128 || !p.ckpt) return hipErrorInvalidValue;
  return launch_linear_d<bf16, 0>(p, s);
}

bool separate_preparation(const PrefillArgs& p) {
  return gdn_stream_chunks(p.T, p.n_sink, p.window) > 0 &&
         (p.gla || !gdn_full_prep(p.B, p.H, p.D, p.bf16) || gdn_segmented(p));
}

hipError_t launch_preparation(const PrefillArgs& p, hipStream_t s) {
  const int nch = gdn_stream_chunks(p.T, p.n_sink, p.window);
  return p.gla ? launch_gla_prep(p, nch, s) : launch_gdn_prep(p, nch, s);
}

hipError_t launch_linear_prefill(const PrefillArgs& p, hipStream_t s, bool* swa_done) {
  if (swa_done) *swa_done = false;
  const int nch = gdn_stream_chunks(p.T, p.n_sink, p.window);
  if (gdn_segmented(p)) {
    if (swa_done) *swa_done = true;
    return launch_gdn_segmented(p, s);
  }
  if (!p.gla && gdn_full_prep(p.B, p.H, p.D, p.bf16)) return launch_gdn_full(p, nch, s, swa_done);
  if (gdn_layer_applies(p)) {
    if (swa_done) *swa_done = true;
    return launch_gdn_layer(p, s);
  }
  if (gdn_linear_layer_applies(p)) return launch_gdn_linear_layer(p, s);
  if (nch > 0 && !p.prepared) {
    const hipError_t e = p.gla ? launch_gla_prep(p, nch, s) : launch_gdn_prep(p, nch, s);
    if (e != hipSuccess) return e;
  }
  if (p.bf16) return launch_linear_m<bf16>(p, s);
  if (p.D != 64) return hipErrorInvalidValue;   // fp32 state tiles fit LDS only at d = 64
  return launch_linear_m<float>(p, s);
}

}  // namespace gdn
