// Chunk preparation for the chunked GLA variant (prefill): everything about a
// 64-token chunk that does not depend on the recurrent state, done for every
// chunk at once so that the sequential scan only keeps the state products.
//
// Method (page "The Key to Going Linear: Analysis-Driven Transformer
// Linearization", section 线性注意力替换机制): GLA update
// S_i = Diag(alpha_i) S_{i-1} + k_i v_i^T with a per-channel forget gate.
// Over a chunk with G_r = inclusive cumsum of log2 alpha (per channel), the
// chunk is exact with
//   O   = (Q 2^G) S0 + A V,   A_rs = [s <= r] sum_c q_r[c] k_s[c] 2^{G_r[c] - G_s[c]}
//   S   = 2^{G_C} o_rows S0 + (K 2^{G_C - G})^T V.
// Outputs per chunk (workspace, element type T unless noted):
//   QG  [64][D]   Q 2^G, columns in acc order (the scan's Q tile layout);
//   KTG [D][64]   (K 2^{G_C - G})^T, tokens in acc order;
//   A   [64][64]  the masked intra-chunk scores, columns in acc order;
//   EGC [D] fp32  2^{G_C}.
// All three operand tiles are bounded by 1 per channel factor.  A needs
// 2^{G_r - G_s}, which would leave the float range if split as
// 2^{G_r} 2^{-G_s} against the chunk start, so each 16-row tile j takes the
// cumulative gate at its row 16j + 7 as reference point M_j: the operands
// q_r 2^{G_r - M_j} and k_s 2^{M_j - G_s} grow by at most the decay of 8
// tokens (clamped at 2^115), and a pair of different tiles (mt > nt) takes the
// per-channel factor 2^{M_mt - M_nt} <= 1 on its key operand.
//
// The delta rule with the same diagonal gate (section 线性注意力替换机制,
// the GDN update with G_t diagonal: S_i = (I - b_i k_i k_i^T) Diag(alpha_i)
// S_{i-1} + b_i k_i v_i^T) is exact over a chunk with
//   L_rs = b_r sum_c k_r[c] k_s[c] 2^{G_r[c] - G_s[c]} (s < r),
//   TB = (I + L)^-1 diag(b),  U = TB V - TB (K 2^G) S0,
//   O  = (Q 2^G) S0 + A U,    S = 2^{G_C} o_rows S0 + (K 2^{G_C - G})^T U,
// derived by unrolling the update over the chunk; L is formed like A (k in
// place of q, the same reference points), the unit lower-triangular inverse
// as in the scalar-gate preparation, and the preparation also writes TB and
// -Wm = -TB (K 2^G).
//
// One workgroup of 8 waves per (chunk, query head, sequence).

#include "common.h"
#include "gdn_prep.h"
#include "launch.h"

namespace gdn {
namespace {

constexpr int kC = 64;
__constant__ const int kGlaTileM[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
__constant__ const int kGlaTileN[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};

template <class T, int D, bool DELTA>
struct GlaPrepSmem {
  static constexpr int PAD = 16 / sizeof(T);
  static constexpr int SK = D + PAD;      // stride of [64][D] tiles
  static constexpr int SC = kC + PAD;     // stride of [*][64] tiles
  static constexpr int oQD = 0;                       // q 2^{G - M}
  static constexpr int oKD = oQD + kC * SK;           // k 2^{M - G}
  // one region, first the cumulative log2 gates (fp32 [64][D]), then, once
  // they are no longer read, K^T 2^{G_C - G} [D][SC] and A [64][SC]
  static constexpr int oU = oKD + kC * SK;
  static constexpr int nG = kC * D;
  static constexpr int nGT = nG * 4 / (int)sizeof(T);   // the gates in T elements
  static constexpr int nKA = D * SC + kC * SC;
  static constexpr int nU = nGT > nKA ? nGT : nKA;
  static constexpr int oKT = oU;
  static constexpr int oA = oU + D * SC;
  // delta rule: k 2^{G - M} (L's left operand), (K 2^G)^T [D][SC], TB [64][SC]
  static constexpr int oKL = oU + nU;
  static constexpr int oKGT = oKL + (DELTA ? kC * SK : 0);
  static constexpr int oTB = oKGT + (DELTA ? D * SC : 0);
  static constexpr int nT = oTB + (DELTA ? kC * SC : 0);
  static constexpr int bytesT = (nT * (int)sizeof(T) + 15) / 16 * 16;
  static constexpr int nMf = 6 * D;                   // tile-pair factors
  // fp32: tile-pair factors, then (delta) the packed solve buffer and b
  static constexpr int nL = DELTA ? prep::PackedL::size : 0;
  static constexpr int bytes = bytesT + 4 * (nMf + nL + (DELTA ? kC : 0));
  static_assert((oU * (int)sizeof(T)) % 16 == 0, "gate region alignment");
  static_assert(((oKL * (int)sizeof(T)) % 16 == 0) && ((oKGT * (int)sizeof(T)) % 16 == 0) &&
                ((oTB * (int)sizeof(T)) % 16 == 0), "delta region alignment");
};

template <class T, int D, bool DELTA>
__global__ __launch_bounds__(512) void gla_prep_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const float* __restrict__ a,
    const float* __restrict__ b, T* __restrict__ wqg, T* __restrict__ wktg, T* __restrict__ wa,
    float* __restrict__ wegc, T* __restrict__ wtb, T* __restrict__ wwm, int B_, int T_, int H,
    int Hkv, int n_sink, int window, int nch) {
  using SM = GlaPrepSmem<T, D, DELTA>;
  constexpr int NTH = 512;
  constexpr int SK = SM::SK;
  constexpr int SC = SM::SC;
  constexpr int VEC = 16 / (int)sizeof(T);
  typedef typename Vec16<T>::type V16;

  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  T* sT = reinterpret_cast<T*>(smem_raw);
  T* QDs = sT + SM::oQD;
  T* KDs = sT + SM::oKD;
  T* KTs = sT + SM::oKT;
  T* As = sT + SM::oA;
  float* Gl = reinterpret_cast<float*>(sT + SM::oU);              // [64][D], aliases K^T and A
  float* Mf = reinterpret_cast<float*>(smem_raw + SM::bytesT);    // [6][D], acc order
  T* KLs = sT + SM::oKL;                                          // delta: k 2^{G - M}
  T* KGTs = sT + SM::oKGT;                                        // delta: (K 2^G)^T
  T* TBs = sT + SM::oTB;                                          // delta: TB
  float* Lf = Mf + SM::nMf;                                       // delta: solve buffer
  float* bet = Lf + SM::nL;                                       // delta: b

  // the query heads of one KV head run back to back on one XCD (shared K)
  const int G = H / Hkv;
  int unit, member;
  if (!xcd_grouped(blockIdx.x, G, B_ * Hkv * nch, unit, member)) return;
  const int c = unit % nch;
  const int g = (unit / nch) % Hkv;
  const int bi = unit / (nch * Hkv);
  const int h = g * G + member;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = wave_id();
  const int l16 = lane & 15;
  const int lg = lane >> 4;
  const int iend = T_ - window;
  const int i0 = n_sink + c * kC;
  const size_t ci = ((size_t)bi * H + h) * nch + c;

  // ---- all global loads of the chunk first (gates, q rows, k rows), so
  // their latency overlaps; b = 0 past the stream end (as a = 1 there)
  if (DELTA && tid < kC) bet[tid] = i0 + tid < iend ? b[(size_t)(bi * T_ + i0 + tid) * H + h] : 0.f;
  constexpr int NA4 = kC * D / 4 / NTH;            // f32x4 gate pieces per thread
  constexpr int NPC = kC * D / VEC / NTH;          // 16-byte q / k pieces per thread
  static_assert(kC * D / 4 % NTH == 0 && kC * D / VEC % NTH == 0, "staging");
  f32x4 ga[NA4];
  V16 qv[NPC], kv[NPC];
  const T* qbase = q + ((size_t)(bi * T_ + i0 + window) * H + h) * D;
  const T* kbase = k + ((size_t)(bi * T_ + i0) * Hkv + g) * D;
#pragma unroll
  for (int j = 0; j < NA4; ++j) {
    const int idx = tid + j * NTH;
    const int r = idx / (D / 4);
    const int cc = (idx % (D / 4)) * 4;
    ga[j] = i0 + r < iend ? *reinterpret_cast<const f32x4*>(a + ((size_t)(bi * T_ + i0 + r) * H + h) * D + cc)
                          : f32x4{1.f, 1.f, 1.f, 1.f};
  }
#pragma unroll
  for (int j = 0; j < NPC; ++j) {
    const int idx = tid + j * NTH;
    const int r = idx / (D / VEC);
    const int cc = (idx % (D / VEC)) * VEC;
    if (i0 + r < iend) {
      qv[j] = *reinterpret_cast<const V16*>(qbase + (size_t)r * H * D + cc);
      kv[j] = *reinterpret_cast<const V16*>(kbase + (size_t)r * Hkv * D + cc);
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        qv[j][e] = from_f32<T>(0.f);
        kv[j][e] = from_f32<T>(0.f);
      }
    }
  }

  // ---- log2 gates, then the per-channel inclusive prefix over the 64 rows:
  // each thread owns one channel and a run of rows
  constexpr int SEG = NTH / D;             // row segments per channel
  constexpr int RPS = kC / SEG;            // rows per segment
#pragma unroll
  for (int j = 0; j < NA4; ++j) {
    const int idx = tid + j * NTH;
    const int r = idx / (D / 4);
    const int cc = (idx % (D / 4)) * 4;
    f32x4 x;
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = __builtin_amdgcn_logf(ga[j][e]);
    *reinterpret_cast<f32x4*>(&Gl[r * D + cc]) = x;
  }
  __syncthreads();
  {
    const int cc = tid % D;
    const int seg = tid / D;
    float run = 0.f;
    float vals[RPS];
#pragma unroll
    for (int j = 0; j < RPS; ++j) vals[j] = Gl[(seg * RPS + j) * D + cc];
#pragma unroll
    for (int j = 0; j < RPS; ++j) {
      run += vals[j];
      vals[j] = run;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < RPS; ++j) Gl[(seg * RPS + j) * D + cc] = vals[j];
    __syncthreads();
    float off = 0.f;
    for (int s2 = 0; s2 < seg; ++s2) off += Gl[((s2 + 1) * RPS - 1) * D + cc];
    __syncthreads();
    if (seg > 0) {
#pragma unroll
      for (int j = 0; j < RPS; ++j) Gl[(seg * RPS + j) * D + cc] = vals[j] + off;
    }
  }
  __syncthreads();

  // ---- scaled operands: Q 2^G (to the workspace), q 2^{G - M}, k 2^{M - G}
  // (LDS, for A) and K^T 2^{G_C - G} (kept in registers until the gates'
  // LDS region is free, then LDS, copied out below); VEC channels of one row
  // per piece, written as runs of 4 (contiguous in acc order)
  T* qg = wqg + ci * (kC * D);
  T ktr[NPC][VEC];
  T kgr[DELTA ? NPC : 1][VEC];
#pragma unroll
  for (int j = 0; j < NPC; ++j) {
    const int idx = tid + j * NTH;
    const int r = idx / (D / VEC);
    const int cb = (idx % (D / VEC)) * VEC;
#pragma unroll
    for (int m = 0; m < VEC / 4; ++m) {
      const int cc = cb + 4 * m;
      const int pc = acc_pos(cc);
      const f32x4 G4 = *reinterpret_cast<const f32x4*>(&Gl[r * D + cc]);
      const f32x4 M4 = *reinterpret_cast<const f32x4*>(&Gl[((r & ~15) + 7) * D + cc]);
      const f32x4 C4 = *reinterpret_cast<const f32x4*>(&Gl[(kC - 1) * D + cc]);
      f32x4 qo, qd, kd, kt, kl, kg;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const float qx = to_f32(qv[j][4 * m + x]);
        const float kx = to_f32(kv[j][4 * m + x]);
        qo[x] = qx * __builtin_amdgcn_exp2f(G4[x]);
        qd[x] = qx * __builtin_amdgcn_exp2f(fminf(G4[x] - M4[x], 115.f));
        kd[x] = kx * __builtin_amdgcn_exp2f(fminf(M4[x] - G4[x], 115.f));
        kt[x] = kx * __builtin_amdgcn_exp2f(fminf(C4[x] - G4[x], 0.f));
        kl[x] = kx * __builtin_amdgcn_exp2f(fminf(G4[x] - M4[x], 115.f));
        kg[x] = kx * __builtin_amdgcn_exp2f(G4[x]);
      }
      store4(qg + r * D + pc, qo);
      store4(&QDs[r * SK + pc], qd);
      store4(&KDs[r * SK + pc], kd);
      if constexpr (DELTA) {
        store4(&KLs[r * SK + pc], kl);
#pragma unroll
        for (int x = 0; x < 4; ++x) kgr[j][4 * m + x] = from_f32<T>(kg[x]);
      }
#pragma unroll
      for (int x = 0; x < 4; ++x) ktr[j][4 * m + x] = from_f32<T>(kt[x]);
    }
  }
  // tile-pair factors 2^{M_mt - M_nt}, pair index mt (mt - 1) / 2 + nt
  for (int i = tid; i < 6 * D; i += NTH) {
    const int pr = i / D;
    const int cc = i % D;
    const int mt = pr < 1 ? 1 : (pr < 3 ? 2 : 3);
    const int nt = pr - mt * (mt - 1) / 2;
    Mf[pr * D + acc_pos(cc)] = __builtin_amdgcn_exp2f(Gl[(16 * mt + 7) * D + cc] - Gl[(16 * nt + 7) * D + cc]);
  }
  if (tid < D) wegc[ci * D + tid] = __builtin_amdgcn_exp2f(Gl[(kC - 1) * D + tid]);
  __syncthreads();   // the gates are no longer read: their region takes K^T and A
#pragma unroll
  for (int j = 0; j < NPC; ++j) {
    const int idx = tid + j * NTH;
    const int r = idx / (D / VEC);
    const int cb = (idx % (D / VEC)) * VEC;
#pragma unroll
    for (int e = 0; e < VEC; ++e) KTs[(cb + e) * SC + acc_pos(r)] = ktr[j][e];
    if constexpr (DELTA) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) KGTs[(cb + e) * SC + acc_pos(r)] = kgr[j][e];
    }
  }

  // ---- A = [s <= r] 2^{G_r - G_s} o (Q K^T) on the 10 lower tiles
  for (int job = wv; job < 10; job += NTH / 64) {
    const int mt = kGlaTileM[job];
    const int nt = kGlaTileN[job];
    f32x4 acc = zero4();
    if (mt == nt) {
#pragma unroll
      for (int p = 0; p < D / 32; ++p)
        acc = mfma(lds_frag8(&QDs[(16 * mt + l16) * SK + 32 * p + 8 * lg]),
                   lds_frag8(&KDs[(16 * nt + l16) * SK + 32 * p + 8 * lg]), acc);
    } else {
      const float* mf = Mf + (mt * (mt - 1) / 2 + nt) * D;
#pragma unroll
      for (int p = 0; p < D / 32; ++p)
        acc = mfma(lds_frag8(&QDs[(16 * mt + l16) * SK + 32 * p + 8 * lg]),
                   lds_frag8_scaled(&KDs[(16 * nt + l16) * SK + 32 * p + 8 * lg], mf + 32 * p + 8 * lg),
                   acc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * mt + 4 * lg + i;
      const int s = 16 * nt + l16;
      As[r * SC + acc_pos(s)] = from_f32<T>(s <= r ? acc[i] : 0.f);
    }
  }
  // delta rule: L = strictly lower (b_r k_r . k_s 2^{G_r - G_s}) on the same
  // tiles, into the packed fp32 solve buffer (zero on and above the diagonal)
  if constexpr (DELTA) {
    for (int job = wv; job < 10; job += NTH / 64) {
      const int mt = kGlaTileM[job];
      const int nt = kGlaTileN[job];
      f32x4 acc = zero4();
      if (mt == nt) {
#pragma unroll
        for (int p = 0; p < D / 32; ++p)
          acc = mfma(lds_frag8(&KLs[(16 * mt + l16) * SK + 32 * p + 8 * lg]),
                     lds_frag8(&KDs[(16 * nt + l16) * SK + 32 * p + 8 * lg]), acc);
      } else {
        const float* mf = Mf + (mt * (mt - 1) / 2 + nt) * D;
#pragma unroll
        for (int p = 0; p < D / 32; ++p)
          acc = mfma(lds_frag8(&KLs[(16 * mt + l16) * SK + 32 * p + 8 * lg]),
                     lds_frag8_scaled(&KDs[(16 * nt + l16) * SK + 32 * p + 8 * lg], mf + 32 * p + 8 * lg),
                     acc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * mt + 4 * lg + i;
        const int s2 = 16 * nt + l16;
        Lf[prep::lidx<prep::PackedL>(r, s2)] = s2 < r ? bet[r] * acc[i] : 0.f;
      }
    }
  }
  // the strictly upper tiles of A are zero
  for (int i = tid; i < 6 * 16 * 16; i += NTH) {
    const int pr = i / 256;
    const int e = i % 256;
    const int mt = pr < 3 ? 0 : (pr < 5 ? 1 : 2);
    const int nt = pr < 3 ? pr + 1 : (pr < 5 ? pr - 1 : 3);
    As[(16 * mt + e / 16) * SC + acc_pos(16 * nt + e % 16)] = from_f32<T>(0.f);
  }
  __syncthreads();

  // ---- copy K^T 2^{G_C - G} and A out as 16-byte pieces (delta rule: by
  // waves 1 .. 7 while wave 0 solves for TB; the solve and what follows it
  // touch neither tile)
  {
    const int t0 = DELTA ? tid - 64 : tid;
    const int nth = DELTA ? NTH - 64 : NTH;
    if (t0 >= 0) {
      T* ktg = wktg + ci * (D * kC);
      T* aa = wa + ci * (kC * kC);
      for (int i = t0; i < D * kC / VEC; i += nth) {
        const int r = i / (kC / VEC);
        const int pc = (i % (kC / VEC)) * VEC;
        *reinterpret_cast<V16*>(ktg + r * kC + pc) = *reinterpret_cast<const V16*>(&KTs[r * SC + pc]);
      }
      for (int i = t0; i < kC * kC / VEC; i += nth) {
        const int r = i / (kC / VEC);
        const int pc = (i % (kC / VEC)) * VEC;
        *reinterpret_cast<V16*>(aa + r * kC + pc) = *reinterpret_cast<const V16*>(&As[r * SC + pc]);
      }
    }
  }

  if constexpr (DELTA) {
    // ---- TB = (I + L)^-1 diag(b) (one wave solves), then -Wm = -TB (K 2^G)
    if (wv == 0) prep::unit_lower_inverse_wave<prep::PackedL>(Lf, lane);
    __syncthreads();
    T* tb = wtb + ci * (kC * kC);
    for (int i = tid; i < kC * kC / 4; i += NTH) {
      const int r = i >> 4;
      const int s0 = (i & 15) * 4;
      const f32x4 tm = (s0 >> 4) <= (r >> 4) ? *reinterpret_cast<const f32x4*>(&Lf[prep::lidx<prep::PackedL>(r, s0)])
                                             : zero4();
      const f32x4 x = tm * *reinterpret_cast<const f32x4*>(&bet[s0]);
      store4(&TBs[r * SC + acc_pos(s0)], x);
      store4(tb + r * kC + acc_pos(s0), x);
    }
    __syncthreads();
    // Wm tile (token rows 16 rt.., d_k columns 16 ct..): TB rows x (K 2^G)^T
    // columns, reduced over the chunk's tokens (acc order in both tiles);
    // staged as [token][d_k in acc order] in the free q 2^{G - M} area
    T* Wst = QDs;
    for (int tile = wv; tile < 4 * (D / 16); tile += NTH / 64) {
      const int rt = tile & 3;
      const int ct = tile >> 2;
      f32x4 acc = zero4();
#pragma unroll
      for (int p = 0; p < 2; ++p)
        acc = mfma(lds_frag8(&TBs[(16 * rt + l16) * SC + 32 * p + 8 * lg]),
                   lds_frag8(&KGTs[(16 * ct + l16) * SC + 32 * p + 8 * lg]), acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) Wst[(16 * rt + 4 * lg + i) * SK + acc_pos(16 * ct + l16)] = from_f32<T>(-acc[i]);
    }
    __syncthreads();
    T* wm = wwm + ci * (kC * D);
    for (int i = tid; i < kC * D / VEC; i += NTH) {
      const int r = i / (D / VEC);
      const int pc = (i % (D / VEC)) * VEC;
      *reinterpret_cast<V16*>(wm + r * D + pc) = *reinterpret_cast<const V16*>(&Wst[r * SK + pc]);
    }
  }

}

template <class T, int D, bool DELTA>
hipError_t launch_gla_prep_t(const PrefillArgs& p, int nch, hipStream_t s) {
  using SM = GlaPrepSmem<T, D, DELTA>;
  auto kern = gla_prep_kernel<T, D, DELTA>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, SM::bytes);
  if (e != hipSuccess) return e;
  const GlaWorkspace w = gla_workspace_layout(p.workspace, p.B, p.H, nch, D, sizeof(T), DELTA);
  hipLaunchKernelGGL(kern, dim3(xcd_grouped_grid((long long)p.B * p.Hkv * nch, p.H / p.Hkv)), dim3(512), SM::bytes, s, (const T*)p.q,
                     (const T*)p.k, p.a, p.b, (T*)w.qg, (T*)w.ktg, (T*)w.a, w.egc, (T*)w.tb, (T*)w.wm, p.B, p.T,
                     p.H, p.Hkv, p.n_sink, p.window, nch);
  return hipGetLastError();
}

template <class T, int D>
hipError_t launch_gla_prep_d(const PrefillArgs& p, int nch, hipStream_t s) {
  return p.dgd ? launch_gla_prep_t<T, D, true>(p, nch, s) : launch_gla_prep_t<T, D, false>(p, nch, s);
}

}  // namespace

GlaWorkspace gla_workspace_layout(void* base, int B, int H, int nch, int D, size_t elt, bool delta) {
  GlaWorkspace w;
  const size_t n = (size_t)B * H * nch;
  unsigned char* p = static_cast<unsigned char*>(base);
  w.qg = p;
  w.ktg = p + n * kC * D * elt;
  w.a = p + 2 * n * kC * D * elt;
  w.egc = reinterpret_cast<float*>(p + 2 * n * kC * D * elt + n * kC * kC * elt);
  size_t off = 2 * n * kC * D * elt + n * kC * kC * elt + n * D * sizeof(float);
  off = (off + 255) / 256 * 256;
  w.tb = delta ? p + off : nullptr;
  off += delta ? n * kC * kC * elt : 0;
  w.wm = delta ? p + off : nullptr;
  off += delta ? n * kC * D * elt : 0;
  w.bytes = off;
  return w;
}

hipError_t launch_gla_prep(const PrefillArgs& p, int nch, hipStream_t s) {
  if (p.bf16) return p.D == 64 ? launch_gla_prep_d<bf16, 64>(p, nch, s) : launch_gla_prep_d<bf16, 128>(p, nch, s);
  return p.D == 64 ? launch_gla_prep_d<float, 64>(p, nch, s) : launch_gla_prep_d<float, 128>(p, nch, s);
}

}  // namespace gdn
