// The whole hybrid layer (prefill, bf16, d = 128) in one pass over q, k, v
// for many (sequence, head) chains: the chunked gated-delta-rule state scan
// and the sink + sliding-window softmax of the same output rows, summed in
// the epilogue, so that q, k and v are read once and o is written once.
//
// Method (page "The Key to Going Linear: Analysis-Driven Transformer
// Linearization"): section 线性注意力替换机制 gives the gated delta rule
// S_i = a_i (I - b_i k_i k_i^T) S_{i-1} + b_i k_i v_i^T; section
// 填补近似缺口的实用设计 keeps n_sink sink tokens and a window of the most
// recent tokens in softmax attention and lets the recurrence cover the rest,
// read with lag `window`: o[t] = S^(t-window)^T q_t + softmax over
// A(t) = { i <= t : i < n_sink or i > t - window }, logits q.k / sqrt(d)
// (section 从 softmax 到 delta 规则的一阶近似).
//
// Chunk form (64 stream tokens i0 .. i0+63, i0 = n_sink + 64 c; g = the
// inclusive prefix sum of log2 a inside the chunk, gamma = 2^g; TB =
// (I + L)^-1 diag(b) from the preparation kernel; derived by unrolling the
// recurrence over the chunk):
//   U = TB V - TB diag(gamma) (K S)           (tokens x d_v)
//   O = diag(gamma) Q S + A U,  A_rs = [s <= r] 2^{g_r - g_s} q_r.k_s
//   S <- gamma_C S + K^T diag(gamma_C / gamma) U
// where Q holds the lagged query rows t = i0 + window + r.  The softmax rows
// of the same chunk attend to the keys (i0 + r, i0 + r + window] and the
// sinks: keys of stream chunks c, c + 1, c + 2 when window <= 128.
//
// Work split: one workgroup of 8 waves per chain.  Waves 0-3 own 32 state
// columns each as fp32 MFMA accumulators for the whole sequence and run the
// state-dependent products.  Waves 4-7 own 16 output rows each: they form
// the chunk's query-key scores (the lower triangle, decayed, is the score
// tile A the state waves need; the rest feeds the softmax), run the softmax
// over the chunk's window and the sinks, add the state waves' rows (handed
// over through LDS) and store o.  They also prefetch the next chunk into
// registers and commit it to LDS at the chunk's end.  K and V rows sit in
// LDS as a ring of three chunks in natural row-major order; transposed
// operands (K^T for the state update, V^T for the value products) come from
// gfx950's transposing LDS reads (ds_read_b64_tr_b16), so no transposed copy
// is staged.  The state update's reduction over tokens therefore reads the
// ring directly, and the state's d_k rows stay in natural order.
//
// MFMA operand conventions (v_mfma_f32_16x16x32_bf16, lane l = 16 g + j):
// A fragment A[j][K_g], B fragment B[K_g][j], D[4 g + i][j]; every product
// here uses K_g = { 4g..4g+3, 16+4g..16+4g+3 } (+ 32 p), the set two stacked
// accumulator tiles provide (see common.h).  Tiles read with plain 16-byte
// LDS reads keep that set contiguous ("acc order": the query tile, TB, A);
// natural-order rows are read as two 8-byte pieces (K as an operand reduced
// over d) or through the transposing reads (K^T, V^T, V).

#include "common.h"
#include "launch.h"

namespace gdn {
namespace {

constexpr int kC = 64;           // chunk length
constexpr int kD = 128;          // head dimension
constexpr int kSR = kD + 8;      // row stride (elements) of [rows][128] tiles
constexpr int kSC = kC + 8;      // row stride of [64][64] tiles
constexpr int kSinkRows = 16;    // sink keys held in LDS (n_sink <= 16)
constexpr int kThreads = 512;

// LDS layout (bf16 elements, then fp32 gates)
constexpr int oKR = 0;                             // K ring [3][64][kSR]
constexpr int oVR = oKR + 3 * kC * kSR;            // V ring [3][64][kSR]
constexpr int oKS = oVR + 3 * kC * kSR;            // sink K [16][kSR]
constexpr int oVS = oKS + kSinkRows * kSR;         // sink V [16][kSR]
constexpr int oQ = oVS + kSinkRows * kSR;          // lagged queries [64][kSR] (acc order); then the hand-over rows
constexpr int oTB = oQ + kC * kSR;                 // TB [64][kSC] (acc order)
constexpr int oA = oTB + kC * kSC;                 // A [64][kSC] (acc order)
constexpr int nLdsT = oA + kC * kSC;
constexpr int kLdsBytes = nLdsT * 2 + 2 * kC * 4;  // + g (log2), gamma
static_assert(kLdsBytes <= 160 * 1024, "one workgroup per compute unit");

typedef __attribute__((address_space(3))) bf16x4* lds_bf16x4_ptr;

// Two transposing 8-byte LDS reads: lane (g, j) receives X[r0 + 4g + i][c0 + j]
// and X[r0 + 16 + 4g + i][c0 + j], i = 0..3, of the row-major bf16 tile X
// (row stride kSR): the operand X^T[c0 + j][K_g] (A side) or X[K_g][c0 + j]
// (B side).  Within each 16-lane group, lane 4 r + c1 addresses row
// r0 + 4g + r at columns c0 + 4 c1 .. + 3, and the hardware hands column
// c0 + j of the group's four rows to lane j.
__device__ __forceinline__ Frag<bf16> tr_frag(const bf16* X, int r0, int c0, int lane) {
  const int g = lane >> 4;
  const int j = lane & 15;
  const bf16* p0 = X + (r0 + 4 * g + (j >> 2)) * kSR + c0 + 4 * (j & 3);
  const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_ptr)(p0));
  const bf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_ptr)(p0 + 16 * kSR));
  Frag<bf16> f;
  f.v = bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return f;
}

// Natural-order row `row` of a [rows][128] tile as an operand reduced over d
// on the set 32 p + K_g (two 8-byte reads).
__device__ __forceinline__ Frag<bf16> row_frag(const bf16* X, int row, int p, int g) {
  return lds_frag44(X + row * kSR + 32 * p + 4 * g, X + row * kSR + 32 * p + 16 + 4 * g);
}

// Sum over lanes l, l^16, l^32, l^48 (the four lane groups of one column).
__device__ __forceinline__ float sum_lane_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float max_lane_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// One 32-key block of the softmax of a wave's 16 query rows: keys kk0 ..
// kk0 + 31 at rows r0 .. r0 + 31 of the tiles K, V (natural order).  half:
// the sink block, 16 rows holding keys 0 .. 15 of which those below n_sink
// are attended; otherwise ring keys (>= n_sink), attended inside the window.
struct KeyPair {
  const bf16* K;
  const bf16* V;
  int r0;
  int kk0;
  bool half;
};

// Softmax over up to NP key pairs for the queries t = t0 + j (lane column
// j), in two phases.  Phase 1 (sm_scores): the scores of the pairs not
// given (have[pair]) from the query fragments qf (S^T tiles: key 4g + i of
// each 16-key half, query j), masked keys set to -inf, and the row maximum.
// Phase 2 (sm_values): weights 2^((s - m) log2(e) / sqrt(d)), their sum (on
// the matrix cores, against a ones operand) and the O^T tiles (d = 16 dt +
// 4g + i, query j).  A pair every row attends in full needs no mask.
template <int NP>
__device__ __forceinline__ float sm_scores(const KeyPair (&kp)[NP], const bool (&use)[NP],
                                           f32x4 (&st)[NP][2], const bool (&have)[NP],
                                           const Frag<bf16> (&qf)[4], int t0, int n_sink,
                                           int window, int T_, int lane) {
  const int g = lane >> 4;
  const int j = lane & 15;
  const int t = t0 + j;
#pragma unroll
  for (int pi = 0; pi < NP; ++pi) {
    if (!use[pi] || have[pi]) continue;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      st[pi][hf] = zero4();
      if (hf == 1 && kp[pi].half) continue;
#pragma unroll
      for (int p = 0; p < 4; ++p) st[pi][hf] = mfma(row_frag(kp[pi].K, kp[pi].r0 + 16 * hf + j, p, g), qf[p], st[pi][hf]);
    }
  }
  float m = -INFINITY;
#pragma unroll
  for (int pi = 0; pi < NP; ++pi) {
    if (!use[pi]) continue;
    const int kk0 = kp[pi].kk0;
    // every key of a ring pair inside every row's window (t - window, t]
    const bool full = !kp[pi].half && kk0 > t0 + 15 - window && kk0 + 31 <= t0 && kk0 + 31 < T_;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (!full) {
          const int kk = kk0 + 16 * hf + 4 * g + i;
          // the sink pair holds keys 0 .. 15, of which only kk < n_sink are
          // sinks (the others, if any, are window keys held in the ring);
          // ring pairs hold keys >= n_sink, attended inside the window
          const bool on = kp[pi].half ? hf == 0 && kk < n_sink && kk <= t
                                      : kk <= t && kk < T_ && kk > t - window;
          if (!on) st[pi][hf][i] = -INFINITY;
        }
        m = fmaxf(m, st[pi][hf][i]);
      }
  }
  m = max_lane_groups(m);
  return m == -INFINITY ? 0.f : m;   // a row with no key (past the sequence): weights 0
}

template <int NP>
__device__ __forceinline__ void sm_values(const KeyPair (&kp)[NP], const bool (&use)[NP],
                                          const f32x4 (&st)[NP][2], float m, int lane,
                                          f32x4 (&oacc)[8], float& inv_l) {
  const float scale = kLog2e / sqrtf((float)kD);
  const float mb = -m * scale;
  Frag<bf16> ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones.v[e] = static_cast<bf16>(1.f);
  f32x4 lacc = zero4();
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) oacc[dt] = zero4();
#pragma unroll
  for (int pi = 0; pi < NP; ++pi) {
    if (!use[pi]) continue;
    f32x4 p0, p1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p0[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(st[pi][0][i], scale, mb));
      p1[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(st[pi][1][i], scale, mb));
    }
    const Frag<bf16> pf = frag_from_acc<bf16>(p0, p1);
    lacc = mfma(ones, pf, lacc);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      Frag<bf16> vf;
      if (kp[pi].half) {
        // the sink pair: its second half weighs 0, so it reads the first
        // 16 rows twice
        const int g = lane >> 4;
        const int j = lane & 15;
        const bf16* p0p = kp[pi].V + (kp[pi].r0 + 4 * g + (j >> 2)) * kSR + 16 * dt + 4 * (j & 3);
        const bf16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_ptr)(p0p));
        vf.v = bf16x8{x[0], x[1], x[2], x[3], x[0], x[1], x[2], x[3]};
      } else {
        vf = tr_frag(kp[pi].V, kp[pi].r0, 16 * dt, lane);
      }
      oacc[dt] = mfma(vf, pf, oacc[dt]);
    }
  }
  // the bf16 weights summed (the same rounding as the weights P V uses)
  inv_l = lacc[0] > 0.f ? 1.f / lacc[0] : 0.f;
}

__global__ __launch_bounds__(kThreads) void gdn_layer_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ w_tb, const float* __restrict__ w_g, bf16* __restrict__ o,
    float* __restrict__ state_out, int B, int T_, int H, int Hkv, int n_sink, int window,
    int nch, int write_state, float w_lin, float w_swa) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  bf16* sm = reinterpret_cast<bf16*>(smem_raw);
  bf16* KR = sm + oKR;
  bf16* VR = sm + oVR;
  bf16* KSk = sm + oKS;
  bf16* VSk = sm + oVS;
  bf16* Qs = sm + oQ;
  bf16* Xs = sm + oQ;             // hand-over rows (after the queries are read)
  bf16* TBs = sm + oTB;
  bf16* As = sm + oA;
  float* Gs = reinterpret_cast<float*>(smem_raw + nLdsT * 2);   // g[64], gamma[64]

  // the G query heads of a KV head are consecutive workgroups on one XCD
  // and share the K and V rows through its L2
  const int G = H / Hkv;
  int unit, member;
  if (!xcd_grouped(blockIdx.x, G, B * Hkv, unit, member)) return;
  const int bi = unit / Hkv;
  const int gk = unit % Hkv;
  const int h = gk * G + member;
  const size_t chain = (size_t)bi * H + h;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = wave_id();
  const int g = lane >> 4;
  const int j = lane & 15;
  const int iend = T_ - window;                   // stream tokens [n_sink, iend)
  const bool scan_wave = wv < 4;
  typedef bf16x8 V16;
  const size_t kvrow = (size_t)Hkv * kD;          // elements between tokens (k, v)
  const size_t qrow = (size_t)H * kD;             // elements between tokens (q, o)
  const bf16* kb = k + ((size_t)bi * T_ * Hkv + gk) * kD;
  const bf16* vb = v + ((size_t)bi * T_ * Hkv + gk) * kD;
  const bf16* qb = q + ((size_t)bi * T_ * H + h) * kD;
  bf16* ob = o + ((size_t)bi * T_ * H + h) * kD;
  V16 zero8;
#pragma unroll
  for (int e = 0; e < 8; ++e) zero8[e] = static_cast<bf16>(0.f);

  // ---------------------------------------------------------- staging
  // 16-byte piece n of a [64][128] tile: row n / 16, columns 8 (n % 16) ..
  // Rows past the sequence repeat its last row (one unconditional load per
  // piece, so the loads of a prefetch stay in flight together).  Their
  // values never count: such keys are masked in the softmax, such query rows
  // are not stored, and stream rows past the chunk's end meet zero rows and
  // columns of TB (the preparation sets b = 0 there), so they add nothing to
  // U, O or the state.
  auto load_rows = [&](const bf16* base, size_t stride, int row0, int n) -> V16 {
    const int r = min(row0 + (n >> 4), T_ - 1);
    const int cp = (n & 15) * 8;
    return *reinterpret_cast<const V16*>(base + (size_t)r * stride + cp);
  };
  auto put_row = [&](bf16* tile, int n, const V16& x) {
    *reinterpret_cast<V16*>(tile + (n >> 4) * kSR + (n & 15) * 8) = x;
  };
  auto put_q = [&](int n, const V16& x) {      // query columns in acc order (runs of 4)
    const int r = n >> 4;
    const int cp = (n & 15) * 8;
    *reinterpret_cast<bf16x4*>(Qs + r * kSR + acc_pos(cp)) = bf16x4{x[0], x[1], x[2], x[3]};
    *reinterpret_cast<bf16x4*>(Qs + r * kSR + acc_pos(cp + 4)) = bf16x4{x[4], x[5], x[6], x[7]};
  };
  auto tb_of = [&](int c) { return w_tb + (chain * nch + c) * (kC * kC); };
  auto g_of = [&](int c) { return w_g + (chain * nch + c) * (2 * kC); };
  auto q_row0 = [&](int c) { return n_sink + c * kC + window; };
  auto kv_row0 = [&](int c) { return n_sink + c * kC; };

  // initial fill: sinks, ring chunks 0..2, chunk 0's queries, TB and gates
  for (int n = tid; n < kSinkRows * 16; n += kThreads) {
    const int r = n >> 4;
    const bool in = r < n_sink && r < T_;
    put_row(KSk, n, in ? *reinterpret_cast<const V16*>(kb + (size_t)r * kvrow + (n & 15) * 8) : zero8);
    put_row(VSk, n, in ? *reinterpret_cast<const V16*>(vb + (size_t)r * kvrow + (n & 15) * 8) : zero8);
  }
  for (int n = tid; n < 3 * 1024; n += kThreads) {
    const int sl = n >> 10;
    put_row(KR + sl * kC * kSR, n & 1023, load_rows(kb, kvrow, kv_row0(sl), n & 1023));
    put_row(VR + sl * kC * kSR, n & 1023, load_rows(vb, kvrow, kv_row0(sl), n & 1023));
  }
  for (int n = tid; n < 1024; n += kThreads) put_q(n, load_rows(qb, qrow, q_row0(0), n));
  *reinterpret_cast<V16*>(TBs + (tid >> 3) * kSC + (tid & 7) * 8) =
      *reinterpret_cast<const V16*>(tb_of(0) + (tid >> 3) * kC + (tid & 7) * 8);
  if (tid < 32) *reinterpret_cast<f32x4*>(Gs + 4 * tid) = *reinterpret_cast<const f32x4*>(g_of(0) + 4 * tid);
  __syncthreads();

  // ---------------------------------------------------------- chunks
  // Both roles run the same barrier sequence per chunk c:
  //   B0  chunk c's queries, TB, gates and ring chunks c .. c+2 are in LDS;
  //   B1  A (the decayed lower scores) is in LDS;
  //   B2  the softmax rows are in LDS (in the query tile, read by then);
  //       every read of TB, the gates and ring slot c % 3 is done;
  //   B3  the state waves have read the softmax rows.
  // Between B2 and B3 the state waves store o and the softmax waves commit
  // the prefetched TB and gates of chunk c+1 and K, V of chunk c+3; after
  // B3 they commit chunk c+1's queries.
  if (scan_wave) {
    // state columns 32 wv .. + 31; natural d_k rows 16 mt + 4 g + i
    const int cw = 32 * wv;
    f32x4 S[8][2];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) S[mt][nt] = zero4();
    for (int c = 0; c < nch; ++c) {
      const int i0 = n_sink + c * kC;
      const bf16* Kc = KR + (c % 3) * kC * kSR;
      const bf16* Vc = VR + (c % 3) * kC * kSR;
      const float* gl = Gs;
      const float* gam = Gs + kC;
      lds_barrier();                     // B0
      // ---- O^T = S^T Q^T   [dv tile nt][query tile rt]
      Frag<bf16> sf[4][2];
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) sf[p][nt] = frag_from_acc<bf16>(S[2 * p][nt], S[2 * p + 1][nt]);
      f32x4 ot[2][4];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) ot[nt][rt] = zero4();
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        Frag<bf16> qf[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) qf[rt] = lds_frag8(Qs + (16 * rt + j) * kSR + 32 * p + 8 * g);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) ot[nt][rt] = mfma(sf[p][nt], qf[rt], ot[nt][rt]);
      }
      // ---- KS = K S   [token tile mt][dv tile nt]
      f32x4 KS[4][2];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) KS[mt][nt] = zero4();
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        Frag<bf16> kf[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) kf[mt] = row_frag(Kc, 16 * mt + j, p, g);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) KS[mt][nt] = mfma(kf[mt], sf[p][nt], KS[mt][nt]);
      }
      // ---- U = TB V - TB diag(gamma) KS   [token tile mt][dv tile nt]
      f32x4 U[4][2];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) U[mt][nt] = zero4();
      const f32x4 neg = f32x4{-1.f, -1.f, -1.f, -1.f};
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        Frag<bf16> tf[4], vf[2], kf[2];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) tf[mt] = lds_frag8(TBs + (16 * mt + j) * kSC + 32 * pp + 8 * g);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) vf[nt] = tr_frag(Vc, 32 * pp, cw + 16 * nt, lane);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          kf[nt] = frag_from_acc_scaled<bf16>(KS[2 * pp][nt], KS[2 * pp + 1][nt], neg, neg);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) U[mt][nt] = mfma(tf[mt], vf[nt], U[mt][nt]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          tf[mt] = lds_frag8_scaled(TBs + (16 * mt + j) * kSC + 32 * pp + 8 * g, gam + 32 * pp + 4 * g,
                                    gam + 32 * pp + 16 + 4 * g);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) U[mt][nt] = mfma(tf[mt], kf[nt], U[mt][nt]);
      }

      lds_barrier();                     // B1: A is in LDS

      // ---- O^T: gamma of each query on the S^T Q^T part, then + U^T A^T
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const float gq = gam[16 * rt + j];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) ot[nt][rt] *= gq;
      }
      const float lgC = gl[kC - 1];
      const float gC = gam[kC - 1];
      Frag<bf16> uf[2][2], us[2][2];
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        f32x4 s0, s1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          s0[i] = __builtin_amdgcn_exp2f(fminf(lgC - gl[32 * pp + 4 * g + i], 0.f));
          s1[i] = __builtin_amdgcn_exp2f(fminf(lgC - gl[32 * pp + 16 + 4 * g + i], 0.f));
        }
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          uf[pp][nt] = frag_from_acc<bf16>(U[2 * pp][nt], U[2 * pp + 1][nt]);
          us[pp][nt] = frag_from_acc_scaled<bf16>(U[2 * pp][nt], U[2 * pp + 1][nt], s0, s1);
        }
      }
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        Frag<bf16> af[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) af[rt] = lds_frag8(As + (16 * rt + j) * kSC + 32 * pp + 8 * g);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) ot[nt][rt] = mfma(uf[pp][nt], af[rt], ot[nt][rt]);
      }
      // ---- S = gamma_C S + K^T diag(gamma_C / gamma) U
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) S[mt][nt] *= gC;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        Frag<bf16> kt[2];
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) kt[pp] = tr_frag(Kc, 32 * pp, 16 * mt, lane);
#pragma unroll
        for (int pp = 0; pp < 2; ++pp)
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) S[mt][nt] = mfma(kt[pp], us[pp][nt], S[mt][nt]);
      }
      lds_barrier();                     // B2: the softmax rows are in LDS
      // ---- o = w_lin o_lin + the softmax rows: buffer stores whose range
      // ends at the sequence's last row (rows past it are dropped), so the
      // stores need no branch
      {
        const long long left = (long long)(T_ - i0 - window) * H * kD * 2;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            ob + (size_t)(i0 + window) * qrow, 0, (int)min(left, 0x7fffffffLL), 0x00020000);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            const int r = 16 * rt + j;
            const int col = cw + 16 * nt + 4 * g;
            const f32x4 x = ot[nt][rt] * w_lin + load4(Xs + r * kSR + col);
            const bf16x4 y = bf16x4{static_cast<bf16>(x[0]), static_cast<bf16>(x[1]), static_cast<bf16>(x[2]),
                                    static_cast<bf16>(x[3])};
            typedef unsigned int u2 __attribute__((ext_vector_type(2)));
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u2, y), rs, (r * (int)qrow + col) * 2, 0, 0);
          }
      }
      lds_barrier();                     // B3: the softmax rows are read
    }
    if (write_state) {
      float* Sg = state_out + chain * kD * kD;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) Sg[(size_t)(16 * mt + 4 * g + i) * kD + cw + 16 * nt + j] = S[mt][nt][i];
    }
    return;
  }

  // ---------------------------------------------------------- softmax waves
  const int jq = wv - 4;              // rows 16 jq .. + 15 of each chunk
  const int ptid = tid - 256;         // prefetch pieces n = ptid + 256 m
  // prologue: rows t < n_sink + window carry no linear branch and attend to
  // every key t' <= t: the sinks and ring chunks 0 and 1 hold them all
  {
    const int nrow = min(n_sink + window, T_);
    for (int t0 = 16 * jq; t0 < nrow; t0 += 64) {
      Frag<bf16> qf[4];
      const int tq = t0 + j;
      const int tl = min(tq, nrow - 1);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const bf16x4 x0 = *reinterpret_cast<const bf16x4*>(qb + (size_t)tl * qrow + 32 * p + 4 * g);
        const bf16x4 x1 = *reinterpret_cast<const bf16x4*>(qb + (size_t)tl * qrow + 32 * p + 16 + 4 * g);
        qf[p].v = bf16x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      }
      const KeyPair kp[5] = {{KSk, VSk, 0, 0, true},
                             {KR, VR, 0, n_sink, false},
                             {KR, VR, 32, n_sink + 32, false},
                             {KR + kC * kSR, VR + kC * kSR, 0, n_sink + 64, false},
                             {KR + kC * kSR, VR + kC * kSR, 32, n_sink + 96, false}};
      bool use[5], have[5];
      f32x4 st[5][2];
#pragma unroll
      for (int pi = 0; pi < 5; ++pi) {
        use[pi] = pi == 0 ? n_sink > 0 : kp[pi].kk0 <= t0 + 15 && kp[pi].kk0 < T_;
        have[pi] = false;
      }
      const float m = sm_scores<5>(kp, use, st, have, qf, t0, n_sink, window, T_, lane);
      f32x4 oacc[8];
      float inv_l;
      sm_values<5>(kp, use, st, m, lane, oacc, inv_l);
      if (tq < nrow) {
        const float f = w_swa * inv_l;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) store4(ob + (size_t)tq * qrow + 16 * dt + 4 * g, oacc[dt] * f);
      }
    }
  }

  V16 pq[4], pt[2], pk[4], pv[4];
  f32x4 pg;
  for (int c = 0; c < nch; ++c) {
    const int i0 = n_sink + c * kC;
    const bf16* Kc = KR + (c % 3) * kC * kSR;
    const bf16* Vc = VR + (c % 3) * kC * kSR;
    const float* gl = Gs;
    lds_barrier();                       // B0: chunk c is in LDS
    // ---- prefetch, committed after the chunk: queries, TB, gates of c + 1
    // and K, V of chunk c + 3.  Always issued (past the last chunk they
    // reread valid rows and are not committed), so that the memory
    // counters the compiler waits on are exact.
    {
      const int cn = min(c + 1, nch - 1);
#pragma unroll
      for (int m = 0; m < 4; ++m) pq[m] = load_rows(qb, qrow, q_row0(cn), ptid + 256 * m);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int n = ptid + 256 * m;
        pt[m] = *reinterpret_cast<const V16*>(tb_of(cn) + (n >> 3) * kC + (n & 7) * 8);
      }
      pg = *reinterpret_cast<const f32x4*>(g_of(cn) + 4 * (ptid & 31));
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        pk[m] = load_rows(kb, kvrow, kv_row0(c + 3), ptid + 256 * m);
        pv[m] = load_rows(vb, kvrow, kv_row0(c + 3), ptid + 256 * m);
      }
    }
    // ---- query-key scores of rows r = 16 jq + j (lane column) against the
    // window (ring chunks c, c+1, c+2) and the sinks; the chunk's own keys
    // also give A
    Frag<bf16> qf[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) qf[p] = lds_frag8(Qs + (16 * jq + j) * kSR + 32 * p + 8 * g);
    f32x4 st[7][2];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      f32x4 acc = zero4();
#pragma unroll
      for (int p = 0; p < 4; ++p) acc = mfma(row_frag(Kc, 16 * kt + j, p, g), qf[p], acc);
      st[kt >> 1][kt & 1] = acc;
    }
    // A rows: [s <= r] 2^{g_r - g_s} q_r.k_s, columns in acc order
    {
      const int r = 16 * jq + j;
      const float lr = gl[r];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const f32x4 ls = *reinterpret_cast<const f32x4*>(gl + 16 * kt + 4 * g);
        f32x4 x;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int s_ = 16 * kt + 4 * g + i;
          x[i] = s_ <= r ? __builtin_amdgcn_exp2f(fminf(lr - ls[i], 0.f)) * st[kt >> 1][kt & 1][i] : 0.f;
        }
        store4(As + r * kSC + acc_pos(16 * kt + 4 * g), x);
      }
    }
    const int t0 = i0 + window + 16 * jq;
    const bf16* K1 = KR + ((c + 1) % 3) * kC * kSR;
    const bf16* V1 = VR + ((c + 1) % 3) * kC * kSR;
    const bf16* K2 = KR + ((c + 2) % 3) * kC * kSR;
    const bf16* V2 = VR + ((c + 2) % 3) * kC * kSR;
    const KeyPair kp[7] = {{Kc, Vc, 0, i0, false},       {Kc, Vc, 32, i0 + 32, false},
                           {K1, V1, 0, i0 + 64, false},  {K1, V1, 32, i0 + 96, false},
                           {K2, V2, 0, i0 + 128, false}, {K2, V2, 32, i0 + 160, false},
                           {KSk, VSk, 0, 0, true}};
    bool use[7], have[7];
#pragma unroll
    for (int pi = 0; pi < 6; ++pi) {
      // some key of the pair may be in some row's window (t - window, t]
      const int kk0 = kp[pi].kk0;
      use[pi] = kk0 + 31 > t0 - window && kk0 <= t0 + 15 && kk0 < T_;
      have[pi] = pi < 2;
    }
    use[6] = n_sink > 0;
    have[6] = false;
    const float m = sm_scores<7>(kp, use, st, have, qf, t0, n_sink, window, T_, lane);
    lds_barrier();                       // B1
    f32x4 oacc[8];
    float inv_l;
    sm_values<7>(kp, use, st, m, lane, oacc, inv_l);
    // ---- the softmax rows, w_swa-weighted, into the query tile ([row][d])
    {
      const int r = 16 * jq + j;
      const float f = w_swa * inv_l;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) store4(Xs + r * kSR + 16 * dt + 4 * g, oacc[dt] * f);
    }
    lds_barrier();                       // B2
    // ---- commit TB and gates of chunk c + 1, K and V of chunk c + 3 (into
    // the ring slot chunk c leaves)
    if (c + 1 < nch) {
#pragma unroll
      for (int m2 = 0; m2 < 2; ++m2) {
        const int n = ptid + 256 * m2;
        *reinterpret_cast<V16*>(TBs + (n >> 3) * kSC + (n & 7) * 8) = pt[m2];
      }
      if (ptid < 32) *reinterpret_cast<f32x4*>(Gs + 4 * ptid) = pg;
    }
    if (kv_row0(c + 3) < T_) {
      bf16* Ks3 = KR + (c % 3) * kC * kSR;
      bf16* Vs3 = VR + (c % 3) * kC * kSR;
#pragma unroll
      for (int m2 = 0; m2 < 4; ++m2) {
        put_row(Ks3, ptid + 256 * m2, pk[m2]);
        put_row(Vs3, ptid + 256 * m2, pv[m2]);
      }
    }
    lds_barrier();                       // B3: the softmax rows are read
    if (c + 1 < nch) {
#pragma unroll
      for (int m2 = 0; m2 < 4; ++m2) put_q(ptid + 256 * m2, pq[m2]);
    }
  }
}

}  // namespace

bool gdn_layer_applies(const PrefillArgs& p) {
  const int nch = gdn_stream_chunks(p.T, p.n_sink, p.window);
  return p.bf16 && !p.gla && p.D == kD && (p.flags & 3) == 3 && !(p.flags & 8) && nch >= 1 &&
         p.window <= 128 && p.n_sink <= kSinkRows && !gdn_full_prep(p.B, p.H, p.D, p.bf16);
}

hipError_t launch_gdn_layer(const PrefillArgs& p, hipStream_t s) {
  const int nch = gdn_stream_chunks(p.T, p.n_sink, p.window);
  hipError_t e = launch_gdn_prep(p, nch, s);
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute((const void*)gdn_layer_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
  if (e != hipSuccess) return e;
  const GdnWorkspace w = gdn_workspace_layout(p.workspace, p.B, p.H, nch, kD, sizeof(bf16), false);
  const dim3 grid(xcd_grouped_grid((long long)p.B * p.Hkv, p.H / p.Hkv));
  hipLaunchKernelGGL(gdn_layer_kernel, grid, dim3(kThreads), kLdsBytes, s, (const bf16*)p.q,
                     (const bf16*)p.k, (const bf16*)p.v, (const bf16*)w.tb, w.g, (bf16*)p.o,
                     p.state_out, p.B, p.T, p.H, p.Hkv, p.n_sink, p.window, nch,
                     (p.flags & 4) ? 1 : 0, p.w_lin, p.w_swa);
  return hipGetLastError();
}

}  // namespace gdn
