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

#include <algorithm>

#include "common.h"
#include "launch.h"

namespace gdn {
namespace {

constexpr int kC = 64;           // chunk length
constexpr int kD = 128;          // head dimension
// Row stride (elements) of every [rows][128] tile (K, V, queries): 288
// bytes.  Measured on gfx950, it keeps the transposing reads and the 16-byte
// row reads free of bank conflicts; the 8-byte row reads it does not suit
// (two-way) are few.
constexpr int kSR = kD + 16;
constexpr int kSV = kSR;
constexpr int kSC = kC + 8;      // row stride of [64][64] tiles
constexpr int kSinkRows = 16;    // sink keys held in LDS (n_sink <= 16)
constexpr int kThreads = 512;

// LDS layout (bf16 elements, then fp32 gates)
constexpr int oKR = 0;                             // K ring [3][64][kSR]
constexpr int oVR = oKR + 3 * kC * kSR;            // V ring [3][64][kSV]
constexpr int oKS = oVR + 3 * kC * kSV;            // sink K [16][kSR]
constexpr int oVS = oKS + kSinkRows * kSR;         // sink V [16][kSV]
constexpr int oQ = oVS + kSinkRows * kSV;          // lagged queries [64][kSR]; then the hand-over rows
constexpr int oTB = oQ + kC * kSR;                 // TB [64][kSC] (acc order)
constexpr int oA = oTB + kC * kSC;                 // A [64][kSC] (acc order)
constexpr int nLdsT = oA + kC * kSC;
// + fp32 per-token gate values of the chunk: g (log2 prefix), gamma = 2^g,
//   -gamma, and 2^(g_C - g) (the decay from each token to the chunk's end)
constexpr int kLdsBytes = nLdsT * 2 + 4 * kC * 4;
static_assert(kLdsBytes <= 160 * 1024, "one workgroup per compute unit");

typedef __attribute__((address_space(3))) bf16x4* lds_bf16x4_ptr;

// Two transposing 8-byte LDS reads: lane (g, j) receives X[r0 + 4g + i][c0 + j]
// and X[r0 + 16 + 4g + i][c0 + j], i = 0..3, of the row-major bf16 tile X
// (row stride SX): the operand X^T[c0 + j][K_g] (A side) or X[K_g][c0 + j]
// (B side).  Within each 16-lane group, lane 4 r + c1 addresses row
// r0 + 4g + r at columns c0 + 4 c1 .. + 3, and the hardware hands column
// c0 + j of the group's four rows to lane j.  The V tiles, read only this
// way, use a 288-byte row stride, which spreads a read's 16 rows x 32
// bytes over distinct banks; the K tiles, mostly read as rows (row_frag),
// use 272 bytes, which does the same for the row reads.
template <int SX = kSR>
__device__ __forceinline__ Frag<bf16> tr_frag(const bf16* X, int r0, int c0, int lane) {
  const int g = lane >> 4;
  const int j = lane & 15;
  const bf16* p0 = X + (r0 + 4 * g + (j >> 2)) * SX + c0 + 4 * (j & 3);
  const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_ptr)(p0));
  const bf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_ptr)(p0 + 16 * SX));
  Frag<bf16> f;
  f.v = bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return f;
}

// Row `row` of a natural-order [rows][128] tile as an operand reduced over
// d on the set 32 p + 8 g .. + 7 (one 16-byte read).  Every product over d
// uses that set: the state's accumulator rows are ordered so that two
// stacked state tiles provide it (see tr_frag_k).
__device__ __forceinline__ Frag<bf16> row_frag8(const bf16* X, int row, int p, int g) {
  return lds_frag8(X + row * kSR + 32 * p + 8 * g);
}

// K^T as the A operand of the state update, producing state tile
// mt = 2 p + hh whose accumulator row 4 g + i holds d_k = 32 p + 8 g + 4 hh + i
// (so that state tiles 2p and 2p+1 stacked as an operand hold d_k
// 32 p + 8 g .. + 7 in order): a transposing read whose 16-lane group
// addresses the rows (tokens) r0 + 4g + r and, in lane 4 r + c1, the columns
// 32 p + 8 c1 + 4 hh .. + 3, which the hardware hands to lanes 4 c1 .. + 3.
__device__ __forceinline__ Frag<bf16> tr_frag_k(const bf16* X, int r0, int p, int hh, int lane) {
  const int g = lane >> 4;
  const int j = lane & 15;
  const bf16* p0 = X + (r0 + 4 * g + (j >> 2)) * kSR + 32 * p + 8 * (j & 3) + 4 * hh;
  const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_ptr)(p0));
  const bf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_ptr)(p0 + 16 * kSR));
  Frag<bf16> f;
  f.v = bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return f;
}

// A transposing read pair at Xl + off and 16 rows below, Xl holding the
// lane's part of the address (row 4 g + j / 4, column 4 (j % 4) of a
// [rows][kSR] tile; see tr_frag).  The loops pass the lane parts of their
// addresses through an empty asm once per chunk: the compiler then adds a
// tile's uniform base to one lane register and folds the remaining
// constant into each instruction's offset, instead of keeping every
// distinct lane offset in a register of its own across the loop.
__device__ __forceinline__ Frag<bf16> tr_at(const bf16* Xl, int off) {
  const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_ptr)(Xl + off));
  const bf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_ptr)(Xl + off + 16 * kSR));
  Frag<bf16> f;
  f.v = bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return f;
}

// The segment states N and S_s in the workspace are fp32 [128][128] in the
// carry's accumulator order: 16 x 16 tiles (row tile, column tile), and in a
// tile lane 16 (r % 16 / 4) + c % 16 holds its 4 rows r % 4 = 0..3, so that
// the carry moves a tile with one 16-byte access per lane.
__device__ __forceinline__ int tile_off(int r, int c) {
  return ((r >> 4) * 8 + (c >> 4)) * 256 + (16 * ((r & 15) >> 2) + (c & 15)) * 4 + (r & 3);
}

// Sum over lanes l, l^16, l^32, l^48 (the four lane groups of one column).
__device__ __forceinline__ float sum_lane_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
// Max of attention scores in one instruction each.  Scores are never NaN
// (finite or -inf; unused sink rows are zero), so the NaN quieting that fmaxf
// needs in IEEE mode (an extra v_max per operand) is left out.
__device__ __forceinline__ float score_max2(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float score_max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float max_lane_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = score_max2(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return score_max2(__uint_as_float(b[0]), __uint_as_float(b[1]));
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

// Softmax over NP key pairs for the queries t = t0 + j (lane column j), in
// two phases and without branches: every pair is processed, keys outside a
// row's window (or past its sinks) weigh exactly 0.  Phase 1 (sm_scores):
// the scores of pairs NG.. from the query fragments qf (the first NG pairs'
// scores are given; S^T tiles: key 4g + i of each 16-key half, query j),
// masked keys set to -inf, and the row maximum.  Phase 2 (sm_values):
// weights 2^((s - m) log2(e) / sqrt(d)), their sum (on the matrix cores,
// against a ones operand) and the O^T tiles (d = 16 dt + 4g + i, query j).
template <int NP, int NG>
__device__ __forceinline__ float sm_scores(const KeyPair (&kp)[NP], f32x4 (&st)[NP][2],
                                           const Frag<bf16> (&qf)[4], int t0, int n_sink,
                                           int window, int lane) {
  const int g = lane >> 4;
  const int j = lane & 15;
  const int t = t0 + j;
#pragma unroll
  for (int pi = NG; pi < NP; ++pi) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      st[pi][hf] = zero4();
      if (hf == 1 && kp[pi].half) continue;
#pragma unroll
      for (int p = 0; p < 4; ++p) st[pi][hf] = mfma(row_frag8(kp[pi].K, kp[pi].r0 + 16 * hf + j, p, g), qf[p], st[pi][hf]);
    }
  }
  float m = -INFINITY;
#pragma unroll
  for (int pi = 0; pi < NP; ++pi) {
    // ring keys (>= n_sink): attended inside the window, kk - t in (-window, 0];
    // the sink pair holds keys 0 .. 15, of which those below n_sink (and <= t)
    // are sinks (the others, if any, are window keys held in the ring)
    const int d0 = kp[pi].kk0 + 4 * g - t + window - 1;      // (kk - t) + window - 1 at i = 0
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kk = kp[pi].kk0 + 16 * hf + 4 * g + i;
        const bool on = kp[pi].half ? hf == 0 && kk < n_sink && kk <= t
                                    : (unsigned)(d0 + 16 * hf + i) < (unsigned)window;
        st[pi][hf][i] = on ? st[pi][hf][i] : -INFINITY;
      }
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
      m = score_max3(score_max3(m, st[pi][hf][0], st[pi][hf][1]), st[pi][hf][2], st[pi][hf][3]);
  }
  m = max_lane_groups(m);
  return m == -INFINITY ? 0.f : m;   // a row with no key (past the sequence): weights 0
}

template <int NP>
__device__ __forceinline__ void sm_values(const KeyPair (&kp)[NP], const f32x4 (&st)[NP][2], float m,
                                          int lane, f32x4 (&oacc)[8], float& inv_l) {
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
        const bf16* p0p = kp[pi].V + (kp[pi].r0 + 4 * g + (j >> 2)) * kSV + 16 * dt + 4 * (j & 3);
        const bf16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_ptr)(p0p));
        vf.v = bf16x8{x[0], x[1], x[2], x[3], x[0], x[1], x[2], x[3]};
      } else {
        vf = tr_frag<kSV>(kp[pi].V, kp[pi].r0, 16 * dt, lane);
      }
      oacc[dt] = mfma(vf, pf, oacc[dt]);
    }
  }
  // the bf16 weights summed (the same rounding as the weights P V uses)
  inv_l = lacc[0] > 0.f ? 1.f / lacc[0] : 0.f;
}

// q, k, v, w_tb and w_g are read through plain (not restrict) pointers on
// purpose: the prefetch loads must stay where they are issued, ahead of the
// chunk's barriers, rather than be moved next to their use.
// LIN_ONLY: the linear branch alone (windows past the ring, the softmax
// branch added by its own launch afterwards): the softmax waves form only A
// and keep the K, V, TB and gates prefetch; the state waves store w_lin o_lin.
// NB: 32-key ring blocks a softmax row group reads besides the sinks: 5 for
// windows up to 128, 3 for windows up to 64.
template <bool LIN_ONLY, int NT, int NB = 5>
__device__ __forceinline__ void gdn_layer_body(
    const bf16* q, const bf16* k, const bf16* v, const bf16* w_tb, const float* w_g,
    bf16* __restrict__ o,
    float* __restrict__ state_out, int B, int T_, int H, int Hkv, int n_sink, int window,
    int nch, int write_state, float w_lin, float w_swa, int seg_len, const float* s_in, int add_o) {
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
  float* Gs = reinterpret_cast<float*>(smem_raw + nLdsT * 2);   // g, gamma, -gamma, 2^(g_C - g) [64 each]

  // the G query heads of a KV head are consecutive workgroups on one XCD
  // and share the K and V rows through its L2
  const int G = H / Hkv;
  constexpr int HALVES = NT == 2 ? 1 : 2;    // workgroups per chain (state columns split)
  int unit, member;
  if (!xcd_grouped(blockIdx.x, G * HALVES, B * Hkv, unit, member)) return;
  const int bi = unit / Hkv;
  const int gk = unit % Hkv;
  const int h = gk * G + member / HALVES;
  const int half = member % HALVES;
  const size_t chain = (size_t)bi * H + h;
  // segment y of the chain: chunks cb .. ce - 1, entered with the state
  // s_in holds for it (segment 0, or no s_in: the zero state)
  const int sg = blockIdx.y;
  const int cb = sg * seg_len;
  const int ce = min(nch, cb + seg_len);

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
  // The prefetch's 4 pieces m of 64 rows from row0, for the thread with
  // piece index n0 (rows n0 / 16 + 16 m): a uniform row base plus a per-lane
  // offset when all 64 rows exist, the clamped form near the end.
  auto load_tile4 = [&](const bf16* base, size_t stride, int row0, int n0, V16 (&x)[4]) {
    if (row0 + kC <= T_) {
      const bf16* rb = base + (size_t)row0 * stride;
      const int off = (n0 >> 4) * (int)stride + (n0 & 15) * 8;
#pragma unroll
      for (int m = 0; m < 4; ++m) x[m] = *reinterpret_cast<const V16*>(rb + off + 16 * m * (int)stride);
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m) x[m] = load_rows(base, stride, row0, n0 + 256 * m);
    }
  };
  auto put_row = [&](bf16* tile, int n, const V16& x) {      // K tiles
    *reinterpret_cast<V16*>(tile + (n >> 4) * kSR + (n & 15) * 8) = x;
  };
  auto put_vrow = [&](bf16* tile, int n, const V16& x) {     // V tiles
    *reinterpret_cast<V16*>(tile + (n >> 4) * kSV + (n & 15) * 8) = x;
  };
  auto put_q = [&](int n, const V16& x) { put_row(Qs, n, x); };
  auto tb_of = [&](int c) { return w_tb + (chain * nch + c) * (kC * kC); };
  // the gate block of a chunk from the 32 f32x4 pieces of (g, gamma): lane
  // l < 32 of one wave holds piece l (g for l < 16, gamma after); g_C is
  // g[63], piece 15's last value
  // (called by a whole wave, l = its lane; lanes 32.. only take part in the
  // shuffle)
  auto put_gates = [&](int l, const f32x4& x) {
    const float gC = __shfl(x[3], 15, 64);
    if (l >= 32) return;
    *reinterpret_cast<f32x4*>(Gs + 4 * l) = x;
    if (l < 16) {
      f32x4 f;
#pragma unroll
      for (int i = 0; i < 4; ++i) f[i] = __builtin_amdgcn_exp2f(fminf(gC - x[i], 0.f));
      *reinterpret_cast<f32x4*>(Gs + 3 * kC + 4 * l) = f;
    } else {
      *reinterpret_cast<f32x4*>(Gs + kC + 4 * l) = -x;     // -gamma at 2 kC + 4 (l - 16)
    }
  };
  auto g_of = [&](int c) { return w_g + (chain * nch + c) * (2 * kC); };
  auto q_row0 = [&](int c) { return n_sink + c * kC + window; };
  auto kv_row0 = [&](int c) { return n_sink + c * kC; };

  // initial fill: sinks, ring chunks cb .. cb + 2, chunk cb's queries, TB
  // and gates
  // (every load is issued before the first LDS store, so that their
  // latencies overlap)
  {
    static_assert(kSinkRows * 16 <= kThreads, "one sink piece per thread");
    V16 fk[6], fv[6], fq[2], fsk = zero8, fsv = zero8, ftb;
    f32x4 fg = zero4();
    const int rs = tid >> 4;
    const bool sin = tid < kSinkRows * 16 && rs < n_sink && rs < T_;
    if (sin) {
      fsk = *reinterpret_cast<const V16*>(kb + (size_t)rs * kvrow + (tid & 15) * 8);
      fsv = *reinterpret_cast<const V16*>(vb + (size_t)rs * kvrow + (tid & 15) * 8);
    }
#pragma unroll
    for (int m = 0; m < 6; ++m) {
      const int n = tid + kThreads * m;
      fk[m] = load_rows(kb, kvrow, kv_row0(cb + (n >> 10)), n & 1023);
      fv[m] = load_rows(vb, kvrow, kv_row0(cb + (n >> 10)), n & 1023);
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) fq[m] = load_rows(qb, qrow, q_row0(cb), tid + kThreads * m);
    ftb = *reinterpret_cast<const V16*>(tb_of(cb) + (tid >> 3) * kC + (tid & 7) * 8);
    if (tid < 64) fg = *reinterpret_cast<const f32x4*>(g_of(cb) + 4 * (tid & 31));
    asm volatile("" ::: "memory");
    if (tid < kSinkRows * 16) {
      put_row(KSk, tid, fsk);
      put_vrow(VSk, tid, fsv);
    }
#pragma unroll
    for (int m = 0; m < 6; ++m) {
      const int n = tid + kThreads * m;
      const unsigned sl = (unsigned)(cb + (n >> 10)) % 3u;
      put_row(KR + sl * kC * kSR, n & 1023, fk[m]);
      put_vrow(VR + sl * kC * kSV, n & 1023, fv[m]);
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) put_q(tid + kThreads * m, fq[m]);
    *reinterpret_cast<V16*>(TBs + (tid >> 3) * kSC + (tid & 7) * 8) = ftb;
    if (tid < 64) put_gates(tid, fg);
  }
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
    // Issue priority to the role whose work bounds the phase, when both
    // waves of a SIMD are ready: the state waves when the softmax waves only
    // form A (here); the softmax waves when they form the softmax rows
    // (below), except between B2 and B3, where the state waves' stores
    // bound the phase and the softmax waves only commit prefetched tiles.
    if constexpr (LIN_ONLY) __builtin_amdgcn_s_setprio(2);
    // state columns 32 wv .. + 31; tile mt's accumulator row 4 g + i holds
    // d_k = 32 (mt / 2) + 8 g + 4 (mt % 2) + i (see tr_frag_k), and column j
    // of tile nt is d_v = 32 wv + 8 (j / 4) + 4 nt + j % 4, so that a lane's
    // two output tiles hold 8 adjacent columns of a row (one 16-byte store)
    // (NT == 1: the workgroup's half of the columns, 16 per wave, column j
    // of the single tile is d_v = cw + j and a lane stores 4 columns)
    const int cw = NT == 2 ? 32 * wv : 64 * half + 16 * wv;

    f32x4 S[8][NT];
    if (s_in && sg > 0) {
      const float* Si = s_in + ((size_t)sg * B * H + chain) * kD * kD;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            S[mt][nt][i] = Si[tile_off(32 * (mt >> 1) + 8 * g + 4 * (mt & 1) + i,
                                       NT == 2 ? cw + 8 * (j >> 2) + 4 * nt + (j & 3) : cw + j)];
    } else {
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) S[mt][nt] = zero4();
    }
    V16 pq[4];
    for (int c = cb; c < ce; ++c) {
      const int i0 = n_sink + c * kC;
      const bf16* Kc = KR + ((unsigned)c % 3u) * kC * kSR;
      const bf16* Vc = VR + ((unsigned)c % 3u) * kC * kSV;
      const float* gam = Gs + kC;
      // lane parts of the LDS addresses: row reads, V^T and K^T reads,
      // [64][64] tiles, hand-over rows
      int l_row = j * kSR + 8 * g, l_tv = (4 * g + (j >> 2)) * kSR + 4 * (j & 3);
      int l_tk = (4 * g + (j >> 2)) * kSR + 8 * (j & 3), l_acc = j * kSC + 8 * g, l_x = j * kSR + 8 * g;
      asm volatile("" : "+v"(l_row), "+v"(l_tv), "+v"(l_tk), "+v"(l_acc), "+v"(l_x));
      lds_barrier();                     // B0
      // ---- prefetch the queries of chunk c + 1, committed after B3.
      // Always issued (past the last chunk they reread valid rows and are
      // not committed), so that the memory counters the compiler waits on
      // are exact.
      load_tile4(qb, qrow, q_row0(min(c + 1, ce - 1)), tid, pq);
      // the chunk's output rows, when the linear branch adds onto what o
      // holds (the softmax branch, written first): read through the same
      // bounded range as the stores (rows past the sequence read as 0)
      typedef unsigned int u2 __attribute__((ext_vector_type(2)));
      u2 po[4];
      if constexpr (NT == 1) {
        const long long left = (long long)(T_ - i0 - window) * H * kD * 2;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            ob + (size_t)(i0 + window) * qrow, 0, (int)min(left, 0x7fffffffLL), 0x00020000);
        if (add_o) {
#pragma unroll
          for (int rt = 0; rt < 4; ++rt)
            po[rt] = __builtin_amdgcn_raw_buffer_load_b64(rs, ((16 * rt + j) * (int)qrow + cw + 4 * g) * 2, 0, 0);
        }
      }
      asm volatile("" ::: "memory");     // issue them here, ahead of the products
      // ---- O^T = S^T Q^T [dv tile nt][query tile rt] and KS = K S [token
      // tile mt][dv tile nt], one d-step at a time (the state's operand
      // fragments of a step are formed from its accumulators when needed)
      f32x4 ot[NT][4], KS[4][NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          ot[nt][rt] = zero4();
          KS[rt][nt] = zero4();
        }
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        Frag<bf16> sf[NT], qf[4], kf[4];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) sf[nt] = frag_from_acc<bf16>(S[2 * p][nt], S[2 * p + 1][nt]);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) qf[rt] = lds_frag8(Qs + l_row + 16 * rt * kSR + 32 * p);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) ot[nt][rt] = mfma(sf[nt], qf[rt], ot[nt][rt]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) kf[mt] = lds_frag8(Kc + l_row + 16 * mt * kSR + 32 * p);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) KS[mt][nt] = mfma(kf[mt], sf[nt], KS[mt][nt]);
      }
      // ---- U = TB V - TB diag(gamma) KS   [token tile mt][dv tile nt];
      // diag(-gamma) is applied to KS's token rows as its fragments form
      Frag<bf16> ksf[2][NT];
      {
        const float* ngam = Gs + 2 * kC;
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          const f32x4 n0 = *reinterpret_cast<const f32x4*>(ngam + 32 * pp + 4 * g);
          const f32x4 n1 = *reinterpret_cast<const f32x4*>(ngam + 32 * pp + 16 + 4 * g);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            ksf[pp][nt] = frag_from_acc_scaled<bf16>(KS[2 * pp][nt], KS[2 * pp + 1][nt], n0, n1);
        }
      }
      f32x4 U[4][NT];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) U[mt][nt] = zero4();
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        Frag<bf16> tf[4], vf[NT];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) tf[mt] = lds_frag8(TBs + l_acc + 16 * mt * kSC + 32 * pp);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          vf[nt] = NT == 2 ? tr_at(Vc + cw + l_tk, 32 * pp * kSR + 4 * nt) : tr_at(Vc + cw + l_tv, 32 * pp * kSR);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) U[mt][nt] = mfma(tf[mt], vf[nt], U[mt][nt]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) U[mt][nt] = mfma(tf[mt], ksf[pp][nt], U[mt][nt]);
      }

      lds_barrier();                     // B1: A is in LDS

      // ---- O^T: gamma of each query on the S^T Q^T part, then + U^T A^T
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const float gq = gam[16 * rt + j];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) ot[nt][rt] *= gq;
      }
      const float gC = gam[kC - 1];
      const float* dec = Gs + 3 * kC;    // 2^(g_C - g_s)
      Frag<bf16> uf[2][NT], us[2][NT];
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        const f32x4 s0 = *reinterpret_cast<const f32x4*>(dec + 32 * pp + 4 * g);
        const f32x4 s1 = *reinterpret_cast<const f32x4*>(dec + 32 * pp + 16 + 4 * g);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          uf[pp][nt] = frag_from_acc<bf16>(U[2 * pp][nt], U[2 * pp + 1][nt]);
          us[pp][nt] = frag_from_acc_scaled<bf16>(U[2 * pp][nt], U[2 * pp + 1][nt], s0, s1);
        }
      }
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        Frag<bf16> af[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) af[rt] = lds_frag8(As + l_acc + 16 * rt * kSC + 32 * pp);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) ot[nt][rt] = mfma(uf[pp][nt], af[rt], ot[nt][rt]);
      }
      // ---- S = gamma_C S + K^T diag(gamma_C / gamma) U
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) S[mt][nt] *= gC;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        Frag<bf16> kt[2];
#pragma unroll
        for (int pp = 0; pp < 2; ++pp)
          kt[pp] = tr_at(Kc + l_tk, 32 * pp * kSR + 32 * (mt >> 1) + 4 * (mt & 1));
#pragma unroll
        for (int pp = 0; pp < 2; ++pp)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) S[mt][nt] = mfma(kt[pp], us[pp][nt], S[mt][nt]);
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
        for (int rt = 0; rt < 4; ++rt) {
          // lane: row 16 rt + j, columns cw + 8 g .. + 7 (tile 0 then tile 1);
          // NT == 1: columns cw + 4 g .. + 3
          const int r = 16 * rt + j;
          if constexpr (NT == 1) {
            static_assert(LIN_ONLY, "the column split serves the linear branch alone");
            f32x4 yv = ot[0][rt] * w_lin;
            if (add_o) {
              const bf16x4 x = __builtin_bit_cast(bf16x4, po[rt]);
              yv += f32x4{static_cast<float>(x[0]), static_cast<float>(x[1]), static_cast<float>(x[2]),
                          static_cast<float>(x[3])};
            }
            const bf16x4 y4{static_cast<bf16>(yv[0]), static_cast<bf16>(yv[1]), static_cast<bf16>(yv[2]),
                            static_cast<bf16>(yv[3])};
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u2, y4), rs, (r * (int)qrow + cw + 4 * g) * 2, 0, 0);
            continue;
          }
          bf16x8 y;
          if constexpr (LIN_ONLY) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
              for (int i = 0; i < 4; ++i) y[4 * nt + i] = static_cast<bf16>(ot[nt][rt][i] * w_lin);
          } else {
            const bf16x8 xs = *reinterpret_cast<const bf16x8*>(Xs + cw + l_x + 16 * rt * kSR);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                y[4 * nt + i] = static_cast<bf16>(__builtin_fmaf(ot[nt][rt][i], w_lin, static_cast<float>(xs[4 * nt + i])));
          }
          typedef unsigned int u4 __attribute__((ext_vector_type(4)));
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, y), rs, (r * (int)qrow + cw + 8 * g) * 2, 0, 0);
        }
      }
      lds_barrier();                     // B3: the softmax rows are read
      if (c + 1 < ce) {
#pragma unroll
        for (int m2 = 0; m2 < 4; ++m2) put_q(tid + 256 * m2, pq[m2]);
      }
    }
    if (write_state) {
      float* Sg = state_out + chain * kD * kD;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            Sg[(size_t)(32 * (mt >> 1) + 8 * g + 4 * (mt & 1) + i) * kD +
               (NT == 2 ? cw + 8 * (j >> 2) + 4 * nt + (j & 3) : cw + j)] = S[mt][nt][i];
    }
    return;
  }

  // ---------------------------------------------------------- softmax waves
  const int jq = wv - 4;              // rows 16 jq .. + 15 of each chunk
  if constexpr (!LIN_ONLY) __builtin_amdgcn_s_setprio(3);
  const int ptid = tid - 256;         // prefetch pieces n = ptid + 256 m
  // prologue (first segment): rows t < n_sink + window carry no linear
  // branch and attend to every key t' <= t: the sinks and ring chunks 0 and
  // 1 hold them all
  if constexpr (!LIN_ONLY) {
    const int nrow = sg == 0 ? min(n_sink + window, T_) : 0;
    for (int t0 = 16 * jq; t0 < nrow; t0 += 64) {
      Frag<bf16> qf[4];
      const int tq = t0 + j;
      const int tl = min(tq, nrow - 1);
#pragma unroll
      for (int p = 0; p < 4; ++p) qf[p].v = *reinterpret_cast<const bf16x8*>(qb + (size_t)tl * qrow + 32 * p + 8 * g);
      const KeyPair kp[5] = {{KSk, VSk, 0, 0, true},
                             {KR, VR, 0, n_sink, false},
                             {KR, VR, 32, n_sink + 32, false},
                             {KR + kC * kSR, VR + kC * kSV, 0, n_sink + 64, false},
                             {KR + kC * kSR, VR + kC * kSV, 32, n_sink + 96, false}};
      f32x4 st[5][2];
      const float m = sm_scores<5, 0>(kp, st, qf, t0, n_sink, window, lane);
      f32x4 oacc[8];
      float inv_l;
      sm_values<5>(kp, st, m, lane, oacc, inv_l);
      if (tq < nrow) {
        const float f = w_swa * inv_l;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) store4(ob + (size_t)tq * qrow + 16 * dt + 4 * g, oacc[dt] * f);
      }
    }
  }

  // Rows r = 16 jq + j of chunk c are the times t = i0 + window + r.  They
  // attend to the ring keys at offsets (from i0) 16 jq + 1 + j .. 16 jq +
  // window + j, all inside the five 32-key blocks pb .. pb + 4, pb = jq / 2
  // (window <= 128); block b holds offsets 32 b .. + 31, rows 32 (b % 2) ..
  // of ring chunk c + b / 2.  Slot 0 is block pb, whose scores the chunk's
  // own score tiles give (blocks 0 and 1 are chunk c); slots 1-3 are blocks
  // 2, 3, 4; slot 4 is block 5 (pb = 1) or block 1 (pb = 0, recomputed so
  // that every wave runs the same code); slot 5 is the sink block.
  const int pb = jq >> 1;
  const int bX = pb ? 5 : 1;
  // A block needs the window mask iff some of its keys lie outside some
  // row's window; the other blocks are attended by all 16 rows.
  auto partial = [&](int b) { return !(32 * b >= 16 * jq + 16 && 32 * b + 31 <= 16 * jq + window); };
  const bool mk0 = partial(pb), mk1 = partial(NB == 3 ? pb + 1 : 2), mk2 = partial(NB == 3 ? pb + 2 : 3),
             mk3 = partial(4), mk4 = partial(bX);
  // key 16 hf + 4 g + i of block b is in row j's window iff
  // e0 + 32 b + 16 hf + i lies in [0, window)
  const int e0 = 4 * g - 16 * jq - j - 1;
  auto mask_block = [&](f32x4 (&x)[2], int b, int e) {
    const int d0 = e + 32 * b;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        x[hf][i] = (unsigned)(d0 + 16 * hf + i) < (unsigned)window ? x[hf][i] : -INFINITY;
  };
  // the sink scores accumulate onto 0 (key 4 g + i < n_sink) or -inf; loop
  // rows are later than every sink, and keys 16 .. 31 of the block are none
  f32x4 sbias;
#pragma unroll
  for (int i = 0; i < 4; ++i) sbias[i] = 4 * g + i < n_sink ? 0.f : -INFINITY;
  const float scale = kLog2e / sqrtf((float)kD);
  Frag<bf16> ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones.v[e] = static_cast<bf16>(1.f);

  V16 pk[4], pv[4], pt[2];
  f32x4 pg;
  for (int c = cb; c < ce; ++c) {
    const int i0 = n_sink + c * kC;
    const bf16* Kc = KR + ((unsigned)c % 3u) * kC * kSR;
    const bf16* Vc = VR + ((unsigned)c % 3u) * kC * kSV;
    const bf16* K1 = KR + ((unsigned)(c + 1) % 3u) * kC * kSR;
    const bf16* V1 = VR + ((unsigned)(c + 1) % 3u) * kC * kSV;
    const bf16* K2 = KR + ((unsigned)(c + 2) % 3u) * kC * kSR;
    const bf16* V2 = VR + ((unsigned)(c + 2) % 3u) * kC * kSV;
    const bf16* KX = KR + ((unsigned)(c + 2 * pb) % 3u) * kC * kSR;
    const bf16* VX = VR + ((unsigned)(c + 2 * pb) % 3u) * kC * kSV;
    const float* gl = Gs;
    // lane parts of the LDS addresses: row reads, V^T reads, A rows
    int l_row = j * kSR + 8 * g, l_tv = (4 * g + (j >> 2)) * kSR + 4 * (j & 3), l_acc = j * kSC + 8 * g;
    asm volatile("" : "+v"(l_row), "+v"(l_tv), "+v"(l_acc));
    lds_barrier();                       // B0: chunk c is in LDS
    // ---- prefetch TB and the gates of chunk c + 1, committed after B2
    // (always issued, as the other prefetches)
    {
      const int cn = min(c + 1, ce - 1);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int n = ptid + 256 * m;
        pt[m] = *reinterpret_cast<const V16*>(tb_of(cn) + (n >> 3) * kC + (n & 7) * 8);
      }
      pg = *reinterpret_cast<const f32x4*>(g_of(cn) + 4 * (ptid & 31));
      asm volatile("" ::: "memory");     // issue them here, ahead of the scores
    }
    // ---- scores (S^T tiles: key 4 g + i of each 16-key half, query j), in
    // batches of two 16-key tiles whose K reads are issued one batch ahead
    // of their products (the scheduling barriers keep that order)
    const int r = 16 * jq + j;
    Frag<bf16> qf[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) qf[p] = lds_frag8(Qs + l_row + 16 * jq * kSR + 32 * p);
    const float lr = gl[r];
    f32x4 ls[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) ls[kt] = *reinterpret_cast<const f32x4*>(gl + 16 * kt + 4 * g);
    auto kfr = [&](const bf16* X, int row0, Frag<bf16> (&f)[4]) {
#pragma unroll
      for (int p = 0; p < 4; ++p) f[p] = lds_frag8(X + l_row + row0 * kSR + 32 * p);
    };
    auto kmma = [&](const Frag<bf16> (&f)[4], f32x4 acc) {
#pragma unroll
      for (int p = 0; p < 4; ++p) acc = mfma(f[p], qf[p], acc);
      return acc;
    };
    if constexpr (LIN_ONLY) {
      // A only: the chunk's own scores, decayed and masked; then the K, V
      // prefetch of chunk c + 3 and the commits, at the same barriers
      f32x4 sa[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        Frag<bf16> kx[4];
        kfr(Kc, 16 * kt, kx);
        sa[kt] = kmma(kx, zero4());
      }
      {
        int jj = j;
        asm volatile("" : "+v"(jj));
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          f32x4 x;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float dec = __builtin_amdgcn_exp2f(fminf(lr - ls[kt][i], 0.f));
            x[i] = kt < jq || (kt == jq && 4 * g + i <= jj) ? dec * sa[kt][i] : 0.f;
          }
          store4(As + l_acc + 16 * jq * kSC + 32 * (kt >> 1) + 4 * (kt & 1), x);
        }
      }
      lds_barrier();                     // B1
      load_tile4(kb, kvrow, kv_row0(c + 3), ptid, pk);
      load_tile4(vb, kvrow, kv_row0(c + 3), ptid, pv);
      asm volatile("" ::: "memory");
      lds_barrier();                     // B2
#pragma unroll
      for (int m2 = 0; m2 < 4; ++m2) {
        put_row(KR + ((unsigned)c % 3u) * kC * kSR, ptid + 256 * m2, pk[m2]);
        put_vrow(VR + ((unsigned)c % 3u) * kC * kSV, ptid + 256 * m2, pv[m2]);
      }
      if (c + 1 < ce) {
#pragma unroll
        for (int m2 = 0; m2 < 2; ++m2) {
          const int n = ptid + 256 * m2;
          *reinterpret_cast<V16*>(TBs + (n >> 3) * kSC + (n & 7) * 8) = pt[m2];
        }
        if (ptid < 64) put_gates(ptid, pg);
      }
      lds_barrier();                     // B3
      continue;
    }
    Frag<bf16> ka[4], kb2[4], kc[4], kd[4];
    f32x4 sa[4], st[6][2];
    kfr(Kc, 0, ka);
    kfr(Kc, 16, kb2);
    __builtin_amdgcn_sched_barrier(0);
    kfr(Kc, 32, kc);
    kfr(Kc, 48, kd);
    sa[0] = kmma(ka, zero4());
    sa[1] = kmma(kb2, zero4());
    __builtin_amdgcn_sched_barrier(0);
    kfr(K1, 0, ka);
    kfr(K1, 16, kb2);
    sa[2] = kmma(kc, zero4());
    sa[3] = kmma(kd, zero4());
    __builtin_amdgcn_sched_barrier(0);
    // NB = 3: the third block pb + 2 is ring chunk c + 1's rows 32 pb .. (for
    // pb = 0 the same rows as block 2, recomputed so that every wave runs the
    // same code)
    kfr(K1, NB == 3 ? 32 * pb : 32, kc);
    kfr(K1, NB == 3 ? 32 * pb + 16 : 48, kd);
    st[1][0] = kmma(ka, zero4());
    st[1][1] = kmma(kb2, zero4());
    // A rows: [s <= r] 2^{g_r - g_s} q_r.k_s, columns in acc order; tile
    // kt is below the diagonal (kt < jq), on it, or above (zero)
    {
      int jj = j;
      asm volatile("" : "+v"(jj));
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        f32x4 x;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float dec = __builtin_amdgcn_exp2f(fminf(lr - ls[kt][i], 0.f));
          x[i] = kt < jq || (kt == jq && 4 * g + i <= jj) ? dec * sa[kt][i] : 0.f;
        }
        store4(As + l_acc + 16 * jq * kSC + 32 * (kt >> 1) + 4 * (kt & 1), x);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NB == 3) {
      kfr(KSk, 0, ka);
      st[2][0] = kmma(kc, zero4());
      st[2][1] = kmma(kd, zero4());
      __builtin_amdgcn_sched_barrier(0);
      st[5][0] = kmma(ka, sbias);
      st[5][1] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      // slot 0: block pb (chunk c's own scores); slot 1: block pb + 1 (block
      // 2 for pb = 1, chunk c's second half for pb = 0); slot 2: block pb + 2
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        st[0][hf] = pb ? sa[2 + hf] : sa[hf];
        st[1][hf] = pb ? st[1][hf] : sa[2 + hf];
      }
    } else {
      kfr(K2, 0, ka);
      kfr(K2, 16, kb2);
      st[2][0] = kmma(kc, zero4());
      st[2][1] = kmma(kd, zero4());
      __builtin_amdgcn_sched_barrier(0);
      kfr(KX, 32, kc);
      kfr(KX, 48, kd);
      st[3][0] = kmma(ka, zero4());
      st[3][1] = kmma(kb2, zero4());
      __builtin_amdgcn_sched_barrier(0);
      kfr(KSk, 0, ka);
      st[4][0] = kmma(kc, zero4());
      st[4][1] = kmma(kd, zero4());
      __builtin_amdgcn_sched_barrier(0);
      st[5][0] = kmma(ka, sbias);
      st[5][1] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) st[0][hf] = pb ? sa[2 + hf] : sa[hf];
    }
    // ---- window masks (blocks with keys outside some row's window) and the
    // row maximum
    // (e0 passes through an empty asm so that the compares stay in the loop:
    // hoisted, their lane masks would not fit the scalar registers)
    int e = e0;
    asm volatile("" : "+v"(e));
    if (mk0) mask_block(st[0], pb, e);
    if constexpr (NB == 3) {
      if (mk1) mask_block(st[1], pb + 1, e);
      if (mk2) mask_block(st[2], pb + 2, e);
    } else {
      if (mk1) mask_block(st[1], 2, e);
      if (mk2) mask_block(st[2], 3, e);
      if (mk3) mask_block(st[3], 4, e);
      if (mk4) mask_block(st[4], bX, e);
    }
    float m = -INFINITY;
#pragma unroll
    for (int sl = 0; sl < 6; ++sl) {
      if (NB == 3 && (sl == 3 || sl == 4)) continue;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        m = score_max3(score_max3(m, st[sl][hf][0], st[sl][hf][1]), st[sl][hf][2], st[sl][hf][3]);
    }
    m = max_lane_groups(m);
    m = m == -INFINITY ? 0.f : m;      // a row with no key (past the sequence): weights 0
    lds_barrier();                       // B1
    // ---- prefetch K, V of chunk c + 3 (committed after B2; always issued,
    // rows past the sequence clamped)
    load_tile4(kb, kvrow, kv_row0(c + 3), ptid, pk);
    load_tile4(vb, kvrow, kv_row0(c + 3), ptid, pv);
    asm volatile("" ::: "memory");       // issue them here, ahead of the softmax
    // ---- weights 2^((s - m) log2(e) / sqrt(d)), their sum (on the matrix
    // cores, against a ones operand) and O^T tiles (d = 16 dt + 4 g + i,
    // query j); the V^T reads of a slot are issued one slot ahead
    const float mb = -m * scale;
    auto vfr = [&](const bf16* X, int r0, Frag<bf16> (&f)[8]) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) f[dt] = tr_at(X + l_tv, r0 * kSR + 16 * dt);
    };
    auto pfr = [&](const f32x4 (&x)[2]) {
      f32x4 p0, p1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p0[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[0][i], scale, mb));
        p1[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[1][i], scale, mb));
      }
      return frag_from_acc<bf16>(p0, p1);
    };
    f32x4 lacc = zero4(), oacc[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) oacc[dt] = zero4();
    auto vmma = [&](const Frag<bf16> (&f)[8], const Frag<bf16>& pf) {
      lacc = mfma(ones, pf, lacc);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) oacc[dt] = mfma(f[dt], pf, oacc[dt]);
    };
    Frag<bf16> va[8], vb2[8], pa, pb2;
    vfr(Vc, 32 * pb, va);
    pa = pfr(st[0]);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NB == 3) {
      vfr(pb ? V1 : Vc, pb ? 0 : 32, vb2);     // block pb + 1
      pb2 = pfr(st[1]);
      vmma(va, pa);
      __builtin_amdgcn_sched_barrier(0);
      vfr(V1, 32 * pb, va);                    // block pb + 2
      pa = pfr(st[2]);
      vmma(vb2, pb2);
      __builtin_amdgcn_sched_barrier(0);
    } else {
      vfr(V1, 0, vb2);
      pb2 = pfr(st[1]);
      vmma(va, pa);
      __builtin_amdgcn_sched_barrier(0);
      vfr(V1, 32, va);
      pa = pfr(st[2]);
      vmma(vb2, pb2);
      __builtin_amdgcn_sched_barrier(0);
      vfr(V2, 0, vb2);
      pb2 = pfr(st[3]);
      vmma(va, pa);
      __builtin_amdgcn_sched_barrier(0);
      vfr(VX, 32, va);
      pa = pfr(st[4]);
      vmma(vb2, pb2);
      __builtin_amdgcn_sched_barrier(0);
    }
    // the sink block: 16 keys, read once and used for both halves (the
    // second half weighs 0)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const bf16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_ptr)(VSk + l_tv + 16 * dt));
      vb2[dt].v = bf16x8{x[0], x[1], x[2], x[3], x[0], x[1], x[2], x[3]};
    }
    pb2 = pfr(st[5]);
    vmma(va, pa);
    __builtin_amdgcn_sched_barrier(0);
    vmma(vb2, pb2);
    // the bf16 weights summed (the same rounding as the weights P V uses)
    const float inv_l = lacc[0] > 0.f ? 1.f / lacc[0] : 0.f;
    // ---- the softmax rows, w_swa-weighted, into the query tile ([row][d])
    {
      const float f = w_swa * inv_l;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) store4(Xs + l_row - 4 * g + 16 * jq * kSR + 16 * dt, oacc[dt] * f);
    }
    lds_barrier();                       // B2
    __builtin_amdgcn_s_setprio(0);       // the state waves' stores bound this phase
    // ---- commit K, V of chunk c + 3 into the ring slot chunk c leaves (past
    // the sequence: its clamped last row, a key no row attends), then TB
    // and the gates of chunk c + 1 (their last reads were before B2)
#pragma unroll
    for (int m2 = 0; m2 < 4; ++m2) {
      put_row(KR + ((unsigned)c % 3u) * kC * kSR, ptid + 256 * m2, pk[m2]);
      put_vrow(VR + ((unsigned)c % 3u) * kC * kSV, ptid + 256 * m2, pv[m2]);
    }
    if (c + 1 < ce) {
#pragma unroll
      for (int m2 = 0; m2 < 2; ++m2) {
        const int n = ptid + 256 * m2;
        *reinterpret_cast<V16*>(TBs + (n >> 3) * kSC + (n & 7) * 8) = pt[m2];
      }
      if (ptid < 64) put_gates(ptid, pg);
    }
    lds_barrier();                       // B3: the softmax rows are read
    __builtin_amdgcn_s_setprio(3);
  }
}

template <int NB>
__global__ __launch_bounds__(kThreads) void gdn_layer_kernel(
    const bf16* q, const bf16* k, const bf16* v, const bf16* w_tb, const float* w_g,
    bf16* __restrict__ o,
    float* __restrict__ state_out, int B, int T_, int H, int Hkv, int n_sink, int window,
    int nch, int write_state, float w_lin, float w_swa, int seg_len, const float* s_in) {
  gdn_layer_body<false, 2, NB>(q, k, v, w_tb, w_g, o, state_out, B, T_, H, Hkv, n_sink, window, nch,
                               write_state, w_lin, w_swa, seg_len, s_in, 0);
}
// the instance for a window: three ring blocks per row group up to 64 keys
inline decltype(&gdn_layer_kernel<5>) layer_kernel_for(int window) {
  return window <= 64 ? gdn_layer_kernel<3> : gdn_layer_kernel<5>;
}

__global__ __launch_bounds__(kThreads) void gdn_linear_layer_kernel(
    const bf16* q, const bf16* k, const bf16* v, const bf16* w_tb, const float* w_g,
    bf16* __restrict__ o,
    float* __restrict__ state_out, int B, int T_, int H, int Hkv, int n_sink, int window,
    int nch, int write_state, float w_lin, int add_o) {
  gdn_layer_body<true, 1>(q, k, v, w_tb, w_g, o, state_out, B, T_, H, Hkv, n_sink, window, nch, write_state,
                          w_lin, 0.f, nch, nullptr, add_o);
}

// ---------------------------------------------------------------------------
// Segmented scan for few chains.  When the chains cannot fill the GPU, each
// chain's stream chunks are cut into P segments of L chunks.  Over a segment
// the state update is affine in the incoming state, S_end = M S_start + N
// (the recurrence is linear in S with the gates, keys and values fixed): N is
// the state the segment's chunks produce from S_start = 0, and M what they
// make of S_start = I with the values set to zero (column k of M is the
// image of the unit state e_k).  After the chunk preparation three launches
// run: the maps of all segments at once (gdn_segmap_kernel), the carry
// S_{s+1} = M_s S_s + N_s from S_0 = 0 (gdn_carry_kernel), and the layer
// kernel on every segment at once from its incoming state S_s.

// The map kernel's chunk inputs reach LDS by direct loads (global_load_lds:
// lane L of a wave writes 16 bytes at base + 16 L, 1 KB per instruction),
// two chunks ahead, into a ring of three slots: K [64][kSR] and V [64][kSV]
// (natural order), TB [64][kSC] (acc order), then g and gamma [64 each]
// fp32 (in a 1 KB block).  A lane whose 16 bytes fall in a row's padding
// (or past the gates) loads the row's first piece again (never read).  46
// instructions per chunk, 6 per wave (the last one three times).
constexpr int oMK = 0;
constexpr int oMV = oMK + kC * kSR * 2;
constexpr int oMTB = oMV + kC * kSV * 2;
constexpr int oMG = oMTB + kC * kSC * 2;
constexpr int kMapSlot = oMG + 1024;
constexpr int kMapBytes = 3 * kMapSlot;
constexpr int kMapDma = 6;              // direct loads per wave per chunk
static_assert(kMapBytes <= 160 * 1024, "one workgroup per compute unit");
static_assert((kC * kSR * 2) % 1024 == 0 && (kC * kSC * 2) % 1024 == 0, "whole 1 KB loads");

// One direct load (16 bytes per lane into LDS at lds + 16 lane).  Written
// as asm so that the compiler, which cannot tell which LDS bytes such a load
// writes, does not wait for it before every transposing LDS read: the
// kernel itself waits (vmcnt) before the barrier that hands a slot over.
// It has no register result; m0 holds the wave-uniform LDS address.
__device__ __forceinline__ void dma16(const void* g, const void* lds) {
  const unsigned la = __builtin_amdgcn_readfirstlane(
      (unsigned)(size_t)(const __attribute__((address_space(3))) void*)lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(la), "v"(g)
               : "memory", "m0");
}

// Maps of segment y of each chain.  Waves 0-3 run the recurrence from the
// zero state on the values (32 columns of N each), waves 4-7 from the
// identity without values (32 columns of M each); the products are those of
// the layer kernel's state waves (KS = K S, U = TB (V - diag(gamma) KS),
// S <- gamma_C S + K^T diag(gamma_C / gamma) U) with the same register
// layouts.  One barrier per chunk.
// Out: N fp32 (tile order, tile_off) and M bf16 ([d_k][column] row-major),
// per (segment, chain).
__global__ __launch_bounds__(kThreads) void gdn_segmap_kernel(
    const bf16* k, const bf16* v, const bf16* w_tb, const float* w_g, bf16* __restrict__ seg_m,
    float* __restrict__ seg_n, int B, int T_, int H, int Hkv, int n_sink, int nch, int seg_len) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  const int G = H / Hkv;
  int unit, member;
  if (!xcd_grouped(blockIdx.x, G, B * Hkv, unit, member)) return;
  const int bi = unit / Hkv;
  const int gk = unit % Hkv;
  const int h = gk * G + member;
  const size_t chain = (size_t)bi * H + h;
  const int sg = blockIdx.y;
  const int cb = sg * seg_len;
  const int ce = min(nch, cb + seg_len);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = wave_id();
  const int g = lane >> 4;
  const int j = lane & 15;
  const bool mw = wv >= 4;              // the map M: identity start, no values
  const int cw = 32 * (wv & 3);
  const size_t kvrow = (size_t)Hkv * kD;
  const bf16* kb = k + ((size_t)bi * T_ * Hkv + gk) * kD;
  const bf16* vb = v + ((size_t)bi * T_ * Hkv + gk) * kD;

  // this wave's direct loads of chunk c into slot sl: list entries wv + 8 m
  // (K pieces 0..17, V 18..35, TB 36..44, the gates 45); rows past the
  // sequence repeat its last row (they meet zero rows and columns of TB)
  auto issue = [&](int c, int sl) {
    const int row0 = n_sink + c * kC;
    const size_t ci = chain * nch + c;
    const unsigned char* base = smem_raw + sl * kMapSlot;
#pragma unroll
    for (int m = 0; m < kMapDma; ++m) {
      const int i = min(wv + 8 * m, 45);
      const void* src;
      int dst;
      if (i < 36) {
        const int n = i < 18 ? i : i - 18;
        const int off = 1024 * n + 16 * lane;
        const int r = off / (kSR * 2);
        const int pc = (off % (kSR * 2)) >> 4;
        const size_t row = (size_t)min(row0 + r, T_ - 1);
        src = (i < 18 ? kb : vb) + row * kvrow + (pc < 16 ? 8 * pc : 0);
        dst = (i < 18 ? oMK : oMV) + 1024 * n;
      } else if (i < 45) {
        const int n = i - 36;
        const int off = 1024 * n + 16 * lane;
        const int r = off / (kSC * 2);
        const int pc = (off % (kSC * 2)) >> 4;
        src = w_tb + ci * (kC * kC) + r * kC + (pc < 8 ? 8 * pc : 0);
        dst = oMTB + 1024 * n;
      } else {
        src = w_g + ci * (2 * kC) + 4 * (lane & 31);
        dst = oMG;
      }
      dma16(src, base + dst);
    }
  };

  // state tile mt's accumulator row 4 g + i is d_k = 32 (mt / 2) + 8 g +
  // 4 (mt % 2) + i; column j of tile nt is 32 (wv % 4) + 8 (j / 4) + 4 nt + j % 4
  auto row_of = [&](int mt, int i) { return 32 * (mt >> 1) + 8 * g + 4 * (mt & 1) + i; };
  auto col_of = [&](int nt) { return cw + 8 * (j >> 2) + 4 * nt + (j & 3); };
  f32x4 S[8][2];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) S[mt][nt][i] = mw && row_of(mt, i) == col_of(nt) ? 1.f : 0.f;

  // chunks cb and cb + 1 (every issue is made, the chunk index clamped, so
  // that each wave always has exactly kMapDma loads per chunk in flight)
  issue(cb, 0);
  issue(min(cb + 1, ce - 1), 1);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0F70 | kMapDma);   // vmcnt(6): chunk cb has landed
  unsigned sl = 0;
  for (int c = cb; c < ce; ++c) {
    const bf16* Kc = reinterpret_cast<const bf16*>(smem_raw + sl * kMapSlot + oMK);
    const bf16* Vc = reinterpret_cast<const bf16*>(smem_raw + sl * kMapSlot + oMV);
    const bf16* TBc = reinterpret_cast<const bf16*>(smem_raw + sl * kMapSlot + oMTB);
    const float* Gc = reinterpret_cast<const float*>(smem_raw + sl * kMapSlot + oMG);
    const unsigned sl2 = sl == 0 ? 2u : sl - 1;      // (sl + 2) % 3: chunk c - 1's slot
    int l_row = j * kSR + 8 * g, l_tk = (4 * g + (j >> 2)) * kSR + 8 * (j & 3), l_acc = j * kSC + 8 * g;
    asm volatile("" : "+v"(l_row), "+v"(l_tk), "+v"(l_acc));
    lds_barrier();                       // chunk c is in slot sl; chunk c - 1's slot is free
    issue(min(c + 2, ce - 1), sl2);
    asm volatile("" ::: "memory");
    // ---- KS = K S [token tile mt][column tile nt]
    f32x4 KS[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) KS[mt][nt] = zero4();
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      Frag<bf16> sf[2], kf[4];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) sf[nt] = frag_from_acc<bf16>(S[2 * p][nt], S[2 * p + 1][nt]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) kf[mt] = lds_frag8(Kc + l_row + 16 * mt * kSR + 32 * p);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) KS[mt][nt] = mfma(kf[mt], sf[nt], KS[mt][nt]);
    }
    // ---- U = TB (V - diag(gamma) KS) (the map waves: no values); the
    // operand X = V - diag(gamma) KS is formed in fp32 and rounded once
    const float* gam = Gc + kC;
    Frag<bf16> xf[2][2];
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      const f32x4 n0 = -*reinterpret_cast<const f32x4*>(gam + 32 * pp + 4 * g);
      const f32x4 n1 = -*reinterpret_cast<const f32x4*>(gam + 32 * pp + 16 + 4 * g);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        float x[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[i] = n0[i] * KS[2 * pp][nt][i];
          x[4 + i] = n1[i] * KS[2 * pp + 1][nt][i];
        }
        if (!mw) {
          // V^T fragment with the same (token, column) per element as KS's
          const Frag<bf16> vf = tr_at(Vc + cw + l_tk, 32 * pp * kSR + 4 * nt);
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] += static_cast<float>(vf.v[e]);
        }
        xf[pp][nt] = frag_from8<bf16>(x);
      }
    }
    f32x4 U[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) U[mt][nt] = zero4();
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      Frag<bf16> tf[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) tf[mt] = lds_frag8(TBc + l_acc + 16 * mt * kSC + 32 * pp);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) U[mt][nt] = mfma(tf[mt], xf[pp][nt], U[mt][nt]);
    }
    // ---- S = gamma_C S + K^T diag(gamma_C / gamma) U
    const float gC = gam[kC - 1];
    const float lgC = Gc[kC - 1];
    Frag<bf16> us[2][2];
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      const f32x4 l0 = *reinterpret_cast<const f32x4*>(Gc + 32 * pp + 4 * g);
      const f32x4 l1 = *reinterpret_cast<const f32x4*>(Gc + 32 * pp + 16 + 4 * g);
      f32x4 s0, s1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s0[i] = __builtin_amdgcn_exp2f(fminf(lgC - l0[i], 0.f));
        s1[i] = __builtin_amdgcn_exp2f(fminf(lgC - l1[i], 0.f));
      }
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) us[pp][nt] = frag_from_acc_scaled<bf16>(U[2 * pp][nt], U[2 * pp + 1][nt], s0, s1);
    }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) S[mt][nt] *= gC;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      Frag<bf16> kt[2];
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) kt[pp] = tr_at(Kc + l_tk, 32 * pp * kSR + 32 * (mt >> 1) + 4 * (mt & 1));
#pragma unroll
      for (int pp = 0; pp < 2; ++pp)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) S[mt][nt] = mfma(kt[pp], us[pp][nt], S[mt][nt]);
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0F70 | kMapDma);   // vmcnt(6): chunk c + 1 has landed
    sl = sl == 2 ? 0u : sl + 1;
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);   // no direct load outlives the workgroup

  const size_t off = ((size_t)sg * B * H + chain) * kD * kD;
  if (mw) {
    // segment 0 starts from the zero state: its M is never used
    if (sg == 0) return;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) seg_m[off + row_of(mt, i) * kD + col_of(nt)] = static_cast<bf16>(S[mt][nt][i]);
  } else {
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) seg_n[off + tile_off(row_of(mt, i), col_of(nt))] = S[mt][nt][i];
  }
}

// The carry over the segments of one chain, for 32 state columns c0 .. c0 +
// 31 (the columns of S are independent): S_1 = N_0, S_{s+1} = M_s S_s + N_s.
// Writes S_1 .. S_{P-1} (the incoming states of segments 1 .. P-1, tile
// order) and, with write_state, S_P (the final state).  Wave w computes rows
// 16 w .. + 15;
// the state passes between steps through LDS as bf16 S^T [column][d_k]; the
// operands of M_s and N_s are loaded kCarryDepth steps ahead (they do not
// depend on the carry), so a step waits only on its own products.
constexpr int kCarryST = kD + 8;    // row stride of S^T in LDS
constexpr int kCarryDepth = 4;
__global__ __launch_bounds__(512) void gdn_carry_kernel(const bf16* __restrict__ seg_m,
                                                        const float* __restrict__ seg_n,
                                                        float* __restrict__ seg_s,
                                                        float* __restrict__ state_out, int C,
                                                        int P, int write_state) {
  __shared__ __attribute__((aligned(16))) bf16 ST[32 * kCarryST];
  const int chain = blockIdx.x >> 2;
  const int c0 = 32 * (blockIdx.x & 3);
  const int lane = threadIdx.x & 63;
  const int wv = wave_id();
  const int g = lane >> 4;
  const int j = lane & 15;
  // accumulator tile u: rows 16 wv + 4 g + i, column c0 + 16 u + j; at(u)
  // is its 4 values' offset in tile order
  auto at = [&](int u) { return (wv * 8 + (c0 >> 4) + u) * 256 + 4 * lane; };
  auto mat = [&](int s) { return ((size_t)s * C + chain) * kD * kD; };
  const int last = write_state ? P : P - 1;   // the last state needed
  // operands of step s (S_{s+1} = M_s S_s + N_s): A fragments of M_s rows
  // 16 wv + j, d_k 32 p + 8 g .. + 7, and N_s
  Frag<bf16> ma[kCarryDepth][4];
  f32x4 na[kCarryDepth][2];
  // (every step loads and stores unconditionally, so that the compiler's
  // memory-counter waits stay exact: loads past the last map reread map
  // P - 1, and the states of steps past the last go to the workspace's
  // spare slot P)
  auto load_step = [&](int q, int s) {
    s = min(s, P - 1);
    const bf16* M = seg_m + mat(s);
    const float* N = seg_n + mat(s);
#pragma unroll
    for (int p = 0; p < 4; ++p)
      ma[q][p].v = *reinterpret_cast<const bf16x8*>(M + (16 * wv + j) * kD + 32 * p + 8 * g);
#pragma unroll
    for (int u = 0; u < 2; ++u) na[q][u] = *reinterpret_cast<const f32x4*>(N + at(u));
  };
  f32x4 acc[2];
  const float* N0 = seg_n + mat(0);
#pragma unroll
  for (int u = 0; u < 2; ++u) acc[u] = *reinterpret_cast<const f32x4*>(N0 + at(u));
  // (the empty asm statements keep the loads in step order, so that a
  // step's wait covers only its own operands)
#pragma unroll
  for (int q = 0; q < kCarryDepth; ++q) {
    load_step(q, 1 + q);
    asm volatile("" ::: "memory");
  }
  for (int s0 = 1; s0 < last; s0 += kCarryDepth) {
#pragma unroll
    for (int q = 0; q < kCarryDepth; ++q) {
      const int s = s0 + q;
      const bool live = s < last;
      // acc holds S_s (past the last step: S_last): out to the segment's
      // incoming state, and as bf16 S^T
      float* So = seg_s + mat(min(s, P));
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        *reinterpret_cast<f32x4*>(So + at(u)) = acc[u];
        bf16x4 x;
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = static_cast<bf16>(acc[u][i]);
        *reinterpret_cast<bf16x4*>(ST + (16 * u + j) * kCarryST + 16 * wv + 4 * g) = x;
      }
      lds_barrier();
      Frag<bf16> sb[2][4];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int p = 0; p < 4; ++p) sb[u][p] = lds_frag8(ST + (16 * u + j) * kCarryST + 32 * p + 8 * g);
      f32x4 nx[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) nx[u] = na[q][u];
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int u = 0; u < 2; ++u) nx[u] = mfma(ma[q][p], sb[u][p], nx[u]);
#pragma unroll
      for (int u = 0; u < 2; ++u) acc[u] = live ? nx[u] : acc[u];
      asm volatile("" ::: "memory");
      load_step(q, s + kCarryDepth);
      lds_barrier();                     // S^T is read before the next step overwrites it
    }
  }
  // acc holds S_last: the final state ([d_k][d_v] row-major), or the last
  // segment's incoming state
  if (last == P) {
    float* So = state_out + (size_t)chain * kD * kD;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) So[(16 * wv + 4 * g + i) * kD + c0 + 16 * u + j] = acc[u][i];
  } else {
    float* So = seg_s + mat(last);
#pragma unroll
    for (int u = 0; u < 2; ++u) *reinterpret_cast<f32x4*>(So + at(u)) = acc[u];
  }
}

}  // namespace

bool gdn_layer_applies(const PrefillArgs& p) {
  const int nch = gdn_stream_chunks(p.T, p.n_sink, p.window);
  return p.bf16 && !p.gla && p.D == kD && (p.flags & 3) == 3 && !(p.flags & 8) && nch >= 1 &&
         p.window <= 128 && p.n_sink <= kSinkRows && !gdn_full_prep(p.B, p.H, p.D, p.bf16);
}

bool gdn_linear_layer_applies(const PrefillArgs& p) {
  // the linear branch (the softmax branch, if asked for, by its own launch
  // afterwards: windows past the layer kernel's ring, or more sinks than it
  // holds), overwriting o, many chains
  const int nch = gdn_stream_chunks(p.T, p.n_sink, p.window);
  return p.bf16 && !p.gla && !p.dgd && p.D == kD && (p.flags & 1) && !(p.flags & 8) && nch >= 1 &&
         !gdn_layer_applies(p) && !gdn_segmented(p) && !gdn_full_prep(p.B, p.H, p.D, p.bf16);
}

hipError_t launch_gdn_linear_layer(const PrefillArgs& p, hipStream_t s, bool add_o) {
  const int nch = gdn_stream_chunks(p.T, p.n_sink, p.window);
  hipError_t e = p.prepared ? hipSuccess : launch_gdn_prep(p, nch, s);
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute((const void*)gdn_linear_layer_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                          kLdsBytes);
  if (e != hipSuccess) return e;
  const GdnWorkspace w = gdn_workspace_layout(p.workspace, p.B, p.H, nch, kD, sizeof(bf16), false);
  // two workgroups per chain, each with half of the state's columns
  const dim3 grid(xcd_grouped_grid((long long)p.B * p.Hkv, 2 * (p.H / p.Hkv)));
  hipLaunchKernelGGL(gdn_linear_layer_kernel, grid, dim3(kThreads), kLdsBytes, s, (const bf16*)p.q,
                     (const bf16*)p.k, (const bf16*)p.v, (const bf16*)w.tb, w.g, (bf16*)p.o,
                     p.state_out, p.B, p.T, p.H, p.Hkv, p.n_sink, p.window, nch,
                     (p.flags & 4) ? 1 : 0, p.w_lin, add_o ? 1 : 0);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // linear branch alone: rows t < n_sink + window carry no linear output
  return (p.flags & 2) ? hipSuccess : launch_zero_head_rows(p, s);
}

hipError_t launch_gdn_layer(const PrefillArgs& p, hipStream_t s) {
  const int nch = gdn_stream_chunks(p.T, p.n_sink, p.window);
  hipError_t e = p.prepared ? hipSuccess : launch_gdn_prep(p, nch, s);
  if (e != hipSuccess) return e;
  const auto kern = layer_kernel_for(p.window);
  e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
  if (e != hipSuccess) return e;
  const GdnWorkspace w = gdn_workspace_layout(p.workspace, p.B, p.H, nch, kD, sizeof(bf16), false);
  const dim3 grid(xcd_grouped_grid((long long)p.B * p.Hkv, p.H / p.Hkv));
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), kLdsBytes, s, (const bf16*)p.q,
                     (const bf16*)p.k, (const bf16*)p.v, (const bf16*)w.tb, w.g, (bf16*)p.o,
                     p.state_out, p.B, p.T, p.H, p.Hkv, p.n_sink, p.window, nch,
                     (p.flags & 4) ? 1 : 0, p.w_lin, p.w_swa, nch, (const float*)nullptr);
  return hipGetLastError();
}

SegPlan gdn_seg_plan(int B, int H, int nch) {
  const long long C = (long long)B * H;
  // one workgroup per compute unit in the map and layer launches
  const long long want = C > 0 ? 256 / C : 0;
  SegPlan pl{1, nch};
  if (want < 4 || nch < 4) return pl;
  pl.P = (int)std::min<long long>(want, nch);
  pl.L = (nch + pl.P - 1) / pl.P;
  pl.P = (nch + pl.L - 1) / pl.L;
  return pl;
}

bool gdn_segmented(int B, int T, int H, int D, int n_sink, int window, int bf16, int gla, int flags) {
  const int nch = gdn_stream_chunks(T, n_sink, window);
  return bf16 && !gla && D == kD && (flags & 3) == 3 && !(flags & 8) && window <= 128 &&
         n_sink <= kSinkRows && gdn_seg_plan(B, H, nch).P >= 4;
}
bool gdn_segmented(const PrefillArgs& p) {
  return gdn_segmented(p.B, p.T, p.H, p.D, p.n_sink, p.window, p.bf16, p.gla, p.flags);
}

SegWorkspace gdn_seg_layout(void* base, int B, int H, int nch) {
  const GdnWorkspace w = gdn_workspace_layout(base, B, H, nch, kD, sizeof(bf16), false);
  const SegPlan pl = gdn_seg_plan(B, H, nch);
  const size_t mats = (size_t)pl.P * B * H * kD * kD;
  const size_t al = 256;
  size_t off = (w.bytes + al - 1) / al * al;
  SegWorkspace s;
  s.light = w;
  unsigned char* b = static_cast<unsigned char*>(base);
  s.m = b + off;
  off += (mats * 2 + al - 1) / al * al;
  s.n = reinterpret_cast<float*>(b + off);
  off += mats * 4;
  s.s = reinterpret_cast<float*>(b + off);
  off += mats * 4 + (size_t)B * H * kD * kD * 4;   // + the carry's spare slot P
  s.bytes = off;
  return s;
}

hipError_t launch_gdn_segmented(const PrefillArgs& p, hipStream_t s) {
  const int nch = gdn_stream_chunks(p.T, p.n_sink, p.window);
  const SegPlan pl = gdn_seg_plan(p.B, p.H, nch);
  const int C = p.B * p.H;
  const bool wst = (p.flags & 4) != 0;
  const int need = wst ? pl.P : pl.P - 1;      // segments whose maps the carry uses
  hipError_t e = p.prepared ? hipSuccess : launch_gdn_prep(p, nch, s);
  if (e != hipSuccess) return e;
  const SegWorkspace w = gdn_seg_layout(p.workspace, p.B, p.H, nch);
  const unsigned gx = xcd_grouped_grid((long long)p.B * p.Hkv, p.H / p.Hkv);
  e = hipFuncSetAttribute((const void*)gdn_segmap_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kMapBytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gdn_segmap_kernel, dim3(gx, need), dim3(kThreads), kMapBytes, s, (const bf16*)p.k,
                     (const bf16*)p.v, (const bf16*)w.light.tb, w.light.g, (bf16*)w.m, w.n, p.B, p.T, p.H,
                     p.Hkv, p.n_sink, nch, pl.L);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gdn_carry_kernel, dim3(4 * C), dim3(512), 0, s, (const bf16*)w.m,
                     (const float*)w.n, w.s, p.state_out, C, pl.P, wst ? 1 : 0);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const auto kern = layer_kernel_for(p.window);
  e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(gx, pl.P), dim3(kThreads), kLdsBytes, s, (const bf16*)p.q,
                     (const bf16*)p.k, (const bf16*)p.v, (const bf16*)w.light.tb, w.light.g, (bf16*)p.o,
                     p.state_out, p.B, p.T, p.H, p.Hkv, p.n_sink, p.window, nch, 0, p.w_lin, p.w_swa,
                     pl.L, (const float*)w.s);
  return hipGetLastError();
}

}  // namespace gdn
