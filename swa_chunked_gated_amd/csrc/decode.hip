// Decode step of the hybrid layer on gfx950, and the cache fill after a
// prefill.
//
// Method (page "The Key to Going Linear: Analysis-Driven Transformer
// Linearization", sections 线性注意力替换机制 and 填补近似缺口的实用设计):
// the new token t attends by softmax to the n_sink sinks and the last
// `window` tokens (itself included); the token that leaves the window,
// e = t - window, is folded into the per-head recurrent state with its own
// gates, and the state is read with q_t.  The two outputs are summed.
//
// Work split: one workgroup per (sequence, query head) runs both branches.
// It streams the head's d x d fp32 state through registers exactly once (one
// read, one write) and, while those loads are in flight, the softmax over
// the cached rows; the G heads of a KV head share an XCD, so a cached row is
// fetched from HBM once per group.  o is written once.  A second small kernel
// (one workgroup per sequence) writes the new token into the freed slot and
// advances pos, after every head has read the evicted entry.
//
// Gated delta rule in one pass over the old state S (a, b: evicted gates):
//   c1 = S^T k_e, c2 = S^T q, u = b (v_e - a c1)
//   S' = a S + k_e u^T,  o_lin = S'^T q = a c2 + u (k_e . q)
// GLA: S' = Diag(alpha) S + k_e v_e^T, o_lin = S^T (alpha * q) + v_e (k_e . q).
// Delta rule with the diagonal gate (mode 2): c1 = S^T (alpha * k_e),
// c2 = S^T (alpha * q), u = b (v_e - c1), S' = Diag(alpha) S + k_e u^T,
// o_lin = c2 + u (k_e . q).
// MODE: 0 the gated delta rule, 1 GLA, 2 the delta rule with the diagonal gate.

#include "common.h"
#include "launch.h"

namespace gdn {
namespace {

constexpr int kStepThreads = 512;

// Slot state of cache slot j for the new token t: -1 not attended, 0 the
// cached entry, 1 the new token (its slot is being overwritten this step).
__device__ __forceinline__ int slot_state_of(int j, int t, int n_sink, int window) {
  if (j < n_sink) return j < t ? 0 : (j == t ? 1 : -1);
  if (t < n_sink) return -1;
  const int r = j - n_sink;
  const int back = ((t - n_sink - r) % window + window) % window;
  return back == 0 ? 1 : (t - back >= n_sink ? 0 : -1);   // latest token of this ring slot
}

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(1))) void* gbl_void_ptr;

// Lane L of the wave loads 16 bytes at g into LDS at base + 16 L; no
// registers are involved.
__device__ __forceinline__ void dma16(const void* g, void* base) {
  __builtin_amdgcn_global_load_lds((gbl_void_ptr)(void*)g, (lds_void_ptr)base, 16, 0, 0);
}

// Wait until at most n vector-memory operations of this wave are outstanding
// (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt at their
// maxima).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | 0x0F70);
}

template <class T, int D, int MR>
struct StepMap {
  static constexpr int CG = D / 4;                 // column groups of 4 floats
  static constexpr int RG = kStepThreads / CG;     // row groups
  static constexpr int R = D / RG;                 // state rows per thread
  static constexpr int NWV = kStepThreads / 64;    // waves
  static constexpr int ROWS = MR * 128 / sizeof(T);   // cache rows staged per pass
  static constexpr int UPR = D * sizeof(T) / 16;   // 16-byte units per cache row
  static constexpr int UPT = ROWS * UPR / kStepThreads;   // staged units per thread
  static constexpr int LPS = kStepThreads / ROWS;  // lanes per row in the logits
  static constexpr int VEC = 16 / sizeof(T);       // elements per unit
  static constexpr int UPL = UPR / LPS;            // units per lane in the logits
  static constexpr int VPT = ROWS / RG;            // V rows per thread in P V
  static_assert(UPT >= 1 && UPL >= 1 && VPT >= 1, "tile shape");
};

// 4 consecutive elements of the I/O type (8 bytes of bf16, 16 of fp32).
template <class T> struct Raw4;
template <> struct Raw4<bf16> { typedef bf16x4 type; };
template <> struct Raw4<float> { typedef f32x4 type; };
__device__ __forceinline__ f32x4 raw4_f32(const bf16x4& x) {
  return f32x4{static_cast<float>(x[0]), static_cast<float>(x[1]), static_cast<float>(x[2]),
               static_cast<float>(x[3])};
}
__device__ __forceinline__ f32x4 raw4_f32(const f32x4& x) { return x; }

// One decode step of one (sequence, query head), both branches in one
// workgroup.  Issue order: the first pass of cached K and V rows goes
// straight to LDS (no registers), then the small per-step vectors, then the
// head's d x d fp32 state, which is streamed through registers exactly once
// (one read, one write).  The softmax over the staged rows runs while the
// state is still arriving.  Workgroups are placed so that the G query heads
// of a KV head run together on one XCD: each cached row comes from HBM once
// and from that XCD's L2 for the other heads.  o is written once, as
// w_lin o_lin + w_swa o_swa (1, 1 for the plain sum).  MR scales
// the rows staged per pass (MR * 128 bytes of each of K and V per head
// dimension): 1 for budgets that fit one pass, 4 for long budgets, whose
// serial passes (one staging round trip each) would otherwise dominate.
template <class T, int MODE, int D, int MR>
__device__ __forceinline__ void decode_step_body(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ a, const float* __restrict__ b, float* __restrict__ state,
    const T* __restrict__ kc, const T* __restrict__ vc, const float* __restrict__ ac,
    const float* __restrict__ bc, const int* __restrict__ pos, T* __restrict__ o, int B, int H,
    int Hkv, int n_sink, int window, int flags, float w_lin, float w_swa) {
  using M = StepMap<T, D, MR>;
  typedef typename Vec16<T>::type V16;
  typedef typename Raw4<T>::type R4;
  constexpr bool GLA = MODE != 0;    // per-channel gate a_e
  constexpr bool DGD = MODE == 2;
  constexpr int VLOAD = 3 * M::UPR + (GLA ? D / 4 : 0);   // 16-byte units of the per-step vectors
  constexpr int VUNITS = (VLOAD + 63) / 64 * 64;
  static_assert(VUNITS <= 64 * M::NWV, "one load per wave");
  const int G = H / Hkv;
  int grp, member;
  if (!xcd_grouped(blockIdx.x, G, B * Hkv, grp, member)) return;
  const int bi = grp / Hkv;
  const int h = (grp % Hkv) * G + member;
  const int bh = bi * H + h;
  const int N = n_sink + window;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = wave_id();
  const int t = pos[bi];
  if (t < 0) return;   // outside the contract (pos >= 0); never index a negative slot
  const bool lin = flags & 1;
  const bool swa = flags & 2;
  const int e = t - window;
  const bool evict = e >= n_sink;
  const int slot = t < n_sink ? t : n_sink + (t - n_sink) % window;
  const int ring = t < n_sink ? -1 : (t - n_sink) % window;

  __shared__ __align__(16) T ks[M::ROWS * D];
  __shared__ __align__(16) T vs[M::ROWS * D];
  __shared__ float lg[M::ROWS];   // logits of the staged rows, log2 domain
  // per-step vectors as loaded: q, k_e, v_e (I/O type), then GLA's a_e (fp32)
  __shared__ __align__(16) unsigned char vecs[VUNITS * 16];
  __shared__ __align__(16) float gates[64];   // GDN: a_e, b_e
  __shared__ float misc[4];
  __shared__ float red[M::NWV * M::CG * 12];
  __shared__ __align__(16) float fin[M::CG * 12];   // c1, c2, c3 per column group
  const T* qv = reinterpret_cast<const T*>(vecs);
  const T* kev = qv + D;
  const T* vev = kev + D;
  const float* aev = GLA ? reinterpret_cast<const float*>(vev + D) : gates;

  // ---- cached K and V rows j0 .. j0 + ROWS - 1 into LDS, row-major; the
  // new token's slot takes its row from k, v; rows past N repeat row N - 1
  // (never used)
  const size_t kvbase = (size_t)grp * N * D;   // cache [B][Hkv][N][D]
  const size_t tokkv = (size_t)grp * D;        // k, v  [B][Hkv][D]
  auto stage = [&](int j0) {
#pragma unroll
    for (int u = 0; u < M::UPT; ++u) {
      const int w0 = (u * M::NWV + wv) * 64;   // first unit of this wave's load
      const int P = w0 + lane;
      const int j = min(j0 + P / M::UPR, N - 1);
      const int c = (P % M::UPR) * M::VEC;
      const T* kg = j == slot ? k + tokkv + c : kc + kvbase + (size_t)j * D + c;
      const T* vg = j == slot ? v + tokkv + c : vc + kvbase + (size_t)j * D + c;
      dma16(kg, ks + (size_t)w0 * M::VEC);
      dma16(vg, vs + (size_t)w0 * M::VEC);
    }
  };
  if (swa) stage(0);
  asm volatile("" ::: "memory");

  // ---- the small per-step vectors, also straight into LDS: wave w loads
  // units 64 w .. 64 w + 63 of [q | k_e | v_e | a_e (GLA)]; units past the
  // end repeat a valid address into padding
  const size_t gb = evict ? ((size_t)bi * window + ring) * H + h : 0;   // gate cache [B][W][H](,D)
  if (wv * 64 < VLOAD) {
    const int P = min(wv * 64 + lane, VLOAD - 1);
    const int vi = P / M::UPR;            // which vector
    const int c = (P % M::UPR) * M::VEC;  // element offset (I/O-type vectors)
    const void* src;
    if (vi == 0) src = q + (size_t)bh * D + c;
    else if (vi == 1) src = kc + kvbase + (size_t)slot * D + c;
    else if (vi == 2) src = vc + kvbase + (size_t)slot * D + c;
    else src = ac + gb * D + (P - 3 * M::UPR) * 4;   // GLA gates, fp32
    dma16(src, vecs + wv * 64 * 16);
  }
  if ((!GLA || DGD) && wv == M::NWV - 1) {
    // gates[0] = a_e (scalar gate), gates[1] = b_e
    const float* src = (lane == 1 || DGD) ? bc + gb : ac + gb;
    __builtin_amdgcn_global_load_lds((gbl_void_ptr)(void*)src, (lds_void_ptr)(void*)gates, 4, 0, 0);
  }
  asm volatile("" ::: "memory");

  // ---- the head's state, streamed once; its loads and stores are marked
  // non-temporal (a step's state is far larger than the caches and is not
  // touched again within the step), which leaves the caches to the rows
  // the heads of a group share
  const int cg = tid % M::CG;
  const int rg = tid / M::CG;
  float* Sg = state + (size_t)bh * D * D;
  f32x4 s[M::R];
#pragma unroll
  for (int r = 0; r < M::R; ++r)
    s[r] = __builtin_nontemporal_load(
        reinterpret_cast<const f32x4*>(Sg + (size_t)(rg + M::RG * r) * D + 4 * cg));

  wait_vmcnt<M::R>();   // every load before the state's has landed (the staged rows)
  lds_barrier();
  if (evict && wv == 0) {
    float acc = 0.f;
    for (int i = lane; i < D; i += 64) acc += to_f32(kev[i]) * to_f32(qv[i]);
    acc = wave_sum(acc);
    if (lane == 0) misc[1] = acc;   // k_e . q
  }

  // ---- softmax over the staged rows, online across passes of ROWS rows
  float p3[4] = {0.f, 0.f, 0.f, 0.f};
  float mx = -INFINITY, den = 0.f;
  if (swa) {
    const float lscale = 1.4426950408889634f / sqrtf((float)D);   // log2(e) / sqrt(d)
    const int kj = tid / M::LPS;
    const int kp = tid % M::LPS;
    for (int j0 = 0; j0 < N; j0 += M::ROWS) {
      if (j0 > 0) {
        lds_barrier();   // every wave is done with the previous pass's rows
        stage(j0);
        wait_vmcnt<0>();
        lds_barrier();
      }
      // logits: LPS lanes per row, units kp, kp + LPS, ... of the row
      {
        const int j = j0 + kj;
        float acc = 0.f;
#pragma unroll
        for (int m = 0; m < M::UPL; ++m) {
          const int c = (kp + M::LPS * m) * M::VEC;
          const V16 kx = *reinterpret_cast<const V16*>(&ks[kj * D + c]);
          const V16 qx = *reinterpret_cast<const V16*>(&qv[c]);
#pragma unroll
          for (int xx = 0; xx < M::VEC; ++xx) acc += to_f32(kx[xx]) * to_f32(qx[xx]);
        }
#pragma unroll
        for (int m = 1; m < M::LPS; m <<= 1) acc += shfl_xor(acc, m);
        if (kp == 0) {
          const bool att = j < N && slot_state_of(j, t, n_sink, window) >= 0;
          lg[kj] = att ? acc * lscale : -INFINITY;
        }
      }
      lds_barrier();
      // running maximum and denominator (every wave keeps its own copy)
      float cm = -INFINITY;
      for (int r = lane; r < M::ROWS; r += 64) cm = fmaxf(cm, lg[r]);
      const float mn = fmaxf(mx, wave_max(cm));
      const float sc = mx == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mx - mn);
      float ps = 0.f;
      for (int r = lane; r < M::ROWS; r += 64) {
        const float l = lg[r];
        ps += l == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(l - mn);
      }
      den = den * sc + wave_sum(ps);
      mx = mn;
#pragma unroll
      for (int xx = 0; xx < 4; ++xx) p3[xx] *= sc;
#pragma unroll 1
      for (int i = 0; i < M::VPT; ++i) {
        const int jj = rg + M::RG * i;
        const float l = lg[jj];
        const f32x4 vv = raw4_f32(*reinterpret_cast<const R4*>(&vs[jj * D + 4 * cg]));
        const float pj = l == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(l - mn);
#pragma unroll
        for (int xx = 0; xx < 4; ++xx) p3[xx] += l == -INFINITY ? 0.f : pj * vv[xx];
      }
    }
  }

  // ---- one pass over the state held in registers: c1 = S^T k_e, c2 = S^T q
  float p1[4] = {0.f, 0.f, 0.f, 0.f};
  float p2[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < M::R; ++r) {
    const int row = rg + M::RG * r;
    float qr = to_f32(qv[row]);
    if (GLA && evict) qr *= aev[row];
    const float kr2 = evict ? to_f32(kev[row]) * (DGD ? aev[row] : 1.f) : 0.f;
#pragma unroll
    for (int xx = 0; xx < 4; ++xx) {
      p1[xx] += s[r][xx] * kr2;
      p2[xx] += s[r][xx] * qr;
    }
  }
  // reduce over row groups: inside the wave, then across the waves
#pragma unroll
  for (int m = M::CG; m < 64; m <<= 1) {
#pragma unroll
    for (int xx = 0; xx < 4; ++xx) {
      p1[xx] += shfl_xor(p1[xx], m);
      p2[xx] += shfl_xor(p2[xx], m);
      p3[xx] += shfl_xor(p3[xx], m);
    }
  }
  if (lane < M::CG) {
#pragma unroll
    for (int xx = 0; xx < 4; ++xx) {
      red[(wv * M::CG + cg) * 12 + xx] = p1[xx];
      red[(wv * M::CG + cg) * 12 + 4 + xx] = p2[xx];
      red[(wv * M::CG + cg) * 12 + 8 + xx] = p3[xx];
    }
  }
  lds_barrier();
  // across the waves: one thread per reduced value, so that few registers
  // are live beside the state
  if (tid < 12 * M::CG) {
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < M::NWV; ++w) acc += red[w * M::CG * 12 + tid];
    fin[tid] = acc;
  }
  lds_barrier();
  const f32x4 c1 = *reinterpret_cast<const f32x4*>(&fin[cg * 12]);
  float olin[4];
  const f32x4 c2 = *reinterpret_cast<const f32x4*>(&fin[cg * 12 + 4]);
  if (evict) {
    const float kqh = misc[1];
    if constexpr (DGD) {
      const float bt = gates[1];
      float u[4];
#pragma unroll
      for (int xx = 0; xx < 4; ++xx) {
        u[xx] = bt * (to_f32(vev[4 * cg + xx]) - c1[xx]);
        olin[xx] = c2[xx] + u[xx] * kqh;
      }
#pragma unroll
      for (int r = 0; r < M::R; ++r) {
        const int row = rg + M::RG * r;
        const float al = aev[row];
        const float kr2 = to_f32(kev[row]);
#pragma unroll
        for (int xx = 0; xx < 4; ++xx) s[r][xx] = al * s[r][xx] + kr2 * u[xx];
      }
    } else if (GLA) {
#pragma unroll
      for (int xx = 0; xx < 4; ++xx) olin[xx] = c2[xx] + to_f32(vev[4 * cg + xx]) * kqh;
#pragma unroll
      for (int r = 0; r < M::R; ++r) {
        const int row = rg + M::RG * r;
        const float al = aev[row];
        const float kr2 = to_f32(kev[row]);
#pragma unroll
        for (int xx = 0; xx < 4; ++xx) s[r][xx] = al * s[r][xx] + kr2 * to_f32(vev[4 * cg + xx]);
      }
    } else {
      const float al = gates[0];
      const float bt = gates[1];
      float u[4];
#pragma unroll
      for (int xx = 0; xx < 4; ++xx) {
        u[xx] = bt * (to_f32(vev[4 * cg + xx]) - al * c1[xx]);
        olin[xx] = al * c2[xx] + u[xx] * kqh;
      }
#pragma unroll
      for (int r = 0; r < M::R; ++r) {
        const float kr2 = to_f32(kev[rg + M::RG * r]);
#pragma unroll
        for (int xx = 0; xx < 4; ++xx) s[r][xx] = al * s[r][xx] + kr2 * u[xx];
      }
    }
#pragma unroll
    for (int r = 0; r < M::R; ++r)
      __builtin_nontemporal_store(s[r], reinterpret_cast<f32x4*>(Sg + (size_t)(rg + M::RG * r) * D + 4 * cg));
  } else {
#pragma unroll
    for (int xx = 0; xx < 4; ++xx) olin[xx] = c2[xx];
  }
  if (rg == 0) {
    const f32x4 c3 = *reinterpret_cast<const f32x4*>(&fin[cg * 12 + 8]);
    const float inv = swa ? w_swa / den : 0.f;
    f32x4 out;
#pragma unroll
    for (int xx = 0; xx < 4; ++xx) out[xx] = (lin ? olin[xx] * w_lin : 0.f) + (swa ? c3[xx] * inv : 0.f);
    store4(o + (size_t)bh * D + 4 * cg, out);
  }
}

#define GDN_DECODE_STEP_PARAMS                                                                  \
  const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,                       \
      const float *__restrict__ a, const float *__restrict__ b, float *__restrict__ state,         \
      const T *__restrict__ kc, const T *__restrict__ vc, const float *__restrict__ ac,             \
      const float *__restrict__ bc, const int *__restrict__ pos, T *__restrict__ o, int B, int H,   \
      int Hkv, int n_sink, int window, int flags, float w_lin, float w_swa
#define GDN_DECODE_STEP_ARGS \
  q, k, v, a, b, state, kc, vc, ac, bc, pos, o, B, H, Hkv, n_sink, window, flags, w_lin, w_swa

// One staged pass (48 KB of LDS): three workgroups per CU, so at most 80
// VGPRs.
template <class T, int MODE, int D>
__global__ __launch_bounds__(kStepThreads) __attribute__((amdgpu_waves_per_eu(6, 8))) void decode_step_kernel(
    GDN_DECODE_STEP_PARAMS) {
  decode_step_body<T, MODE, D, 1>(GDN_DECODE_STEP_ARGS);
}

// Long budgets: four times the rows per pass (145 KB of LDS, one workgroup
// per CU).
template <class T, int MODE, int D>
__global__ __launch_bounds__(kStepThreads) void decode_step_wide_kernel(GDN_DECODE_STEP_PARAMS) {
  decode_step_body<T, MODE, D, 4>(GDN_DECODE_STEP_ARGS);
}

#undef GDN_DECODE_STEP_PARAMS
#undef GDN_DECODE_STEP_ARGS

// After every head has read the evicted entry: store the new token in its
// slot (and its gates at its ring index) and advance pos.  One workgroup per
// sequence.
template <class T, int MODE>
__global__ __launch_bounds__(256) void decode_commit_kernel(
    const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ a,
    const float* __restrict__ b, T* __restrict__ kc, T* __restrict__ vc, float* __restrict__ ac,
    float* __restrict__ bc, int* __restrict__ pos, int H, int Hkv, int D, int n_sink, int window) {
  const int bi = blockIdx.x;
  const int t = pos[bi];
  if (t < 0) return;
  const int N = n_sink + window;
  const int slot = t < n_sink ? t : n_sink + (t - n_sink) % window;
  for (int i = threadIdx.x; i < Hkv * D; i += blockDim.x) {
    const int g = i / D;
    const int d = i % D;
    const size_t dst = ((size_t)(bi * Hkv + g) * N + slot) * D + d;
    kc[dst] = k[(size_t)bi * Hkv * D + i];
    vc[dst] = v[(size_t)bi * Hkv * D + i];
  }
  if (t >= n_sink) {
    const int ring = (t - n_sink) % window;
    const size_t gb = ((size_t)bi * window + ring) * H;
    if (MODE != 0) {
      for (int i = threadIdx.x; i < H * D; i += blockDim.x) ac[gb * D + i] = a[(size_t)bi * H * D + i];
      if (MODE == 2)
        for (int i = threadIdx.x; i < H; i += blockDim.x) bc[gb + i] = b[(size_t)bi * H + i];
    } else {
      for (int i = threadIdx.x; i < H; i += blockDim.x) {
        ac[gb + i] = a[(size_t)bi * H + i];
        bc[gb + i] = b[(size_t)bi * H + i];
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) pos[bi] = t + 1;
}

// Cache contents after a prefill of T tokens: sinks 0..min(n_sink,T)-1 in
// their slots, window tokens max(n_sink, T-window)..T-1 in ring slots, their
// gates at ring index (i - n_sink) mod window; unwritten slots are zeroed.
template <class T, int MODE>
__global__ __launch_bounds__(256) void cache_fill_kernel(
    const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ a,
    const float* __restrict__ b, T* __restrict__ kc, T* __restrict__ vc,
    float* __restrict__ ac, float* __restrict__ bc, int T_, int H, int Hkv, int D,
    int n_sink, int window) {
  const int j = blockIdx.x;   // slot
  const int bi = blockIdx.y;
  const int N = n_sink + window;
  int tok = -1;
  int ring = -1;
  if (j < n_sink) {
    tok = j < T_ ? j : -1;
  } else if (T_ > n_sink) {
    ring = j - n_sink;
    const int back = ((T_ - 1 - n_sink - ring) % window + window) % window;
    tok = T_ - 1 - back;
    if (tok < n_sink) tok = -1;
  }
  for (int i = threadIdx.x; i < Hkv * D; i += blockDim.x) {
    const int g = i / D;
    const int d = i % D;
    const size_t dst = ((size_t)(bi * Hkv + g) * N + j) * D + d;
    if (tok >= 0) {
      const size_t src = ((size_t)(bi * T_ + tok) * Hkv + g) * D + d;
      kc[dst] = k[src];
      vc[dst] = v[src];
    } else {
      kc[dst] = from_f32<T>(0.f);
      vc[dst] = from_f32<T>(0.f);
    }
  }
  if (ring >= 0) {
    const size_t gb = ((size_t)bi * window + ring) * H;
    const size_t src = ((size_t)bi * T_ + (tok >= 0 ? tok : 0)) * H;
    if (MODE != 0) {
      for (int i = threadIdx.x; i < H * D; i += blockDim.x)
        ac[gb * D + i] = tok >= 0 ? a[src * D + i] : 0.f;
      if (MODE == 2)
        for (int i = threadIdx.x; i < H; i += blockDim.x) bc[gb + i] = tok >= 0 ? b[src + i] : 0.f;
    } else {
      for (int i = threadIdx.x; i < H; i += blockDim.x) {
        ac[gb + i] = tok >= 0 ? a[src + i] : 0.f;
        bc[gb + i] = tok >= 0 ? b[src + i] : 0.f;
      }
    }
  }
}

template <class T, int MODE, int D>
hipError_t launch_decode_t(const DecodeArgs& p, hipStream_t s) {
  const int G = p.H / p.Hkv;
  const dim3 grid(xcd_grouped_grid((long long)p.B * p.Hkv, G));
  // one pass of 128 / sizeof(T) rows holds the whole budget: the narrow kernel
  auto kern = p.n_sink + p.window <= (int)(128 / sizeof(T)) ? decode_step_kernel<T, MODE, D>
                                                             : decode_step_wide_kernel<T, MODE, D>;
  hipLaunchKernelGGL(kern, grid, dim3(kStepThreads), 0, s, (const T*)p.q, (const T*)p.k,
                     (const T*)p.v, p.a, p.b, p.state, (const T*)p.k_cache, (const T*)p.v_cache,
                     p.a_cache, p.b_cache, p.pos, (T*)p.o, p.B, p.H, p.Hkv, p.n_sink, p.window,
                     p.flags, p.w_lin, p.w_swa);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_commit_kernel<T, MODE>), dim3(p.B), dim3(256), 0, s, (const T*)p.k,
                     (const T*)p.v, p.a, p.b, (T*)p.k_cache, (T*)p.v_cache, p.a_cache, p.b_cache,
                     p.pos, p.H, p.Hkv, D, p.n_sink, p.window);
  return hipGetLastError();
}

template <class T>
hipError_t launch_decode_d(const DecodeArgs& p, hipStream_t s) {
  if (p.gla && p.dgd) return p.D == 64 ? launch_decode_t<T, 2, 64>(p, s) : launch_decode_t<T, 2, 128>(p, s);
  if (p.gla) return p.D == 64 ? launch_decode_t<T, 1, 64>(p, s) : launch_decode_t<T, 1, 128>(p, s);
  return p.D == 64 ? launch_decode_t<T, 0, 64>(p, s) : launch_decode_t<T, 0, 128>(p, s);
}

}  // namespace

size_t decode_lds_bytes(int G, int N, int D, int gla, int elt) {
  (void)G;
  const size_t rows = (N <= 128 / elt ? 1 : 4) * 128 / (size_t)elt;   // staged cache rows
  const size_t tiles = 2 * rows * (size_t)D * (size_t)elt;          // K and V
  const size_t vunits = 3 * (size_t)D * elt / 16 + (gla ? (size_t)D / 4 : 0);
  const size_t vecs = (vunits + 63) / 64 * 64 * 16;                 // q, k_e, v_e (, a_e)
  const size_t floats = rows + 64 + 4 + (kStepThreads / 64 + 1) * ((size_t)D / 4) * 12;
  return tiles + vecs + floats * sizeof(float);
}

hipError_t launch_decode(const DecodeArgs& p, hipStream_t s) {
  return p.bf16 ? launch_decode_d<bf16>(p, s) : launch_decode_d<float>(p, s);
}

hipError_t launch_cache_from_prefill(const CacheArgs& p, hipStream_t s) {
  const dim3 grid(p.n_sink + p.window, p.B);
#define GDN_CACHE_LAUNCH(ET, MODE)                                                                 \
  hipLaunchKernelGGL((cache_fill_kernel<ET, MODE>), grid, dim3(256), 0, s, (const ET*)p.k,         \
                     (const ET*)p.v, p.a, p.b, (ET*)p.k_cache, (ET*)p.v_cache, p.a_cache,         \
                     p.b_cache, p.T, p.H, p.Hkv, p.D, p.n_sink, p.window)
  const int mode = p.gla ? (p.dgd ? 2 : 1) : 0;
  if (p.bf16) {
    if (mode == 2) GDN_CACHE_LAUNCH(bf16, 2); else if (mode == 1) GDN_CACHE_LAUNCH(bf16, 1); else GDN_CACHE_LAUNCH(bf16, 0);
  } else {
    if (mode == 2) GDN_CACHE_LAUNCH(float, 2); else if (mode == 1) GDN_CACHE_LAUNCH(float, 1); else GDN_CACHE_LAUNCH(float, 0);
  }
#undef GDN_CACHE_LAUNCH
  return hipGetLastError();
}

}  // namespace gdn
