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
// Work split: one workgroup per (sequence, KV head).  It reads the evicted
// ring slot and every cached key/value once for the G query heads of the
// group, then streams each head's d x d fp32 state through registers exactly
// once (one read, one write).  The new token is written into the freed ring
// slot only after a workgroup barrier, so every head of the group has read
// the evicted entry first.  `pos` is advanced by a second tiny kernel so that
// no workgroup can see another's increment.
//
// Gated delta rule in one pass over the old state S (a, b: evicted gates):
//   c1 = S^T k_e, c2 = S^T q, u = b (v_e - a c1)
//   S' = a S + k_e u^T,  o_lin = S'^T q = a c2 + u (k_e . q)
// GLA: S' = Diag(alpha) S + k_e v_e^T, o_lin = S^T (alpha * q) + v_e (k_e . q).

#include "common.h"
#include "launch.h"

namespace gdn {
namespace {

constexpr int kDecThreads = 256;
constexpr int kMaxG = 16;

template <int D>
struct StateMap {
  static constexpr int CG = D / 4;                 // column groups of 4 floats
  static constexpr int RG = kDecThreads / CG;      // row groups
  static constexpr int R = D / RG;                 // rows per thread
};

template <class T, bool GLA, int D>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ a, const float* __restrict__ b, float* __restrict__ state,
    T* __restrict__ kc, T* __restrict__ vc, float* __restrict__ ac, float* __restrict__ bc,
    const int* __restrict__ pos, T* __restrict__ o, int H, int Hkv, int n_sink, int window,
    int flags) {
  using M = StateMap<D>;
  const int g = blockIdx.x;
  const int bi = blockIdx.y;
  const int G = H / Hkv;
  const int N = n_sink + window;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = wave_id();
  const int t = pos[bi];
  if (t < 0) return;   // outside the contract (pos >= 0); never index a negative slot
  const int e = t - window;
  const bool evict = e >= n_sink;
  const int slot = t < n_sink ? t : n_sink + (t - n_sink) % window;
  const int ring = t < n_sink ? -1 : (t - n_sink) % window;

  extern __shared__ float sm[];
  float* qs = sm;                       // [G][D]   queries of the group
  float* kt = qs + G * D;               // [D]      new key
  float* vt = kt + D;                   // [D]      new value
  float* ke = vt + D;                   // [D]      evicted key
  float* ve = ke + D;                   // [D]      evicted value
  float* ae = ve + D;                   // [G] or [G][D] evicted a
  float* be = ae + (GLA ? G * D : G);   // [G]      evicted b
  float* kq = be + G;                   // [G]      k_e . q_h
  float* osw = kq + G;                  // [G][D]   softmax output
  float* red = osw + G * D;             // [4][CG][8] cross-wave partials
  float* lg = red + 4 * M::CG * 8;      // [G][N]   logits, then probabilities

  const size_t kvbase = (size_t)(bi * Hkv + g) * N * D;     // cache [B][Hkv][N][D]
  const size_t tokkv = (size_t)(bi * Hkv + g) * D;          // k, v  [B][Hkv][D]
  const int h0 = g * G;

  // ---- stage the small per-step vectors in LDS
  for (int i = tid; i < G * D; i += kDecThreads)
    qs[i] = to_f32(q[(size_t)(bi * H + h0) * D + i]);
  for (int i = tid; i < D; i += kDecThreads) {
    kt[i] = to_f32(k[tokkv + i]);
    vt[i] = to_f32(v[tokkv + i]);
    if (evict) {
      ke[i] = to_f32(kc[kvbase + (size_t)slot * D + i]);
      ve[i] = to_f32(vc[kvbase + (size_t)slot * D + i]);
    }
  }
  if (evict) {
    const size_t gb = ((size_t)bi * window + ring) * H + h0;   // gate cache [B][W][H](,D)
    if (GLA) {
      for (int i = tid; i < G * D; i += kDecThreads) ae[i] = ac[gb * D + i];
    } else {
      for (int i = tid; i < G; i += kDecThreads) ae[i] = ac[gb + i];
    }
    if (!GLA)
      for (int i = tid; i < G; i += kDecThreads) be[i] = bc[gb + i];
  }
  lds_barrier();

  // ---- k_e . q_h per head
  if (evict) {
    for (int hh = wv; hh < G; hh += kDecThreads / 64) {
      float s = 0.f;
      for (int i = lane; i < D; i += 64) s += ke[i] * qs[hh * D + i];
      s = wave_sum(s);
      if (lane == 0) kq[hh] = s;
    }
  }

  // ---- softmax branch: logits over the N cache slots (new token in its slot)
  const bool do_swa = (flags & 2) != 0;
  if (do_swa) {
    const float scale = 1.0f / sqrtf((float)D);
    for (int j = tid; j < N; j += kDecThreads) {
      bool valid;
      bool isnew;
      if (j < n_sink) {
        valid = j <= t;
        isnew = j == t;
      } else if (t < n_sink) {
        valid = false;
        isnew = false;
      } else {
        const int r = j - n_sink;
        const int back = ((t - n_sink - r) % window + window) % window;
        const int tok = t - back;               // latest token of this ring slot
        valid = tok >= n_sink;
        isnew = back == 0;
      }
      float acc[kMaxG];
#pragma unroll
      for (int hh = 0; hh < kMaxG; ++hh) acc[hh] = 0.f;
      if (valid) {
        for (int d0 = 0; d0 < D; d0 += 4) {
          float kk[4];
          if (isnew) {
#pragma unroll
            for (int x = 0; x < 4; ++x) kk[x] = kt[d0 + x];
          } else {
            f32x4 t4 = load4(kc + kvbase + (size_t)j * D + d0);
#pragma unroll
            for (int x = 0; x < 4; ++x) kk[x] = t4[x];
          }
#pragma unroll
          for (int hh = 0; hh < kMaxG; ++hh) {
            if (hh < G) {
#pragma unroll
              for (int x = 0; x < 4; ++x) acc[hh] += kk[x] * qs[hh * D + d0 + x];
            }
          }
        }
      }
#pragma unroll
      for (int hh = 0; hh < kMaxG; ++hh)
        if (hh < G) lg[hh * N + j] = valid ? acc[hh] * scale : -INFINITY;
    }
    lds_barrier();
    for (int hh = wv; hh < G; hh += kDecThreads / 64) {
      float m = -INFINITY;
      for (int j = lane; j < N; j += 64) m = fmaxf(m, lg[hh * N + j]);
      m = wave_max(m);
      float s = 0.f;
      for (int j = lane; j < N; j += 64) {
        const float x = lg[hh * N + j];
        const float p = x == -INFINITY ? 0.f : __expf(x - m);
        lg[hh * N + j] = p;
        s += p;
      }
      s = wave_sum(s);
      const float inv = 1.0f / s;
      for (int j = lane; j < N; j += 64) lg[hh * N + j] *= inv;
    }
    lds_barrier();
    {
      const int c = tid % D;
      const int hg = tid / D;
      constexpr int HS = kDecThreads / D;
      float acc[kMaxG];
#pragma unroll
      for (int x = 0; x < kMaxG; ++x) acc[x] = 0.f;
      for (int j = 0; j < N; ++j) {
        // probability 0 marks invalid slots; skip their (possibly unwritten) rows
        bool any = false;
        for (int hh = hg; hh < G; hh += HS) any |= lg[hh * N + j] != 0.f;
        if (!any) continue;
        bool isnew;
        if (j < n_sink) {
          isnew = j == t;
        } else {
          const int r = j - n_sink;
          isnew = ((t - n_sink - r) % window + window) % window == 0;
        }
        const float vv = isnew ? vt[c] : to_f32(vc[kvbase + (size_t)j * D + c]);
#pragma unroll
        for (int x = 0; x < kMaxG; ++x) {
          const int hh = hg + x * HS;
          if (hh < G) acc[x] += lg[hh * N + j] * vv;
        }
      }
#pragma unroll
      for (int x = 0; x < kMaxG; ++x) {
        const int hh = hg + x * HS;
        if (hh < G) osw[hh * D + c] = acc[x];
      }
    }
  }

  // ---- linear branch: stream each head's state once
  const int cg = tid % M::CG;
  const int rg = tid / M::CG;
  for (int hh = 0; hh < G; ++hh) {
    const int h = h0 + hh;
    float* Sg = state + (size_t)(bi * H + h) * D * D;
    f32x4 s[M::R];
#pragma unroll
    for (int r = 0; r < M::R; ++r)
      s[r] = *reinterpret_cast<const f32x4*>(Sg + (size_t)(rg + M::RG * r) * D + 4 * cg);
    lds_barrier();   // osw / kq / previous head's `red` reads are complete
    float p1[4] = {0.f, 0.f, 0.f, 0.f};
    float p2[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < M::R; ++r) {
      const int row = rg + M::RG * r;
      float qr = qs[hh * D + row];
      if (GLA && evict) qr *= ae[hh * D + row];
      const float kr = evict ? ke[row] : 0.f;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        p1[x] += s[r][x] * kr;
        p2[x] += s[r][x] * qr;
      }
    }
    // reduce over row groups: inside the wave, then across the 4 waves
#pragma unroll
    for (int m = M::CG; m < 64; m <<= 1) {
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        p1[x] += shfl_xor(p1[x], m);
        p2[x] += shfl_xor(p2[x], m);
      }
    }
    if (lane < M::CG) {
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        red[(wv * M::CG + cg) * 8 + x] = p1[x];
        red[(wv * M::CG + cg) * 8 + 4 + x] = p2[x];
      }
    }
    lds_barrier();
    float c1[4], c2[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      c1[x] = 0.f;
      c2[x] = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        c1[x] += red[(w * M::CG + cg) * 8 + x];
        c2[x] += red[(w * M::CG + cg) * 8 + 4 + x];
      }
    }
    float olin[4];
    if (evict) {
      const float kqh = kq[hh];
      if (GLA) {
#pragma unroll
        for (int x = 0; x < 4; ++x) olin[x] = c2[x] + ve[4 * cg + x] * kqh;
#pragma unroll
        for (int r = 0; r < M::R; ++r) {
          const int row = rg + M::RG * r;
          const float al = ae[hh * D + row];
          const float kr = ke[row];
#pragma unroll
          for (int x = 0; x < 4; ++x) s[r][x] = al * s[r][x] + kr * ve[4 * cg + x];
        }
      } else {
        const float al = ae[hh];
        const float bt = be[hh];
        float u[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          u[x] = bt * (ve[4 * cg + x] - al * c1[x]);
          olin[x] = al * c2[x] + u[x] * kqh;
        }
#pragma unroll
        for (int r = 0; r < M::R; ++r) {
          const float kr = ke[rg + M::RG * r];
#pragma unroll
          for (int x = 0; x < 4; ++x) s[r][x] = al * s[r][x] + kr * u[x];
        }
      }
#pragma unroll
      for (int r = 0; r < M::R; ++r)
        *reinterpret_cast<f32x4*>(Sg + (size_t)(rg + M::RG * r) * D + 4 * cg) = s[r];
    } else {
#pragma unroll
      for (int x = 0; x < 4; ++x) olin[x] = c2[x];
    }
    if (rg == 0) {
      f32x4 out;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        float val = 0.f;
        if (flags & 1) val += olin[x];
        if (do_swa) val += osw[hh * D + 4 * cg + x];
        out[x] = val;
      }
      store4(o + (size_t)(bi * H + h) * D + 4 * cg, out);
    }
  }

  // ---- store the new token into its slot (every head has read the old entry)
  lds_barrier();
  for (int i = tid; i < D; i += kDecThreads) {
    kc[kvbase + (size_t)slot * D + i] = k[tokkv + i];
    vc[kvbase + (size_t)slot * D + i] = v[tokkv + i];
  }
  if (ring >= 0) {
    const size_t gb = ((size_t)bi * window + ring) * H + h0;
    if (GLA) {
      for (int i = tid; i < G * D; i += kDecThreads) ac[gb * D + i] = a[(size_t)(bi * H + h0) * D + i];
    } else {
      for (int i = tid; i < G; i += kDecThreads) ac[gb + i] = a[bi * H + h0 + i];
      for (int i = tid; i < G; i += kDecThreads) bc[gb + i] = b[bi * H + h0 + i];
    }
  }
}

__global__ void advance_pos_kernel(int* __restrict__ pos, int B) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < B) pos[i] += 1;
}

// Cache contents after a prefill of T tokens: sinks 0..min(n_sink,T)-1 in
// their slots, window tokens max(n_sink, T-window)..T-1 in ring slots, their
// gates at ring index (i - n_sink) mod window; unwritten slots are zeroed.
template <class T, bool GLA>
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
    if (GLA) {
      for (int i = threadIdx.x; i < H * D; i += blockDim.x)
        ac[gb * D + i] = tok >= 0 ? a[src * D + i] : 0.f;
    } else {
      for (int i = threadIdx.x; i < H; i += blockDim.x) {
        ac[gb + i] = tok >= 0 ? a[src + i] : 0.f;
        bc[gb + i] = tok >= 0 ? b[src + i] : 0.f;
      }
    }
  }
}

template <class T, bool GLA, int D>
hipError_t launch_decode_t(const DecodeArgs& p, hipStream_t s) {
  const int G = p.H / p.Hkv;
  const size_t lds = decode_lds_bytes(G, p.n_sink + p.window, D, GLA);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)decode_kernel<T, GLA, D>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((decode_kernel<T, GLA, D>), dim3(p.Hkv, p.B), dim3(kDecThreads), lds, s,
                     (const T*)p.q, (const T*)p.k, (const T*)p.v, p.a, p.b, p.state,
                     (T*)p.k_cache, (T*)p.v_cache, p.a_cache, p.b_cache, p.pos, (T*)p.o, p.H,
                     p.Hkv, p.n_sink, p.window, p.flags);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(advance_pos_kernel, dim3((p.B + 255) / 256), dim3(256), 0, s, p.pos, p.B);
  return hipGetLastError();
}

template <class T>
hipError_t launch_decode_d(const DecodeArgs& p, hipStream_t s) {
  if (p.gla) return p.D == 64 ? launch_decode_t<T, true, 64>(p, s) : launch_decode_t<T, true, 128>(p, s);
  return p.D == 64 ? launch_decode_t<T, false, 64>(p, s) : launch_decode_t<T, false, 128>(p, s);
}

}  // namespace

size_t decode_lds_bytes(int G, int N, int D, int gla) {
  const size_t floats = (size_t)G * D + 4 * (size_t)D + (gla ? (size_t)G * D : (size_t)G) + 2 * (size_t)G +
                        (size_t)G * D + 4 * (size_t)(D / 4) * 8 + (size_t)G * N;
  return floats * sizeof(float);
}

hipError_t launch_decode(const DecodeArgs& p, hipStream_t s) {
  return p.bf16 ? launch_decode_d<bf16>(p, s) : launch_decode_d<float>(p, s);
}

hipError_t launch_cache_from_prefill(const CacheArgs& p, hipStream_t s) {
  const dim3 grid(p.n_sink + p.window, p.B);
#define GDN_CACHE_LAUNCH(ET, GLA)                                                                  \
  hipLaunchKernelGGL((cache_fill_kernel<ET, GLA>), grid, dim3(256), 0, s, (const ET*)p.k,          \
                     (const ET*)p.v, p.a, p.b, (ET*)p.k_cache, (ET*)p.v_cache, p.a_cache,         \
                     p.b_cache, p.T, p.H, p.Hkv, p.D, p.n_sink, p.window)
  if (p.bf16) {
    if (p.gla) GDN_CACHE_LAUNCH(bf16, true); else GDN_CACHE_LAUNCH(bf16, false);
  } else {
    if (p.gla) GDN_CACHE_LAUNCH(float, true); else GDN_CACHE_LAUNCH(float, false);
  }
#undef GDN_CACHE_LAUNCH
  return hipGetLastError();
}

}  // namespace gdn
