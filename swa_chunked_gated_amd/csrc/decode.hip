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
// Work split: the softmax branch runs first, one workgroup per (sequence,
// KV head) for its G query heads, so every cached row is read once; the
// linear branch then streams each head's d x d fp32 state through registers
// exactly once (one read, one write), one workgroup per (sequence, query
// head), and adds its output.  A third small kernel (one workgroup per
// sequence) writes the new token into the freed slot and advances pos,
// after every head has read the evicted entry.
//
// Gated delta rule in one pass over the old state S (a, b: evicted gates):
//   c1 = S^T k_e, c2 = S^T q, u = b (v_e - a c1)
//   S' = a S + k_e u^T,  o_lin = S'^T q = a c2 + u (k_e . q)
// GLA: S' = Diag(alpha) S + k_e v_e^T, o_lin = S^T (alpha * q) + v_e (k_e . q).

#include "common.h"
#include "launch.h"

namespace gdn {
namespace {

constexpr int kSwaThreads = 256;
constexpr int kStateThreads = 512;
constexpr int kMaxG = 16;
constexpr int kSlotChunk = 64;   // cache rows staged in LDS at a time

// Slot state of cache slot j for the new token t: -1 not attended, 0 the
// cached entry, 1 the new token (its slot is being overwritten this step).
__device__ __forceinline__ int slot_state_of(int j, int t, int n_sink, int window) {
  if (j < n_sink) return j < t ? 0 : (j == t ? 1 : -1);
  if (t < n_sink) return -1;
  const int r = j - n_sink;
  const int back = ((t - n_sink - r) % window + window) % window;
  return back == 0 ? 1 : (t - back >= n_sink ? 0 : -1);   // latest token of this ring slot
}

// Softmax branch of the decode step for the G query heads of one KV head:
// each cached K and V row is staged through LDS once (both fetched together)
// and used by all G heads.  Writes o (I/O type) = the softmax output of each
// head.
template <class T, int D>
__global__ __launch_bounds__(kSwaThreads) void decode_swa_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ kc, const T* __restrict__ vc, const int* __restrict__ pos,
    T* __restrict__ o, int B, int H, int Hkv, int n_sink, int window) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int SPH = kSwaThreads / D;      // slot phases of the P V sum
  constexpr int SR = D + VEC;               // staged row stride
  typedef typename Vec16<T>::type V16;
  const int G = H / Hkv;
  const int grp = blockIdx.x;               // (sequence, KV head)
  const int bi = grp / Hkv;
  const int g = grp % Hkv;
  const int N = n_sink + window;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = wave_id();
  const int t = pos[bi];
  if (t < 0) return;   // outside the contract (pos >= 0); never index a negative slot

  extern __shared__ float sm[];
  float* qs = sm;                           // [G][D]
  float* kt = qs + G * D;                   // [D] new key
  float* vt = kt + D;                       // [D] new value
  float* lg = vt + D;                       // [G][N] logits, then probabilities
  T* ks = reinterpret_cast<T*>((reinterpret_cast<uintptr_t>(lg + G * N) + 15) & ~(uintptr_t)15);
  T* vs = ks + kSlotChunk * SR;             // [64][SR] staged K and V rows

  const size_t kvbase = (size_t)grp * N * D;     // cache [B][Hkv][N][D]
  const size_t tokkv = (size_t)grp * D;          // k, v  [B][Hkv][D]
  // K and V rows of slots j0 .. j0 + nj - 1 (the new token's slot from k, v;
  // slots not attended as zeros): fetched into registers, then stored to LDS
  constexpr int PER = (kSlotChunk * (D / VEC) + kSwaThreads - 1) / kSwaThreads;
  V16 kr[PER], vr[PER];
  auto fetch = [&](int j0, int nj) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = tid + u * kSwaThreads;
      const int jj = i / (D / VEC);
      const int c = (i % (D / VEC)) * VEC;
      const int st = jj < nj ? slot_state_of(j0 + jj, t, n_sink, window) : -1;
      if (st == 0) {
        kr[u] = *reinterpret_cast<const V16*>(kc + kvbase + (size_t)(j0 + jj) * D + c);
        vr[u] = *reinterpret_cast<const V16*>(vc + kvbase + (size_t)(j0 + jj) * D + c);
      } else {
#pragma unroll
        for (int xx = 0; xx < VEC; ++xx) {
          kr[u][xx] = from_f32<T>(0.f);
          vr[u][xx] = from_f32<T>(0.f);
        }
      }
    }
  };
  auto store = [&](int j0, int nj) {
    lds_barrier();   // kt / vt are in place; the previous chunk's reads are done
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = tid + u * kSwaThreads;
      const int jj = i / (D / VEC);
      const int c = (i % (D / VEC)) * VEC;
      if (jj < kSlotChunk) {
        const int st = jj < nj ? slot_state_of(j0 + jj, t, n_sink, window) : -1;
        if (st == 1) {
#pragma unroll
          for (int xx = 0; xx < VEC; ++xx) {
            kr[u][xx] = from_f32<T>(kt[c + xx]);
            vr[u][xx] = from_f32<T>(vt[c + xx]);
          }
        }
        *reinterpret_cast<V16*>(&ks[jj * SR + c]) = kr[u];
        *reinterpret_cast<V16*>(&vs[jj * SR + c]) = vr[u];
      }
    }
    lds_barrier();
  };
  // the first chunk's rows are requested before the small per-step vectors
  fetch(0, min(kSlotChunk, N));
  for (int i = tid; i < G * D; i += kSwaThreads) qs[i] = to_f32(q[((size_t)bi * H + g * G) * D + i]);
  for (int i = tid; i < D; i += kSwaThreads) {
    kt[i] = to_f32(k[tokkv + i]);
    vt[i] = to_f32(v[tokkv + i]);
  }

  // ---- logits: thread (slot, head) takes a whole dot product
  const float scale = 1.0f / sqrtf((float)D);
  for (int j0 = 0; j0 < N; j0 += kSlotChunk) {
    const int nj = min(kSlotChunk, N - j0);
    if (j0 > 0) fetch(j0, nj);
    store(j0, nj);
    for (int i = tid; i < nj * G; i += kSwaThreads) {
      const int jj = i % nj;
      const int hh = i / nj;
      float acc = 0.f;
#pragma unroll 4
      for (int d = 0; d < D; d += VEC) {
        const V16 kx = *reinterpret_cast<const V16*>(&ks[jj * SR + d]);
#pragma unroll
        for (int xx = 0; xx < VEC; ++xx) acc += to_f32(kx[xx]) * qs[hh * D + d + xx];
      }
      lg[hh * N + j0 + jj] = slot_state_of(j0 + jj, t, n_sink, window) >= 0 ? acc * scale : -INFINITY;
    }
  }
  lds_barrier();
  // ---- softmax per head (wave w takes heads w, w + 4, ...)
  for (int hh = wv; hh < G; hh += kSwaThreads / 64) {
    float* l = lg + hh * N;
    float m = -INFINITY;
    for (int j = lane; j < N; j += 64) m = fmaxf(m, l[j]);
    m = wave_max(m);
    float sum = 0.f;
    for (int j = lane; j < N; j += 64) {
      const float xv = l[j];
      const float pr = xv == -INFINITY ? 0.f : __expf(xv - m);
      l[j] = pr;
      sum += pr;
    }
    sum = wave_sum(sum);
    const float inv = 1.0f / sum;
    for (int j = lane; j < N; j += 64) l[j] *= inv;
  }
  lds_barrier();
  // ---- o = P V: thread (column c, head hh) sums over the slots; SPH heads
  // per pass of the workgroup
  const int c = tid % D;
  for (int h0 = 0; h0 < G; h0 += SPH) {
    const int hh = h0 + tid / D;
    float acc = 0.f;
    if (N > kSlotChunk) {
      // several chunks: restage V chunk by chunk (all threads take part)
      for (int j0 = 0; j0 < N; j0 += kSlotChunk) {
        const int nj = min(kSlotChunk, N - j0);
        fetch(j0, nj);
        store(j0, nj);
        if (hh < G)
          for (int jj = 0; jj < nj; ++jj) acc += lg[hh * N + j0 + jj] * to_f32(vs[jj * SR + c]);
      }
    } else if (hh < G) {
#pragma unroll 8
      for (int jj = 0; jj < N; ++jj) acc += lg[hh * N + jj] * to_f32(vs[jj * SR + c]);
    }
    if (hh < G) o[((size_t)bi * H + g * G + hh) * D + c] = from_f32<T>(acc);
  }
}

template <int D>
struct StateMap {
  static constexpr int CG = D / 4;                 // column groups of 4 floats
  static constexpr int RG = kStateThreads / CG;    // row groups
  static constexpr int R = D / RG;                 // rows per thread
  static constexpr int NWV = kStateThreads / 64;   // waves
};

// Linear branch of the decode step, one workgroup per (sequence, query
// head): the head's d x d fp32 state is streamed through registers exactly
// once (one read, one write), its loads issued before anything else.  With
// the softmax branch, o already holds its output and the linear output is
// added to it.
template <class T, bool GLA, int D>
__global__ __launch_bounds__(kStateThreads) void decode_state_kernel(
    const T* __restrict__ q, const float* __restrict__ a, const float* __restrict__ b,
    float* __restrict__ state, const T* __restrict__ kc, const T* __restrict__ vc,
    const float* __restrict__ ac, const float* __restrict__ bc, const int* __restrict__ pos,
    T* __restrict__ o, int B, int H, int Hkv, int n_sink, int window, int flags) {
  using M = StateMap<D>;
  const int bh = blockIdx.x;
  const int bi = bh / H;
  const int h = bh % H;
  const int g = h / (H / Hkv);
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

  // ---- the head's state is streamed once: issue its loads before anything else
  const int cg = tid % M::CG;
  const int rg = tid / M::CG;
  float* Sg = state + (size_t)bh * D * D;
  f32x4 s[M::R];
#pragma unroll
  for (int r = 0; r < M::R; ++r)
    s[r] = *reinterpret_cast<const f32x4*>(Sg + (size_t)(rg + M::RG * r) * D + 4 * cg);

  __shared__ float qs[D], ke[D], ve[D], ae[D], misc[4];
  __shared__ float red[M::NWV * M::CG * 8];
  const size_t kvbase = ((size_t)bi * Hkv + g) * N * D;
  for (int i = tid; i < D; i += kStateThreads) {
    qs[i] = to_f32(q[(size_t)bh * D + i]);
    if (evict) {
      ke[i] = to_f32(kc[kvbase + (size_t)slot * D + i]);
      ve[i] = to_f32(vc[kvbase + (size_t)slot * D + i]);
    }
  }
  if (evict) {
    const size_t gb = ((size_t)bi * window + ring) * H + h;   // gate cache [B][W][H](,D)
    if (GLA) {
      for (int i = tid; i < D; i += kStateThreads) ae[i] = ac[gb * D + i];
    } else if (tid == 0) {
      ae[0] = ac[gb];
      misc[0] = bc[gb];
    }
  }
  lds_barrier();
  if (evict && wv == 0) {
    float acc = 0.f;
    for (int i = lane; i < D; i += 64) acc += ke[i] * qs[i];
    acc = wave_sum(acc);
    if (lane == 0) misc[1] = acc;   // k_e . q
  }

  // ---- one pass over the state held in registers: c1 = S^T k_e, c2 = S^T q
  float p1[4] = {0.f, 0.f, 0.f, 0.f};
  float p2[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < M::R; ++r) {
    const int row = rg + M::RG * r;
    float qr = qs[row];
    if (GLA && evict) qr *= ae[row];
    const float kr = evict ? ke[row] : 0.f;
#pragma unroll
    for (int xx = 0; xx < 4; ++xx) {
      p1[xx] += s[r][xx] * kr;
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
    }
  }
  if (lane < M::CG) {
#pragma unroll
    for (int xx = 0; xx < 4; ++xx) {
      red[(wv * M::CG + cg) * 8 + xx] = p1[xx];
      red[(wv * M::CG + cg) * 8 + 4 + xx] = p2[xx];
    }
  }
  lds_barrier();
  float c1[4], c2[4];
#pragma unroll
  for (int xx = 0; xx < 4; ++xx) {
    c1[xx] = 0.f;
    c2[xx] = 0.f;
#pragma unroll
    for (int w = 0; w < M::NWV; ++w) {
      c1[xx] += red[(w * M::CG + cg) * 8 + xx];
      c2[xx] += red[(w * M::CG + cg) * 8 + 4 + xx];
    }
  }
  float olin[4];
  if (evict) {
    const float kqh = misc[1];
    if (GLA) {
#pragma unroll
      for (int xx = 0; xx < 4; ++xx) olin[xx] = c2[xx] + ve[4 * cg + xx] * kqh;
#pragma unroll
      for (int r = 0; r < M::R; ++r) {
        const int row = rg + M::RG * r;
        const float al = ae[row];
        const float kr = ke[row];
#pragma unroll
        for (int xx = 0; xx < 4; ++xx) s[r][xx] = al * s[r][xx] + kr * ve[4 * cg + xx];
      }
    } else {
      const float al = ae[0];
      const float bt = misc[0];
      float u[4];
#pragma unroll
      for (int xx = 0; xx < 4; ++xx) {
        u[xx] = bt * (ve[4 * cg + xx] - al * c1[xx]);
        olin[xx] = al * c2[xx] + u[xx] * kqh;
      }
#pragma unroll
      for (int r = 0; r < M::R; ++r) {
        const float kr = ke[rg + M::RG * r];
#pragma unroll
        for (int xx = 0; xx < 4; ++xx) s[r][xx] = al * s[r][xx] + kr * u[xx];
      }
    }
#pragma unroll
    for (int r = 0; r < M::R; ++r)
      *reinterpret_cast<f32x4*>(Sg + (size_t)(rg + M::RG * r) * D + 4 * cg) = s[r];
  } else {
#pragma unroll
    for (int xx = 0; xx < 4; ++xx) olin[xx] = c2[xx];
  }
  if (rg == 0 && (flags & 1)) {
    T* orow = o + (size_t)bh * D + 4 * cg;
    f32x4 out;
#pragma unroll
    for (int xx = 0; xx < 4; ++xx) out[xx] = olin[xx];
    if (flags & 2) out += load4(orow);
    store4(orow, out);
  }
}

// After every head has read the evicted entry: store the new token in its
// slot (and its gates at its ring index) and advance pos.  One workgroup per
// sequence.
template <class T, bool GLA>
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
    if (GLA) {
      for (int i = threadIdx.x; i < H * D; i += blockDim.x) ac[gb * D + i] = a[(size_t)bi * H * D + i];
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
  if (p.flags & 2) {
    const size_t lds = decode_lds_bytes(G, p.n_sink + p.window, D, GLA, (int)sizeof(T));
    if (lds > 64 * 1024) {
      hipError_t e = hipFuncSetAttribute((const void*)decode_swa_kernel<T, D>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((decode_swa_kernel<T, D>), dim3(p.B * p.Hkv), dim3(kSwaThreads), lds, s,
                       (const T*)p.q, (const T*)p.k, (const T*)p.v, (const T*)p.k_cache,
                       (const T*)p.v_cache, p.pos, (T*)p.o, p.B, p.H, p.Hkv, p.n_sink, p.window);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((decode_state_kernel<T, GLA, D>), dim3(p.B * p.H), dim3(kStateThreads), 0, s,
                     (const T*)p.q, p.a, p.b, p.state, (const T*)p.k_cache, (const T*)p.v_cache,
                     p.a_cache, p.b_cache, p.pos, (T*)p.o, p.B, p.H, p.Hkv, p.n_sink, p.window,
                     p.flags);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_commit_kernel<T, GLA>), dim3(p.B), dim3(256), 0, s, (const T*)p.k,
                     (const T*)p.v, p.a, p.b, (T*)p.k_cache, (T*)p.v_cache, p.a_cache, p.b_cache,
                     p.pos, p.H, p.Hkv, D, p.n_sink, p.window);
  return hipGetLastError();
}

template <class T>
hipError_t launch_decode_d(const DecodeArgs& p, hipStream_t s) {
  if (p.gla) return p.D == 64 ? launch_decode_t<T, true, 64>(p, s) : launch_decode_t<T, true, 128>(p, s);
  return p.D == 64 ? launch_decode_t<T, false, 64>(p, s) : launch_decode_t<T, false, 128>(p, s);
}

}  // namespace

size_t decode_lds_bytes(int G, int N, int D, int gla, int elt) {
  (void)gla;
  const size_t floats = (size_t)G * D + 2 * (size_t)D + (size_t)G * N;
  const size_t ints = 0;
  const size_t staging = 2 * (size_t)kSlotChunk * (D + 16 / elt) * elt;   // K and V rows of the I/O type
  return floats * sizeof(float) + ints * sizeof(int) + 16 + staging;
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
