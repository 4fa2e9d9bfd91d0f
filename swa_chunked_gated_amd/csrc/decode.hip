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
// Work split: one workgroup per (sequence, query head).  Its d x d fp32
// state is streamed through registers exactly once (one read, one write);
// the loads are issued first so they overlap the softmax over the cached
// rows.  The G heads of a KV group are mapped to one XCD so the cached rows
// they share are fetched from HBM once.  A second small kernel (one
// workgroup per sequence) then writes the new token into the freed slot and
// advances pos, after every head has read the evicted entry.
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
constexpr int kSlotChunk = 64;   // cache rows staged in LDS at a time

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
    const T* __restrict__ kc, const T* __restrict__ vc, const float* __restrict__ ac,
    const float* __restrict__ bc, const int* __restrict__ pos, T* __restrict__ o, int B, int H,
    int Hkv, int n_sink, int window, int flags) {
  using M = StateMap<D>;
  const int G = H / Hkv;
  // block -> (KV group, head in group); the G heads of a group share
  // blockIdx.x mod 8 so they run on one XCD and share its L2 for the cache rows
  const int NG = B * Hkv;
  int grp, hh;
  const int x = blockIdx.x;
  if (NG % 8 == 0) {
    grp = (x / (8 * G)) * 8 + x % 8;
    hh = (x / 8) % G;
  } else {
    grp = x / G;
    hh = x % G;
  }
  const int bi = grp / Hkv;
  const int g = grp % Hkv;
  const int h = g * G + hh;
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
  float* Sg = state + (size_t)(bi * H + h) * D * D;
  f32x4 s[M::R];
#pragma unroll
  for (int r = 0; r < M::R; ++r)
    s[r] = *reinterpret_cast<const f32x4*>(Sg + (size_t)(rg + M::RG * r) * D + 4 * cg);

  extern __shared__ float sm[];
  float* qs = sm;                       // [D]   query of this head
  float* kt = qs + D;                   // [D]   new key
  float* vt = kt + D;                   // [D]   new value
  float* ke = vt + D;                   // [D]   evicted key
  float* ve = ke + D;                   // [D]   evicted value
  float* ae = ve + D;                   // [D]   evicted a (GLA: per channel; GDN: ae[0])
  float* misc = ae + D;                 // [4]   b_e, k_e . q
  float* osw = misc + 4;                // [D]   softmax output
  float* red = osw + D;                 // [4][CG][8] cross-wave partials
  float* lg = red + 4 * M::CG * 8;      // [N]   logits, then probabilities
  int* slot_state = reinterpret_cast<int*>(lg + N);                      // [N]
  // [64][D + pad] staged cache rows, 16-byte aligned
  T* kvs = reinterpret_cast<T*>((reinterpret_cast<uintptr_t>(slot_state + N) + 15) & ~(uintptr_t)15);

  const size_t kvbase = (size_t)(bi * Hkv + g) * N * D;     // cache [B][Hkv][N][D]
  const size_t tokkv = (size_t)(bi * Hkv + g) * D;          // k, v  [B][Hkv][D]

  // ---- stage the small per-step vectors in LDS
  for (int i = tid; i < D; i += kDecThreads) {
    qs[i] = to_f32(q[(size_t)(bi * H + h) * D + i]);
    kt[i] = to_f32(k[tokkv + i]);
    vt[i] = to_f32(v[tokkv + i]);
    if (evict) {
      ke[i] = to_f32(kc[kvbase + (size_t)slot * D + i]);
      ve[i] = to_f32(vc[kvbase + (size_t)slot * D + i]);
    }
  }
  if (evict) {
    const size_t gb = ((size_t)bi * window + ring) * H + h;   // gate cache [B][W][H](,D)
    if (GLA) {
      for (int i = tid; i < D; i += kDecThreads) ae[i] = ac[gb * D + i];
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

  // ---- softmax branch over the N cache slots (the new token in its slot).
  // Slot states are computed once; cached K and V rows are staged through
  // LDS 64 slots at a time with coalesced 16-byte loads.
  const bool do_swa = (flags & 2) != 0;
  if (do_swa) {
    const float scale = 1.0f / sqrtf((float)D);
    for (int j = tid; j < N; j += kDecThreads) {
      int st;   // -1: not attended, 0: cached entry, 1: the new token
      if (j < n_sink) {
        st = j < t ? 0 : (j == t ? 1 : -1);
      } else if (t < n_sink) {
        st = -1;
      } else {
        const int r = j - n_sink;
        const int back = ((t - n_sink - r) % window + window) % window;
        st = back == 0 ? 1 : (t - back >= n_sink ? 0 : -1);   // latest token of this ring slot
      }
      slot_state[j] = st;
    }
    lds_barrier();
    constexpr int VEC = 16 / sizeof(T);
    for (int j0 = 0; j0 < N; j0 += kSlotChunk) {
      const int nj = min(kSlotChunk, N - j0);
      for (int i = tid; i < nj * (D / VEC); i += kDecThreads) {
        const int jj = i / (D / VEC);
        const int c = (i % (D / VEC)) * VEC;
        const int st = slot_state[j0 + jj];
        typename Vec16<T>::type kv;
        if (st == 0) {
          kv = *reinterpret_cast<const typename Vec16<T>::type*>(kc + kvbase + (size_t)(j0 + jj) * D + c);
        } else {
#pragma unroll
          for (int xx = 0; xx < VEC; ++xx) kv[xx] = from_f32<T>(st == 1 ? kt[c + xx] : 0.f);
        }
        *reinterpret_cast<typename Vec16<T>::type*>(&kvs[jj * (D + VEC) + c]) = kv;
      }
      lds_barrier();
      // 4 threads per slot, each a quarter of the dot product (all 256 threads
      // take part: nj * 4 <= 256, and inactive slots compute on zeros)
      {
        const int jj = tid >> 2;
        const int part = tid & 3;
        float acc = 0.f;
        if (jj < nj) {
#pragma unroll 8
          for (int d = part * (D / 4); d < (part + 1) * (D / 4); ++d)
            acc += to_f32(kvs[jj * (D + VEC) + d]) * qs[d];
        }
        acc += shfl_xor(acc, 1);
        acc += shfl_xor(acc, 2);
        if (part == 0 && jj < nj) lg[j0 + jj] = slot_state[j0 + jj] >= 0 ? acc * scale : -INFINITY;
      }
      lds_barrier();
    }
    if (wv == 0) {
      float m = -INFINITY;
      for (int j = lane; j < N; j += 64) m = fmaxf(m, lg[j]);
      m = wave_max(m);
      float sum = 0.f;
      for (int j = lane; j < N; j += 64) {
        const float xv = lg[j];
        const float pr = xv == -INFINITY ? 0.f : __expf(xv - m);
        lg[j] = pr;
        sum += pr;
      }
      sum = wave_sum(sum);
      const float inv = 1.0f / sum;
      for (int j = lane; j < N; j += 64) lg[j] *= inv;
    }
    {
      // 256 threads: column c and slot phase sph (256 / D phases), reduced at the end
      constexpr int SPH = kDecThreads / D;
      const int c = tid % D;
      const int sph = tid / D;
      float acc = 0.f;
      for (int j0 = 0; j0 < N; j0 += kSlotChunk) {
        const int nj = min(kSlotChunk, N - j0);
        lds_barrier();   // probabilities are final / previous chunk's reads are done
        for (int i = tid; i < nj * (D / VEC); i += kDecThreads) {
          const int jj = i / (D / VEC);
          const int cc = (i % (D / VEC)) * VEC;
          const int st = slot_state[j0 + jj];
          typename Vec16<T>::type vv;
          if (st == 0) {
            vv = *reinterpret_cast<const typename Vec16<T>::type*>(vc + kvbase + (size_t)(j0 + jj) * D + cc);
          } else {
#pragma unroll
            for (int xx = 0; xx < VEC; ++xx) vv[xx] = from_f32<T>(st == 1 ? vt[cc + xx] : 0.f);
          }
          *reinterpret_cast<typename Vec16<T>::type*>(&kvs[jj * (D + VEC) + cc]) = vv;
        }
        lds_barrier();
        for (int jj = sph; jj < nj; jj += SPH) acc += lg[j0 + jj] * to_f32(kvs[jj * (D + VEC) + c]);
      }
      lds_barrier();
      red[tid] = acc;
      lds_barrier();
      if (tid < D) {
        float tot = 0.f;
        for (int p2 = 0; p2 < SPH; ++p2) tot += red[p2 * D + tid];
        osw[tid] = tot;
      }
    }
  }
  lds_barrier();   // osw, misc and the red buffer are settled

  // ---- linear branch: one pass over the state held in registers
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
  // reduce over row groups: inside the wave, then across the 4 waves
#pragma unroll
  for (int m = M::CG; m < 64; m <<= 1) {
#pragma unroll
    for (int xx = 0; xx < 4; ++xx) {
      p1[xx] += shfl_xor(p1[xx], m);
      p2[xx] += shfl_xor(p2[xx], m);
    }
  }
  lds_barrier();   // the softmax's use of `red` is over
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
    for (int w = 0; w < 4; ++w) {
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
  if (rg == 0) {
    f32x4 out;
#pragma unroll
    for (int xx = 0; xx < 4; ++xx) {
      float val = 0.f;
      if (flags & 1) val += olin[xx];
      if (do_swa) val += osw[4 * cg + xx];
      out[xx] = val;
    }
    store4(o + (size_t)(bi * H + h) * D + 4 * cg, out);
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
  const size_t lds = decode_lds_bytes(G, p.n_sink + p.window, D, GLA, (int)sizeof(T));
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)decode_kernel<T, GLA, D>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((decode_kernel<T, GLA, D>), dim3(p.B * p.H), dim3(kDecThreads), lds, s,
                     (const T*)p.q, (const T*)p.k, (const T*)p.v, p.a, p.b, p.state,
                     (const T*)p.k_cache, (const T*)p.v_cache, p.a_cache, p.b_cache, p.pos, (T*)p.o,
                     p.B, p.H, p.Hkv, p.n_sink, p.window, p.flags);
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
  (void)G;
  (void)gla;
  const size_t floats = 8 * (size_t)D + 4 + 4 * (size_t)(D / 4) * 8 + (size_t)N;
  const size_t ints = (size_t)N;
  const size_t staging = (size_t)kSlotChunk * (D + 16 / elt) * elt;   // cache rows of the I/O type
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
