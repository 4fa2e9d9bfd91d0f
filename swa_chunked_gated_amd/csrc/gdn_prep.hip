// Chunk preparation kernel of the chunked gated delta rule (prefill): the
// part of each 64-token chunk's work that does not depend on the recurrent
// state (gdn_prep.h), done for every chunk at once, one wave per (chunk,
// query head, sequence), so that the sequential scan over chunks only keeps
// the state-dependent products.

#include "common.h"
#include "gdn_prep.h"
#include "launch.h"

namespace gdn {
namespace {

using prep::kC;
using prep::PrepSmem;

template <class T, int D, bool FULL, bool TM = false, int SH = 1>
__global__ __launch_bounds__(256) void gdn_prep_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ a, const float* __restrict__ b, T* __restrict__ wtb,
    T* __restrict__ wwm, T* __restrict__ wktg, T* __restrict__ wa,
    float* __restrict__ wut, float* __restrict__ wg, int T_, int H, int Hkv, int n_sink,
    int window, int nch, T* __restrict__ wtm) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  // The G query heads of one (chunk, KV head) read the same K rows: GW of
  // them (blockDim.x / 64, a divisor of G) are the waves of one workgroup, so
  // their reads meet on one compute unit, and the G / GW workgroups of the
  // unit run on one XCD and share the rows through its L2; y is the sequence.
  // Each wave has its own slice of the LDS; with SH = 4 (GW = 4) the four
  // waves also share the chunk's K K^T.
  const int G = H / Hkv;
  const int GW = blockDim.x >> 6;
  const int wv = wave_id();
  int unit, member;
  if (!xcd_grouped(blockIdx.x, G / GW, nch * Hkv, unit, member)) return;
  const int c = unit % nch;
  const int h = (unit / nch) * G + member * GW + wv;
  if constexpr (SH > 1) {
    prep::gdn_prep_chunk<T, D, FULL, false, TM, SH>(q, k, v, a, b, wtb, wwm, wktg, wa, wut, wg, T_, H,
                                                    Hkv, n_sink, window, nch, c, h, blockIdx.y, smem_raw,
                                                    wtm, wv);
  } else {
    prep::gdn_prep_chunk<T, D, FULL, false, TM>(q, k, v, a, b, wtb, wwm, wktg, wa, wut, wg, T_, H, Hkv,
                                                n_sink, window, nch, c, h, blockIdx.y,
                                                smem_raw + wv * PrepSmem<T, D, FULL>::bytes, wtm);
  }
}

// Waves per workgroup of the preparation kernel: query heads of one KV head,
// up to 4 (48 KiB of LDS for the light preparation); one for the full
// preparation, whose 45 KiB per wave leave no room for more.
template <class T, int D, bool FULL>
int prep_heads_per_workgroup(int G) {
  if (FULL) return 1;
  return G % 4 == 0 ? 4 : G % 2 == 0 ? 2 : 1;
}

template <class T, int D, bool FULL, bool TM>
hipError_t launch_prep_kernel(const PrefillArgs& p, int nch, void* tm, hipStream_t s) {
  using SM = PrepSmem<T, D, FULL>;
  const int G = p.H / p.Hkv;
  const int GW = prep_heads_per_workgroup<T, D, FULL>(G);
  auto kern = gdn_prep_kernel<T, D, FULL, TM>;
  if constexpr (!FULL) {
    if (GW == 4) kern = gdn_prep_kernel<T, D, FULL, TM, 4>;
  }
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     GW * SM::bytes);
  if (e != hipSuccess) return e;
  const GdnWorkspace w = gdn_workspace_layout(p.workspace, p.B, p.H, nch, D, sizeof(T), FULL);
  const dim3 grid(xcd_grouped_grid((long long)nch * p.Hkv, G / GW), p.B);
  hipLaunchKernelGGL(kern, grid, dim3(64 * GW), GW * SM::bytes, s, (const T*)p.q,
                     (const T*)p.k, (const T*)p.v, p.a, p.b, (T*)w.tb, (T*)w.wm,
                     (T*)w.ktg, (T*)w.a, w.ut, w.g, p.T, p.H, p.Hkv, p.n_sink, p.window, nch, (T*)tm);
  return hipGetLastError();
}

template <class T, int D, bool FULL>
hipError_t launch_prep_t(const PrefillArgs& p, int nch, hipStream_t s) {
  return launch_prep_kernel<T, D, FULL, false>(p, nch, nullptr, s);
}

template <class T, int D>
hipError_t launch_prep_d(const PrefillArgs& p, int nch, hipStream_t s) {
  if constexpr (sizeof(T) == 4 && D == 128) {
    return hipErrorInvalidValue;   // fp32 linear branch runs at d = 64 only
  } else {
    if constexpr (sizeof(T) == 2) {
      if (gdn_full_prep(p.B, p.H, p.D, 1) && !gdn_segmented(p)) return launch_prep_t<T, D, true>(p, nch, s);
    }
    return launch_prep_t<T, D, false>(p, nch, s);
  }
}

}  // namespace

bool gdn_full_prep(int B, int H, int D, int bf16) {
  // bf16 and the scan fills fewer workgroups than the GPU has compute units:
  // every state-independent product comes from the preparation kernel
  return bf16 && (long long)B * H * (D == 128 ? 2 : 1) < 256;
}

GdnWorkspace gdn_workspace_layout(void* base, int B, int H, int nch, int D, size_t elt, bool full) {
  GdnWorkspace w;
  const size_t n = (size_t)B * H * nch;
  unsigned char* p = static_cast<unsigned char*>(base);
  size_t off = 0;
  w.tb = full ? nullptr : p + off;
  off += full ? 0 : n * kC * kC * elt;
  w.wm = full ? p + off : nullptr;
  off += full ? n * kC * D * elt : 0;
  w.ktg = full ? p + off : nullptr;
  off += full ? n * D * kC * elt : 0;
  w.a = full ? p + off : nullptr;
  off += full ? n * kC * kC * elt : 0;
  w.ut = full ? reinterpret_cast<float*>(p + off) : nullptr;
  off += full ? n * D * kC * sizeof(float) : 0;
  w.g = reinterpret_cast<float*>(p + off);
  off += n * 2 * kC * sizeof(float);
  w.ready = full ? reinterpret_cast<uint64_t*>(p + off) : nullptr;
  off += full ? n * sizeof(uint64_t) : 0;
  w.done = full ? reinterpret_cast<uint64_t*>(p + off) : nullptr;
  off += full ? n * (D / 16) * sizeof(uint64_t) : 0;
  w.bytes = off;
  return w;
}

hipError_t launch_gdn_prep_tm(const PrefillArgs& p, int nch, void* tm, hipStream_t s) {
  if (!p.bf16 || p.D != 128) return hipErrorInvalidValue;
  return launch_prep_kernel<bf16, 128, false, true>(p, nch, tm, s);
}

hipError_t launch_gdn_prep(const PrefillArgs& p, int nch, hipStream_t s) {
  if (p.bf16) return p.D == 64 ? launch_prep_d<bf16, 64>(p, nch, s) : launch_prep_d<bf16, 128>(p, nch, s);
  return p.D == 64 ? launch_prep_d<float, 64>(p, nch, s) : launch_prep_d<float, 128>(p, nch, s);
}

}  // namespace gdn
