// Softmax branch of the hybrid layer over sinks + sliding window (prefill),
// flash-style, for gfx950: the kernel over swa_tiles (swa_tile.h).
//
// Method (page "The Key to Going Linear: Analysis-Driven Transformer
// Linearization", section 填补近似缺口的实用设计): query t attends with
// softmax to A(t) = { i <= t : i < n_sink or i > t - window }: the sink tokens
// keep full attention and the window holds the most recent tokens, the
// current one included.  Logits are q.k / sqrt(d) (section 从 softmax 到
// delta 规则的一阶近似, Lemma 1).
//
// Work split: one workgroup per (sequence, up to 4 query heads sharing one
// KV head, run of TPW consecutive tiles of QT query rows); each wave owns 32
// query rows of one head.  The next key block is fetched into registers
// (16-byte loads; unguarded when the block is whole) while the current one
// is used from LDS (two LDS buffers), across tiles.  At short budgets with
// many tiles per workgroup (swa_ring_kernel) the key blocks instead stay
// resident in LDS across 64-row tiles and each tile stages one new block.
// Keys are visited in two phases, the sinks [0, n_sink) and then the window
// [max(n_sink, t0 - window + 1), t_end), so a key in both ranges is counted
// once.  64-key blocks of K (row-major) and V (transposed) are staged in LDS
// once and shared by every head of the group.
//
// The product is computed transposed, S^T = K Q^T, so each lane's
// accumulator column is one query: the running max and sum stay per lane
// (plus one butterfly over the 4 lane groups), and the probabilities feed
// O^T += V^T P^T straight from registers (the "acc" reduction set).
// Exponentials use exp2 with log2(e) folded into the scale.  A 16-key tile
// that no query of the wave can see is skipped.
//
// Epilogue: o = O / l, plus the value o already holds on rows t >= add_from
// (the linear branch, or the caller's values when accumulating), cast to the
// output type.

#include "common.h"
#include "launch.h"
#include "swa_tile.h"

namespace gdn {
namespace {

using swa::kNQ;
// most consecutive 64-row tiles per workgroup of the resident-block kernel
constexpr int kRingTiles = 16;

template <class T, int D, int NW>
__global__ __launch_bounds__(64 * NW, 2) void swa_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                      const T* __restrict__ v, T* __restrict__ o,
                                                      int T_, int H, int Hkv, int HPW, int QT, int TPW,
                                                      int n_sink, int window, int add_from,
                                                      float w_swa) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[swa::SwaSmem<T, D>::bytes];
  swa::swa_tiles<T, D, NW, false>(q, k, v, o, T_, H, Hkv, HPW, QT, TPW, n_sink, window, add_from,
                                  blockIdx.x, blockIdx.y, blockIdx.z, reinterpret_cast<T*>(lds),
                                  nullptr, 0, 0, 0, w_swa);
}

// Four query heads of one KV head, 64-row tiles (two waves per head), key
// blocks resident in LDS across the workgroup's TPW consecutive tiles (short
// budgets, many tiles per workgroup; bf16 only, whose key blocks are 64 keys).
template <class T, int D>
__global__ __launch_bounds__(512) void swa_ring_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                       const T* __restrict__ v, T* __restrict__ o,
                                                       int T_, int H, int Hkv, int TPW, int n_sink,
                                                       int window, int add_from, float w_swa) {
  static_assert(swa::KeyBlock<T>::n == 64, "64-row tiles advance by one key block");
  __shared__ __attribute__((aligned(16))) unsigned char lds[swa::SwaSmem<T, D>::ring_bytes];
  swa::swa_tiles<T, D, 8, false, true>(q, k, v, o, T_, H, Hkv, 4, 64, TPW, n_sink, window, add_from,
                                       blockIdx.x, blockIdx.y, blockIdx.z, reinterpret_cast<T*>(lds),
                                       nullptr, 0, 0, 0, w_swa);
}

template <class T>
__global__ void zero_head_rows_kernel(T* __restrict__ o, int T_, int H, int D, int N) {
  const int rows = min(N, T_);
  const size_t per_seq = (size_t)rows * H * D;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int bi = blockIdx.y;
  if (idx < per_seq) o[(size_t)bi * T_ * H * D + idx] = from_f32<T>(0.f);
}

template <class T, int D>
hipError_t launch_swa_t(const PrefillArgs& p, int add_from, hipStream_t s) {
  // heads per workgroup: the largest power of two (<= 4) dividing G; one
  // wave per head and 32 query rows (two waves when a group has one head),
  // so two 4-wave workgroups fit on a CU.  Each workgroup walks TPW
  // consecutive query tiles with one continuous K/V prefetch pipeline.
  const int G = p.H / p.Hkv;
  int HPW = 1;
  while (HPW < 4 && G % (2 * HPW) == 0) HPW *= 2;
  if constexpr (sizeof(T) == 2) {
    // resident key blocks: a 64-row tile's window must fit in three aligned
    // 64-key blocks (window <= 129) and the sinks in one; worth it when every
    // workgroup walks at least four tiles
    if (HPW == 4 && p.n_sink <= 64 && p.window <= 129) {
      const int nt64 = (p.T + 63) / 64;
      const int groups4 = p.H / 4;
      int TPW = 1;
      while (TPW < kRingTiles && (size_t)((nt64 + 2 * TPW - 1) / (2 * TPW)) * groups4 * p.B >= 1024) TPW *= 2;
      if (std::min(TPW, nt64) >= 4) {
        const dim3 grid((nt64 + TPW - 1) / TPW, groups4, p.B);
        hipLaunchKernelGGL((swa_ring_kernel<T, D>), grid, dim3(512), 0, s, (const T*)p.q, (const T*)p.k,
                           (const T*)p.v, (T*)p.o, p.T, p.H, p.Hkv, TPW, p.n_sink, p.window, add_from,
                           p.w_swa);
        return hipGetLastError();
      }
    }
  }
  const int QT = HPW == 1 ? 64 : 32;
  const int waves = HPW * (QT / (16 * kNQ));
  const int ntiles = (p.T + QT - 1) / QT;
  const int groups = p.H / HPW;
  // keep at least ~4 workgroups per CU of work before batching tiles; long
  // budgets do not batch (each tile's key loop is long enough to amortise
  // its pipeline start, and more workgroups run at once: budget 896 is
  // fastest with one tile per workgroup, budget 128 with eight)
  int TPW = 1;
  if (p.n_sink + p.window < 512)
    while (TPW < 8 && (size_t)((ntiles + 2 * TPW - 1) / (2 * TPW)) * groups * p.B >= 2048) TPW *= 2;
  const dim3 grid((ntiles + TPW - 1) / TPW, groups, p.B);
#define GDN_SWA_LAUNCH(NWV)                                                                         \
  hipLaunchKernelGGL((swa_kernel<T, D, NWV>), grid, dim3(64 * NWV), 0, s, (const T*)p.q,           \
                     (const T*)p.k, (const T*)p.v, (T*)p.o, p.T, p.H, p.Hkv, HPW, QT, TPW,         \
                     p.n_sink, p.window, add_from, p.w_swa)
  if (waves == 2) GDN_SWA_LAUNCH(2);
  else GDN_SWA_LAUNCH(4);
#undef GDN_SWA_LAUNCH
  return hipGetLastError();
}

}  // namespace

hipError_t launch_swa_prefill(const PrefillArgs& p, int add_from, hipStream_t s) {
  if (swa_long_applies(p)) return launch_swa_long(p, add_from, s);
  if (p.bf16) return p.D == 64 ? launch_swa_t<bf16, 64>(p, add_from, s) : launch_swa_t<bf16, 128>(p, add_from, s);
  return p.D == 64 ? launch_swa_t<float, 64>(p, add_from, s) : launch_swa_t<float, 128>(p, add_from, s);
}

hipError_t launch_zero_head_rows(const PrefillArgs& p, hipStream_t s) {
  const int N = p.n_sink + p.window;
  const size_t per_seq = (size_t)std::min(N, p.T) * p.H * p.D;
  if (per_seq == 0) return hipSuccess;
  const dim3 grid((unsigned)((per_seq + 255) / 256), p.B);
  if (p.bf16)
    hipLaunchKernelGGL(zero_head_rows_kernel<bf16>, grid, dim3(256), 0, s, (bf16*)p.o, p.T, p.H, p.D, N);
  else
    hipLaunchKernelGGL(zero_head_rows_kernel<float>, grid, dim3(256), 0, s, (float*)p.o, p.T, p.H, p.D, N);
  return hipGetLastError();
}

}  // namespace gdn
