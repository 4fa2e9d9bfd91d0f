// C-ABI front end of the hybrid layer library: host-side validation, then the
// launches on the caller's stream.  See include/gdn_hybrid.h for the contract.

#include <cmath>

#include "gdn_hybrid.h"

#include <stdint.h>

#include <atomic>
#include <initializer_list>
#include <mutex>

#include "launch.h"

namespace {

std::atomic<int> g_last_hip_error{0};
std::atomic<int> g_faults{0};
std::atomic<int> g_wait_us{100000};   // 0.1 s

int launched(hipError_t e) {
  if (e == hipSuccess) return GDN_OK;
  g_last_hip_error.store((int)e);
  return GDN_ELAUNCH;
}

bool dims_ok(int B, int T, int H, int Hkv, int dk, int dv, int n_sink, int window, int dtype,
             int update) {
  if (B < 1 || T < 0 || H < 1 || Hkv < 1 || H % Hkv != 0) return false;
  if (dk != dv || (dk != 64 && dk != 128)) return false;
  if (n_sink < 0 || window < 1) return false;
  if (dtype != GDN_F32 && dtype != GDN_BF16) return false;
  if (update != GDN_DELTA && update != GDN_GLA && update != GDN_DELTA_DIAG) return false;
  // index arithmetic: (b*T + t) fits int, element counts fit 2^40
  if ((int64_t)B * T >= (int64_t)1 << 31) return false;
  if ((int64_t)B * T * H * dk >= (int64_t)1 << 40) return false;
  if ((int64_t)n_sink + window >= (int64_t)1 << 30) return false;
  return true;
}

// The backward pass: bf16 GDN at d = 128 (the query tile, head and sequence
// are grid dimensions).
int backward_supported(int B, int T, int H, int Hkv, int dk, int dv, int n_sink, int window,
                       int dtype, int update) {
  if (!dims_ok(B, T, H, Hkv, dk, dv, n_sink, window, dtype, update)) return GDN_EINVAL;
  if (update != GDN_DELTA || dtype != GDN_BF16 || dk != 128) return GDN_EUNSUPPORTED;
  if ((T + 63) / 64 > 65535 || H > 65535 || B > 65535) return GDN_EUNSUPPORTED;
  return GDN_OK;
}

// Tensor arguments are read and written with 16-byte vector accesses: every
// pointer must be 16-byte aligned (NULL passes; whether a NULL is allowed is
// checked separately).
bool aligned16(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs)
    if (((uintptr_t)p & 15u) != 0) return false;
  return true;
}

}  // namespace

// Device-resident prefill workspace of the allocation-free entry point
// (gdn_hybrid_prefill_noalloc): one copy per GPU, alive until the process
// ends.  Host code never passes `scratch` itself to a kernel (in host code
// the name is a host-side stand-in, not a device address): it uses the
// address hipGetSymbolAddress returns for the current device.
constexpr size_t kScratchBytes = size_t(256) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Address of the current device's scratch array, looked up once per device
// (with that device current) and kept.
int scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    g_last_hip_error.store((int)e);
    return GDN_ELAUNCH;
  }
  if (dev < 0 || dev >= kMaxDevices) return GDN_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      g_last_hip_error.store((int)(e != hipSuccess ? e : hipErrorInvalidSymbol));
      return GDN_ELAUNCH;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GDN_OK;
}

}  // namespace

namespace gdn {
TestFaults test_faults() {
  return TestFaults{g_faults.load(), (uint64_t)g_wait_us.load() * 100u};
}
}  // namespace gdn

extern "C" {

int gdn_hybrid_set_test_faults(int faults, int wait_us) {
  if (faults < 0 || faults > 3 || wait_us < 1 || wait_us > 1000000) return GDN_EINVAL;
  g_faults.store(faults);
  g_wait_us.store(wait_us);
  return GDN_OK;
}

int gdn_hybrid_version(void) { return 10000; }

const char* gdn_hybrid_strerror(int code) {
  switch (code) {
    case GDN_OK: return "ok";
    case GDN_EINVAL: return "invalid argument";
    case GDN_EUNSUPPORTED: return "unsupported parameter combination";
    case GDN_EWORKSPACE: return "workspace too small";
    case GDN_ELAUNCH: return "HIP kernel launch failed";
    default: return "unknown error";
  }
}

int gdn_hybrid_last_hip_error(void) { return g_last_hip_error.load(); }

namespace {
bool prefill_flags_ok(int flags) {
  if (flags < 1 || flags > 63 || (flags & 7) == 0) return false;
  return (flags & (GDN_PREPARE_ONLY | GDN_PREPARED)) != (GDN_PREPARE_ONLY | GDN_PREPARED);
}

// Workspace the linear branch of this call needs (0 unless the gated delta
// rule recurrence runs over at least one chunk).
size_t prefill_workspace_bytes(int B, int T, int H, int dk, int n_sink, int window, int dtype,
                               int update, int flags) {
  const bool rec = (flags & GDN_BRANCH_LINEAR) || (flags & GDN_WRITE_STATE);
  if (!rec) return 0;
  const int nch = gdn::gdn_stream_chunks(T, n_sink, window);
  if (nch == 0) return 0;
  const size_t elt = dtype == GDN_BF16 ? 2 : 4;
  if (update == GDN_DELTA && gdn::gdn_segmented(B, T, H, dk, n_sink, window, elt == 2, 0, flags & 15))
    return gdn::gdn_seg_layout(nullptr, B, H, nch).bytes;
  if (update != GDN_DELTA)
    return gdn::gla_workspace_layout(nullptr, B, H, nch, dk, elt, update == GDN_DELTA_DIAG).bytes;
  return gdn::gdn_workspace_layout(nullptr, B, H, nch, dk, elt, gdn::gdn_full_prep(B, H, dk, elt == 2)).bytes;
}
}  // namespace

int gdn_hybrid_prefill_workspace(int B, int T, int H, int Hkv, int dk, int dv, int n_sink,
                                 int window, int dtype, int update, int flags, size_t* bytes) {
  if (!bytes) return GDN_EINVAL;
  if (!dims_ok(B, T, H, Hkv, dk, dv, n_sink, window, dtype, update)) return GDN_EINVAL;
  if (!prefill_flags_ok(flags)) return GDN_EINVAL;
  *bytes = prefill_workspace_bytes(B, T, H, dk, n_sink, window, dtype, update, flags);
  return GDN_OK;
}

int gdn_hybrid_prefill(const void* q, const void* k, const void* v, const float* a,
                       const float* b, void* o, float* state_out, int B, int T, int H, int Hkv,
                       int dk, int dv, int n_sink, int window, int dtype, int update, int flags,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return gdn_hybrid_prefill_weighted(q, k, v, a, b, o, state_out, B, T, H, Hkv, dk, dv, n_sink,
                                     window, dtype, update, flags, 1.f, 1.f, workspace,
                                     workspace_bytes, stream);
}

namespace {
// Validation and launch of a prefill; with use_scratch the workspace is the
// device's scratch array (workspace / workspace_bytes are ignored).
int prefill_impl(const void* q, const void* k, const void* v, const float* a, const float* b,
                 void* o, float* state_out, int B, int T, int H, int Hkv, int dk, int dv,
                 int n_sink, int window, int dtype, int update, int flags, float w_lin,
                 float w_swa, void* workspace, size_t workspace_bytes, bool use_scratch,
                 void* stream) {
  if (!dims_ok(B, T, H, Hkv, dk, dv, n_sink, window, dtype, update)) return GDN_EINVAL;
  if (!std::isfinite(w_lin) || !std::isfinite(w_swa)) return GDN_EINVAL;
  if (!prefill_flags_ok(flags)) return GDN_EINVAL;
  const bool prep_only = flags & GDN_PREPARE_ONLY;
  const bool prepared = flags & GDN_PREPARED;
  flags &= 15;
  const bool lin = flags & GDN_BRANCH_LINEAR;
  const bool swa = flags & GDN_BRANCH_SOFTMAX;
  const bool wst = flags & GDN_WRITE_STATE;
  const bool acc = flags & GDN_ACCUMULATE;
  const bool needs_rec = lin || wst;
  if (!q || !k || !v) return GDN_EINVAL;
  if ((lin || swa) && !o) return GDN_EINVAL;
  if (needs_rec && !a) return GDN_EINVAL;
  if (needs_rec && update != GDN_GLA && !b) return GDN_EINVAL;
  if (wst && !state_out) return GDN_EINVAL;
  if (!aligned16({q, k, v, a, b, o, state_out})) return GDN_EINVAL;
  if (needs_rec && dtype == GDN_F32 && dk != 64) return GDN_EUNSUPPORTED;
  const size_t need = prefill_workspace_bytes(B, T, H, dk, n_sink, window, dtype, update, flags);
  if (use_scratch) {
    if (need > kScratchBytes) return GDN_EWORKSPACE;
    workspace = nullptr;
    workspace_bytes = 0;
    if (need > 0) {
      const int rc = scratch_of_current_device(&workspace);
      if (rc) return rc;
      workspace_bytes = kScratchBytes;
    }
  }
  if (need > 0 && (!workspace || workspace_bytes < need)) return GDN_EWORKSPACE;
  if (need > 0 && ((uintptr_t)workspace & 255u) != 0) return GDN_EINVAL;
  if (T == 0 && !wst) return GDN_OK;

  gdn::PrefillArgs p{q, k, v, a, b, o, state_out, B, T, H, Hkv, dk, n_sink, window,
                     dtype == GDN_BF16, update != GDN_DELTA, flags, workspace, w_lin, w_swa};
  p.dgd = update == GDN_DELTA_DIAG;
  hipStream_t s = (hipStream_t)stream;
  if (prep_only || prepared) {
    if (!needs_rec || !gdn::separate_preparation(p)) return GDN_EUNSUPPORTED;
    if (prep_only) return launched(gdn::launch_preparation(p, s));
    p.prepared = true;
  }
  const int N = n_sink + window;
  // The linear kernel writes (or adds) rows t >= N and, for a linear-only
  // overwrite, zeroes rows t < N itself; the softmax kernel then adds what o
  // holds on rows t >= add_from.
  const bool run_linear = wst || (lin && T > N);
  // Both branches on the linear-only layer kernel (many chains, windows past
  // the one-pass layer's ring): the softmax launch writes every row first,
  // then the layer kernel adds the linear rows (its reads of o overlap its
  // chunk work, where the softmax launch's would stall it).
  if (swa && lin && T > N && gdn::gdn_linear_layer_applies(p)) {
    int rc = launched(gdn::launch_swa_prefill(p, T, s));
    if (rc) return rc;
    return launched(gdn::launch_gdn_linear_layer(p, s, true));
  }
  bool swa_done = false;
  if (run_linear) {
    int rc = launched(gdn::launch_linear_prefill(p, s, &swa_done));
    if (rc) return rc;
  }
  if (swa && !swa_done) {
    const int add_from = acc ? 0 : ((lin && T > N) ? N : T);
    return launched(gdn::launch_swa_prefill(p, add_from, s));
  }
  if (lin && !acc && !run_linear) return launched(gdn::launch_zero_head_rows(p, s));
  return GDN_OK;
}
}  // namespace

int gdn_hybrid_prefill_weighted(const void* q, const void* k, const void* v, const float* a,
                                const float* b, void* o, float* state_out, int B, int T, int H,
                                int Hkv, int dk, int dv, int n_sink, int window, int dtype,
                                int update, int flags, float w_lin, float w_swa, void* workspace,
                                size_t workspace_bytes, void* stream) {
  return prefill_impl(q, k, v, a, b, o, state_out, B, T, H, Hkv, dk, dv, n_sink, window, dtype,
                      update, flags, w_lin, w_swa, workspace, workspace_bytes, false, stream);
}

size_t gdn_hybrid_noalloc_max_workspace(void) { return kScratchBytes; }

int gdn_hybrid_prefill_noalloc(const void* q, const void* k, const void* v, const float* a,
                               const float* b, void* o, float* state_out, int B, int T, int H,
                               int Hkv, int dk, int dv, int n_sink, int window, int dtype,
                               int update, int flags, void* stream) {
  return prefill_impl(q, k, v, a, b, o, state_out, B, T, H, Hkv, dk, dv, n_sink, window, dtype,
                      update, flags, 1.f, 1.f, nullptr, 0, true, stream);
}

int gdn_hybrid_prefill_backward_workspace(int B, int T, int H, int Hkv, int dk, int dv, int n_sink,
                                          int window, int dtype, int update, size_t* bytes) {
  if (!bytes) return GDN_EINVAL;
  const int rc = backward_supported(B, T, H, Hkv, dk, dv, n_sink, window, dtype, update);
  if (rc) return rc;
  *bytes = gdn::gdn_bwd_layout(nullptr, B, T, H, n_sink, window).bytes;
  return GDN_OK;
}

int gdn_hybrid_prefill_backward(const void* q, const void* k, const void* v, const float* a,
                                const float* b, const void* d_o, const float* d_state, float* dq,
                                float* dk, float* dv, float* da, float* db, int B, int T, int H,
                                int Hkv, int dk_, int dv_, int n_sink, int window, int dtype,
                                int update, float w_lin, float w_swa, void* workspace,
                                size_t workspace_bytes, void* stream) {
  const int rc = backward_supported(B, T, H, Hkv, dk_, dv_, n_sink, window, dtype, update);
  if (rc) return rc;
  if (!std::isfinite(w_lin) || !std::isfinite(w_swa)) return GDN_EINVAL;
  if (!q || !k || !v || !a || !b || !d_o || !dq || !dk || !dv || !da || !db) return GDN_EINVAL;
  if (!aligned16({q, k, v, a, b, d_o, d_state, dq, dk, dv, da, db})) return GDN_EINVAL;
  const size_t need = gdn::gdn_bwd_layout(nullptr, B, T, H, n_sink, window).bytes;
  if (!workspace || workspace_bytes < need) return GDN_EWORKSPACE;
  if (((uintptr_t)workspace & 255u) != 0) return GDN_EINVAL;
  if (T == 0) return GDN_OK;
  gdn::BwdArgs p{q, k, v, a, b, d_o, d_state, dq, dk, dv, da, db, B, T, H, Hkv, n_sink, window,
                 w_lin, w_swa, workspace};
  return launched(gdn::launch_gdn_backward(p, (hipStream_t)stream));
}

int gdn_hybrid_decode(const void* q, const void* k, const void* v, const float* a, const float* b,
                      float* state, void* k_cache, void* v_cache, float* a_cache, float* b_cache,
                      int* pos, void* o, int B, int H, int Hkv, int dk, int dv, int n_sink,
                      int window, int dtype, int update, int flags, void* stream) {
  return gdn_hybrid_decode_weighted(q, k, v, a, b, state, k_cache, v_cache, a_cache, b_cache, pos,
                                    o, B, H, Hkv, dk, dv, n_sink, window, dtype, update, flags, 1.f,
                                    1.f, stream);
}

int gdn_hybrid_decode_weighted(const void* q, const void* k, const void* v, const float* a,
                               const float* b, float* state, void* k_cache, void* v_cache,
                               float* a_cache, float* b_cache, int* pos, void* o, int B, int H,
                               int Hkv, int dk, int dv, int n_sink, int window, int dtype,
                               int update, int flags, float w_lin, float w_swa, void* stream) {
  if (!dims_ok(B, 1, H, Hkv, dk, dv, n_sink, window, dtype, update)) return GDN_EINVAL;
  if (!std::isfinite(w_lin) || !std::isfinite(w_swa)) return GDN_EINVAL;
  if (flags < 1 || flags > 3) return GDN_EINVAL;
  if (!q || !k || !v || !a || !state || !k_cache || !v_cache || !a_cache || !pos || !o)
    return GDN_EINVAL;
  if (update != GDN_GLA && (!b || !b_cache)) return GDN_EINVAL;
  if (!aligned16({q, k, v, a, b, state, k_cache, v_cache, a_cache, b_cache, pos, o})) return GDN_EINVAL;
  const int G = H / Hkv;
  if (G > 16) return GDN_EUNSUPPORTED;
  if ((int64_t)G * (n_sink + window) > 12288) return GDN_EUNSUPPORTED;
  if (gdn::decode_lds_bytes(G, n_sink + window, dk, update != GDN_DELTA, dtype == GDN_BF16 ? 2 : 4) > 160 * 1024)
    return GDN_EUNSUPPORTED;
  gdn::DecodeArgs p{q, k, v, a, b, state, k_cache, v_cache, a_cache, b_cache, pos, o,
                    B, H, Hkv, dk, n_sink, window, dtype == GDN_BF16, update != GDN_DELTA, flags,
                    w_lin, w_swa};
  p.dgd = update == GDN_DELTA_DIAG;
  return launched(gdn::launch_decode(p, (hipStream_t)stream));
}

int gdn_hybrid_cache_from_prefill(const void* k, const void* v, const float* a, const float* b,
                                  void* k_cache, void* v_cache, float* a_cache, float* b_cache,
                                  int B, int T, int H, int Hkv, int dk, int dv, int n_sink,
                                  int window, int dtype, int update, void* stream) {
  if (!dims_ok(B, T, H, Hkv, dk, dv, n_sink, window, dtype, update)) return GDN_EINVAL;
  if (!k_cache || !v_cache || !a_cache) return GDN_EINVAL;
  if (update != GDN_GLA && !b_cache) return GDN_EINVAL;
  if (T > 0 && (!k || !v || !a)) return GDN_EINVAL;
  if (T > 0 && update != GDN_GLA && !b) return GDN_EINVAL;
  if (!aligned16({k, v, a, b, k_cache, v_cache, a_cache, b_cache})) return GDN_EINVAL;
  gdn::CacheArgs p{k, v, a, b, k_cache, v_cache, a_cache, b_cache, B, T, H, Hkv, dk,
                   n_sink, window, dtype == GDN_BF16, update != GDN_DELTA};
  p.dgd = update == GDN_DELTA_DIAG;
  return launched(gdn::launch_cache_from_prefill(p, (hipStream_t)stream));
}

int shortconv_qkv(const void* q, const void* k, const void* v, const float* wq, const float* wk,
                  const float* wv, void* q_out, void* k_out, void* v_out, int B, int T, int H,
                  int Hkv, int d, int ksize, float rope_theta, int pos0, int flags, int dtype,
                  void* stream) {
  if (!dims_ok(B, T, H, Hkv, d, d, 0, 1, dtype, GDN_DELTA)) return GDN_EINVAL;
  if (!q || !k || !v || !wq || !wk || !wv || !q_out || !k_out || !v_out) return GDN_EINVAL;
  if (!aligned16({q, k, v, wq, wk, wv, q_out, k_out, v_out})) return GDN_EINVAL;
  if (ksize < 1 || ksize > 8) return GDN_EUNSUPPORTED;
  if (flags < 0 || flags > 3) return GDN_EINVAL;
  if ((flags & GDN_ROPE) && !(rope_theta > 0.f)) return GDN_EINVAL;
  if (pos0 < 0 || (int64_t)pos0 + T >= (int64_t)1 << 30) return GDN_EINVAL;
  // the sequence and the 64-token tile are grid dimensions
  if (B > 65535 || (T + 63) / 64 > 65535) return GDN_EUNSUPPORTED;
  if (T == 0) return GDN_OK;
  gdn::ShortConvArgs p{q, k, v, wq, wk, wv, q_out, k_out, v_out, B, T, H, Hkv, d, ksize,
                       rope_theta, pos0, flags, dtype == GDN_BF16};
  return launched(gdn::launch_shortconv(p, (hipStream_t)stream));
}

int shortconv_history_from_prefill(const void* q, const void* k, const void* v, float* hist_q,
                                   float* hist_k, float* hist_v, int B, int T, int H, int Hkv, int d,
                                   int ksize, float rope_theta, int pos0, int flags, int dtype,
                                   void* stream) {
  if (!dims_ok(B, T, H, Hkv, d, d, 0, 1, dtype, GDN_DELTA)) return GDN_EINVAL;
  if (ksize < 1 || ksize > 8) return GDN_EUNSUPPORTED;
  if (flags < 0 || flags > 3) return GDN_EINVAL;
  if ((flags & GDN_ROPE) && !(rope_theta > 0.f)) return GDN_EINVAL;
  if (pos0 < 0 || (int64_t)pos0 + T >= (int64_t)1 << 30) return GDN_EINVAL;
  if (B > 65535) return GDN_EUNSUPPORTED;   // the sequence is a grid dimension
  if (ksize == 1) return GDN_OK;   // no history to keep
  if (!hist_q || !hist_k || !hist_v) return GDN_EINVAL;
  if (T > 0 && (!q || !k || !v)) return GDN_EINVAL;
  if (!aligned16({q, k, v, hist_q, hist_k, hist_v})) return GDN_EINVAL;
  gdn::ShortConvArgs p{q, k, v, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, B, T, H, Hkv,
                       d, ksize, rope_theta, pos0, flags, dtype == GDN_BF16};
  float* const hist[3] = {hist_q, hist_k, hist_v};
  return launched(gdn::launch_shortconv_history(p, hist, (hipStream_t)stream));
}

int shortconv_qkv_decode(const void* q, const void* k, const void* v, const float* wq,
                         const float* wk, const float* wv, float* hist_q, float* hist_k,
                         float* hist_v, const int* pos, void* q_out, void* k_out, void* v_out, int B,
                         int H, int Hkv, int d, int ksize, float rope_theta, int pos0, int flags,
                         int dtype, void* stream) {
  if (!dims_ok(B, 1, H, Hkv, d, d, 0, 1, dtype, GDN_DELTA)) return GDN_EINVAL;
  if (!q || !k || !v || !wq || !wk || !wv || !pos || !q_out || !k_out || !v_out) return GDN_EINVAL;
  if (ksize < 1 || ksize > 8) return GDN_EUNSUPPORTED;
  if (ksize > 1 && (!hist_q || !hist_k || !hist_v)) return GDN_EINVAL;
  if (B > 65535) return GDN_EUNSUPPORTED;   // the sequence is a grid dimension
  if (flags < 0 || flags > 3) return GDN_EINVAL;
  if ((flags & GDN_ROPE) && !(rope_theta > 0.f)) return GDN_EINVAL;
  if (pos0 < 0 || pos0 >= 1 << 30) return GDN_EINVAL;
  if (!aligned16({q, k, v, wq, wk, wv, hist_q, hist_k, hist_v, pos, q_out, k_out, v_out}))
    return GDN_EINVAL;
  gdn::ShortConvArgs p{q, k, v, wq, wk, wv, q_out, k_out, v_out, B, 1, H, Hkv, d, ksize,
                       rope_theta, pos0, flags, dtype == GDN_BF16};
  float* const hist[3] = {hist_q, hist_k, hist_v};
  return launched(gdn::launch_shortconv_decode(p, hist, pos, (hipStream_t)stream));
}

}  // extern "C"
