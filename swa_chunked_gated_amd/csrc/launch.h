// Internal launchers shared by the kernel files and the C-ABI front end.
// Every launcher assumes its arguments were validated by the front end.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* a;
  const float* b;
  void* o;
  float* state_out;
  int B, T, H, Hkv, D;
  int n_sink, window;
  int bf16;     // 1: q/k/v/o are bf16, 0: fp32
  int gla;      // 1: GLA diagonal-gate update, 0: gated delta rule
  int flags;    // GDN_BRANCH_LINEAR | GDN_BRANCH_SOFTMAX | GDN_WRITE_STATE
  void* workspace;   // chunk preparation results (gated delta rule), see GdnWorkspace
  float w_lin = 1.f;   // branch weights: o = w_lin o_lin + w_swa o_swa
  float w_swa = 1.f;
  bool prepared = false;   // the workspace already holds the chunk preparation
  int dgd = 0;   // with gla = 1: the delta rule with a diagonal gate (b used)
  void* ckpt = nullptr;    // backward pass: states entering each chunk (bf16 [d][d])
};

// Workspace of the gated delta rule prefill, per (sequence, head, chunk), as
// consecutive arrays (I/O element type; token reduction index in acc order):
//   light preparation: TB = Tm diag(b) [64][64], then g, gamma [2][64] fp32
//   (the scan forms Tm diag(b gamma) from TB and gamma);
//   full preparation (bf16): -Wm [64][D] with d_k in natural order,
//   K^T 2^{g_C - g} [D][64] whose row r holds d_k index acc_pos(r), the
//   scores A [64][64], (TB V)^T [D][64] fp32 (tokens in natural order),
//   g, gamma [2][64] fp32, one uint64 ready flag per chunk, and d / 16
//   uint64 flags per chunk that publish the scan's output rows.
struct GdnWorkspace {
  void* tb;
  void* wm;
  void* ktg;
  void* a;
  float* ut;         // full preparation: (Tm diag(b) V)^T [D][64] fp32
  float* g;
  uint64_t* ready;   // full preparation: per-chunk ready flags
  uint64_t* done;    // full preparation: per-chunk scan-output flags (d / 64 * 4 each)
  size_t bytes;
};
// Full preparation (everything state-independent precomputed) for bf16 when
// the scan alone cannot fill the GPU.
bool gdn_full_prep(int B, int H, int D, int bf16);
GdnWorkspace gdn_workspace_layout(void* base, int B, int H, int nch, int D, size_t elt, bool full);
// Full preparation and state scan (bf16, d = 64 or 128): one kernel whose
// preparation workgroups publish chunks to its scan workgroups when the scan
// leaves half of the GPU free, else the preparation kernel then the scan.
hipError_t launch_gdn_full(const PrefillArgs& p, int nch, hipStream_t s, bool* swa_done);
// Workspace of the GLA prefill: for each (sequence, head, chunk) Q 2^G
// [64][D], (K 2^{G_C - G})^T [D][64], A [64][64] (I/O type, reduction index in
// acc order) and 2^{G_C} [D] fp32, as four consecutive arrays.
// Workspace of the per-channel-gate prefill, per (sequence, head, chunk):
// Q 2^G [64][D], (K 2^{G_C - G})^T [D][64], A [64][64], 2^{G_C} [D] fp32;
// the diagonal-gate delta rule adds TB = Tm diag(b) [64][64] and
// -Wm = -TB (K 2^G) [64][D] (d_k in acc order).
struct GlaWorkspace {
  void* qg;
  void* ktg;
  void* a;
  float* egc;
  void* tb;    // delta only
  void* wm;    // delta only
  size_t bytes;
};
GlaWorkspace gla_workspace_layout(void* base, int B, int H, int nch, int D, size_t elt, bool delta);
// Chunks of the linear stream of a sequence of length T.
inline int gdn_stream_chunks(int T, int n_sink, int window) {
  const long long n = (long long)T - window - n_sink;
  return n > 0 ? (int)((n + 63) / 64) : 0;
}

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* a;
  const float* b;
  float* state;
  void* k_cache;
  void* v_cache;
  float* a_cache;
  float* b_cache;
  int* pos;
  void* o;
  int B, H, Hkv, D;
  int n_sink, window;
  int bf16, gla, flags;   // gla: per-channel gates (GLA, or the diagonal-gate delta rule)
  float w_lin = 1.f;   // branch weights: o = w_lin o_lin + w_swa o_swa
  float w_swa = 1.f;
  int dgd = 0;   // with gla = 1: the delta rule with a diagonal gate (b used)
};

struct CacheArgs {
  const void* k;
  const void* v;
  const float* a;
  const float* b;
  void* k_cache;
  void* v_cache;
  float* a_cache;
  float* b_cache;
  int B, T, H, Hkv, D;
  int n_sink, window;
  int bf16, gla;   // gla: per-channel gates (GLA, or the diagonal-gate delta rule)
  int dgd = 0;     // the diagonal-gate delta rule: b cached too
};

struct ShortConvArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* wq;
  const float* wk;
  const float* wv;
  void* q_out;
  void* k_out;
  void* v_out;
  int B, T, H, Hkv, D, ksize;
  float rope_theta;
  int pos0, flags, bf16;
};

// Linear branch (chunked GDN or GLA): writes (GDN_ACCUMULATE: adds to) o rows
// t >= n_sink + window when the linear branch is selected, zeroes rows
// t < n_sink + window for a linear-only overwrite, and writes the final
// state when asked.
// *swa_done is set when the softmax branch was computed in the same launch.
hipError_t launch_linear_prefill(const PrefillArgs& a, hipStream_t s, bool* swa_done);
// The whole layer in one pass over q, k, v (light preparation, then one
// kernel running the state scan and the softmax rows of each chunk): bf16
// GDN at d = 128 with both branches and no accumulation, many chains,
// window <= 128 and n_sink <= 16.
// Whether the linear branch of p runs a separate chunk-preparation launch
// (false when there is no stream chunk or the one-launch path applies), and
// that launch alone.
bool separate_preparation(const PrefillArgs& p);
hipError_t launch_preparation(const PrefillArgs& p, hipStream_t s);
bool gdn_layer_applies(const PrefillArgs& p);
hipError_t launch_gdn_layer(const PrefillArgs& p, hipStream_t s);
// The same layer kernel for the linear branch alone (overwriting o; the
// softmax branch, when asked for, runs as its own launch after it): bf16
// GDN, d = 128, many chains, when the one-pass layer does not apply.
bool gdn_linear_layer_applies(const PrefillArgs& p);
// add_o: add the linear rows onto what o holds (the softmax branch, launched
// before it) instead of storing them.
hipError_t launch_gdn_linear_layer(const PrefillArgs& p, hipStream_t s, bool add_o = false);
// Segmented scan (bf16 GDN at d = 128, both branches, no accumulation,
// window <= 128, n_sink <= 16, too few chains to fill the GPU): each chain's
// P segments of L chunks each; P = 1 when the chains fill the GPU.
struct SegPlan {
  int P, L;
};
SegPlan gdn_seg_plan(int B, int H, int nch);
bool gdn_segmented(int B, int T, int H, int D, int n_sink, int window, int bf16, int gla, int flags);
bool gdn_segmented(const PrefillArgs& p);
// Its workspace: the light preparation's, then per (segment, chain) the
// map M (bf16), the state N (fp32) and the incoming state S (fp32, one
// more spare segment), each [128][128] row-major.
struct SegWorkspace {
  GdnWorkspace light;
  void* m;
  float* n;
  float* s;
  size_t bytes;
};
SegWorkspace gdn_seg_layout(void* base, int B, int H, int nch);
// Preparation (unless prepared), maps, carry, and the layer kernel per segment.
hipError_t launch_gdn_segmented(const PrefillArgs& p, hipStream_t s);
// Chunk preparation of the gated delta rule / of GLA into a.workspace (nch chunks).
hipError_t launch_gdn_prep(const PrefillArgs& a, int nch, hipStream_t s);
// The backward pass's preparation (bf16, d = 128): the light preparation
// into a.workspace, plus Tm [64][64] (natural order) per chunk into tm.
hipError_t launch_gdn_prep_tm(const PrefillArgs& a, int nch, void* tm, hipStream_t s);
// The backward pass's forward sweep (bf16 GDN, d = 128, light preparation
// in a.workspace): writes the state entering every chunk to a.ckpt.
hipError_t launch_linear_ckpt(const PrefillArgs& a, hipStream_t s);
hipError_t launch_gla_prep(const PrefillArgs& a, int nch, hipStream_t s);
// Softmax branch: writes every row of o, adding the value o already holds
// on rows t >= add_from.
hipError_t launch_swa_prefill(const PrefillArgs& a, int add_from, hipStream_t s);
// The long-budget softmax kernel (bf16, d = 128, window >= 256): key blocks
// reach LDS by direct loads three blocks ahead.  launch_swa_prefill routes
// there when swa_long_applies.
bool swa_long_applies(const PrefillArgs& a);
hipError_t launch_swa_long(const PrefillArgs& a, int add_from, hipStream_t s);
// Zero rows t < n_sink + window of o (linear-only output).
hipError_t launch_zero_head_rows(const PrefillArgs& a, hipStream_t s);

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);
hipError_t launch_cache_from_prefill(const CacheArgs& a, hipStream_t s);
hipError_t launch_shortconv(const ShortConvArgs& a, hipStream_t s);
// Short-conv decode step (a.T unused; pos [B] on the device) and the history
// after a prefill of a.T tokens; hist = {q, k, v} histories [B][ks-1][C] fp32.
hipError_t launch_shortconv_decode(const ShortConvArgs& a, float* const hist[3], const int* pos,
                                   hipStream_t s);
hipError_t launch_shortconv_history(const ShortConvArgs& a, float* const hist[3], hipStream_t s);

// Backward pass (bf16 GDN at d = 128): gradients of sum(do * o) +
// sum(d_state * S_final) into fp32 dq [B,T,H,d], dk, dv [B,T,Hkv,d], da, db
// [B,T,H] (overwritten).
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* a;
  const float* b;
  const void* d_o;
  const float* d_state;     // may be null (zero)
  float* dq;
  float* dk;
  float* dv;
  float* da;
  float* db;
  int B, T, H, Hkv;
  int n_sink, window;
  float w_lin, w_swa;
  void* workspace;
};
// Its workspace: the light preparation's, then per (sequence, head, chunk)
// Tm (bf16 [64][64]), the state entering the chunk and the gradient of the
// state leaving it (bf16 [128][128] each), then per (sequence, head, row) the
// softmax log-sum-exp and D = do.o, and the sink keys' partial dK, dV per
// 64-row query tile (fp32).
struct BwdWorkspace {
  GdnWorkspace light;
  void* tm;
  void* s0;
  void* ds1;
  float* stats;
  float* pk;
  float* pv;
  size_t bytes;
};
BwdWorkspace gdn_bwd_layout(void* base, int B, int T, int H, int n_sink, int window);
hipError_t launch_gdn_backward(const BwdArgs& a, hipStream_t s);

// Time bound of the in-kernel waits on flags published by other workgroups
// of the same launch (100 MHz real-time counter ticks), and faults injected
// by tests (bit 0: the preparation publishes no ready flags; bit 1: the scan
// publishes no done flags).  Process-wide; set by gdn_hybrid_set_test_faults.
struct TestFaults {
  int faults;
  uint64_t wait_ticks;
};
TestFaults test_faults();

// Dynamic LDS bytes the decode kernel needs (the front end checks the limit).
size_t decode_lds_bytes(int G, int N, int D, int gla, int elt);

}  // namespace gdn
