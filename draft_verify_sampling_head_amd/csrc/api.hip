// api.hip -- the C ABI of libdspark.so (declared in include/dspark.h).
// Host-side argument checks, workspace sizing, then kernel enqueues.  No call
// allocates, frees or synchronises (dspark_get_status aside, which reads the
// status word with a blocking copy by design).
#include "dspark.h"

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "launch.hpp"
#include "workspace.hpp"

using namespace dspark;

namespace dspark {

namespace {
std::mutex g_sw_mu;
bool g_sw_init = false;
Switches g_sw{};

void init_switches_locked() {
  if (g_sw_init) return;
  const char* dk = std::getenv("DSPARK_DRAFT_KERNEL");
  g_sw.force_per_step = (dk && std::strcmp(dk, "steps") == 0) ? 1 : 0;
  g_sw.draft_kernel = (dk && std::strcmp(dk, "pipe") == 0) ? 1 : 0;
  g_sw.rnn_cell_valu = std::getenv("DSPARK_RNN_CELL_VALU") ? 1 : 0;
  const char* sl = std::getenv("DSPARK_BARRIER_SPINS");
  g_sw.barrier_spins = sl ? (uint32_t)std::strtoul(sl, nullptr, 10) : 0u;
  const char* pl = std::getenv("DSPARK_PERSIST_LAUNCH");
  g_sw.persist_launch = (pl && std::strcmp(pl, "coop") == 0) ? 1 : 0;
  g_sw_init = true;
}
}  // namespace

Switches switches() {
  std::lock_guard<std::mutex> lk(g_sw_mu);
  init_switches_locked();
  return g_sw;
}

hipError_t launch_coresident(const void* fn, dim3 grid, dim3 block, void** args, size_t lds,
                             hipStream_t st) {
  // Every grid passed here is at most one workgroup per compute unit, and the
  // dispatcher spreads workgroups over the XCDs in turn, so on a device with
  // nothing else running a plain launch is resident at once.  The cooperative
  // launch guarantees it whatever else runs, at the price of the runtime's
  // synchronisation around the kernel (about 20 us per launch, measured).
  if (switches().persist_launch == 0) return hipLaunchKernel(fn, grid, block, args, lds, st);
  return hipLaunchCooperativeKernel(fn, grid, block, args, lds, st);
}

}  // namespace dspark

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
bool dtype_ok(dspark_dtype t) { return t == DSPARK_F32 || t == DSPARK_BF16; }

dspark_status rank_check(int r) {
  if (r < 0) return DSPARK_E_INVALID;
  if (r > 512 || (r % 16) != 0) return DSPARK_E_UNSUPPORTED;
  return DSPARK_OK;
}

dspark_status shape_check(int R, int gamma, int V) {
  if (R < 0 || gamma < 1 || V < 1) return DSPARK_E_INVALID;
  if (gamma > 32) return DSPARK_E_UNSUPPORTED;
  return DSPARK_OK;
}

dspark_status hip_status(hipError_t e) { return e == hipSuccess ? DSPARK_OK : DSPARK_E_HIP; }

__global__ void k_store_u32(uint32_t* p, uint32_t v) {
  if (threadIdx.x == 0) *p = v;
}

}  // namespace

extern "C" {

size_t dspark_workspace_bytes(int R, int gamma, int V, int r, int d) {
  (void)r;
  (void)d;
  if (R < 0 || gamma < 1 || V < 1) return 0;
  return ws_layout(R, gamma, V).total;
}

const char* dspark_status_string(dspark_status s) {
  switch (s) {
    case DSPARK_OK: return "DSPARK_OK";
    case DSPARK_E_INVALID: return "DSPARK_E_INVALID";
    case DSPARK_E_UNSUPPORTED: return "DSPARK_E_UNSUPPORTED";
    case DSPARK_E_WORKSPACE: return "DSPARK_E_WORKSPACE";
    case DSPARK_E_HIP: return "DSPARK_E_HIP";
  }
  return "DSPARK_E_UNKNOWN";
}

const char* dspark_version(void) { return "dspark-mi355x 0.2 (gfx950)"; }

dspark_status dspark_set_switch(int key, int64_t value) {
  std::lock_guard<std::mutex> lk(g_sw_mu);
  init_switches_locked();
  switch (key) {
    case DSPARK_SWITCH_FORCE_PER_STEP:
      if (value != 0 && value != 1) return DSPARK_E_INVALID;
      g_sw.force_per_step = (int)value;
      return DSPARK_OK;
    case DSPARK_SWITCH_RNN_CELL_VALU:
      if (value != 0 && value != 1) return DSPARK_E_INVALID;
      g_sw.rnn_cell_valu = (int)value;
      return DSPARK_OK;
    case DSPARK_SWITCH_BARRIER_SPINS:
      if (value < 0 || value > 0xFFFFFFFFll) return DSPARK_E_INVALID;
      g_sw.barrier_spins = (uint32_t)value;
      return DSPARK_OK;
    case DSPARK_SWITCH_DRAFT_KERNEL:
      if (value != 0 && value != 1) return DSPARK_E_INVALID;
      g_sw.draft_kernel = (int)value;
      return DSPARK_OK;
    case DSPARK_SWITCH_PERSIST_LAUNCH:
      if (value < 0 || value > 1) return DSPARK_E_INVALID;
      g_sw.persist_launch = (int)value;
      return DSPARK_OK;
  }
  return DSPARK_E_INVALID;
}

int64_t dspark_get_switch(int key) {
  std::lock_guard<std::mutex> lk(g_sw_mu);
  init_switches_locked();
  switch (key) {
    case DSPARK_SWITCH_FORCE_PER_STEP: return g_sw.force_per_step;
    case DSPARK_SWITCH_RNN_CELL_VALU: return g_sw.rnn_cell_valu;
    case DSPARK_SWITCH_BARRIER_SPINS: return g_sw.barrier_spins;
    case DSPARK_SWITCH_DRAFT_KERNEL: return g_sw.draft_kernel;
    case DSPARK_SWITCH_PERSIST_LAUNCH: return g_sw.persist_launch;
  }
  return -1;
}

dspark_status dspark_clear_status(void* ws, size_t ws_bytes, hipStream_t stream) {
  DSPARK_ABI_RANGE();
  if (!ws || ws_bytes < 256 || !aligned16(ws)) return DSPARK_E_INVALID;
  hipLaunchKernelGGL(k_store_u32, dim3(1), dim3(64), 0, stream, reinterpret_cast<uint32_t*>(ws), 0u);
  return hip_status(hipGetLastError());
}

dspark_status dspark_get_status(const void* ws, size_t ws_bytes, uint32_t* flags) {
  DSPARK_ABI_RANGE();
  if (!ws || !flags || ws_bytes < 256) return DSPARK_E_INVALID;
  return hip_status(hipMemcpy(flags, ws, sizeof(uint32_t), hipMemcpyDeviceToHost));
}

static dspark_status draft_impl(int R, int gamma, int V, int r, float T, uint64_t seed,
                                uint64_t round, const void* U, dspark_dtype U_dt, const void* W1,
                                const void* W2t, dspark_dtype W_dt, const int32_t* x0, int32_t* x,
                                float* logp_d, float* lse_d, float* margin, void* ws,
                                size_t ws_bytes, hipStream_t stream, hipEvent_t* ev_begin,
                                hipEvent_t* ev_end, int* n_timed, bool dry = false) {
  dspark_status s = shape_check(R, gamma, V);
  if (s != DSPARK_OK) return s;
  if ((s = rank_check(r)) != DSPARK_OK) return s;
  if (!(T >= 0.f) || !std::isfinite(T)) return DSPARK_E_INVALID;
  if (!dtype_ok(U_dt) || !dtype_ok(W_dt)) return DSPARK_E_INVALID;
  if (R == 0) return DSPARK_OK;
  if (!U || !x0 || !x || !logp_d || !lse_d || !ws) return DSPARK_E_INVALID;
  if (r > 0 && (!W1 || !W2t)) return DSPARK_E_INVALID;
  if (r > 0 && (!aligned16(W1) || !aligned16(W2t))) return DSPARK_E_UNSUPPORTED;
  if (!aligned16(ws)) return DSPARK_E_INVALID;
  if (ws_bytes < ws_layout(R, gamma, V).total) return DSPARK_E_WORKSPACE;
  if (dry) return DSPARK_OK;
  return hip_status(launch_draft(R, gamma, V, r, T, seed, round, U, U_dt == DSPARK_BF16, W1, W2t,
                                 W_dt == DSPARK_BF16, x0, x, logp_d, lse_d, margin,
                                 draft_ws(ws, R, gamma, V), stream, ev_begin, ev_end, n_timed));
}

dspark_status dspark_draft_markov(int R, int gamma, int V, int r, float T, uint64_t seed,
                                  uint64_t round, const void* U, dspark_dtype U_dt, const void* W1,
                                  const void* W2t, dspark_dtype W_dt, const int32_t* x0,
                                  int32_t* x, float* logp_d, float* lse_d, float* margin, void* ws,
                                  size_t ws_bytes, hipStream_t stream) {
  DSPARK_ABI_RANGE();
  return draft_impl(R, gamma, V, r, T, seed, round, U, U_dt, W1, W2t, W_dt, x0, x, logp_d, lse_d,
                    margin, ws, ws_bytes, stream, nullptr, nullptr, nullptr);
}

dspark_status dspark_draft_markov_profiled(int R, int gamma, int V, int r, float T, uint64_t seed,
                                           uint64_t round, const void* U, dspark_dtype U_dt,
                                           const void* W1, const void* W2t, dspark_dtype W_dt,
                                           const int32_t* x0, int32_t* x, float* logp_d,
                                           float* lse_d, float* margin, void* ws, size_t ws_bytes,
                                           hipStream_t stream, hipEvent_t* ev_begin,
                                           hipEvent_t* ev_end, int* n_timed) {
  DSPARK_ABI_RANGE();
  if (!ev_begin || !ev_end) return DSPARK_E_INVALID;
  if (n_timed) *n_timed = 0;
  return draft_impl(R, gamma, V, r, T, seed, round, U, U_dt, W1, W2t, W_dt, x0, x, logp_d, lse_d,
                    margin, ws, ws_bytes, stream, ev_begin, ev_end, n_timed);
}

size_t dspark_rnn_workspace_bytes(int R, int gamma, int V, int r, int d) {
  (void)d;
  if (R < 0 || gamma < 1 || V < 1 || r < 0) return 0;
  return rnn_ws_layout(R, gamma, V, r).total;
}

static dspark_status draft_rnn_impl(int R, int gamma, int V, int r, int d, float T,
                                    uint64_t seed, uint64_t round, const void* U,
                                    dspark_dtype U_dt, const void* W1, const void* W2t,
                                    dspark_dtype W_dt, const void* Wr, const void* h,
                                    dspark_dtype h_dt, const int32_t* x0, int32_t* x,
                                    float* logp_d, float* lse_d, float* margin, void* feat,
                                    float* state, void* ws, size_t ws_bytes, hipStream_t stream,
                                    hipEvent_t* ev_begin, hipEvent_t* ev_end, int* n_timed) {
  dspark_status s = shape_check(R, gamma, V);
  if (s != DSPARK_OK) return s;
  if (d < 1) return DSPARK_E_INVALID;
  if ((s = rank_check(r)) != DSPARK_OK) return s;
  if (r == 0) return DSPARK_E_UNSUPPORTED;
  if (!(T >= 0.f) || !std::isfinite(T)) return DSPARK_E_INVALID;
  if (!dtype_ok(U_dt) || !dtype_ok(W_dt) || !dtype_ok(h_dt)) return DSPARK_E_INVALID;
  if (R == 0) return DSPARK_OK;
  if (!U || !W1 || !W2t || !Wr || !h || !x0 || !x || !logp_d || !lse_d || !feat || !ws)
    return DSPARK_E_INVALID;
  if (!aligned16(W1) || !aligned16(W2t) || !aligned16(feat)) return DSPARK_E_UNSUPPORTED;
  if (!aligned16(ws)) return DSPARK_E_INVALID;
  const RnnWsLayout RL = rnn_ws_layout(R, gamma, V, r);
  if (ws_bytes < RL.total) return DSPARK_E_WORKSPACE;
  char* w = reinterpret_cast<char*>(ws);
  RnnArgs a{};
  a.R = R; a.gamma = gamma; a.V = V; a.rank = r; a.d = d;
  a.W1 = W1; a.Wr = Wr; a.h = h; a.w_bf16 = W_dt == DSPARK_BF16; a.h_bf16 = h_dt == DSPARK_BF16;
  a.x0 = x0; a.x = x;
  a.P = reinterpret_cast<float*>(w + RL.P);
  a.state = state ? state : reinterpret_cast<float*>(w + RL.state);
  a.feat = feat;
  a.status = reinterpret_cast<uint32_t*>(w + ws_layout(R, gamma, V).header);
  return hip_status(launch_draft(R, gamma, V, r, T, seed, round, U, U_dt == DSPARK_BF16, W1, W2t,
                                 W_dt == DSPARK_BF16, x0, x, logp_d, lse_d, margin,
                                 draft_ws(ws, R, gamma, V), stream, ev_begin, ev_end, n_timed, &a));
}

dspark_status dspark_draft_rnn(int R, int gamma, int V, int r, int d, float T, uint64_t seed,
                               uint64_t round, const void* U, dspark_dtype U_dt, const void* W1,
                               const void* W2t, dspark_dtype W_dt, const void* Wr, const void* h,
                               dspark_dtype h_dt, const int32_t* x0, int32_t* x, float* logp_d,
                               float* lse_d, float* margin, void* feat, float* state, void* ws,
                               size_t ws_bytes, hipStream_t stream) {
  DSPARK_ABI_RANGE();
  return draft_rnn_impl(R, gamma, V, r, d, T, seed, round, U, U_dt, W1, W2t, W_dt, Wr, h, h_dt,
                        x0, x, logp_d, lse_d, margin, feat, state, ws, ws_bytes, stream, nullptr,
                        nullptr, nullptr);
}

dspark_status dspark_draft_rnn_profiled(int R, int gamma, int V, int r, int d, float T,
                                        uint64_t seed, uint64_t round, const void* U,
                                        dspark_dtype U_dt, const void* W1, const void* W2t,
                                        dspark_dtype W_dt, const void* Wr, const void* h,
                                        dspark_dtype h_dt, const int32_t* x0, int32_t* x,
                                        float* logp_d, float* lse_d, float* margin, void* feat,
                                        float* state, void* ws, size_t ws_bytes,
                                        hipStream_t stream, hipEvent_t* ev_begin,
                                        hipEvent_t* ev_end, int* n_timed) {
  DSPARK_ABI_RANGE();
  if (!ev_begin || !ev_end) return DSPARK_E_INVALID;
  if (n_timed) *n_timed = 0;
  return draft_rnn_impl(R, gamma, V, r, d, T, seed, round, U, U_dt, W1, W2t, W_dt, Wr, h, h_dt,
                        x0, x, logp_d, lse_d, margin, feat, state, ws, ws_bytes, stream, ev_begin,
                        ev_end, n_timed);
}

static dspark_status confidence_impl(int R, int gamma, int d, int r, int V, const void* h,
                                     dspark_dtype h_dt, const void* W1, dspark_dtype W_dt,
                                     const void* w, dspark_dtype w_dt, const float* sts_T,
                                     const int32_t* x, float* c, bool logits, hipStream_t stream, bool dry = false) {
  if (R < 0 || gamma < 1 || d < 1) return DSPARK_E_INVALID;
  if (gamma > 32) return DSPARK_E_UNSUPPORTED;
  dspark_status s = rank_check(r);
  if (s != DSPARK_OK) return s;
  if (!dtype_ok(h_dt) || !dtype_ok(W_dt) || !dtype_ok(w_dt)) return DSPARK_E_INVALID;
  if (R == 0) return DSPARK_OK;
  if (!h || !w || !x || !c) return DSPARK_E_INVALID;
  if (r > 0 && (!W1 || V < 1)) return DSPARK_E_INVALID;
  ConfArgs a{};
  a.R = R; a.gamma = gamma; a.d = d; a.rank = r; a.V = V; a.h = h; a.W1 = W1; a.w = w;
  a.sts = sts_T; a.x = x; a.c = c; a.status = nullptr; a.logits = logits;
  const size_t hs = h_dt == DSPARK_BF16 ? 2 : 4, ws_ = w_dt == DSPARK_BF16 ? 2 : 4;
  const size_t es = W_dt == DSPARK_BF16 ? 2 : 4;
  a.vec_h = aligned16(h) && aligned16(w) && ((size_t)d * hs) % 16 == 0 && hs == ws_;
  a.vec_e = r > 0 && aligned16(W1) && aligned16(reinterpret_cast<const char*>(w) + (size_t)d * ws_) &&
            ((size_t)r * es) % 16 == 0 && es == ws_;
  if (dry) return DSPARK_OK;
  return hip_status(launch_confidence(a, h_dt == DSPARK_BF16, W_dt == DSPARK_BF16,
                                      w_dt == DSPARK_BF16, stream));
}

dspark_status dspark_confidence(int R, int gamma, int d, int r, int V, const void* h,
                                dspark_dtype h_dt, const void* W1, dspark_dtype W_dt,
                                const void* w, dspark_dtype w_dt, const float* sts_T,
                                const int32_t* x, float* c, hipStream_t stream) {
  DSPARK_ABI_RANGE();
  return confidence_impl(R, gamma, d, r, V, h, h_dt, W1, W_dt, w, w_dt, sts_T, x, c, false,
                         stream);
}

dspark_status dspark_confidence_logits(int R, int gamma, int d, int r, int V, const void* h,
                                       dspark_dtype h_dt, const void* W1, dspark_dtype W_dt,
                                       const void* w, dspark_dtype w_dt, const int32_t* x,
                                       float* z, hipStream_t stream) {
  DSPARK_ABI_RANGE();
  return confidence_impl(R, gamma, d, r, V, h, h_dt, W1, W_dt, w, w_dt, nullptr, x, z, true,
                         stream);
}

dspark_status dspark_prefix_schedule(int R, int gamma, const float* c, const double* sps,
                                     int N_max, int enabled, int32_t* ell, float* a,
                                     int32_t* N_out, double* theta_best, hipStream_t stream) {
  DSPARK_ABI_RANGE();
  if (R < 0 || gamma < 1) return DSPARK_E_INVALID;
  if (gamma > 32) return DSPARK_E_UNSUPPORTED;
  if (R == 0) return DSPARK_OK;
  if (!c || !sps || !ell) return DSPARK_E_INVALID;
  if (N_max < R) return DSPARK_E_INVALID;
  // static verification sends the whole block: R (gamma + 1) tokens must fit
  if (!enabled && (int64_t)N_max < (int64_t)R * (gamma + 1)) return DSPARK_E_INVALID;
  if ((int64_t)R * gamma > 16384) return DSPARK_E_UNSUPPORTED;
  SchedArgs sa{};
  sa.R = R; sa.gamma = gamma; sa.N_max = N_max; sa.enabled = enabled ? 1 : 0;
  sa.c = c; sa.sps = sps; sa.ell = ell; sa.a = a; sa.N_out = N_out; sa.theta = theta_best;
  return hip_status(launch_schedule(sa, stream));
}

dspark_status dspark_async_schedule(int R, int gamma, const float* c, const double* sps,
                                    int N_max, const int32_t* K_in, int32_t* K_plan, int32_t* ell,
                                    float* a, int32_t* N_out, double* theta, double* theta_plan,
                                    hipStream_t stream) {
  DSPARK_ABI_RANGE();
  if (R < 0 || gamma < 1) return DSPARK_E_INVALID;
  if (gamma > 32) return DSPARK_E_UNSUPPORTED;
  if (R == 0) return DSPARK_OK;
  if (!c || !sps || !ell || !K_in || !K_plan) return DSPARK_E_INVALID;
  if (N_max < R) return DSPARK_E_INVALID;
  if ((int64_t)R * gamma > 16384) return DSPARK_E_UNSUPPORTED;
  SchedArgs sa{};
  sa.R = R; sa.gamma = gamma; sa.N_max = N_max; sa.enabled = 1; sa.mode = 1;
  sa.c = c; sa.sps = sps; sa.ell = ell; sa.a = a; sa.N_out = N_out; sa.theta = theta;
  sa.K_in = K_in; sa.K_plan = K_plan; sa.theta_plan = theta_plan;
  return hip_status(launch_schedule(sa, stream));
}

static dspark_status schedule_pack_impl(int R, int gamma, int mode, const float* c,
                                        const double* sps, int N_max, const int32_t* K_in,
                                        int32_t* K_plan, const int32_t* x, int32_t* ell, float* a,
                                        int32_t* N_out, double* theta, double* theta_plan,
                                        int32_t* cu, int32_t* flat, int32_t* marker_req,
                                        int32_t* marker_pos, hipStream_t stream, bool dry) {
  if (R < 0 || gamma < 1) return DSPARK_E_INVALID;
  if (mode < 0 || mode > 2) return DSPARK_E_INVALID;
  if (gamma > 32) return DSPARK_E_UNSUPPORTED;
  if (R == 0) return DSPARK_OK;
  if (!c || !sps || !ell || !x || !cu || !flat) return DSPARK_E_INVALID;
  if (mode == 2 && (!K_in || !K_plan)) return DSPARK_E_INVALID;
  if (N_max < R) return DSPARK_E_INVALID;
  if (mode == 0 && (int64_t)N_max < (int64_t)R * (gamma + 1)) return DSPARK_E_INVALID;
  if ((int64_t)R * gamma > 16384) return DSPARK_E_UNSUPPORTED;
  SchedArgs sa{};
  sa.R = R; sa.gamma = gamma; sa.N_max = N_max; sa.enabled = mode != 0; sa.mode = mode == 2;
  sa.c = c; sa.sps = sps; sa.ell = ell; sa.a = a; sa.N_out = N_out; sa.theta = theta;
  sa.K_in = K_in; sa.K_plan = K_plan; sa.theta_plan = theta_plan;
  sa.pack = true;
  PackArgs& p = sa.pk;
  p.R = R; p.width = gamma + 1; p.rows = x; p.cu = cu; p.flat = flat;
  p.marker_req = marker_req; p.marker_pos = marker_pos;
  p.slots = (int64_t)R * (gamma + 1);
  if (dry) return DSPARK_OK;
  return hip_status(launch_schedule(sa, stream));
}

dspark_status dspark_schedule_pack(int R, int gamma, int mode, const float* c, const double* sps,
                                   int N_max, const int32_t* K_in, int32_t* K_plan,
                                   const int32_t* x, int32_t* ell, float* a, int32_t* N_out,
                                   double* theta, double* theta_plan, int32_t* cu, int32_t* flat,
                                   int32_t* marker_req, int32_t* marker_pos, hipStream_t stream) {
  DSPARK_ABI_RANGE();
  return schedule_pack_impl(R, gamma, mode, c, sps, N_max, K_in, K_plan, x, ell, a, N_out, theta,
                            theta_plan, cu, flat, marker_req, marker_pos, stream, false);
}

static dspark_status pack_impl(int R, int width, const int32_t* rows, const int32_t* len,
                               int len_offset, int32_t* cu, int32_t* flat, int32_t* marker_req,
                               int32_t* marker_pos, int32_t* N_out, void* ws, size_t ws_bytes,
                               hipStream_t stream, bool dry) {
  if (R < 0 || width < 1) return DSPARK_E_INVALID;
  if (R == 0) return DSPARK_OK;
  if (!rows || !len || !cu || !flat) return DSPARK_E_INVALID;
  if ((int64_t)R * width >= ((int64_t)1 << 31)) return DSPARK_E_UNSUPPORTED;
  if (ws && (ws_bytes < 256 || !aligned16(ws))) return DSPARK_E_WORKSPACE;
  PackArgs p{};
  p.R = R; p.width = width; p.len_offset = len_offset; p.rows = rows; p.len = len; p.cu = cu;
  p.flat = flat; p.marker_req = marker_req; p.marker_pos = marker_pos; p.N_out = N_out;
  p.status = reinterpret_cast<uint32_t*>(ws);
  p.slots = (int64_t)R * width;
  if (dry) return DSPARK_OK;
  return hip_status(launch_pack(p, stream));
}

dspark_status dspark_pack(int R, int width, const int32_t* rows, const int32_t* len,
                          int len_offset, int32_t* cu, int32_t* flat, int32_t* marker_req,
                          int32_t* marker_pos, int32_t* N_out, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  DSPARK_ABI_RANGE();
  return pack_impl(R, width, rows, len, len_offset, cu, flat, marker_req, marker_pos, N_out, ws,
                   ws_bytes, stream, false);
}

dspark_status dspark_pack_tiered(int R, int width, const int32_t* rows, const int32_t* len,
                                 int len_offset, const int32_t* tiers, int n_tiers, int pad_token,
                                 int64_t slots, int32_t* cu, int32_t* flat, int32_t* marker_req,
                                 int32_t* marker_pos, int32_t* N_out, int32_t* N_pad, void* ws,
                                 size_t ws_bytes, hipStream_t stream) {
  DSPARK_ABI_RANGE();
  if (R < 0 || width < 1) return DSPARK_E_INVALID;
  if (n_tiers < 0 || (n_tiers > 0 && !tiers)) return DSPARK_E_INVALID;
  if (n_tiers > kMaxTiers) return DSPARK_E_UNSUPPORTED;
  if (slots < (int64_t)R * width) return DSPARK_E_INVALID;
  for (int k = 0; k < n_tiers; ++k) {
    if (tiers[k] < 1 || tiers[k] > slots) return DSPARK_E_INVALID;
    if (k > 0 && tiers[k] <= tiers[k - 1]) return DSPARK_E_INVALID;
  }
  if (R == 0) return DSPARK_OK;
  if (!rows || !len || !cu || !flat) return DSPARK_E_INVALID;
  if (slots >= ((int64_t)1 << 31)) return DSPARK_E_UNSUPPORTED;
  if (ws && (ws_bytes < 256 || !aligned16(ws))) return DSPARK_E_WORKSPACE;
  PackArgs p{};
  p.R = R; p.width = width; p.len_offset = len_offset; p.rows = rows; p.len = len; p.cu = cu;
  p.flat = flat; p.marker_req = marker_req; p.marker_pos = marker_pos; p.N_out = N_out;
  p.status = reinterpret_cast<uint32_t*>(ws);
  p.slots = slots; p.ntiers = n_tiers; p.pad_token = pad_token; p.N_pad = N_pad;
  for (int k = 0; k < n_tiers; ++k) p.tiers[k] = tiers[k];
  return hip_status(launch_pack(p, stream));
}

static dspark_status verify_impl(int R, int gamma, int V, int r, float T, uint64_t seed,
                                 uint64_t round, const int32_t* ell, const int32_t* cu,
                                 const void* target, dspark_dtype t_dt, int target_layout,
                                 const int32_t* x, const float* logp_d, const float* lse_d,
                                 const void* U, dspark_dtype U_dt, const void* W1, const void* W2t,
                                 dspark_dtype W_dt, int32_t* m, int32_t* tau, int32_t* emitted,
                                 int32_t* next_anchor, float* logp_t, void* ws, size_t ws_bytes,
                                 hipStream_t stream, const int32_t* cap, int32_t* m_full,
                                 const void* feat = nullptr, bool dry = false) {
  dspark_status s = shape_check(R, gamma, V);
  if (s != DSPARK_OK) return s;
  if ((s = rank_check(r)) != DSPARK_OK) return s;
  if (!(T >= 0.f) || !std::isfinite(T)) return DSPARK_E_INVALID;
  if (!dtype_ok(t_dt) || !dtype_ok(U_dt) || !dtype_ok(W_dt)) return DSPARK_E_INVALID;
  if (target_layout != 0 && target_layout != 1) return DSPARK_E_INVALID;
  if (R == 0) return DSPARK_OK;
  if (t_dt != U_dt) return DSPARK_E_UNSUPPORTED;
  if (!ell || !cu || !target || !x || !m || !tau || !emitted || !next_anchor || !ws)
    return DSPARK_E_INVALID;
  if (T > 0.f && (!logp_d || !lse_d || !U)) return DSPARK_E_INVALID;
  if (T > 0.f && r > 0 && (!W1 || !W2t)) return DSPARK_E_INVALID;
  if (r > 0 && T > 0.f && (!aligned16(W1) || !aligned16(W2t))) return DSPARK_E_UNSUPPORTED;
  if (!aligned16(ws)) return DSPARK_E_INVALID;
  if (ws_bytes < ws_layout(R, gamma, V).total) return DSPARK_E_WORKSPACE;
  if (dry) return DSPARK_OK;
  return hip_status(launch_verify(R, gamma, V, r, T, seed, round, ell, cu, target, target_layout,
                                  x, logp_d, lse_d, U, U_dt == DSPARK_BF16, W1, W2t,
                                  W_dt == DSPARK_BF16, m, tau, emitted, next_anchor, logp_t, ws,
                                  stream, cap, m_full, feat));
}

size_t dspark_sts_workspace_bytes(int n) {
  return n < 0 ? 0
               : 256 + ws_align((size_t)n * 8) +
                     (size_t)kStsMaxGrid * kStsMaxSlices * kStsMaxBins * sizeof(double);
}

dspark_status dspark_sts_fit(int n, int gamma, const float* z, const int32_t* m, const float* grid,
                             int G, int nbins, float* t_out, double* ece_out, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  DSPARK_ABI_RANGE();
  if (n < 0 || gamma < 1 || G < 1 || nbins < 1) return DSPARK_E_INVALID;
  if (G > kStsMaxGrid || nbins > kStsMaxBins) return DSPARK_E_UNSUPPORTED;
  if (!grid) return DSPARK_E_INVALID;
  for (int g = 0; g < G; ++g)
    if (!(grid[g] > 0.f) || !std::isfinite(grid[g])) return DSPARK_E_INVALID;
  if (n == 0) return DSPARK_E_INVALID;      // nothing to calibrate on
  if (!z || !m || !t_out || !ws) return DSPARK_E_INVALID;
  if (!aligned16(ws)) return DSPARK_E_INVALID;
  if (ws_bytes < dspark_sts_workspace_bytes(n)) return DSPARK_E_WORKSPACE;
  StsArgs a{};
  a.n = n; a.gamma = gamma; a.G = G; a.nbins = nbins; a.z = z; a.m = m;
  char* w = reinterpret_cast<char*>(ws);
  a.A = reinterpret_cast<double*>(w + 256);
  a.part = reinterpret_cast<double*>(w + 256 + ws_align((size_t)n * 8));
  // slices of at least 2048 examples (16 per thread), at most 32 per temperature
  a.S = std::max(1, std::min(kStsMaxSlices, (n + 2047) / 2048));
  a.t_out = t_out; a.ece_out = ece_out;
  for (int g = 0; g < G; ++g) a.grid[g] = grid[g];
  return hip_status(launch_sts_fit(a, stream));
}

static dspark_status acceptance_rate_impl(int R, int gamma, int V, int r, float T,
                                          const void* target, dspark_dtype t_dt, const int32_t* x,
                                          const float* lse_d, const void* U, dspark_dtype U_dt,
                                          const void* W1, const void* W2t, dspark_dtype W_dt,
                                          float* c_star, void* ws, size_t ws_bytes,
                                          hipStream_t stream, const void* feat) {
  dspark_status s = shape_check(R, gamma, V);
  if (s != DSPARK_OK) return s;
  if ((s = rank_check(r)) != DSPARK_OK) return s;
  if (!(T >= 0.f) || !std::isfinite(T)) return DSPARK_E_INVALID;
  if (!dtype_ok(t_dt) || !dtype_ok(U_dt) || !dtype_ok(W_dt)) return DSPARK_E_INVALID;
  if (R == 0) return DSPARK_OK;
  if (t_dt != U_dt) return DSPARK_E_UNSUPPORTED;
  if (!target || !x || !c_star || !ws) return DSPARK_E_INVALID;
  if (T > 0.f && (!lse_d || !U)) return DSPARK_E_INVALID;
  if (T > 0.f && r > 0 && (!W1 || !W2t)) return DSPARK_E_INVALID;
  if (r > 0 && T > 0.f && (!aligned16(W1) || !aligned16(W2t))) return DSPARK_E_UNSUPPORTED;
  if (!aligned16(ws)) return DSPARK_E_INVALID;
  if (ws_bytes < ws_layout(R, gamma, V).total) return DSPARK_E_WORKSPACE;
  return hip_status(launch_acceptance_rate(R, gamma, V, r, T, target, x, lse_d, U,
                                           U_dt == DSPARK_BF16, W1, W2t, W_dt == DSPARK_BF16,
                                           c_star, ws, stream, feat));
}

dspark_status dspark_acceptance_rate(int R, int gamma, int V, int r, float T, const void* target,
                                     dspark_dtype t_dt, const int32_t* x, const float* lse_d,
                                     const void* U, dspark_dtype U_dt, const void* W1,
                                     const void* W2t, dspark_dtype W_dt, float* c_star, void* ws,
                                     size_t ws_bytes, hipStream_t stream) {
  DSPARK_ABI_RANGE();
  return acceptance_rate_impl(R, gamma, V, r, T, target, t_dt, x, lse_d, U, U_dt, W1, W2t, W_dt,
                              c_star, ws, ws_bytes, stream, nullptr);
}

dspark_status dspark_acceptance_rate_features(int R, int gamma, int V, int r, float T,
                                              const void* target, dspark_dtype t_dt,
                                              const int32_t* x, const float* lse_d, const void* U,
                                              dspark_dtype U_dt, const void* feat,
                                              const void* W2t, dspark_dtype W_dt, float* c_star,
                                              void* ws, size_t ws_bytes, hipStream_t stream) {
  DSPARK_ABI_RANGE();
  if (r == 0 && R > 0) return DSPARK_E_UNSUPPORTED;
  if (R > 0 && !feat) return DSPARK_E_INVALID;
  // the features take W1's place in the argument checks
  return acceptance_rate_impl(R, gamma, V, r, T, target, t_dt, x, lse_d, U, U_dt, feat, W2t, W_dt,
                              c_star, ws, ws_bytes, stream, feat);
}

dspark_status dspark_verify(int R, int gamma, int V, int r, float T, uint64_t seed, uint64_t round,
                            const int32_t* ell, const int32_t* cu, const void* target,
                            dspark_dtype t_dt, int target_layout, const int32_t* x,
                            const float* logp_d, const float* lse_d, const void* U,
                            dspark_dtype U_dt, const void* W1, const void* W2t, dspark_dtype W_dt,
                            int32_t* m, int32_t* tau, int32_t* emitted, int32_t* next_anchor,
                            float* logp_t, void* ws, size_t ws_bytes, hipStream_t stream) {
  DSPARK_ABI_RANGE();
  return verify_impl(R, gamma, V, r, T, seed, round, ell, cu, target, t_dt, target_layout, x,
                     logp_d, lse_d, U, U_dt, W1, W2t, W_dt, m, tau, emitted, next_anchor, logp_t,
                     ws, ws_bytes, stream, nullptr, nullptr);
}

dspark_status dspark_verify_features(int R, int gamma, int V, int r, float T, uint64_t seed,
                                     uint64_t round, const int32_t* ell, const int32_t* cu,
                                     const void* target, dspark_dtype t_dt, int target_layout,
                                     const int32_t* x, const float* logp_d, const float* lse_d,
                                     const void* U, dspark_dtype U_dt, const void* feat,
                                     const void* W2t, dspark_dtype W_dt, int32_t* m, int32_t* tau,
                                     int32_t* emitted, int32_t* next_anchor, float* logp_t,
                                     void* ws, size_t ws_bytes, hipStream_t stream) {
  DSPARK_ABI_RANGE();
  if (r == 0 && R > 0) return DSPARK_E_UNSUPPORTED;
  if (R > 0 && !feat) return DSPARK_E_INVALID;
  // the features take W1's place in the argument checks
  return verify_impl(R, gamma, V, r, T, seed, round, ell, cu, target, t_dt, target_layout, x,
                     logp_d, lse_d, U, U_dt, feat, W2t, W_dt, m, tau, emitted, next_anchor,
                     logp_t, ws, ws_bytes, stream, nullptr, nullptr, feat);
}

dspark_status dspark_verify_cap_accept_features(int R, int gamma, int V, int r, float T,
                                                uint64_t seed, uint64_t round, const int32_t* ell,
                                                const int32_t* cap, const int32_t* cu,
                                                const void* target, dspark_dtype t_dt,
                                                int target_layout, const int32_t* x,
                                                const float* logp_d, const float* lse_d,
                                                const void* U, dspark_dtype U_dt, const void* feat,
                                                const void* W2t, dspark_dtype W_dt, int32_t* m,
                                                int32_t* tau, int32_t* emitted,
                                                int32_t* next_anchor, int32_t* m_full,
                                                float* logp_t, void* ws, size_t ws_bytes,
                                                hipStream_t stream) {
  DSPARK_ABI_RANGE();
  if (R > 0 && !cap) return DSPARK_E_INVALID;
  if (r == 0 && R > 0) return DSPARK_E_UNSUPPORTED;
  if (R > 0 && !feat) return DSPARK_E_INVALID;
  // the features take W1's place in the argument checks
  return verify_impl(R, gamma, V, r, T, seed, round, ell, cu, target, t_dt, target_layout, x,
                     logp_d, lse_d, U, U_dt, feat, W2t, W_dt, m, tau, emitted, next_anchor,
                     logp_t, ws, ws_bytes, stream, cap, m_full, feat);
}

dspark_status dspark_verify_cap_accept(int R, int gamma, int V, int r, float T, uint64_t seed,
                                       uint64_t round, const int32_t* ell, const int32_t* cap,
                                       const int32_t* cu, const void* target, dspark_dtype t_dt,
                                       int target_layout, const int32_t* x, const float* logp_d,
                                       const float* lse_d, const void* U, dspark_dtype U_dt,
                                       const void* W1, const void* W2t, dspark_dtype W_dt,
                                       int32_t* m, int32_t* tau, int32_t* emitted,
                                       int32_t* next_anchor, int32_t* m_full, float* logp_t,
                                       void* ws, size_t ws_bytes, hipStream_t stream) {
  DSPARK_ABI_RANGE();
  if (R > 0 && !cap) return DSPARK_E_INVALID;
  return verify_impl(R, gamma, V, r, T, seed, round, ell, cu, target, t_dt, target_layout, x,
                     logp_d, lse_d, U, U_dt, W1, W2t, W_dt, m, tau, emitted, next_anchor, logp_t,
                     ws, ws_bytes, stream, cap, m_full);
}

dspark_status dspark_round_markov(const dspark_round_markov_args* a, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  DSPARK_ABI_RANGE();
  if (!a) return DSPARK_E_INVALID;
  if (a->sched_mode < 0 || a->sched_mode > 2) return DSPARK_E_INVALID;
  // every call's checks first (nothing enqueued), then the five calls
  for (int pass = 0; pass < 2; ++pass) {
    const bool dry = pass == 0;
    dspark_status s = draft_impl(a->R, a->gamma, a->V, a->r, a->T, a->seed, a->round, a->U,
                                 a->U_dt, a->W1, a->W2t, a->W_dt, a->x0, a->x, a->logp_d,
                                 a->lse_d, nullptr, ws, ws_bytes, stream, nullptr, nullptr,
                                 nullptr, dry);
    if (s != DSPARK_OK) return s;
    s = confidence_impl(a->R, a->gamma, a->d, a->r, a->V, a->h, a->h_dt, a->W1, a->W_dt, a->w,
                        a->w_dt, a->sts_T, a->x, a->c, false, stream, dry);
    if (s != DSPARK_OK) return s;
    s = schedule_pack_impl(a->R, a->gamma, a->sched_mode, a->c, a->sps, a->N_max, a->K_in,
                           a->K_plan, a->x, a->ell, a->a, a->N, a->theta, a->theta_plan, a->cu,
                           a->flat, a->marker_req, a->marker_pos, stream, dry);
    if (s != DSPARK_OK) return s;
    s = verify_impl(a->R, a->gamma, a->V, a->r, a->T, a->seed, a->round, a->ell, a->cu, a->target,
                    a->t_dt, a->target_layout, a->x, a->logp_d, a->lse_d, a->U, a->U_dt, a->W1,
                    a->W2t, a->W_dt, a->m, a->tau, a->emitted, a->next_anchor, a->logp_t, ws,
                    ws_bytes, stream, nullptr, nullptr, nullptr, dry);
    if (s != DSPARK_OK) return s;
    s = pack_impl(a->R, a->gamma + 1, a->emitted, a->tau, 0, a->cu_out, a->flat_out, nullptr,
                  nullptr, a->N_out, ws, ws_bytes, stream, dry);
    if (s != DSPARK_OK) return s;
  }
  return DSPARK_OK;
}

}  // extern "C"
