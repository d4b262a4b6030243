// launch.hpp -- internal host/device interface between the C ABI and kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"
#include <rocprofiler-sdk-roctx/roctx.h>

namespace dspark {

// A marker range over one C-ABI call, named after the entry point: a
// profiler's marker trace (rocprofv3 --marker-trace) shows each call's host
// span next to the kernels it enqueued.  Without a tool attached the two
// calls return at once.
struct AbiRange {
  explicit AbiRange(const char* name) { roctxRangePush(name); }
  ~AbiRange() { roctxRangePop(); }
  AbiRange(const AbiRange&) = delete;
  AbiRange& operator=(const AbiRange&) = delete;
};
#define DSPARK_ABI_RANGE() ::dspark::AbiRange dspark_abi_range_(__func__)

// Test and measurement switches of the library (dspark_set_switch): read
// once from the environment (DSPARK_DRAFT_KERNEL=steps, DSPARK_RNN_CELL_VALU,
// DSPARK_BARRIER_SPINS) the first time they are needed, replaced only by an
// explicit dspark_set_switch call.
struct Switches {
  int force_per_step;      // 1: the per-step draft schedule for every shape
  int rnn_cell_valu;       // 1: the RNN head's per-step schedule with the vector-ALU cell
  uint32_t barrier_spins;  // polls before a cross-workgroup wait gives up
  int draft_kernel;        // persistent draft: 0 one grid barrier per step, 1 pipelined
  int persist_launch;      // launches that need a co-resident grid: 0 plain, 1 cooperative
};
// Polls before a cross-workgroup wait gives up when barrier_spins is 0.
constexpr uint32_t kBarrierSpins = 1u << 24;
Switches switches();

// Launch of a kernel whose workgroups wait for one another (grid
// barriers): the grid (at most one workgroup per compute unit)
// must be co-resident.  By the switch: a plain launch (resident at once when
// nothing else occupies the device; while other work holds compute units the
// waits last until it drains, and they are bounded: a wait that gives up
// reports DSPARK_FLAG_BARRIER), or a cooperative launch (the runtime
// guarantees residency or fails the launch).
hipError_t launch_coresident(const void* fn, dim3 grid, dim3 block, void** args, size_t lds,
                             hipStream_t st);

enum { kRowsDraft = 0, kRowsVerifyPacked = 1, kRowsVerifyDense = 2, kRowsAll = 3 };
enum { kModeSample = 0, kModeGreedy = 1, kModeResid = 2 };

// Streaming per-chunk statistics of rows with no bias.
struct RowStatsArgs {
  const void* base;        // U (draft) or target (verify)
  int kind;                // kRows*
  int R, gamma, k, V, nch;
  const int32_t* cu;       // verify: offsets; N = cu[R]
  int nrows_cap;           // draft: R; verify: R*(gamma+1)
  float scale2;            // log2(e) / T (sampling) -- unused for greedy
  bool vec_ok;             // rows are 16-byte aligned
  float2* L;               // [row][nch] (raw max M_c, sum exp((x - M_c)/T)); greedy: (M_c, -)
  int* I;                  // [row][nch] argmax (greedy)
  uint32_t* status;
  uint32_t* zero_me;       // nullable: cleared by the first thread (work counter)
  int segs, cps;           // filled by the launcher
};

// Per-chunk statistics of rows carrying the Markov bias (draft or residual).
struct MarkovArgs {
  int R, gamma, k, V, rank, nch, nrows_cap;
  const void* U;
  const void* W1v;
  const void* W2tv;
  const uint16_t* W1;      // bf16 views (MFMA path)
  const uint16_t* W2t;
  const int32_t* x0;       // draft anchors
  const int32_t* x;        // [R][gamma+1]
  bool feat_rows;          // W1 holds per-position features [R][gamma][rank] (RNN head)
  float scale2;
  bool u_vec_ok;
  float2* L;               // [row][nch] as RowStatsArgs; residual: (0, sum max(0, p_t - p_d))
  int* I;
  // residual rows
  const int32_t* rej_count;
  const int4* rej;         // (request, position k, target row, verify row)
  const void* target;
  const float2* lse_t;     // [verify row] (raw max, log-normaliser relative to it)
  const float* lse_d;
  bool overlap;            // residual rows: sum min(p_t, p_d) instead of max(0, p_t - p_d)
  uint32_t* status;
  // filled by the launcher
  int cg, nrg, ncg;        // chunks per workgroup, 256-row groups, chunk groups
};

struct ConfArgs {
  int R, gamma, d, rank, V;
  const void* h;
  const void* W1;
  const void* w;
  const float* sts;
  const int32_t* x;
  float* c;                // sigmoid(z / t), or z itself when logits is set
  bool vec_h, vec_e, logits;
  uint32_t* status;
};

constexpr int kMaxTiers = 32;

struct PackArgs {
  int R, width, len_offset;
  const int32_t* rows;
  const int32_t* len;
  int32_t* cu;
  int32_t* flat;
  int32_t* marker_req;
  int32_t* marker_pos;
  int32_t* N_out;
  uint32_t* status;
  int64_t slots;            // length of flat / markers (>= R * width)
  int ntiers;               // 0: no tier padding
  int pad_token;
  int32_t* N_pad;           // nullable
  int tiers[kMaxTiers];     // ascending
};

struct SchedArgs {
  int R, gamma, N_max, enabled;
  int mode;                 // 0: Algorithm 1 (early stop); 1: asynchronous (top-K + plan)
  const float* c;
  const double* sps;
  int32_t* ell;
  float* a;
  int32_t* N_out;
  double* theta;
  const int32_t* K_in;      // mode 1: capacity planned two rounds earlier
  int32_t* K_plan;          // mode 1: capacity planned from this round
  double* theta_plan;       // mode 1 (nullable)
  bool pack;                // also pack the verify batch: pk.rows with length ell + 1
  PackArgs pk;              // (pk.len, pk.len_offset unused)
};

constexpr int kStsMaxBins = 64;
constexpr int kStsMaxGrid = 256;
constexpr int kStsMaxSlices = 32;

struct StsArgs {
  int n, gamma, G, nbins;
  int S;                     // example slices per temperature (1..kStsMaxSlices)
  const float* z;            // [n][gamma] raw confidence logits
  const int32_t* m;          // [n] accepted drafts
  double* A;                 // [n] workspace: cumulative product of earlier positions
  double* part;              // [G][nbins][S] workspace: per-slice signed bin sums
  float* t_out;              // [gamma]
  double* ece_out;           // [gamma] nullable
  float grid[kStsMaxGrid];   // candidate temperatures, in search order
};

// RNN draft head: the recurrent cell that produces the bias features e_k.
struct RnnArgs {
  int R, gamma, V, rank, d;
  const void* W1;          // [V][rank] token embeddings (W dtype)
  const void* Wr;          // [3 rank][2 rank + d] gate / candidate / output rows (W dtype)
  const void* h;           // [R][gamma][d] backbone hidden states
  bool w_bf16, h_bf16;
  const int32_t* x0;       // [R] anchors
  const int32_t* x;        // [R][gamma+1] drafted tokens (x[i][k-1] read at step k)
  float* P;                // [R*gamma][3 rank] workspace: the h part of the projection
  float* state;            // [R][gamma][rank] s_1 .. s_gamma
  void* feat;              // [R][gamma][rank] e_1 .. e_gamma (W dtype)
  uint32_t* status;
};

hipError_t launch_rnn_hproj(const RnnArgs& a, hipStream_t st);
hipError_t launch_rnn_cell(const RnnArgs& a, int k, hipStream_t st);

hipError_t launch_sts_fit(const StsArgs& a, hipStream_t st);
hipError_t launch_row_stats(const RowStatsArgs& a, bool bf16, bool greedy, hipStream_t st);
hipError_t launch_markov_stats(const MarkovArgs& a, bool u_bf16, bool w_bf16, int mode,
                               hipStream_t st);

hipError_t launch_confidence(const ConfArgs& a, bool h_bf16, bool w1_bf16, bool w_bf16,
                             hipStream_t st);
hipError_t launch_pack(const PackArgs& a, hipStream_t st);
hipError_t launch_schedule(const SchedArgs& a, hipStream_t st);
struct DraftWs;
struct DraftPickArgs;
bool launch_draft_pipe(const DraftPickArgs& p, bool greedy, float scale2, int grid,
                       uint32_t spin_limit, const DraftWs& ws, hipStream_t st, hipEvent_t* ev_begin,
                       hipEvent_t* ev_end, int* n_timed, hipError_t* err);
hipError_t launch_draft(int R, int gamma, int V, int rank, float T, uint64_t seed, uint64_t round,
                        const void* U, bool u_bf16, const void* W1, const void* W2t, bool w_bf16,
                        const int32_t* x0, int32_t* x, float* logp_d, float* lse_d, float* margin,
                        const DraftWs& ws, hipStream_t st, hipEvent_t* ev_begin = nullptr,
                        hipEvent_t* ev_end = nullptr, int* n_timed = nullptr,
                        const RnnArgs* rnn = nullptr);
bool launch_resid_slices(int R, int gamma, int V, int rank, float T, const void* U,
                         const void* W1, const void* W2t, const void* target, const int32_t* x,
                         const int32_t* rej_count, const int4* rej, const float2* lse_t,
                         const float* lse_d, float2* L, uint32_t* status, hipStream_t st,
                         hipError_t* err, bool overlap = false, bool feat_rows = false);
hipError_t launch_acceptance_rate(int R, int gamma, int V, int rank, float T, const void* target,
                                  const int32_t* x, const float* lse_d, const void* U, bool u_bf16,
                                  const void* W1, const void* W2t, bool w_bf16, float* c_star,
                                  void* ws, hipStream_t st, const void* feat = nullptr);
hipError_t launch_verify(int R, int gamma, int V, int rank, float T, uint64_t seed, uint64_t round,
                         const int32_t* ell, const int32_t* cu, const void* target, int layout,
                         const int32_t* x, const float* logp_d, const float* lse_d,
                         const void* U, bool u_bf16, const void* W1, const void* W2t, bool w_bf16,
                         int32_t* m, int32_t* tau, int32_t* emitted, int32_t* next_anchor,
                         float* logp_t, void* ws, hipStream_t st, const int32_t* cap = nullptr,
                         int32_t* m_full = nullptr, const void* feat = nullptr);

}  // namespace dspark
