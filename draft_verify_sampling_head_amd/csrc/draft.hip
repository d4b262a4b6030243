// draft.hip -- Markov draft head: the gamma-step sequential chain.
//
// DSpark summary page, Method details (causal block distribution, Markov
// head): p_k(v | x_0, x_<k) = softmax(U_k + W1[x_{k-1}] W2)(v), sampled left to
// right.  Each step k is two launches on the caller's stream:
//   1. per-chunk statistics of s = (U_k + bias)/T for every row (stats.hip);
//   2. k_draft_pick, one wave per request: the row normaliser from the chunk
//      log-masses, the chunk-level Gumbel pick, then the in-chunk pick after
//      rebuilding the 128 scores of the chosen chunk (bias by FMA chain).
// The next step's statistics read x_k written by step 1's pick, so stream
// order is the only synchronisation; nothing returns to the host.
#include "launch.hpp"
#include "sampling.hpp"
#include "workspace.hpp"

namespace dspark {

struct DraftPickArgs {
  int R, gamma, k, V, rank, nch;
  float invT;               // 1/T (sampling)
  uint64_t seed, round;
  const void* U;
  const void* W1;
  const void* W2t;
  const int32_t* x0;
  int32_t* x;
  float* logp_d;
  float* lse_d;
  float* margin;
  const float2* L;          // [R][nch] chunk (max, scaled sum) or (max, -) when greedy
  const int* I;             // [R][nch] chunk argmax (greedy)
  uint32_t* status;
};

// One 256-thread block per request.
template <typename UT, typename WT, bool GREEDY>
__global__ __launch_bounds__(256) void k_draft_pick(DraftPickArgs a) {
  __shared__ BlockScratch sh;
  const int i = blockIdx.x;
  const int tid = threadIdx.x;
  const int k = a.k;
  const int64_t xo = (int64_t)i * (a.gamma + 1);
  const int prev = (k == 1) ? a.x0[i] : a.x[xo + k - 1];
  const float2* Lr = a.L + (int64_t)i * a.nch;
  int xk;
  float logp, lse, gap = INFINITY;
  if (GREEDY) {
    float v = -INFINITY;
    int idx = 0x7FFFFFFF;
    const int* Ir = a.I + (int64_t)i * a.nch;
    for (int c = tid; c < a.nch; c += 256) argmax_merge(v, idx, Lr[c].x, Ir[c]);
    block_argmax(v, idx, sh);
    xk = idx;
    lse = v;
    logp = 0.f;
    if (xk < 0 || xk >= a.V) { set_flag(a.status, kFlagNonFinite); xk = 0; }
  } else {
    float m = -INFINITY;
    for (int c = tid; c < a.nch; c += 256) m = fmaxf(m, Lr[c].x);
    m = block_max(m, sh);
    const bool want_gap = a.margin != nullptr;
    float srel;
    const PickResult pc = block_pick_chunk(Lr, a.nch, m, a.invT, a.seed, a.round, kTagDraftChunk,
                                           (uint32_t)i, (uint32_t)k, want_gap, &srel, sh);
    const float lse_rel = logf(srel);
    lse = m * a.invT + lse_rel;
    int c = pc.idx;
    if (c < 0) { set_flag(a.status, kFlagNonFinite); c = 0; }
    const int base = c * kChunk;
    // rebuild the 128 scores of the chosen chunk: thread t covers entry
    // base + t/2 and one half of the rank
    const int v = base + (tid >> 1), h = tid & 1;
    const bool in = v < a.V;
    float b = 0.f;
    if (a.rank > 0 && in) {
      const int pv = (prev >= 0 && prev < a.V) ? prev : 0;
      const WT* erow = reinterpret_cast<const WT*>(a.W1) + (int64_t)pv * a.rank;
      b = markov_bias_half(erow, reinterpret_cast<const WT*>(a.W2t), a.rank, v, h);
    }
    b += __shfl_xor(b, 1);
    const UT* urow = reinterpret_cast<const UT*>(a.U) + ((int64_t)i * a.gamma + (k - 1)) * a.V;
    const float s = in ? (Elem<UT>::get(urow, v) + b - m) * a.invT : -INFINITY;
    const PickResult pe = block_pick_in_chunk(s, base, a.seed, a.round, kTagDraftElem,
                                              (uint32_t)i, (uint32_t)k, want_gap, sh);
    xk = pe.idx;
    if (xk < 0) { set_flag(a.status, kFlagNonFinite); xk = base; }
    // the winner's score: held by thread 2*(xk - base)
    __syncthreads();
    if (tid == 2 * (xk - base)) sh.g[0] = s;
    __syncthreads();
    logp = sh.g[0] - lse_rel;
    gap = fminf(pc.gap, pe.gap);
  }
  if (tid == 0) {
    if (k == 1) a.x[xo] = a.x0[i];
    a.x[xo + k] = xk;
    const int64_t o = (int64_t)i * a.gamma + (k - 1);
    a.logp_d[o] = logp;
    a.lse_d[o] = lse;
    if (a.margin) a.margin[o] = gap;
  }
}

hipError_t launch_draft(int R, int gamma, int V, int rank, float T, uint64_t seed, uint64_t round,
                        const void* U, bool u_bf16, const void* W1, const void* W2t, bool w_bf16,
                        const int32_t* x0, int32_t* x, float* logp_d, float* lse_d, float* margin,
                        void* ws, hipStream_t st, hipEvent_t* ev_begin, hipEvent_t* ev_end) {
  const WsLayout L = ws_layout(R, gamma, V);
  char* w = reinterpret_cast<char*>(ws);
  uint32_t* status = reinterpret_cast<uint32_t*>(w + L.header);
  float2* Lc = reinterpret_cast<float2*>(w + L.draft_l);
  int* Ic = reinterpret_cast<int*>(w + L.draft_i);
  const int nch = (V + kChunk - 1) / kChunk;
  const bool greedy = (T == 0.f);
  const float scale2 = greedy ? 1.f : kLog2e / T;
  const size_t usz = u_bf16 ? 2 : 4;
  const bool u_vec = ((reinterpret_cast<uintptr_t>(U) & 15) == 0) && (((size_t)V * usz) % 16 == 0);
  for (int k = 1; k <= gamma; ++k) {
    hipError_t e;
    if (ev_begin && (e = hipEventRecord(ev_begin[k - 1], st)) != hipSuccess) return e;
    if (rank == 0) {
      RowStatsArgs a{};
      a.base = U; a.kind = kRowsDraft; a.R = R; a.gamma = gamma; a.k = k; a.V = V; a.nch = nch;
      a.nrows_cap = R; a.scale2 = scale2; a.vec_ok = u_vec; a.L = Lc; a.I = Ic;
      a.status = status;
      e = launch_row_stats(a, u_bf16, greedy, st);
    } else {
      MarkovArgs a{};
      a.R = R; a.gamma = gamma; a.k = k; a.V = V; a.rank = rank; a.nch = nch; a.nrows_cap = R;
      a.U = U; a.W1v = W1; a.W2tv = W2t; a.x0 = x0; a.x = x; a.scale2 = scale2; a.u_vec_ok = u_vec;
      a.L = Lc; a.I = Ic; a.status = status;
      e = launch_markov_stats(a, u_bf16, w_bf16, greedy ? kModeGreedy : kModeSample, st);
    }
    if (e != hipSuccess) return e;
    if (ev_end && (e = hipEventRecord(ev_end[k - 1], st)) != hipSuccess) return e;
    DraftPickArgs p{};
    p.R = R; p.gamma = gamma; p.k = k; p.V = V; p.rank = rank; p.nch = nch;
    p.invT = greedy ? 1.f : 1.f / T; p.seed = seed; p.round = round;
    p.U = U; p.W1 = W1; p.W2t = W2t; p.x0 = x0; p.x = x; p.logp_d = logp_d; p.lse_d = lse_d;
    p.margin = margin; p.L = Lc; p.I = Ic; p.status = status;
#define DSPARK_PICK(UT_, WT_, G_) \
    hipLaunchKernelGGL((k_draft_pick<UT_, WT_, G_>), dim3(R), dim3(256), 0, st, p)
    if (u_bf16 && w_bf16) { if (greedy) DSPARK_PICK(uint16_t, uint16_t, true); else DSPARK_PICK(uint16_t, uint16_t, false); }
    else if (u_bf16)      { if (greedy) DSPARK_PICK(uint16_t, float, true);    else DSPARK_PICK(uint16_t, float, false); }
    else if (w_bf16)      { if (greedy) DSPARK_PICK(float, uint16_t, true);    else DSPARK_PICK(float, uint16_t, false); }
    else                  { if (greedy) DSPARK_PICK(float, float, true);       else DSPARK_PICK(float, float, false); }
#undef DSPARK_PICK
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace dspark
