// verify.hip -- lossless rejection-sampling verification.
//
// DSpark summary page, Background (x_k accepted with probability
// min(1, p_t(x_k)/p_d(x_k)), left to right, the first rejection drops the
// rest); MTP survey page, section 2.2 (resample the rejected position from
// norm(max(0, p_t - p_d)); after a fully accepted prefix draw the bonus token
// from the next target distribution; tau = m + 1; greedy reduction).
// Launches, all sized by capacity so N, m and the rejections stay on device:
//   1. k_row_stats over the N verify rows: chunk log-masses of t/T (or chunk
//      maxima at T = 0); also clears the residual work counter.
//   2. k_row_norm, one wave per verify row: the row normaliser (raw maximum,
//      log-sum above it) or, at T = 0, the row argmax.
//   3. k_verify_scan, one workgroup per request: lane k-1 of the first wave
//      evaluates position k (log p_t(x_k), its uniform, the accept test) for
//      every k at once and a ballot finds the first rejection; then either the
//      bonus draw (chunked Gumbel-max on the row after the accepted prefix)
//      or a residual work item.  Cap-accept (DeepSpec analysis page, section
//      5.4, DSpark in SGLang: the verify modes): with a commit window C below
//      the accepted count m, the first C + 1 tokens of the sequence are
//      committed, the last being the accepted draft x_{C+1}; no draw is made.
//   4. residual chunk masses for the listed (request, position) rows: the
//      draft scores are rebuilt with the Markov bias (MFMA) and combined with
//      the target row into max(0, p_t - p_d) per chunk.
//   5. k_resid_pick, one workgroup per work item: chunk pick and in-chunk pick
//      on log max(0, p_t - p_d); zero mass falls back to p_t.
#include "launch.hpp"
#include "sampling.hpp"
#include "workspace.hpp"

namespace dspark {

struct VerifyArgs {
  int R, gamma, V, rank, nch, layout;
  bool all_rows;        // every dense row R*(gamma+1), not cu[R] (acceptance-rate pass)
  float invT;
  bool greedy;
  uint64_t seed, round;
  const int32_t* ell;
  const int32_t* cu;
  const void* target;
  const int32_t* x;
  const float* logp_d;
  const float* lse_d;
  const void* U;
  const void* W1;
  const void* W2t;
  const void* feat;     // nullable: per-position bias features [R][gamma][rank] (RNN head)
  int32_t* m;
  int32_t* tau;
  int32_t* emitted;
  int32_t* next_anchor;
  float* logp_t;
  const int32_t* cap;   // nullable: commit window per request (cap-accept)
  int32_t* m_full;      // nullable: accepted count over the whole window
  const float2* vl;     // [q][nch] chunk (max, scaled sum) of verify rows
  const int* vi;        // [q][nch] chunk argmax (greedy)
  float2* lse_t;        // [q] (raw row max, log-normaliser relative to it)
  int32_t* rej_count;
  int4* rej;            // (request, position, target row, verify row q)
  const float2* rl;     // [slot][nch] residual chunk masses (0, sum)
  uint32_t* status;
};

__device__ __forceinline__ int64_t target_row(const VerifyArgs& a, int i, int j) {
  return a.layout == 0 ? (int64_t)a.cu[i] + j : (int64_t)i * (a.gamma + 1) + j;
}

// Row normaliser of every verify row q < N: (raw max, log sum_c S_c
// exp((M_c - max)/T)); at T = 0 (row max, bits of the first argmax).
__global__ __launch_bounds__(256) void k_row_norm(VerifyArgs a) {
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nwaves = gridDim.x * 4;
  const int N = a.all_rows ? a.R * (a.gamma + 1) : min(a.cu[a.R], a.R * (a.gamma + 1));
  for (int q = wave; q < N; q += nwaves) {
    if (a.greedy) {
      float v;
      int am;
      argmax_chunks(a.vl + (int64_t)q * a.nch, a.vi + (int64_t)q * a.nch, a.nch, v, am);
      if ((threadIdx.x & 63) == 0) a.lse_t[q] = make_float2(v, __int_as_float(am));
    } else {
      const RowNorm rn = row_norm(a.vl + (int64_t)q * a.nch, a.nch, a.invT);
      if ((threadIdx.x & 63) == 0) a.lse_t[q] = make_float2(rn.m, rn.lse_rel);
    }
  }
}

template <typename TT>
__global__ __launch_bounds__(256) void k_verify_scan(VerifyArgs a) {
  __shared__ BlockScratch sh;
  __shared__ int s_m, s_rej;
  const int i = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  int L = a.ell[i];
  if (L < 0 || L > a.gamma) { if (tid == 0) set_flag(a.status, kFlagBadLen); L = L < 0 ? 0 : a.gamma; }
  const int q0 = a.cu[i];
  const int32_t* xi = a.x + (int64_t)i * (a.gamma + 1);
  const TT* tgt = reinterpret_cast<const TT*>(a.target);
  if (tid < 64) {
    // lane k-1 evaluates position k
    const int k = lane + 1;
    bool rej = false;
    if (k <= L) {
      const float2 nt = a.lse_t[q0 + k - 1];
      int xk = xi[k];
      if (xk < 0 || xk >= a.V) { set_flag(a.status, kFlagBadToken); xk = 0; }
      if (a.greedy) {
        rej = xk != __float_as_int(nt.y);
        if (a.logp_t) a.logp_t[(int64_t)i * a.gamma + (k - 1)] = 0.f;
      } else {
        const float lp = (Elem<TT>::get(tgt + target_row(a, i, k - 1) * a.V, xk) - nt.x) * a.invT
                         - nt.y;
        if (a.logp_t) a.logp_t[(int64_t)i * a.gamma + (k - 1)] = lp;
        const uint4 blk = stream_block(a.seed, a.round, kTagAccept, (uint32_t)i, (uint32_t)k, 0u);
        const float lu = log_uniform(blk.x);
        const float rhs = lp - a.logp_d[(int64_t)i * a.gamma + (k - 1)];
        rej = !(lu < rhs);
      }
    } else if (k <= a.gamma && a.logp_t) {
      a.logp_t[(int64_t)i * a.gamma + (k - 1)] = 0.f;
    }
    const uint64_t bal = __ballot(rej);
    if (lane == 0) {
      s_rej = bal != 0;
      s_m = bal ? (__builtin_ctzll(bal)) : L;   // first rejected position k = m + 1
    }
  }
  __syncthreads();
  int m = s_m;
  bool rejected = s_rej != 0;
  int y = -1;
  // cap-accept: when more drafts were accepted than the commit window holds,
  // the window closes on the accepted draft x_{C+1} (no correction, no bonus)
  bool closed = false;
  if (a.cap) {
    int C = a.cap[i];
    if (C < 0) { if (tid == 0) set_flag(a.status, kFlagBadLen); C = 0; }
    if (C > L) C = L;
    if (tid == 0 && a.m_full) a.m_full[i] = m;
    if (m > C) {
      closed = true;
      m = C;
      rejected = false;
    }
  }
  if (closed) {
    y = xi[m + 1];                      // the accepted draft that closes the window
    if (y < 0 || y >= a.V) y = 0;       // (flagged by the scan above)
  } else if (a.greedy) {
    // correction: the argmax of the first mismatching row; bonus: of row L
    y = __float_as_int(a.lse_t[q0 + m].y);
    if (y < 0 || y >= a.V) { if (tid == 0) set_flag(a.status, kFlagNonFinite); y = 0; }
  } else if (!rejected) {
    // bonus token from the target row after the accepted prefix
    const int q = q0 + L;
    const float2 nt = a.lse_t[q];
    float srel;
    const PickResult pc = block_pick_chunk<256>(a.vl + (int64_t)q * a.nch, a.nch, nt.x, a.invT,
                                                a.seed, a.round, kTagBonusChunk, (uint32_t)i,
                                                (uint32_t)(L + 1), false, &srel, sh);
    const int c = pc.idx < 0 ? 0 : pc.idx;
    if (pc.idx < 0 && tid == 0) set_flag(a.status, kFlagNonFinite);
    const TT* trow = tgt + target_row(a, i, L) * a.V;
    const int v = c * kChunk + (tid >> 1);
    const float s = (v < a.V) ? (Elem<TT>::get(trow, v) - nt.x) * a.invT : -INFINITY;
    const PickResult pe = block_pick_in_chunk<256>(s, c * kChunk, a.seed, a.round, kTagBonusElem,
                                                   (uint32_t)i, (uint32_t)(L + 1), false, sh);
    y = pe.idx < 0 ? c * kChunk : pe.idx;
  } else if (tid == 0) {
    const int slot = atomicAdd(a.rej_count, 1);
    a.rej[slot] = make_int4(i, m + 1, (int)target_row(a, i, m), q0 + m);
  }
  // outputs (a rejected sampled position gets its token from k_resid_pick)
  int32_t* em = a.emitted + (int64_t)i * (a.gamma + 1);
  const bool have_y = closed || a.greedy || !rejected;
  for (int q = tid; q <= a.gamma; q += 256)
    em[q] = (q < m) ? xi[q + 1] : ((q == m && have_y) ? y : -1);
  if (tid == 0) {
    a.m[i] = m;
    a.tau[i] = m + 1;
    if (have_y) a.next_anchor[i] = y;
  }
}

template <typename UT, typename WT>
__global__ __launch_bounds__(256) void k_resid_pick(VerifyArgs a) {
  __shared__ BlockScratch sh;
  const int slot = blockIdx.x;
  const int tid = threadIdx.x;
  if (slot >= *a.rej_count) return;
  const int4 e = a.rej[slot];
  const int i = e.x, k = e.y, trow_i = e.z, q = e.w;
  const UT* trow = reinterpret_cast<const UT*>(a.target) + (int64_t)trow_i * a.V;
  const float2* Lq = a.rl + (int64_t)slot * a.nch;
  const float2 nt = a.lse_t[q];
  // chunk pick on the residual masses (keys log S_c + G_c); srel = total mass
  float mass;
  const PickResult pr = block_pick_chunk<256>(Lq, a.nch, 0.f, 1.f, a.seed, a.round, kTagResidChunk,
                                              (uint32_t)i, (uint32_t)k, false, &mass, sh);
  const int v_off = tid >> 1, h = tid & 1;
  int y;
  if (mass > 0.f) {
    const int c = pr.idx < 0 ? 0 : pr.idx;
    const int v = c * kChunk + v_off;
    const UT* urow = reinterpret_cast<const UT*>(a.U) + ((int64_t)i * a.gamma + (k - 1)) * a.V;
    int prev = a.x[(int64_t)i * (a.gamma + 1) + (k - 1)];
    if (prev < 0 || prev >= a.V) prev = 0;
    const WT* erow = a.feat ? reinterpret_cast<const WT*>(a.feat) + ((int64_t)i * a.gamma + (k - 1)) * a.rank
                            : reinterpret_cast<const WT*>(a.W1) + (int64_t)prev * a.rank;
    const float lse_d = a.lse_d[(int64_t)i * a.gamma + (k - 1)];
    float b = 0.f;
    if (a.rank > 0 && v < a.V) b = markov_bias_half(erow, reinterpret_cast<const WT*>(a.W2t), a.rank, v, h);
    b += __shfl_xor(b, 1);
    float s = -INFINITY;
    if (v < a.V) {
      const float sd = (Elem<UT>::get(urow, v) + b) * a.invT;
      const float pt = expf((Elem<UT>::get(trow, v) - nt.x) * a.invT - nt.y);
      const float pd = expf(sd - lse_d);
      const float d = pt - pd;
      s = d > 0.f ? logf(d) : -INFINITY;
    }
    const PickResult pe = block_pick_in_chunk<256>(s, c * kChunk, a.seed, a.round, kTagResidElem,
                                                   (uint32_t)i, (uint32_t)k, false, sh);
    y = pe.idx;
    if (y < 0) {
      // the chunk's mass vanished on re-evaluation (rounding): keep the chunk's first entry
      if (tid == 0) set_flag(a.status, kFlagNonFinite);
      y = c * kChunk;
    }
  } else {
    // zero residual mass: sample p_t of the same row
    float srel;
    const PickResult pc = block_pick_chunk<256>(a.vl + (int64_t)q * a.nch, a.nch, nt.x, a.invT,
                                                a.seed, a.round, kTagResidChunk, (uint32_t)i,
                                                (uint32_t)k, false, &srel, sh);
    const int c = pc.idx < 0 ? 0 : pc.idx;
    const int v = c * kChunk + v_off;
    const float s = (v < a.V) ? (Elem<UT>::get(trow, v) - nt.x) * a.invT : -INFINITY;
    const PickResult pe = block_pick_in_chunk<256>(s, c * kChunk, a.seed, a.round, kTagResidElem,
                                                   (uint32_t)i, (uint32_t)k, false, sh);
    y = pe.idx < 0 ? c * kChunk : pe.idx;
  }
  if (tid == 0) {
    a.emitted[(int64_t)i * (a.gamma + 1) + (k - 1)] = y;
    a.next_anchor[i] = y;
  }
}

// ------------------------------------------------- acceptance rate c*
// c*_k = sum_v min(p_d^k(v), p_t^k(v)) for every request and block position
// (DSpark summary page, Method details: the confidence head's supervision
// target, one minus the total variation between draft and target).  One pass
// over every dense target row gives the row normalisers; then one launch of
// the residual kernels in overlap mode covers a work list of all R * gamma
// (request, position) rows (p_d rebuilt from U and the Markov bias exactly as
// for a rejection; W2 is streamed once), and one wave per row adds the chunk
// masses.  The list and the masses reuse the target-row statistics buffers,
// which are free once the normalisers exist.  At T == 0 the distributions
// are point masses: c* = [x_k == argmax of target row k-1].
// items q0 .. q0+n-1, q = i * gamma + (k - 1): request i, position k, target row
// i*(gamma+1) + k-1
__global__ __launch_bounds__(256) void k_cstar_list(int gamma, int q0, int n, int4* list,
                                                     int32_t* count) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j < n) {
    const int q = q0 + j;
    const int i = q / gamma, k = q % gamma + 1;
    const int row = i * (gamma + 1) + (k - 1);
    list[j] = make_int4(i, k, row, row);
  }
  if (j == 0) *count = n;
}

__global__ __launch_bounds__(256) void k_cstar_sum(int items, int nch, const float2* L,
                                                    float* c_star) {
  const int q = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (q >= items) return;
  const int lane = threadIdx.x & 63;
  float s = 0.f;
  for (int c = lane; c < nch; c += 64) s += L[(int64_t)q * nch + c].y;
  s = wave_sum(s);
  if (lane == 0) c_star[q] = s;
}

__global__ __launch_bounds__(256) void k_cstar_greedy(int R, int gamma, int V, const int32_t* x,
                                                       const float2* lse_t, float* c_star,
                                                       uint32_t* status) {
  const int item = blockIdx.x * 256 + threadIdx.x;
  if (item >= R * gamma) return;
  const int i = item / gamma, k = item % gamma + 1;
  const int am = __float_as_int(lse_t[i * (gamma + 1) + (k - 1)].y);
  const int xk = x[(int64_t)i * (gamma + 1) + k];
  if (xk < 0 || xk >= V) set_flag(status, kFlagBadToken);
  c_star[item] = (xk == am) ? 1.f : 0.f;
}

hipError_t launch_acceptance_rate(int R, int gamma, int V, int rank, float T, const void* target,
                                  const int32_t* x, const float* lse_d, const void* U, bool u_bf16,
                                  const void* W1, const void* W2t, bool w_bf16, float* c_star,
                                  void* ws, hipStream_t st, const void* feat) {
  const WsLayout L = ws_layout(R, gamma, V);
  char* w = reinterpret_cast<char*>(ws);
  uint32_t* hdr = reinterpret_cast<uint32_t*>(w + L.header);
  const int nch = (V + kChunk - 1) / kChunk;
  const bool greedy = (T == 0.f);
  const size_t usz = u_bf16 ? 2 : 4;
  const bool t_vec = ((reinterpret_cast<uintptr_t>(target) & 15) == 0) && (((size_t)V * usz) % 16 == 0);
  const bool u_vec = ((reinterpret_cast<uintptr_t>(U) & 15) == 0) && (((size_t)V * usz) % 16 == 0);
  const int rows = R * (gamma + 1);

  RowStatsArgs rs{};
  rs.base = target; rs.kind = kRowsAll;
  rs.R = R; rs.gamma = gamma; rs.k = 0; rs.V = V; rs.nch = nch; rs.cu = nullptr;
  rs.nrows_cap = rows;
  rs.scale2 = greedy ? 1.f : kLog2e / T;
  rs.vec_ok = t_vec;
  rs.L = reinterpret_cast<float2*>(w + L.ver_l);
  rs.I = reinterpret_cast<int*>(w + L.ver_i);
  rs.status = hdr;
  rs.zero_me = nullptr;
  hipError_t e = launch_row_stats(rs, u_bf16, greedy, st);
  if (e != hipSuccess) return e;

  VerifyArgs a{};
  a.R = R; a.gamma = gamma; a.V = V; a.rank = rank; a.nch = nch; a.layout = 1; a.all_rows = true;
  a.invT = greedy ? 1.f : 1.f / T; a.greedy = greedy;
  a.vl = rs.L; a.vi = rs.I;
  a.lse_t = reinterpret_cast<float2*>(w + L.lse_t);
  a.status = hdr;
  hipLaunchKernelGGL(k_row_norm, dim3(min(4096, (rows + 3) / 4)), dim3(256), 0, st, a);
  if (greedy) {
    hipLaunchKernelGGL(k_cstar_greedy, dim3((R * gamma + 255) / 256), dim3(256), 0, st, R, gamma,
                       V, x, a.lse_t, c_star, hdr);
    return hipGetLastError();
  }
  // the list takes the argmax buffer (unused at T > 0) and the masses the
  // chunk statistics (read by k_row_norm only): all R*gamma items at once when
  // the list fits (at least 4 chunks), else in batches of what fits
  const int items = R * gamma;
  int32_t* count = reinterpret_cast<int32_t*>(hdr + 1);
  int4* list = reinterpret_cast<int4*>(w + L.ver_i);
  float2* rl = reinterpret_cast<float2*>(w + L.ver_l);
  const int cap = (int)std::min<size_t>((size_t)items, (L.lse_t - L.ver_i) / sizeof(int4));
  // rows of the bias features: W1[x_{k-1}] (Markov head) or the draft's own
  // per-position features (RNN head)
  const void* E = feat ? feat : W1;
  for (int q0 = 0; q0 < items; q0 += cap) {
    const int n = std::min(cap, items - q0);
    hipLaunchKernelGGL(k_cstar_list, dim3((n + 255) / 256), dim3(256), 0, st, gamma, q0, n, list,
                       count);
    if (u_bf16 && w_bf16 && rank > 0 && u_vec && t_vec &&
        launch_resid_slices(n, gamma, V, rank, T, U, E, W2t, target, x, count, list, a.lse_t,
                            lse_d, rl, hdr, st, &e, true, feat != nullptr)) {
      if (e != hipSuccess) return e;
    } else {
      MarkovArgs ma{};
      ma.R = R; ma.gamma = gamma; ma.k = 0; ma.V = V; ma.rank = rank; ma.nch = nch;
      ma.nrows_cap = n;
      ma.U = U; ma.W1v = E; ma.W2tv = W2t; ma.x0 = nullptr; ma.x = x; ma.feat_rows = feat != nullptr;
      ma.scale2 = kLog2e / T;
      ma.u_vec_ok = u_vec && t_vec;
      ma.L = rl; ma.I = nullptr;
      ma.rej_count = count; ma.rej = list; ma.target = target; ma.lse_t = a.lse_t;
      ma.lse_d = lse_d; ma.status = hdr; ma.overlap = true;
      e = launch_markov_stats(ma, u_bf16, w_bf16 && rank > 0, kModeResid, st);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_cstar_sum, dim3((n + 3) / 4), dim3(256), 0, st, n, nch, rl,
                       c_star + q0);
  }
  return hipGetLastError();
}

hipError_t launch_verify(int R, int gamma, int V, int rank, float T, uint64_t seed, uint64_t round,
                         const int32_t* ell, const int32_t* cu, const void* target, int layout,
                         const int32_t* x, const float* logp_d, const float* lse_d,
                         const void* U, bool u_bf16, const void* W1, const void* W2t, bool w_bf16,
                         int32_t* m, int32_t* tau, int32_t* emitted, int32_t* next_anchor,
                         float* logp_t, void* ws, hipStream_t st, const int32_t* cap,
                         int32_t* m_full, const void* feat) {
  const WsLayout L = ws_layout(R, gamma, V);
  char* w = reinterpret_cast<char*>(ws);
  uint32_t* hdr = reinterpret_cast<uint32_t*>(w + L.header);
  const int nch = (V + kChunk - 1) / kChunk;
  const bool greedy = (T == 0.f);
  const size_t usz = u_bf16 ? 2 : 4;
  const bool t_vec = ((reinterpret_cast<uintptr_t>(target) & 15) == 0) && (((size_t)V * usz) % 16 == 0);
  const bool u_vec = ((reinterpret_cast<uintptr_t>(U) & 15) == 0) && (((size_t)V * usz) % 16 == 0);

  RowStatsArgs rs{};
  rs.base = target;
  rs.kind = layout == 0 ? kRowsVerifyPacked : kRowsVerifyDense;
  rs.R = R; rs.gamma = gamma; rs.k = 0; rs.V = V; rs.nch = nch; rs.cu = cu;
  rs.nrows_cap = R * (gamma + 1);
  rs.scale2 = greedy ? 1.f : kLog2e / T;
  rs.vec_ok = t_vec;
  rs.L = reinterpret_cast<float2*>(w + L.ver_l);
  rs.I = reinterpret_cast<int*>(w + L.ver_i);
  rs.status = hdr;
  rs.zero_me = hdr + 1;
  hipError_t e = launch_row_stats(rs, u_bf16, greedy, st);
  if (e != hipSuccess) return e;

  VerifyArgs a{};
  a.R = R; a.gamma = gamma; a.V = V; a.rank = rank; a.nch = nch; a.layout = layout;
  a.invT = greedy ? 1.f : 1.f / T; a.greedy = greedy; a.seed = seed; a.round = round;
  a.ell = ell; a.cu = cu; a.target = target; a.x = x; a.logp_d = logp_d; a.lse_d = lse_d;
  a.U = U; a.W1 = W1; a.W2t = W2t; a.m = m; a.tau = tau; a.emitted = emitted;
  a.next_anchor = next_anchor; a.logp_t = logp_t; a.cap = cap; a.m_full = m_full;
  a.feat = feat;
  a.vl = rs.L; a.vi = rs.I;
  a.lse_t = reinterpret_cast<float2*>(w + L.lse_t);
  a.rej_count = reinterpret_cast<int32_t*>(hdr + 1);
  a.rej = reinterpret_cast<int4*>(w + L.rej);
  a.rl = reinterpret_cast<float2*>(w + L.draft_l);
  a.status = hdr;
  {
    const int rows = R * (gamma + 1);
    const int grid = min(4096, (rows + 3) / 4);
    hipLaunchKernelGGL(k_row_norm, dim3(grid), dim3(256), 0, st, a);
  }
  if (u_bf16) hipLaunchKernelGGL((k_verify_scan<uint16_t>), dim3(R), dim3(256), 0, st, a);
  else hipLaunchKernelGGL((k_verify_scan<float>), dim3(R), dim3(256), 0, st, a);
  e = hipGetLastError();
  if (e != hipSuccess || greedy) return e;

  // rows of the bias features: W1[x_{k-1}] (Markov head) or the draft's own
  // per-position features (RNN head)
  const void* E = feat ? feat : W1;
  if (u_bf16 && w_bf16 && rank > 0 && u_vec && t_vec &&
      launch_resid_slices(R, gamma, V, rank, T, U, E, W2t, target, x, a.rej_count, a.rej,
                          a.lse_t, lse_d, const_cast<float2*>(a.rl), hdr, st, &e, false,
                          feat != nullptr)) {
    if (e != hipSuccess) return e;
  } else {
    // per-tile kernel for the other shapes
    MarkovArgs ma{};
    ma.R = R; ma.gamma = gamma; ma.k = 0; ma.V = V; ma.rank = rank; ma.nch = nch; ma.nrows_cap = R;
    ma.U = U; ma.W1v = E; ma.W2tv = W2t; ma.x0 = nullptr; ma.x = x; ma.feat_rows = feat != nullptr;
    ma.scale2 = kLog2e / T;
    ma.u_vec_ok = u_vec && t_vec;
    ma.L = const_cast<float2*>(a.rl); ma.I = nullptr;
    ma.rej_count = a.rej_count; ma.rej = a.rej; ma.target = target; ma.lse_t = a.lse_t;
    ma.lse_d = lse_d; ma.status = hdr;
    e = launch_markov_stats(ma, u_bf16, w_bf16 && rank > 0, kModeResid, st);
    if (e != hipSuccess) return e;
  }
#define DSPARK_RP(UT_, WT_) hipLaunchKernelGGL((k_resid_pick<UT_, WT_>), dim3(R), dim3(256), 0, st, a)
  if (u_bf16 && w_bf16) DSPARK_RP(uint16_t, uint16_t);
  else if (u_bf16) DSPARK_RP(uint16_t, float);
  else if (w_bf16) DSPARK_RP(float, uint16_t);
  else DSPARK_RP(float, float);
#undef DSPARK_RP
  return hipGetLastError();
}

}  // namespace dspark
