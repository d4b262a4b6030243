// verify.hip -- lossless rejection-sampling verification.
//
// DSpark summary page, Background (x_k accepted with probability
// min(1, p_t(x_k)/p_d(x_k)), left to right, the first rejection drops the
// rest); MTP survey page, section 2.2 (resample the rejected position from
// norm(max(0, p_t - p_d)); after a fully accepted prefix draw the bonus token
// from the next target distribution; tau = m + 1; greedy reduction).
// Launches, all sized by capacity so N, m and the rejections stay on device:
//   1. k_verify_rows, one workgroup per verify row: the row's chunk
//      log-masses of t/T (chunk maxima at T = 0) and normaliser, the accept
//      test of the position it decides (log p_t(x_k), its uniform), the bonus
//      draw from a request's last row; the workgroup that completes a request
//      finds its first rejection by a ballot over the published outcomes and
//      writes the outputs, or lists a residual work item.  Cap-accept
//      (DeepSpec analysis page, section 5.4, DSpark in SGLang: the verify
//      modes): with a commit window C below the accepted count m, the first
//      C + 1 tokens of the sequence are committed, the last being the accepted
//      draft x_{C+1}; no draw is made.  Rows of more than kVrMaxChunks chunks
//      take three launches instead: k_row_stats, k_row_norm (one wave per
//      row) and k_verify_scan (one workgroup per request).
//   2. residual chunk masses for the listed (request, position) rows: the
//      draft scores are rebuilt with the Markov bias (MFMA) and combined with
//      the target row into max(0, p_t - p_d) per chunk.
//   3. k_resid_pick, one workgroup per work item: chunk pick and in-chunk pick
//      on log max(0, p_t - p_d); zero mass falls back to p_t.

#include <atomic>

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
  // fused verify rows
  float2* vl_out;       // = vl, written by the fused kernel
  int* req_done;        // [R] rows finished per request
  int* ybonus;          // [R] bonus token drawn from the request's last row
  int* acc;             // [R][gamma] outcome of each tested position (1 = rejected)
  uint32_t* epoch_word; // header word raised by workgroup 0 once the counters are clear
  uint32_t epoch;       // this call's epoch from the host (below 2^31), or 0: taken on the device
  uint32_t* last_word;  // header word: device epochs used so far (the last call's, counted)
  int* rows_done;       // header word: rows of this call finished (device epochs only)
  uint32_t spin_limit;  // polls before the wait for the epoch gives up
  float scale2;         // log2(e) / T (chunk sums), 1 at T = 0
  bool vec_ok;          // 16-byte loads of target rows
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

// The accept scan of request i and its outputs, by one workgroup of NT
// threads, from the row normalisers and chunk statistics in memory (the
// three-launch verify for rows too long to keep in LDS).
template <int NT, typename TT>
__device__ inline void scan_request(const VerifyArgs& a, int i, int q0, BlockScratch& sh,
                                    int* s_m, int* s_rej) {
  const int tid = threadIdx.x, lane = tid & 63;
  int L = a.ell[i];
  if (L < 0 || L > a.gamma) { if (tid == 0) set_flag(a.status, kFlagBadLen); L = L < 0 ? 0 : a.gamma; }
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
      *s_rej = bal != 0;
      *s_m = bal ? (__builtin_ctzll(bal)) : L;   // first rejected position k = m + 1
    }
  }
  __syncthreads();
  int m = *s_m;
  bool rejected = *s_rej != 0;
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
    const PickResult pc = block_pick_chunk<NT>(a.vl + (int64_t)q * a.nch, a.nch, nt.x, a.invT,
                                               a.seed, a.round, kTagBonusChunk, (uint32_t)i,
                                               (uint32_t)(L + 1), false, &srel, sh);
    const int c = pc.idx < 0 ? 0 : pc.idx;
    if (pc.idx < 0 && tid == 0) set_flag(a.status, kFlagNonFinite);
    const TT* trow = tgt + target_row(a, i, L) * a.V;
    const int v = c * kChunk + tid / (NT / kChunk);
    const float sc = (v < a.V) ? (Elem<TT>::get(trow, v) - nt.x) * a.invT : -INFINITY;
    const PickResult pe = block_pick_in_chunk<NT>(sc, c * kChunk, a.seed, a.round, kTagBonusElem,
                                                  (uint32_t)i, (uint32_t)(L + 1), false, sh);
    y = pe.idx < 0 ? c * kChunk : pe.idx;
  } else if (tid == 0) {
    const int slot = atomicAdd(a.rej_count, 1);
    a.rej[slot] = make_int4(i, m + 1, (int)target_row(a, i, m), q0 + m);
  }
  // outputs (a rejected sampled position gets its token from k_resid_pick)
  int32_t* em = a.emitted + (int64_t)i * (a.gamma + 1);
  const bool have_y = closed || a.greedy || !rejected;
  for (int q = tid; q <= a.gamma; q += NT)
    em[q] = (q < m) ? xi[q + 1] : ((q == m && have_y) ? y : -1);
  if (tid == 0) {
    a.m[i] = m;
    a.tau[i] = m + 1;
    if (have_y) a.next_anchor[i] = y;
  }
}

template <typename TT>
__global__ __launch_bounds__(256) void k_verify_scan(VerifyArgs a) {
  __shared__ BlockScratch sh;
  __shared__ int s_m, s_rej;
  const int i = blockIdx.x;
  scan_request<256, TT>(a, i, a.cu[i], sh, &s_m, &s_rej);
}

// ------------------------------------------------------- fused verify rows
// One launch for the verify rows: statistics of every verify row, its
// normaliser, every position's accept test, and the accept scan of every
// request.  One workgroup of kVrThreads per verify row q = cu[i] + j:
//   1. finds its request i (the one whose offsets hold q) and streams the
//      target row into per-chunk statistics in LDS (each wave one batch of
//      kVrUnr loads per lane, the arithmetic of the stand-alone statistics
//      kernel);
//   2. writes them to memory (read later by the residual kernels), reduces
//      them to the row normaliser and publishes it (device-coherent store);
//   3. j < ell_i: tests position k = j + 1 (log p_t(x_k) is this row's) and
//      publishes the outcome; j == ell_i at T > 0: draws the bonus token from
//      its own statistics (used if the whole block is accepted);
//   4. counts itself done for request i; the workgroup that completes the
//      request finds the first rejection from the published outcomes and
//      writes the request's outputs.
// After step 3 only the first wave goes on (the counter update, the scan);
// the others write the chunk statistics out and leave.
// The completion counters and the residual count are cleared inside the
// launch by workgroup 0, which then raises the launch's epoch in a header
// word; a workgroup waits for that epoch (bounded) before its counter update.
// Workgroup 0 is dispatched before every other, so the wait ends.  The epoch
// comes from a per-process host counter, or, for a call captured in a graph
// (where a host value would be frozen into every replay), from the device: a
// count of the device epochs used so far, kept in a second header word and
// advanced by the row that completes the call's count.
constexpr int kVrThreads = 512;
constexpr int kVrWaves = kVrThreads / 64;
constexpr int kVrUnr = 8;                   // 16-byte loads in flight per lane
constexpr int kVrMaxChunks = 4096;          // per-row statistics held in LDS

// The scan of request i from the outcomes its rows published in this launch,
// by one wave: one round of device-coherent loads, a ballot, the outputs.
template <bool GREEDY>
__device__ inline void scan_published(const VerifyArgs& a, int i, int q0, int L) {
  const int lane = threadIdx.x & 63;
  const int32_t* xi = a.x + (int64_t)i * (a.gamma + 1);
  const int k = lane + 1;
  const bool rej_k = k <= L && ld_coh(a.acc + (int64_t)i * a.gamma + (k - 1)) != 0;
  int yl = -1;
  if (GREEDY && lane <= L) yl = __float_as_int(ld_coh2(a.lse_t + q0 + lane).y);   // argmax of row `lane`
  if (!GREEDY && lane == 0) yl = ld_coh(a.ybonus + i);
  if (k > L && k <= a.gamma && a.logp_t) a.logp_t[(int64_t)i * a.gamma + (k - 1)] = 0.f;
  const uint64_t bal = __ballot(rej_k);
  int m = bal ? __builtin_ctzll(bal) : L;       // first rejected position k = m + 1
  int y = __shfl(yl, GREEDY ? m : 0);
  bool rejected = bal != 0;
  bool closed = false;
  if (a.cap) {
    int C = a.cap[i];
    if (C < 0) { if (lane == 0) set_flag(a.status, kFlagBadLen); C = 0; }
    if (C > L) C = L;
    if (lane == 0 && a.m_full) a.m_full[i] = m;
    if (m > C) {
      closed = true;
      m = C;
      rejected = false;
    }
  }
  if (closed) {
    y = xi[m + 1];                      // the accepted draft that closes the window
    if (y < 0 || y >= a.V) y = 0;       // (flagged by the position's test)
  } else if (GREEDY || !rejected) {
    // greedy: the argmax of row m; sampled: the bonus token drawn from row L
    if (y < 0 || y >= a.V) { if (lane == 0) set_flag(a.status, kFlagNonFinite); y = 0; }
  } else if (lane == 0) {
    const int slot = atomicAdd(a.rej_count, 1);
    a.rej[slot] = make_int4(i, m + 1, (int)target_row(a, i, m), q0 + m);
  }
  int32_t* em = a.emitted + (int64_t)i * (a.gamma + 1);
  const bool have_y = closed || GREEDY || !rejected;
  for (int q = lane; q <= a.gamma; q += 64)
    em[q] = (q < m) ? xi[q + 1] : ((q == m && have_y) ? y : -1);
  if (lane == 0) {
    a.m[i] = m;
    a.tau[i] = m + 1;
    if (have_y) a.next_anchor[i] = y;
  }
}

template <typename T, bool GREEDY>
__global__ __launch_bounds__(kVrThreads) void k_verify_rows(VerifyArgs a) {
  extern __shared__ __align__(16) unsigned char vr_lds[];
  float2* sL = reinterpret_cast<float2*>(vr_lds);
  int* sI = reinterpret_cast<int*>(vr_lds + (size_t)a.nch * sizeof(float2));
  __shared__ BlockScratch sh;
  __shared__ int s_i, s_lo, s_hi, s_ell;
  const int tid = threadIdx.x, wv = tid >> 6;
  const int q = blockIdx.x;
  const int N = min(a.cu[a.R], a.R * (a.gamma + 1));
  // this call's epoch.  From the host when the call is enqueued directly;
  // under graph capture a host value would be frozen into every replay, so
  // then it is taken on the device: the count of device epochs used so far
  // plus one, with the top bit set so that it never equals a host epoch.
  // Every workgroup reads that count before any row of the call is counted
  // (it moves only once every row has been), so all agree.
  const bool dev_epoch = a.epoch == 0;
  uint32_t E = a.epoch;
  if (dev_epoch && tid == 0)
    E = ((__hip_atomic_load(a.last_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u) & 0x7FFFFFFFu) |
        0x80000000u;
  if (q == 0) {
    for (int t = tid; t < a.R; t += kVrThreads) st_coh(a.req_done + t, 0);
    if (tid == 0) { st_coh(a.rej_count, 0); st_coh(a.rows_done, 0); }
    __builtin_amdgcn_s_waitcnt(0x0F70);         // vmcnt(0): the clears have completed
    __syncthreads();
    if (tid == 0) {
      __hip_atomic_store(a.epoch_word, E, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (dev_epoch && N <= 0)
        __hip_atomic_store(a.last_word, E & 0x7FFFFFFFu, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (q >= N) return;
  // (thread 0) wait for this call's epoch, bounded; false if the wait gave up.
  // A wait that gives up leaves its row uncounted, so it records the epoch as
  // finished itself: the next call then starts from a new epoch.
  auto epoch_ready = [&]() {
    uint32_t spins = 0;
    while (__hip_atomic_load(a.epoch_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != E) {
      if (++spins >= a.spin_limit) {
        atomicOr(a.status, kFlagBarrier);
        if (dev_epoch)
          __hip_atomic_store(a.last_word, E & 0x7FFFFFFFu, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return false;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    return true;
  };
  // (thread 0, after epoch_ready) with a device epoch, count row q; the last
  // row of the call records the epoch as used.  (One counter for the whole
  // call: its updates serialise, which costs about 9 us at 462 rows, so
  // directly enqueued calls use the host epoch and skip it.)
  auto count_row = [&]() {
    if (dev_epoch &&
        __hip_atomic_fetch_add(a.rows_done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1 == N)
      __hip_atomic_store(a.last_word, E & 0x7FFFFFFFu, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  // the request whose offsets hold q, and its scheduled length
  if (tid == 0) s_i = -1;
  __syncthreads();
  for (int t = tid; t < a.R; t += kVrThreads) {
    const int lo = a.cu[t], hi = a.cu[t + 1], el = a.ell[t];
    if (lo <= q && q < hi) { s_i = t; s_lo = lo; s_hi = hi; s_ell = el; }
  }
  __syncthreads();
  const int i = s_i;
  if (i < 0) {                                  // offsets not ascending
    if (tid == 0) {
      set_flag(a.status, kFlagBadLen);
      if (epoch_ready()) count_row();
    }
    return;
  }
  const int q0 = s_lo, nrows = s_hi - s_lo, j = q - q0;
  if (nrows > a.gamma + 1) {                    // more rows than the block holds
    if (tid == 0) {
      set_flag(a.status, kFlagBadLen);
      if (epoch_ready()) count_row();
    }
    return;
  }
  int L = s_ell;
  if (L < 0 || L > a.gamma || L > nrows - 1) {
    if (tid == 0 && j == 0) set_flag(a.status, kFlagBadLen);
    L = min(max(L, 0), min(a.gamma, nrows - 1));
  }
  const int64_t row = a.layout == 0 ? (int64_t)q : (int64_t)i * (a.gamma + 1) + j;
  const T* rp = reinterpret_cast<const T*>(a.target) + row * a.V;
  // the token this row tests and its draft log-probability, fetched ahead
  int xk = 0;
  float lpd = 0.f;
  if (tid == 0 && j < L) {
    xk = a.x[(int64_t)i * (a.gamma + 1) + j + 1];
    if (!GREEDY) lpd = a.logp_d[(int64_t)i * a.gamma + j];
  }

  // 1. chunk statistics of the row into LDS: batches of CPB chunks per wave
  constexpr int CPB = 64 * kVrUnr / (kChunk * (int)sizeof(T) / 16);
  for (int c0 = wv * CPB; c0 < a.nch; c0 += kVrWaves * CPB)
    row_segment<T, GREEDY, kVrUnr>(rp, a.V, c0, min(a.nch, c0 + CPB), a.scale2, a.vec_ok, sL, sI,
                                   a.status);
  // the tested token's score (its row was just streamed), in flight during
  // the reductions below
  float tk = 0.f;
  if (!GREEDY && tid == 0 && j < L) tk = Elem<T>::get(rp, (xk < 0 || xk >= a.V) ? 0 : xk);
  __syncthreads();

  // 2. the row normaliser (raw maximum, log-sum above it), or at T = 0 the
  // row maximum and its first argmax
  float2 nt;
  if (GREEDY) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
    for (int c = tid; c < a.nch; c += kVrThreads) argmax_merge(bv, bi, sL[c].x, sI[c]);
    block_argmax<kVrThreads>(bv, bi, sh);
    nt = make_float2(bv, __int_as_float(bi));
  } else {
    float mx = -INFINITY;
    for (int c = tid; c < a.nch; c += kVrThreads) mx = fmaxf(mx, sL[c].x);
    const float m = block_max<kVrThreads>(mx, sh);
    float sum = 0.f;
    if (m != -INFINITY) {
      for (int c = tid; c < a.nch; c += kVrThreads) {
        const float2 v = sL[c];
        if (v.y > 0.f) sum += v.y * expf((v.x - m) * a.invT);
      }
    }
    sum = block_sum<kVrThreads>(sum, sh);
    nt = (m == -INFINITY) ? make_float2(-INFINITY, -INFINITY)
                          : make_float2(m, sum > 0.f ? logf(sum) : -INFINITY);
  }
  if (tid == 0) st_coh2(a.lse_t + q, nt);

  // 3. the test of position j + 1, or the bonus draw from the last row
  if (tid == 0 && j < L) {
    const int k = j + 1;
    if (xk < 0 || xk >= a.V) { set_flag(a.status, kFlagBadToken); xk = 0; }
    int rej;
    if (GREEDY) {
      rej = xk != __float_as_int(nt.y);
      if (a.logp_t) a.logp_t[(int64_t)i * a.gamma + j] = 0.f;
    } else {
      const float lp = (tk - nt.x) * a.invT - nt.y;
      if (a.logp_t) a.logp_t[(int64_t)i * a.gamma + j] = lp;
      const uint4 blk = stream_block(a.seed, a.round, kTagAccept, (uint32_t)i, (uint32_t)k, 0u);
      rej = !(log_uniform(blk.x) < lp - lpd);
    }
    st_coh(a.acc + (int64_t)i * a.gamma + j, rej);
  }
  if (!GREEDY && j == L) {
    const PickResult pc = block_pick_chunk<kVrThreads>(sL, a.nch, nt.x, a.invT, a.seed, a.round,
                                                       kTagBonusChunk, (uint32_t)i,
                                                       (uint32_t)(L + 1), false, nullptr, sh);
    const int c = pc.idx < 0 ? 0 : pc.idx;
    if (pc.idx < 0 && tid == 0) set_flag(a.status, kFlagNonFinite);
    const int v = c * kChunk + tid / (kVrThreads / kChunk);
    const float sc = (v < a.V) ? (Elem<T>::get(rp, v) - nt.x) * a.invT : -INFINITY;
    const PickResult pe = block_pick_in_chunk<kVrThreads>(sc, c * kChunk, a.seed, a.round,
                                                          kTagBonusElem, (uint32_t)i,
                                                          (uint32_t)(L + 1), false, sh);
    if (tid == 0) st_coh(a.ybonus + i, pe.idx < 0 ? c * kChunk : pe.idx);
  }
  // the chunk statistics, read only by the residual kernels of later
  // launches, are written by the other waves, which then leave
  if (wv != 0) {
    if (!GREEDY) {
      float2* gL = a.vl_out + (int64_t)q * a.nch;
      for (int c = tid - 64; c < a.nch; c += kVrThreads - 64) gL[c] = sL[c];
    }
    return;
  }
  const int lane = tid;

  // 4. done with row q: the wave's stores have completed, then one counter
  // update; the wave that completes request i scans it
  __builtin_amdgcn_s_waitcnt(0x0F70);
  int last = 0;
  if (lane == 0 && epoch_ready()) {
    const int done = __hip_atomic_fetch_add(a.req_done + i, 1, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
    last = done + 1 == nrows;
    count_row();
  }
  if (!__shfl(last, 0)) return;
  scan_published<GREEDY>(a, i, q0, L);
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

// A new host epoch for every directly enqueued fused verify launch: in
// [1, 2^31) (0 and the top bit are the device epochs' marks).
static uint32_t next_verify_epoch() {
  static std::atomic<uint32_t> counter{0};
  for (;;) {
    const uint32_t e = (counter.fetch_add(1, std::memory_order_relaxed) + 1) & 0x7FFFFFFFu;
    if (e != 0) return e;
  }
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

  VerifyArgs a{};
  a.R = R; a.gamma = gamma; a.V = V; a.rank = rank; a.nch = nch; a.layout = layout;
  a.invT = greedy ? 1.f : 1.f / T; a.greedy = greedy; a.seed = seed; a.round = round;
  a.ell = ell; a.cu = cu; a.target = target; a.x = x; a.logp_d = logp_d; a.lse_d = lse_d;
  a.U = U; a.W1 = W1; a.W2t = W2t; a.m = m; a.tau = tau; a.emitted = emitted;
  a.next_anchor = next_anchor; a.logp_t = logp_t; a.cap = cap; a.m_full = m_full;
  a.feat = feat;
  a.vl = reinterpret_cast<const float2*>(w + L.ver_l);
  a.vi = reinterpret_cast<const int*>(w + L.ver_i);
  a.lse_t = reinterpret_cast<float2*>(w + L.lse_t);
  a.rej_count = reinterpret_cast<int32_t*>(hdr + 1);
  a.rej = reinterpret_cast<int4*>(w + L.rej);
  a.rl = reinterpret_cast<float2*>(w + L.draft_l);
  a.status = hdr;
  a.scale2 = greedy ? 1.f : kLog2e / T;
  a.vec_ok = t_vec;
  const int rows = R * (gamma + 1);
  hipError_t e;
  if (nch <= kVrMaxChunks) {
    // statistics, normalisers and the accept scan in one launch
    a.vl_out = reinterpret_cast<float2*>(w + L.ver_l);
    a.req_done = reinterpret_cast<int*>(w + L.vaux);
    a.ybonus = a.req_done + R;
    a.acc = a.ybonus + R;
    a.epoch_word = hdr + 3;
    // a host epoch for a call enqueued directly; 0 (epoch taken on the device)
    // for a call being captured into a graph
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if ((e = hipStreamIsCapturing(st, &cs)) != hipSuccess) return e;
    a.epoch = cs == hipStreamCaptureStatusNone ? next_verify_epoch() : 0u;
    a.last_word = hdr + 4;
    a.rows_done = reinterpret_cast<int*>(hdr + 5);
    a.spin_limit = switches().barrier_spins ? switches().barrier_spins : kBarrierSpins;
    const size_t lds = (size_t)nch * (greedy ? 12 : 8);
#define DSPARK_VR(T_, G_) hipLaunchKernelGGL((k_verify_rows<T_, G_>), dim3(rows), dim3(kVrThreads), lds, st, a)
    if (u_bf16) { if (greedy) DSPARK_VR(uint16_t, true); else DSPARK_VR(uint16_t, false); }
    else        { if (greedy) DSPARK_VR(float, true);    else DSPARK_VR(float, false); }
#undef DSPARK_VR
  } else {
    // rows too long for the statistics to stay in LDS: three launches
    RowStatsArgs rs{};
    rs.base = target;
    rs.kind = layout == 0 ? kRowsVerifyPacked : kRowsVerifyDense;
    rs.R = R; rs.gamma = gamma; rs.k = 0; rs.V = V; rs.nch = nch; rs.cu = cu;
    rs.nrows_cap = rows;
    rs.scale2 = a.scale2;
    rs.vec_ok = t_vec;
    rs.L = reinterpret_cast<float2*>(w + L.ver_l);
    rs.I = reinterpret_cast<int*>(w + L.ver_i);
    rs.status = hdr;
    rs.zero_me = hdr + 1;
    e = launch_row_stats(rs, u_bf16, greedy, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_row_norm, dim3(min(4096, (rows + 3) / 4)), dim3(256), 0, st, a);
    if (u_bf16) hipLaunchKernelGGL((k_verify_scan<uint16_t>), dim3(R), dim3(256), 0, st, a);
    else hipLaunchKernelGGL((k_verify_scan<float>), dim3(R), dim3(256), 0, st, a);
  }
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
