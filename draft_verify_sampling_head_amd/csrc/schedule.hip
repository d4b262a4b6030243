// schedule.hip -- hardware-aware prefix scheduler (one workgroup).
//
// DSpark summary page, Method details ("greedy solution and causality",
// Algorithm 1).  Survival a_{r,j} = prod_{i<=j} c_{r,i} is a left-to-right
// float32 running product per request.  Candidates (r, j) with a > 0 are
// ordered by a descending, then r, then j ascending -- a total order -- by
// sorting 64-bit keys (~bits(a) << 32 | r*32 + j-1).  Since c <= 1 makes a
// non-increasing in j, each request's keys are already an ascending run: up
// to four keys per thread the runs, padded to a power of two, are merged
// bottom-up (merge path: each thread finds its output range by a binary
// search and merges it from LDS into registers).  Larger shapes, and runs out
// of order (some c outside [0, 1]), take a stable LSD radix sort of the keys'
// high halves (four 8-bit passes; ranks among equal digits from wave
// ballots, offsets from one block scan of per-wave digit counts per pass),
// which leaves equal values of a in (r, j) order.  Admitting the q first
// candidates gives B = R + q and tau_q = R + sum of their a; in 2^-32 fixed
// point the sums are exact, so a block-wide prefix sum yields every tau_q at
// once, and
// Theta_q = (tau_q * 2^-32) * SPS(B) is one double product (0 past N_max).
// The sequential rule "admit while Theta improves, stop at the first
// non-improvement" admits exactly the candidates before the first q with
// Theta_q <= Theta_{q-1}; a block-wide min finds that q.  ell_r is then the
// largest admitted position of request r (admitted positions of a request are
// always a prefix 1..ell_r, because a is non-increasing in j).
//
// The rule reads the order only up to its first stop, a few hundred
// positions for real confidence curves.  So Algorithm 1 first orders only a
// selected prefix of about 512 keys (histograms of the keys' high bits find
// it; it is ranked bucket by bucket) and decides on it with one position per
// thread; the whole sort above runs only when the stop is not inside that
// prefix, or when too many equal keys make the prefix too long.
//
// The asynchronous form used in production (same page, Supplementary details,
// the scheduler in production) sorts the same keys and takes two decisions
// from the one sort: admission of the first min(K_in, N_max) - R candidates
// (K_in = verify capacity in tokens planned two rounds earlier; clamped to
// [0, |E|]; no Theta test), and the plan K_plan = R + q* where q* is the first
// maximiser of Theta_q over q = 0..|E| (global search: every thread keeps the
// first maximum of its own positions, then one block-wide (max Theta, min q)
// reduction).
//
// With pack set, the same workgroup then packs the verify batch (the drafted
// rows x with lengths ell + 1, anchors included) as the stand-alone pack
// kernel does, from the lengths it has just left in LDS: the scheduler's
// decision and the batch it implies cost one launch.
#include "launch.hpp"
#include "pack.hpp"

namespace dspark {

constexpr int kSchedMaxKeys = 16384;
constexpr int kSchedThreads = 1024;

__device__ __forceinline__ int64_t fixed32(float a) {
  return __double2ll_rn((double)a * 4294967296.0);
}

__device__ __forceinline__ double theta_of(int64_t tau, int B, int N_max, const double* sps) {
  return (B > N_max) ? 0.0 : ((double)tau * 0x1p-32) * sps[B];
}

__device__ inline int64_t block_sum_i64(int64_t v, int64_t* lds) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  if (lane == 0) lds[wv] = v;
  __syncthreads();
  int64_t t = 0;
  for (int q = 0; q < kSchedThreads / 64; ++q) t += lds[q];
  __syncthreads();
  return t;
}

__device__ inline int64_t block_exscan_i64(int64_t v, int64_t* lds) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int64_t inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t y = __shfl_up(inc, o);
    if (lane >= o) inc += y;
  }
  if (lane == 63) lds[wv] = inc;
  __syncthreads();
  int64_t before = 0;
  for (int q = 0; q < wv; ++q) before += lds[q];
  __syncthreads();
  return before + inc - v;
}

// (max th, then min q) over the workgroup: the first maximum of Theta_q when
// every thread holds the first maximum of its own ascending positions.
__device__ inline void block_argmax_first(double& th, int& q, double* ldsd, int* ldsi) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const double oth = __shfl_xor(th, o);
    const int oq = __shfl_xor(q, o);
    if (oth > th || (oth == th && oq < q)) { th = oth; q = oq; }
  }
  if (lane == 0) { ldsd[wv] = th; ldsi[wv] = q; }
  __syncthreads();
  th = ldsd[0];
  q = ldsi[0];
  for (int w = 1; w < kSchedThreads / 64; ++w) {
    const double oth = ldsd[w];
    const int oq = ldsi[w];
    if (oth > th || (oth == th && oq < q)) { th = oth; q = oq; }
  }
  __syncthreads();
}

__device__ inline int block_min_i(int v, int* lds) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, __shfl_xor(v, o));
  if (lane == 0) lds[wv] = v;
  __syncthreads();
  int t = lds[0];
  for (int q = 1; q < kSchedThreads / 64; ++q) t = min(t, lds[q]);
  __syncthreads();
  return t;
}

// Stable LSD radix sort of keys[0, P) by their high 32 bits: four passes of
// eight bits.  Wave w owns positions [w S, w S + S), S = 64 EPT, read in EPT
// rounds of 64 consecutive positions.  In a round the lanes holding the same
// digit are found by matching the digit's bits across the wave (eight
// ballots); a key's rank among the equal digits of its wave before it is the
// wave's count of that digit so far plus the matching lanes below it.  One
// exclusive scan of the per-wave digit counts in (digit, wave) order gives
// every key its place.  Keys whose high halves are equal keep their buffer
// order, which the caller makes ascending in the low halves, so the result
// is the order of the whole 64-bit keys.  Thread t ends with the sorted
// positions [t EPT, t EPT + EPT) in v.
template <int EPT>
__device__ __forceinline__ void radix_sort_hi32(uint64_t (&v)[EPT], uint64_t* keys,
                                                uint32_t* whist, int* scan_lds) {
  constexpr int S = 64 * EPT;
  constexpr int NW = kSchedThreads / 64;
  static_assert(NW * 256 == 4 * kSchedThreads, "four counts per thread in the scan");
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const uint64_t below = (1ull << lane) - 1;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 32 + 8 * pass;
    for (int t = tid; t < NW * 256; t += kSchedThreads) whist[t] = 0;
    uint64_t k[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) k[e] = keys[wv * S + e * 64 + lane];
    __syncthreads();                          // counts cleared, every key read
    uint32_t rank[EPT];
    int dig[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int d = (int)(k[e] >> shift) & 255;
      uint64_t peers = ~0ull;
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const uint64_t bb = __ballot((d >> b) & 1);
        peers &= ((d >> b) & 1) ? bb : ~bb;
      }
      const int leader = __builtin_ctzll(peers);
      uint32_t base = 0;
      if (lane == leader) {
        base = whist[wv * 256 + d];
        whist[wv * 256 + d] = base + (uint32_t)__popcll(peers);
      }
      base = __shfl(base, leader);
      rank[e] = base + (uint32_t)__popcll(peers & below);
      dig[e] = d;
    }
    __syncthreads();
    // offsets: exclusive scan of the counts, entry d * NW + w for digit d of wave w
    uint32_t c4[4], sum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = 4 * tid + q;
      c4[q] = whist[(idx % NW) * 256 + idx / NW];
      sum += c4[q];
    }
    int total;
    uint32_t pre = (uint32_t)block_exclusive_scan((int)sum, scan_lds, &total);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = 4 * tid + q;
      whist[(idx % NW) * 256 + idx / NW] = pre;
      pre += c4[q];
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < EPT; ++e) keys[whist[wv * 256 + dig[e]] + rank[e]] = k[e];
    __syncthreads();
  }
#pragma unroll
  for (int e = 0; e < EPT; ++e) v[e] = keys[tid * EPT + e];
}

// Bottom-up merge of the ascending runs of length run0 (a power of two) in
// keys[0, P); thread t ends with the sorted positions [t EPT, t EPT + EPT) in
// v.  Per level, thread t's output range lies inside one pair of runs
// (2 run >= EPT): a binary search over the merge path finds how many of its
// first outputs come from the left run, then EPT steps merge from LDS (ties
// take the left run).  The outputs are written back after a barrier.
template <int EPT>
__device__ __forceinline__ void merge_sort_runs(uint64_t (&v)[EPT], uint64_t* keys, int P, int run0) {
  const int o0 = threadIdx.x * EPT;
  if (run0 >= P) {
#pragma unroll
    for (int e = 0; e < EPT; ++e) v[e] = keys[o0 + e];
    return;
  }
  for (int run = run0; run < P; run *= 2) {
    const int base = o0 & ~(2 * run - 1);
    const int d = o0 - base;
    const uint64_t* A = keys + base;
    const uint64_t* B = keys + base + run;
    int lo = max(0, d - run), hi = min(d, run);
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (A[mid] <= B[d - mid - 1]) lo = mid + 1;
      else hi = mid;
    }
    int i = lo, j = d - lo;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const uint64_t x = (i < run) ? A[i] : ~0ull;
      const uint64_t y = (j < run) ? B[j] : ~0ull;
      const bool ta = (j >= run) || (i < run && x <= y);
      v[e] = ta ? x : y;
      i += ta ? 1 : 0;
      j += ta ? 0 : 1;
    }
    __syncthreads();
    if (2 * run < P) {
#pragma unroll
      for (int e = 0; e < EPT; ++e) keys[o0 + e] = v[e];
      __syncthreads();
    }
  }
}

// Algorithm 1 reads the sorted order only up to its first stop, which for
// real confidence curves lies a few hundred positions in, however many
// candidates there are.  So before sorting everything, the kSelK smallest
// keys (largest a) are selected: a histogram of 12 bits of the keys' high
// halves (bits 19..30: exponent and four mantissa bits of a; bit 31 is the
// same for every candidate) finds the bucket in which the count reaches
// kSelK; if more than kSelMax keys lie up to that bucket, a second histogram
// of the next 12 bits, over that bucket's keys alone, finds the crossing
// there.  The selected set is every key whose prefix (12 or 24 bits) does not
// exceed the crossing one, so it is a prefix of the full order: keys with
// equal prefixes are all in or all out.  Ordering the set: with one level,
// the exclusive scan of the bucket counts is each bucket's first position, so
// every key is scattered into its bucket's range and ranked against the keys
// of its own bucket only; after a second level the keys are ranked against
// the whole set.  The keys are distinct, so the ranks are a permutation.
// Thread t receives positions [t EPT, t EPT + EPT) in v, sentinels past the
// set.  Returns the set's size n, or -1 when more than kSelMax keys tie on
// the prefixes around the crossing; *total is the number of candidates.  The
// caller sorts everything when -1 comes back, or when the admission scan over
// the n positions finds no stop and n < *total.
constexpr int kSelK = 512;
constexpr int kSelMax = 1024;
constexpr int kSelBins = 4 * kSchedThreads;

template <int EPT>
__device__ int select_sorted_prefix(uint64_t (&v)[EPT], const uint64_t* keys, int P,
                                    uint32_t* whist, uint64_t* ssel, int* sel, int64_t* red64,
                                    int* total) {
  static_assert(kSelBins == (kSchedThreads / 64) * 256, "the bins fill the radix count buffer");
  static_assert(kSelBins * 4 >= kSelMax * 8, "the ranked keys fit the bins' buffer");
  static_assert(kSchedMaxKeys < 65536, "bucket offsets and counts fit 16 bits");
  const int tid = threadIdx.x;
  // one histogram level: bins (k >> shift) & 0xFFF over the candidates (only
  // those of level-1 bucket b1 when inb); returns the crossing bin of `need`
  // (the last bin when the count never reaches it), the count before it and
  // the count through it; n_all = count of everything histogrammed.  Each
  // thread then leaves, in its own four bins, the bin's first position in
  // the high half and zero in the low half (the scatter's running count).
  auto level = [&](int shift, bool inb, uint32_t b1, int need, int& b, int& before_b,
                   int& through_b, int& n_all) {
    for (int t = tid; t < kSelBins; t += kSchedThreads) whist[t] = 0;
    if (tid == 0) { sel[0] = kSelBins - 1; sel[1] = 0; sel[2] = -1; sel[4] = 0; }
    __syncthreads();
    for (int q = tid; q < P; q += kSchedThreads) {
      const uint64_t k = keys[q];
      if (k != ~0ull && (!inb || (uint32_t)((k >> 51) & 0xFFFu) == b1))
        atomicAdd(&whist[(uint32_t)(k >> shift) & 0xFFFu], 1u);
    }
    __syncthreads();
    int c[4], s = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) { c[q] = (int)whist[4 * tid + q]; s += c[q]; }
    int cum = (int)block_exscan_i64(s, red64);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (cum < need && cum + c[q] >= need) { sel[0] = 4 * tid + q; sel[1] = cum; sel[2] = cum + c[q]; }
      whist[4 * tid + q] = (uint32_t)cum << 16;
      cum += c[q];
    }
    if (tid == kSchedThreads - 1) sel[3] = cum;
    __syncthreads();
    b = sel[0];
    before_b = sel[1];
    n_all = sel[3];
    through_b = sel[2] < 0 ? n_all : sel[2];
    __syncthreads();                           // sel is rewritten next
  };
  int b1, cb1, nb1, n_all;
  level(51, false, 0u, kSelK, b1, cb1, nb1, n_all);
  *total = n_all;
  uint64_t* out = reinterpret_cast<uint64_t*>(whist);
  int n = nb1;
  int r = 0;
  uint64_t x = 0;
  if (nb1 <= kSelMax) {
    // one level: scatter into the buckets, rank inside the bucket
    for (int q = tid; q < P; q += kSchedThreads) {
      const uint64_t k = keys[q];
      const uint32_t d1 = (uint32_t)((k >> 51) & 0xFFFu);
      if (k != ~0ull && (int)d1 <= b1) {
        const uint32_t w = atomicAdd(&whist[d1], 1u);
        ssel[(w >> 16) + (w & 0xFFFFu)] = k;
      }
    }
    __syncthreads();
    if (tid < n) {
      x = ssel[tid];
      const uint32_t w = whist[(uint32_t)((x >> 51) & 0xFFFu)];
      const int s0 = (int)(w >> 16), cnt = (int)(w & 0xFFFFu);
      r = s0;
      int i = 0;
      for (; i + 4 <= cnt; i += 4) {
        const uint64_t y0 = ssel[s0 + i], y1 = ssel[s0 + i + 1], y2 = ssel[s0 + i + 2],
                       y3 = ssel[s0 + i + 3];
        r += (y0 < x ? 1 : 0) + (y1 < x ? 1 : 0) + (y2 < x ? 1 : 0) + (y3 < x ? 1 : 0);
      }
      for (; i < cnt; ++i) r += (ssel[s0 + i] < x) ? 1 : 0;
    }
  } else {
    // second level inside the crossing bucket; the selected keys are ranked
    // against all of them
    int b2, cb2, nb2, n_b1;
    level(39, true, (uint32_t)b1, kSelK - cb1, b2, cb2, nb2, n_b1);
    n = cb1 + nb2;
    if (n > kSelMax) return -1;
    for (int q = tid; q < P; q += kSchedThreads) {
      const uint64_t k = keys[q];
      if (k == ~0ull) continue;
      const int d1 = (int)((k >> 51) & 0xFFFu), d2 = (int)((k >> 39) & 0xFFFu);
      if (d1 < b1 || (d1 == b1 && d2 <= b2)) ssel[atomicAdd(&sel[4], 1)] = k;
    }
    __syncthreads();
    if (tid < n) {
      x = ssel[tid];
      int i = 0;
      for (; i + 4 <= n; i += 4) {
        const uint64_t y0 = ssel[i], y1 = ssel[i + 1], y2 = ssel[i + 2], y3 = ssel[i + 3];
        r += (y0 < x ? 1 : 0) + (y1 < x ? 1 : 0) + (y2 < x ? 1 : 0) + (y3 < x ? 1 : 0);
      }
      for (; i < n; ++i) r += (ssel[i] < x) ? 1 : 0;
    }
  }
  __syncthreads();                             // the bins are read; out overwrites them
  if (tid < n) out[r] = x;
  __syncthreads();
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int p = tid * EPT + e;
    v[e] = (p < n) ? out[p] : ~0ull;
  }
  return n;
}

template <int EPT>
__device__ __forceinline__ void schedule_body(const SchedArgs& a, int G2, uint64_t* keys, int64_t* red64,
                                              int* red32, const int* kin_l, uint32_t* whist,
                                              int* scan_lds, uint64_t* ssel, int* sel) {
  const int tid = threadIdx.x;
  const int R = a.R, G = a.gamma;
  const int P = kSchedThreads * EPT;
  // G2 > 0: request r's keys sit at r*G2 + j (runs padded to G2, a power of
  // two); G2 == 0: packed at r*G + j
  const int stride = G2 > 0 ? G2 : G;
  const int p0 = tid * EPT;

  // SPS(B) for every batch size this thread's positions can reach
  // (B = R + p0 .. R + p0 + EPT, clamped to N_max: Theta is 0 past it),
  // fetched first so the admission pass after the sort reads registers (up
  // to 8 positions per thread; the 16-position form, which has no registers
  // to spare, reads them where they are used)
  constexpr int NSV = EPT <= 8 ? EPT + 1 : 1;
  double sv[NSV];
#pragma unroll
  for (int e = 0; e < NSV; ++e) sv[e] = a.sps[min(R + p0 + e, a.N_max)];
  // Theta at B = R + p0 + e (e known at compile time after unrolling)
  auto theta_here = [&](int64_t tau, int e) {
    const int B = R + p0 + e;
    return (B > a.N_max) ? 0.0 : ((double)tau * 0x1p-32) * (EPT <= 8 ? sv[e] : a.sps[B]);
  };

  // survival products (left to right, float32) and sort keys
  int64_t part = 0;
  int unsorted = 0;
  const bool vec4 = (G % 4) == 0 && (reinterpret_cast<uintptr_t>(a.c) & 15) == 0;
  for (int r = tid; r < R; r += kSchedThreads) {
    const float* cr = a.c + (int64_t)r * G;
    float cv[32];
    if (vec4) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float4 f = (4 * q < G) ? reinterpret_cast<const float4*>(cr)[q] : make_float4(0.f, 0.f, 0.f, 0.f);
        cv[4 * q] = f.x; cv[4 * q + 1] = f.y; cv[4 * q + 2] = f.z; cv[4 * q + 3] = f.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 32; ++j) cv[j] = (j < G) ? cr[j] : 0.f;
    }
    float acc = 1.f;
    uint64_t prevkey = 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      if (j < G) {
        acc = __fmul_rn(acc, cv[j]);
        if (a.a) a.a[(int64_t)r * G + j] = acc;
        const uint64_t key = (acc > 0.f)
            ? ((uint64_t)(0xFFFFFFFFu - __float_as_uint(acc)) << 32) | (uint32_t)(r * 32 + j)
            : ~0ull;
        unsorted |= key < prevkey;
        prevkey = key;
        keys[r * stride + j] = key;
        part += fixed32(acc);
      }
    }
    for (int j = G; j < stride; ++j) keys[r * stride + j] = ~0ull;
  }
  for (int q = R * stride + tid; q < P; q += kSchedThreads) keys[q] = ~0ull;
  unsorted = __syncthreads_or(unsorted);

  if (!a.enabled) {
    const int64_t tau = ((int64_t)R << 32) + block_sum_i64(part, red64);
    int* ell_l = reinterpret_cast<int*>(keys);        // (the keys are not read again)
    for (int r = tid; r < R; r += kSchedThreads) {
      a.ell[r] = G;
      ell_l[r] = G;
    }
    if (tid == 0) {
      const int B = R * (G + 1);
      if (a.N_out) *a.N_out = B;
      if (a.theta) *a.theta = theta_of(tau, B, a.N_max, a.sps);
    }
    return;
  }

  // Admission over sorted positions in v: thread t owns [t*EPT, t*EPT + EPT),
  // and the first sentinel ends the candidates.  Fixed-point prefix sums give
  // tau at every position.  Returns the number of candidates admitted; mode 1
  // also writes the plan, so it is decided once.
  uint64_t v[EPT];
  auto decide = [&]() -> int {
    int64_t local = 0;
#pragma unroll
    for (int e = 0; e < EPT; ++e)
      if (v[e] != ~0ull) local += fixed32(__uint_as_float(0xFFFFFFFFu - (uint32_t)(v[e] >> 32)));
    int64_t tau = ((int64_t)R << 32) + block_exscan_i64(local, red64);  // tau before p0
    int first_stop = 0x7FFFFFFF, firstsent = 0x7FFFFFFF;
    // asynchronous form: first maximum of Theta_q over this thread's q = p + 1
    // (thread 0 also holds q = 0)
    double pbest = -__builtin_inf();
    int pq = 0x7FFFFFFF;
    if (a.mode == 1 && tid == 0) { pbest = theta_here((int64_t)R << 32, 0); pq = 0; }
    bool stopped = false;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int p = p0 + e;
      if (v[e] == ~0ull) { if (firstsent == 0x7FFFFFFF) firstsent = p; stopped = true; }
      if (!stopped) {
        const int64_t tau_next = tau + fixed32(__uint_as_float(0xFFFFFFFFu - (uint32_t)(v[e] >> 32)));
        const double after = theta_here(tau_next, e + 1);
        if (a.mode == 0) {
          const double before = theta_here(tau, e);
          if (!(after > before)) { first_stop = p; stopped = true; }
        } else if (after > pbest) {
          pbest = after;
          pq = p + 1;
        }
        tau = tau_next;
      }
    }
    // number of candidates = position of the first sentinel key
    int E = block_min_i(firstsent, red32);
    if (E > P) E = P;
    int adm;
    if (a.mode == 0) {
      adm = block_min_i(first_stop, red32);
      if (adm > E) adm = E;
    } else {
      const int cap = min(*kin_l, a.N_max);
      adm = max(0, min(cap - R, E));
      block_argmax_first(pbest, pq, reinterpret_cast<double*>(red64), red32);
      if (tid == 0) {
        *a.K_plan = R + pq;
        if (a.theta_plan) *a.theta_plan = pbest;
      }
    }
    return adm;
  };

  // Algorithm 1 first tries the selected prefix of the order; the whole sort
  // (ascending: a descending, then r, then j) runs when that cannot decide,
  // and always for the asynchronous form, whose plan scans every position.
  // Up to four keys per thread with ascending padded runs it is the run
  // merge; otherwise (more keys, or runs out of order) the radix sort, which
  // keeps equal values of a in the buffer's (r, j) order.
  // Algorithm 1 over the selected prefix (at most kSelMax positions, in
  // order in srt): one position per thread, p = tid, so each thread makes a
  // single Theta comparison instead of scanning EPT positions in sequence.
  // Same arithmetic as decide(): Theta before and after admitting p.
  auto decide_prefix = [&](const uint64_t* srt, int n) -> int {
    const int p = tid;
    const bool valid = p < n;
    const uint64_t k = valid ? srt[p] : ~0ull;
    const int64_t fa = valid ? fixed32(__uint_as_float(0xFFFFFFFFu - (uint32_t)(k >> 32))) : 0;
    const int B0 = R + p;
    const double s0 = (valid && B0 <= a.N_max) ? a.sps[B0] : 0.0;
    const double s1 = (valid && B0 + 1 <= a.N_max) ? a.sps[B0 + 1] : 0.0;
    const int64_t tau = ((int64_t)R << 32) + block_exscan_i64(fa, red64);   // tau before p
    int stop = 0x7FFFFFFF;
    if (valid) {
      const double before = (B0 > a.N_max) ? 0.0 : ((double)tau * 0x1p-32) * s0;
      const double after = (B0 + 1 > a.N_max) ? 0.0 : ((double)(tau + fa) * 0x1p-32) * s1;
      if (!(after > before)) stop = p;
    }
    return min(block_min_i(stop, red32), n);
  };

  int admitted = -1;
  if (a.mode == 0) {
    int total = 0;
    const int n = select_sorted_prefix<EPT>(v, keys, P, whist, ssel, sel, red64, &total);
    if (n >= 0) {
      admitted = decide_prefix(reinterpret_cast<const uint64_t*>(whist), n);
      if (admitted >= n && n < total) admitted = -1;   // no stop inside the prefix
    }
  }
  if (admitted < 0) {
    bool merged = false;
    if constexpr (EPT <= 4) {
      if (G2 > 0 && !unsorted) {
        merge_sort_runs<EPT>(v, keys, P, G2);
        merged = true;
      }
    }
    if (!merged) radix_sort_hi32<EPT>(v, keys, whist, scan_lds);
    __syncthreads();
    admitted = decide();
  }

  // ell_r = largest admitted position of request r, by LDS atomics in the
  // (now free) key buffer, then written out
  int* ell_l = reinterpret_cast<int*>(keys);
  for (int r = tid; r < R; r += kSchedThreads) ell_l[r] = 0;
  __syncthreads();
  int64_t mine = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int p = p0 + e;
    if (p < admitted) {
      const uint32_t lo = (uint32_t)v[e];
      atomicMax(&ell_l[lo >> 5], (int)(lo & 31u) + 1);
      mine += fixed32(__uint_as_float(0xFFFFFFFFu - (uint32_t)(v[e] >> 32)));
    }
  }
  if (tid == 0 && a.N_out) *a.N_out = R + admitted;
  // Theta of the admitted prefix (exact integer sum)
  const int64_t tau_adm = ((int64_t)R << 32) + block_sum_i64(mine, red64);   // (has barriers)
  for (int r = tid; r < R; r += kSchedThreads) a.ell[r] = ell_l[r];
  // Theta of the admitted prefix, from the thread whose SPS values reach
  // B = R + admitted
  const int owner = min(admitted / EPT, kSchedThreads - 1);
  if (tid == owner && a.theta) {
    double th = theta_here(tau_adm, 0);
#pragma unroll
    for (int e = 1; e <= EPT; ++e)
      if (p0 + e == admitted) th = theta_here(tau_adm, e);
    *a.theta = th;
  }
}

__global__ __launch_bounds__(kSchedThreads) void k_schedule(SchedArgs a) {
  static_assert(kSchedThreads == kPackThreads, "the pack runs on the scheduler's workgroup");
  __shared__ uint64_t keys[kSchedMaxKeys];
  __shared__ int64_t red64[kSchedThreads / 64];
  __shared__ int red32[kSchedThreads / 64];
  __shared__ int pk_lds[kPackLds];
  // per-wave digit counts of the radix sort; the selection's bins, then its
  // selected and ranked keys
  __shared__ __align__(16) uint32_t whist[kSchedThreads / 64 * 256];
  __shared__ uint64_t ssel[kSelMax];                       // the selection's keys
  __shared__ int sel[8];
  __shared__ int kin_l;
  // K_in is read once, before K_plan (which may be the same address) is written
  if (threadIdx.x == 0) kin_l = (a.mode == 1) ? *a.K_in : 0;
  // runs padded to a power of two up to four keys per thread (the run
  // merge), else packed keys (R gamma <= kSchedMaxKeys, checked by the host)
  int G2 = 1;
  while (G2 < a.gamma) G2 *= 2;
  int n = a.R * G2;
  if (n > 4 * kSchedThreads) { G2 = 0; n = a.R * a.gamma; }
  if (n <= kSchedThreads) schedule_body<1>(a, G2, keys, red64, red32, &kin_l, whist, pk_lds, ssel, sel);
  else if (n <= 2 * kSchedThreads) schedule_body<2>(a, G2, keys, red64, red32, &kin_l, whist, pk_lds, ssel, sel);
  else if (n <= 4 * kSchedThreads) schedule_body<4>(a, G2, keys, red64, red32, &kin_l, whist, pk_lds, ssel, sel);
  else if (n <= 8 * kSchedThreads) schedule_body<8>(a, G2, keys, red64, red32, &kin_l, whist, pk_lds, ssel, sel);
  else schedule_body<16>(a, G2, keys, red64, red32, &kin_l, whist, pk_lds, ssel, sel);
  // verify-batch pack of x with the lengths ell + 1 just decided (every path
  // of the body leaves ell in LDS at the start of the key buffer)
  if (a.pack) {
    __syncthreads();
    // ell in the first R ints of the key buffer; the offsets after them
    // (2 R + 1 <= 2 * 16384 ints of the 32768 the buffer holds, except at R = 16384)
    int* kb = reinterpret_cast<int*>(keys);
    const int* ell_l = kb;
    pack_rows_block(a.pk, [&](int r) { return ell_l[r] + 1; }, pk_lds, kb + a.R,
                    2 * kSchedMaxKeys - a.R);
  }
}

hipError_t launch_schedule(const SchedArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_schedule, dim3(1), dim3(kSchedThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace dspark
