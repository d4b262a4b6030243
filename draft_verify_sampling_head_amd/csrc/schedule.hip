// schedule.hip -- hardware-aware prefix scheduler (one workgroup).
//
// DSpark summary page, Method details ("greedy solution and causality",
// Algorithm 1).  Survival a_{r,j} = prod_{i<=j} c_{r,i} is a left-to-right
// float32 running product per request.  Candidates (r, j) with a > 0 are
// ordered by a descending, then r, then j ascending -- a total order -- by
// sorting 64-bit keys (~bits(a) << 32 | r*32 + j-1) in LDS (bitonic network,
// 1024 threads).  Admitting the q first candidates gives B = R + q and
// tau_q = R + sum of their a; in 2^-32 fixed point the sums are exact, so a
// block-wide prefix sum yields every tau_q at once, and
// Theta_q = (tau_q * 2^-32) * SPS(B) is one double product (0 past N_max).
// The sequential rule "admit while Theta improves, stop at the first
// non-improvement" admits exactly the candidates before the first q with
// Theta_q <= Theta_{q-1}; a block-wide min finds that q.  ell_r is then the
// largest admitted position of request r (admitted positions of a request are
// always a prefix 1..ell_r, because a is non-increasing in j).
#include "launch.hpp"

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

__global__ __launch_bounds__(kSchedThreads) void k_schedule(SchedArgs a) {
  __shared__ uint64_t keys[kSchedMaxKeys];
  __shared__ int64_t red64[kSchedThreads / 64];
  __shared__ int red32[kSchedThreads / 64];
  const int tid = threadIdx.x;
  const int R = a.R, G = a.gamma;
  const int n = R * G;
  int P = 1;
  while (P < n) P <<= 1;

  // survival products (left to right, float32) and sort keys
  int64_t part = 0;
  for (int r = tid; r < R; r += kSchedThreads) {
    float acc = 1.f;
    for (int j = 1; j <= G; ++j) {
      acc = __fmul_rn(acc, a.c[(int64_t)r * G + (j - 1)]);
      if (a.a) a.a[(int64_t)r * G + (j - 1)] = acc;
      keys[r * G + (j - 1)] = (acc > 0.f)
          ? ((uint64_t)(0xFFFFFFFFu - __float_as_uint(acc)) << 32) | (uint32_t)(r * 32 + (j - 1))
          : ~0ull;
      part += fixed32(acc);
    }
  }
  for (int q = n + tid; q < P; q += kSchedThreads) keys[q] = ~0ull;
  __syncthreads();

  if (!a.enabled) {
    const int64_t tau = ((int64_t)R << 32) + block_sum_i64(part, red64);
    for (int r = tid; r < R; r += kSchedThreads) a.ell[r] = G;
    if (tid == 0) {
      const int B = R * (G + 1);
      if (a.N_out) *a.N_out = B;
      if (a.theta) *a.theta = theta_of(tau, B, a.N_max, a.sps);
    }
    return;
  }

  // bitonic sort, ascending keys = a descending, then r, then j
  for (int kk = 2; kk <= P; kk <<= 1) {
    for (int j = kk >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < P; i += kSchedThreads) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const uint64_t x = keys[i], y = keys[ixj];
          const bool up = (i & kk) == 0;
          if ((x > y) == up) { keys[i] = y; keys[ixj] = x; }
        }
      }
      __syncthreads();
    }
  }

  // fixed-point prefix sums over the sorted order; thread t owns positions
  // [t*PT, t*PT + PT)
  const int PT = (P + kSchedThreads - 1) / kSchedThreads;
  const int p0 = tid * PT;
  int64_t local = 0;
  for (int p = p0; p < p0 + PT && p < P; ++p) {
    const uint64_t key = keys[p];
    if (key != ~0ull) local += fixed32(__uint_as_float(0xFFFFFFFFu - (uint32_t)(key >> 32)));
  }
  int64_t tau = ((int64_t)R << 32) + block_exscan_i64(local, red64);  // tau before p0
  int first_stop = 0x7FFFFFFF;
  for (int p = p0; p < p0 + PT && p < P; ++p) {
    const uint64_t key = keys[p];
    if (key == ~0ull) break;
    const int64_t tau_next = tau + fixed32(__uint_as_float(0xFFFFFFFFu - (uint32_t)(key >> 32)));
    const double before = theta_of(tau, R + p, a.N_max, a.sps);
    const double after = theta_of(tau_next, R + p + 1, a.N_max, a.sps);
    if (!(after > before)) { first_stop = p; break; }
    tau = tau_next;
  }
  // number of candidates = position of the first sentinel key
  int firstsent = 0x7FFFFFFF;
  for (int p = p0; p < p0 + PT && p < P; ++p)
    if (keys[p] == ~0ull) { firstsent = p; break; }
  int E = block_min_i(firstsent, red32);
  if (E > P) E = P;
  int admitted = block_min_i(first_stop, red32);
  if (admitted > E) admitted = E;

  for (int r = tid; r < R; r += kSchedThreads) a.ell[r] = 0;
  __threadfence();
  __syncthreads();
  for (int p = tid; p < admitted; p += kSchedThreads) {
    const uint32_t lo = (uint32_t)keys[p];
    atomicMax(&a.ell[lo >> 5], (int)(lo & 31u) + 1);
  }
  if (tid == 0) {
    if (a.N_out) *a.N_out = R + admitted;
  }
  // Theta of the admitted prefix: the thread owning position admitted-1 knows
  // tau there; recompute it from a block sum instead (exact integers).
  int64_t mine = 0;
  for (int p = p0; p < p0 + PT && p < admitted; ++p)
    mine += fixed32(__uint_as_float(0xFFFFFFFFu - (uint32_t)(keys[p] >> 32)));
  const int64_t tau_adm = ((int64_t)R << 32) + block_sum_i64(mine, red64);
  if (tid == 0 && a.theta) *a.theta = theta_of(tau_adm, R + admitted, a.N_max, a.sps);
}

hipError_t launch_schedule(const SchedArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_schedule, dim3(1), dim3(kSchedThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace dspark
