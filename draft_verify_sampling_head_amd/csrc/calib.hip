// calib.hip -- sequential temperature scaling (STS) fit of the confidence head.
//
// DSpark summary page, Method details (post-hoc calibration) and the MTP
// survey page, 4.2.3: on held-out blocks the per-position temperatures t_k of
// c_k = sigmoid(z_k / t_k) are fitted left to right, each by a 1-D grid search
// that minimises the expected calibration error (ECE) of the cumulative
// product A_k = prod_{j<=k} c_j against the event "the prefix 1..k was
// accepted", with the earlier positions' temperatures already fixed.
//
// ECE over nbins equal-width bins of [0, 1] (bin = min(floor(A nbins),
// nbins - 1)):  ECE = (1/n) sum_b | sum_{i in b} (A_i - y_i) |.
// Everything is evaluated in double.  Per position k, three launches:
//   k_sts_ece    a (slice, temperature) grid of 128-thread workgroups: each
//                thread accumulates its examples' (A - y) into its own LDS
//                column of bins, the columns are added in a fixed order and
//                the slice's signed bin sums are written out.
//   k_sts_pick   per temperature, the slices' bin sums added in slice order,
//                then |.| summed over bins; the first grid index with the
//                smallest ECE.  Fixed orders throughout: the result does not
//                depend on scheduling.
//   k_sts_apply  A_i *= sigmoid(z_ik / t_k) for the next position.
#include "launch.hpp"

namespace dspark {

constexpr int kStsThreads = 128;

__device__ __forceinline__ double sigmoid_d(double x) { return 1.0 / (1.0 + exp(-x)); }

__global__ __launch_bounds__(kStsThreads) void k_sts_ece(StsArgs a, int k) {
  __shared__ double D[kStsMaxBins * kStsThreads];
  const int tid = threadIdx.x;
  const int sl = blockIdx.x, g = blockIdx.y;
  const double t = (double)a.grid[g];
  const int nb = a.nbins;
  const int per = (a.n + a.S - 1) / a.S;
  const int i0 = sl * per, i1 = min(a.n, i0 + per);
  for (int b = 0; b < nb; ++b) D[b * kStsThreads + tid] = 0.0;
  for (int i = i0 + tid; i < i1; i += kStsThreads) {
    const double prev = (k == 1) ? 1.0 : a.A[i];
    const double A = prev * sigmoid_d((double)a.z[(int64_t)i * a.gamma + (k - 1)] / t);
    int b = (int)floor(A * nb);
    b = b < 0 ? 0 : (b > nb - 1 ? nb - 1 : b);
    D[b * kStsThreads + tid] += A - (a.m[i] >= k ? 1.0 : 0.0);
  }
  __syncthreads();
  if (tid < nb) {
    double s = 0.0;
    for (int q = 0; q < kStsThreads; ++q) s += D[tid * kStsThreads + q];
    a.part[((int64_t)g * nb + tid) * a.S + sl] = s;
  }
}

constexpr int kStsPickThreads = 1024;

__global__ __launch_bounds__(kStsPickThreads) void k_sts_pick(StsArgs a, int k) {
  __shared__ double absb[kStsMaxGrid * kStsMaxBins];
  __shared__ double ece[kStsMaxGrid];
  const int tid = threadIdx.x;
  const int nb = a.nbins;
  // |sum over slices| per (temperature, bin), slices added in order
  for (int p = tid; p < a.G * nb; p += kStsPickThreads) {
    const double* q = a.part + (int64_t)p * a.S;
    double s = 0.0;
    for (int sl = 0; sl < a.S; ++sl) s += q[sl];
    absb[p] = fabs(s);
  }
  __syncthreads();
  if (tid < a.G) {
    double e = 0.0;
    for (int b = 0; b < nb; ++b) e += absb[tid * nb + b];
    ece[tid] = e / (double)a.n;
  }
  __syncthreads();
  if (tid != 0) return;
  int best = 0;
  double be = ece[0];
  for (int q = 1; q < a.G; ++q) {
    if (ece[q] < be) { be = ece[q]; best = q; }
  }
  a.t_out[k - 1] = a.grid[best];
  if (a.ece_out) a.ece_out[k - 1] = be;
}

__global__ __launch_bounds__(256) void k_sts_apply(StsArgs a, int k) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= a.n) return;
  const double t = (double)a.t_out[k - 1];
  const double prev = (k == 1) ? 1.0 : a.A[i];
  a.A[i] = prev * sigmoid_d((double)a.z[(int64_t)i * a.gamma + (k - 1)] / t);
}

hipError_t launch_sts_fit(const StsArgs& a, hipStream_t st) {
  for (int k = 1; k <= a.gamma; ++k) {
    hipLaunchKernelGGL(k_sts_ece, dim3(a.S, a.G), dim3(kStsThreads), 0, st, a, k);
    hipLaunchKernelGGL(k_sts_pick, dim3(1), dim3(kStsPickThreads), 0, st, a, k);
    if (k < a.gamma)
      hipLaunchKernelGGL(k_sts_apply, dim3((a.n + 255) / 256), dim3(256), 0, st, a, k);
  }
  return hipGetLastError();
}

}  // namespace dspark
