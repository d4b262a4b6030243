// conf_pack.hip -- confidence head and ragged pack.
//
// Confidence head (DSpark summary page, Method details, confidence head and
// STS calibration): c_k = sigmoid(w^T [h_k ; W1[x_{k-1}]] / t_k).  One wave
// per (request, position): a 16-byte-vectorised dot product of length d + r
// with float32 partial sums and a wave tree reduction.  Bound by reading h.
//
// Ragged pack (DSpark summary page, Supplementary details, variable-length
// routing; CSDN article 3.3, flatten + marker tensors): one workgroup scans
// the lengths (block-wide exclusive scan, 1024 at a time with a carry) and
// scatters every request's tokens to their flattened slots, writing the
// offsets and the (request, position) markers; slots past N are set to -1.
#include "launch.hpp"
#include "pack.hpp"

namespace dspark {

// ------------------------------------------------------------- confidence
template <typename A>
__device__ __forceinline__ int vec_n() { return 16 / (int)sizeof(A); }

template <typename A>
__device__ __forceinline__ void unpack(const A* p, float* o);
template <>
__device__ __forceinline__ void unpack<uint16_t>(const uint16_t* p, float* o) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  o[0] = bf16_lo(u.x); o[1] = bf16_hi(u.x); o[2] = bf16_lo(u.y); o[3] = bf16_hi(u.y);
  o[4] = bf16_lo(u.z); o[5] = bf16_hi(u.z); o[6] = bf16_lo(u.w); o[7] = bf16_hi(u.w);
}
template <>
__device__ __forceinline__ void unpack<float>(const float* p, float* o) {
  const float4 u = *reinterpret_cast<const float4*>(p);
  o[0] = u.x; o[1] = u.y; o[2] = u.z; o[3] = u.w;
}

// Partial dot product of a[0..n) and b[0..n) over this lane's slots; the
// vector path needs both operands 16-byte aligned with the same element size.
template <typename A, typename B>
__device__ __forceinline__ float lane_dot(const A* a, const B* b, int n, bool vec) {
  const int lane = threadIdx.x & 63;
  float acc = 0.f;
  if (vec && sizeof(A) == sizeof(B)) {
    constexpr int W = 16 / sizeof(A);
    constexpr int UNR = 4;                  // 16-byte loads of each operand in flight per lane
    int j = lane * W;
    // four independent accumulators: the loads of four steps are issued
    // together instead of one dependent step at a time
    float part[UNR] = {0.f, 0.f, 0.f, 0.f};
    for (; j + (UNR - 1) * 64 * W + W <= n; j += UNR * 64 * W) {
      float x[UNR][W], y[UNR][W];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        unpack<A>(a + j + u * 64 * W, x[u]);
        unpack<B>(b + j + u * 64 * W, y[u]);
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u)
#pragma unroll
        for (int e = 0; e < W; ++e) part[u] = fmaf(x[u][e], y[u][e], part[u]);
    }
    acc = (part[0] + part[1]) + (part[2] + part[3]);
    for (; j + W <= n; j += 64 * W) {
      float x[W], y[W];
      unpack<A>(a + j, x);
      unpack<B>(b + j, y);
#pragma unroll
      for (int e = 0; e < W; ++e) acc = fmaf(x[e], y[e], acc);
    }
    // tail (n not a multiple of the vector width): the lane that would own it
    if (j < n) for (int e = j; e < n; ++e) acc = fmaf(Elem<A>::get(a, e), Elem<B>::get(b, e), acc);
  } else {
    for (int j = lane; j < n; j += 64) acc = fmaf(Elem<A>::get(a, j), Elem<B>::get(b, j), acc);
  }
  return acc;
}

template <typename HT, typename WT, typename VT>
__global__ __launch_bounds__(256) void k_confidence(ConfArgs a) {
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= a.R * a.gamma) return;
  const int i = item / a.gamma, k = item % a.gamma + 1;
  const HT* h = reinterpret_cast<const HT*>(a.h) + (int64_t)item * a.d;
  const VT* w = reinterpret_cast<const VT*>(a.w);
  // the token x_{k-1} is loaded first: its W1 row's address is then ready
  // when the h part is done
  int prev = a.rank > 0 ? a.x[(int64_t)i * (a.gamma + 1) + (k - 1)] : 0;
  float z = lane_dot(h, w, a.d, a.vec_h);
  if (a.rank > 0) {
    if (prev < 0 || prev >= a.V) { set_flag(a.status, kFlagBadToken); prev = 0; }
    const WT* e = reinterpret_cast<const WT*>(a.W1) + (int64_t)prev * a.rank;
    z += lane_dot(e, w + a.d, a.rank, a.vec_e);
  }
  z = wave_sum(z);
  if ((threadIdx.x & 63) == 0) {
    const float t = a.sts ? a.sts[k - 1] : 1.f;
    a.c[item] = a.logits ? z : 1.f / (1.f + expf(-z / t));
  }
}

hipError_t launch_confidence(const ConfArgs& a, bool h_bf16, bool w1_bf16, bool w_bf16,
                             hipStream_t st) {
  const int grid = (a.R * a.gamma + 3) / 4;
#define DSPARK_CONF(H_, W_, V_) \
  hipLaunchKernelGGL((k_confidence<H_, W_, V_>), dim3(grid), dim3(256), 0, st, a)
  if (h_bf16) {
    if (w1_bf16) { if (w_bf16) DSPARK_CONF(uint16_t, uint16_t, uint16_t); else DSPARK_CONF(uint16_t, uint16_t, float); }
    else         { if (w_bf16) DSPARK_CONF(uint16_t, float, uint16_t);    else DSPARK_CONF(uint16_t, float, float); }
  } else {
    if (w1_bf16) { if (w_bf16) DSPARK_CONF(float, uint16_t, uint16_t);    else DSPARK_CONF(float, uint16_t, float); }
    else         { if (w_bf16) DSPARK_CONF(float, float, uint16_t);       else DSPARK_CONF(float, float, float); }
  }
#undef DSPARK_CONF
  return hipGetLastError();
}

// ------------------------------------------------------------------- pack
constexpr int kPackCuLds = 8192;            // offsets kept in LDS up to R = 8191

__global__ __launch_bounds__(kPackThreads) void k_pack(PackArgs a) {
  __shared__ int lds[kPackLds];
  __shared__ int cu_l[kPackCuLds];
  pack_rows_block(a, [&](int r) { return a.len[r] + a.len_offset; }, lds, cu_l, kPackCuLds);
}

hipError_t launch_pack(const PackArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_pack, dim3(1), dim3(kPackThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace dspark
