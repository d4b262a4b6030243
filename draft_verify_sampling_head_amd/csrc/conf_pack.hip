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
    int j = lane * W;
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
  float z = lane_dot(h, w, a.d, a.vec_h);
  if (a.rank > 0) {
    int prev = a.x[(int64_t)i * (a.gamma + 1) + (k - 1)];
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
// Exclusive scan of one value per thread over a 1024-thread block; returns
// the thread's prefix and writes the block total to *total.
__device__ inline int block_exclusive_scan(int v, int* lds_waves, int* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(inc, o);
    if (lane >= o) inc += y;
  }
  if (lane == 63) lds_waves[wv] = inc;
  __syncthreads();
  if (wv == 0) {
    int t = (lane < 16) ? lds_waves[lane] : 0;
    int ti = t;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const int y = __shfl_up(ti, o);
      if (lane >= o) ti += y;
    }
    if (lane < 16) lds_waves[16 + lane] = ti - t;
    if (lane == 15) lds_waves[32] = ti;
  }
  __syncthreads();
  const int res = lds_waves[16 + wv] + inc - v;
  *total = lds_waves[32];
  __syncthreads();
  return res;
}

__global__ __launch_bounds__(1024) void k_pack(PackArgs a) {
  __shared__ int lds[40];
  const int tid = threadIdx.x;
  int carry = 0;
  for (int base = 0; base < a.R; base += 1024) {
    const int r = base + tid;
    int l = 0;
    if (r < a.R) {
      l = a.len[r] + a.len_offset;
      if (l < 0 || l > a.width) {
        set_flag(a.status, kFlagBadLen);
        l = l < 0 ? 0 : a.width;
      }
    }
    int tot;
    const int pos = carry + block_exclusive_scan(l, lds, &tot);
    if (r < a.R) {
      a.cu[r] = pos;
      const int32_t* src = a.rows + (int64_t)r * a.width;
      for (int j = 0; j < l; ++j) {
        a.flat[pos + j] = src[j];
        if (a.marker_req) a.marker_req[pos + j] = r;
        if (a.marker_pos) a.marker_pos[pos + j] = j;
      }
    }
    carry += tot;
  }
  // graph-tier padding: the smallest tier that holds the packed total
  int npad = carry;
  if (a.ntiers > 0) {
    int t = -1;
    for (int k = 0; k < a.ntiers; ++k)
      if (a.tiers[k] >= carry) { t = a.tiers[k]; break; }
    if (t < 0) {
      if (tid == 0) set_flag(a.status, kFlagTier);
      t = carry;
    }
    npad = t;
  }
  if (tid == 0) {
    a.cu[a.R] = carry;
    if (a.N_out) *a.N_out = carry;
    if (a.N_pad) *a.N_pad = npad;
  }
  for (int64_t q = carry + tid; q < a.slots; q += 1024) {
    a.flat[q] = q < npad ? a.pad_token : -1;
    if (a.marker_req) a.marker_req[q] = -1;
    if (a.marker_pos) a.marker_pos[q] = -1;
  }
}

hipError_t launch_pack(const PackArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_pack, dim3(1), dim3(1024), 0, st, a);
  return hipGetLastError();
}

}  // namespace dspark
