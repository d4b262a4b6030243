// rnn.hip -- RNN draft head: the recurrent cell that produces the bias features.
//
// DSpark summary page, Method details (RNN head): instead of the first-order
// transition bias W1[x_{k-1}] W2 of the Markov head, a gated recurrent state
// carries the whole in-block prefix.  With z_k = [s_{k-1} ; W1[x_{k-1}] ; h_k]
// (s_0 = 0) and one projection Wr [3r][2r + d] whose row blocks are the gate,
// the candidate and the output parts,
//   g = sigmoid(Wr_g z_k),  s_k = g * s_{k-1} + (1 - g) * tanh(Wr_c z_k),
//   e_k = tanh(Wr_o z_k),   bias_k = W2^T e_k,
// and x_k is sampled from softmax((U_k + bias_k) / T) exactly as for the
// Markov head.  e_k is handed to the W2 contraction in the weights' dtype.
//
// Split of the projection:
//   k_rnn_hproj_mfma : the h part for every block position at once (it does not
//                      depend on the drafted tokens): P = h Wr_h^T, an
//                      (R gamma) x d x 3r bf16 contraction on MFMA with fp32
//                      accumulation (bf16 products are exact in fp32).
//   k_rnn_hproj_valu : the same for float32 operands or unaligned rows.
//   k_rnn_cell       : per step, the recurrent part [s_{k-1} ; W1[x_{k-1}]]
//                      (2r inputs) in fp32 on the VALU, plus P, then the gates,
//                      s_k and e_k.  A workgroup owns 16 requests x 16 state
//                      entries with their gate, candidate and output rows, so
//                      the cell completes locally.
#include <algorithm>

#include "launch.hpp"

namespace dspark {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

namespace {

template <typename T> __device__ __forceinline__ float ld_f(const T* p, int64_t i);
template <> __device__ __forceinline__ float ld_f<float>(const float* p, int64_t i) { return p[i]; }
template <> __device__ __forceinline__ float ld_f<uint16_t>(const uint16_t* p, int64_t i) {
  return __uint_as_float((uint32_t)p[i] << 16);
}

// float32 -> bf16, round to nearest, ties to even (finite inputs; NaN kept quiet)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
template <typename T> __device__ __forceinline__ void st_f(T* p, int64_t i, float v);
template <> __device__ __forceinline__ void st_f<float>(float* p, int64_t i, float v) { p[i] = v; }
template <> __device__ __forceinline__ void st_f<uint16_t>(uint16_t* p, int64_t i, float v) {
  p[i] = f32_to_bf16(v);
}

// ------------------------------------------------------------- h projection
// P[m][q] = sum_t h[m][t] Wr[q][2r + t], m < M = R gamma, q < N = 3r.
// 256 threads, a 64 x 64 output tile; wave w computes the 32 x 32 quarter
// (w >> 1, w & 1) as 2 x 2 tiles of v_mfma_f32_16x16x32_bf16.  Operand lane
// (l & 15, l >> 4) holds row l & 15 of its 16-row tile, k-values 8 (l >> 4) +
// [0, 8) of the 32-wide k-step; result lane (n, g) holds rows 4 g + [0, 4) of
// column n.
constexpr int kHT = 64;

__global__ __launch_bounds__(256) void k_rnn_hproj_mfma(const uint16_t* __restrict__ h,
                                                         const uint16_t* __restrict__ Wr, int M,
                                                         int N, int d, int ldw, int wcol,
                                                         float* __restrict__ P) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int m0 = blockIdx.x * kHT + 32 * (wv >> 1);
  const int n0 = blockIdx.y * kHT + 32 * (wv & 1);
  const int rl = lane & 15, kg = lane >> 4;
  const uint16_t* arow[2];
  const uint16_t* brow[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    arow[t] = h + (int64_t)min(m0 + 16 * t + rl, M - 1) * d + 8 * kg;
    brow[t] = Wr + (int64_t)min(n0 + 16 * t + rl, N - 1) * ldw + wcol + 8 * kg;
  }
  f32x4_t acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const bf16x8_t zero = {};
  const int ksteps = (d + 31) / 32;
  bf16x8_t A[2], B[2], An[2], Bn[2];
  auto load = [&](bf16x8_t (&Ao)[2], bf16x8_t (&Bo)[2], int ks) __attribute__((always_inline)) {
    const bool in = ks * 32 + 8 * kg < d;   // d is a multiple of 8: a group is all in or all out
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      Ao[t] = in ? *reinterpret_cast<const bf16x8_t*>(arow[t] + 32 * ks) : zero;
      Bo[t] = in ? *reinterpret_cast<const bf16x8_t*>(brow[t] + 32 * ks) : zero;
    }
  };
  load(A, B, 0);
  for (int ks = 0; ks < ksteps; ++ks) {
    if (ks + 1 < ksteps) load(An, Bn, ks + 1);
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[a], B[b], acc[a][b], 0, 0, 0);
#pragma unroll
    for (int t = 0; t < 2; ++t) { A[t] = An[t]; B[t] = Bn[t]; }
  }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int n = n0 + 16 * b + rl;
      if (n >= N) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + 16 * a + 4 * kg + i;
        if (m < M) P[(int64_t)m * N + n] = acc[a][b][i];
      }
    }
}

// One wave per output: lanes stride the contraction, then a wave sum.
template <typename HT, typename WT>
__global__ __launch_bounds__(256) void k_rnn_hproj_valu(const HT* __restrict__ h,
                                                         const WT* __restrict__ Wr, int M, int N,
                                                         int d, int ldw, int wcol,
                                                         float* __restrict__ P) {
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * 4;
  for (int64_t o = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); o < (int64_t)M * N; o += nw) {
    const int m = (int)(o / N), q = (int)(o % N);
    const HT* hr = h + (int64_t)m * d;
    const WT* wr = Wr + (int64_t)q * ldw + wcol;
    float acc = 0.f;
    for (int t = lane; t < d; t += 64) acc = fmaf(ld_f(hr, t), ld_f(wr, t), acc);
    acc = wave_sum(acc);
    if (lane == 0) P[o] = acc;
  }
}

// ---------------------------------------------------------------- the cell
// Workgroup (request tile rt, state tile jt): requests 16 rt + [0, 16), state
// entries j = 16 jt + [0, 16).  Thread t: request 16 rt + (t >> 4), entry
// 16 jt + (t & 15); it accumulates the gate, candidate and output rows of its
// entry against its request's recurrent input over the 2r columns, staged
// through LDS in chunks of kKC columns (as fp32).
constexpr int kKC = 64;
constexpr int kKP = kKC + 4;                 // padded LDS row (float4 reads stay conflict-light)

template <typename WT>
__global__ __launch_bounds__(256) void k_rnn_cell(RnnArgs a, int k) {
  __shared__ float Z[16 * kKP];
  __shared__ float W[48 * kKP];
  __shared__ int PV[16];
  const int tid = threadIdx.x;
  const int r = a.rank, nin = 2 * r, ldw = 2 * r + a.d;
  const int req0 = blockIdx.x * 16, j0 = blockIdx.y * 16;
  const int rr = tid >> 4, jj = tid & 15;
  const WT* W1 = reinterpret_cast<const WT*>(a.W1);
  const WT* Wr = reinterpret_cast<const WT*>(a.Wr);
  if (tid < 16) {
    const int req = req0 + tid;
    int prev = 0;
    if (req < a.R) {
      prev = (k == 1) ? a.x0[req] : a.x[(int64_t)req * (a.gamma + 1) + (k - 1)];
      if (prev < 0 || prev >= a.V) { set_flag(a.status, kFlagBadToken); prev = 0; }
    }
    PV[tid] = prev;
  }
  __syncthreads();
  float pg = 0.f, pc = 0.f, po = 0.f;
  for (int q0 = 0; q0 < nin; q0 += kKC) {
    // stage z[16][kKC] and the 48 weight rows [gate | candidate | output] x 16
    for (int idx = tid; idx < 16 * kKC; idx += 256) {
      const int row = idx / kKC, col = idx % kKC, q = q0 + col;
      const int req = req0 + row;
      float v = 0.f;
      if (req < a.R && q < nin) {
        if (q < r) v = (k == 1) ? 0.f : a.state[((int64_t)req * a.gamma + (k - 2)) * r + q];
        else v = ld_f(W1, (int64_t)PV[row] * r + (q - r));
      }
      Z[row * kKP + col] = v;
    }
    for (int idx = tid; idx < 48 * kKC; idx += 256) {
      const int row = idx / kKC, col = idx % kKC, q = q0 + col;
      const int part = row >> 4, j = j0 + (row & 15);
      float v = 0.f;
      if (j < r && q < nin) v = ld_f(Wr, (int64_t)(part * r + j) * ldw + q);
      W[row * kKP + col] = v;
    }
    __syncthreads();
    const float4* zr = reinterpret_cast<const float4*>(Z + rr * kKP);
    const float4* gr = reinterpret_cast<const float4*>(W + jj * kKP);
    const float4* cr = reinterpret_cast<const float4*>(W + (16 + jj) * kKP);
    const float4* orw = reinterpret_cast<const float4*>(W + (32 + jj) * kKP);
#pragma unroll 4
    for (int c = 0; c < kKC / 4; ++c) {
      const float4 z = zr[c], g = gr[c], cc = cr[c], o = orw[c];
      pg = fmaf(g.x, z.x, pg); pg = fmaf(g.y, z.y, pg); pg = fmaf(g.z, z.z, pg); pg = fmaf(g.w, z.w, pg);
      pc = fmaf(cc.x, z.x, pc); pc = fmaf(cc.y, z.y, pc); pc = fmaf(cc.z, z.z, pc); pc = fmaf(cc.w, z.w, pc);
      po = fmaf(o.x, z.x, po); po = fmaf(o.y, z.y, po); po = fmaf(o.z, z.z, po); po = fmaf(o.w, z.w, po);
    }
    __syncthreads();
  }
  const int req = req0 + rr, j = j0 + jj;
  if (req >= a.R || j >= r) return;
  const int64_t pos = (int64_t)req * a.gamma + (k - 1);
  const float* Pr = a.P + pos * 3 * r;
  pg += Pr[j];
  pc += Pr[r + j];
  po += Pr[2 * r + j];
  const float sp = (k == 1) ? 0.f : a.state[(pos - 1) * r + j];
  const float g = 1.f / (1.f + expf(-pg));
  const float s = g * sp + (1.f - g) * tanhf(pc);
  const float e = tanhf(po);
  if (!isfinite(pg) || !isfinite(pc) || !isfinite(po)) set_flag(a.status, kFlagNonFinite);
  a.state[pos * r + j] = s;
  st_f(reinterpret_cast<WT*>(a.feat), pos * r + j, e);
}

}  // namespace

hipError_t launch_rnn_hproj(const RnnArgs& a, hipStream_t st) {
  const int M = a.R * a.gamma, N = 3 * a.rank, ldw = 2 * a.rank + a.d, wcol = 2 * a.rank;
  if (M == 0) return hipSuccess;
  const bool aligned = ((reinterpret_cast<uintptr_t>(a.h) | reinterpret_cast<uintptr_t>(a.Wr)) & 15) == 0;
  if (a.h_bf16 && a.w_bf16 && aligned && (a.d % 8) == 0) {
    hipLaunchKernelGGL(k_rnn_hproj_mfma, dim3((M + kHT - 1) / kHT, (N + kHT - 1) / kHT), dim3(256),
                       0, st, reinterpret_cast<const uint16_t*>(a.h),
                       reinterpret_cast<const uint16_t*>(a.Wr), M, N, a.d, ldw, wcol, a.P);
    return hipGetLastError();
  }
  const int64_t waves = (int64_t)M * N;
  const int grid = (int)std::min<int64_t>(8192, (waves + 3) / 4);
#define DSPARK_HP(HT_, WT_)                                                                        \
  hipLaunchKernelGGL((k_rnn_hproj_valu<HT_, WT_>), dim3(grid), dim3(256), 0, st,                   \
                     reinterpret_cast<const HT_*>(a.h), reinterpret_cast<const WT_*>(a.Wr), M, N,   \
                     a.d, ldw, wcol, a.P)
  if (a.h_bf16 && a.w_bf16) DSPARK_HP(uint16_t, uint16_t);
  else if (a.h_bf16) DSPARK_HP(uint16_t, float);
  else if (a.w_bf16) DSPARK_HP(float, uint16_t);
  else DSPARK_HP(float, float);
#undef DSPARK_HP
  return hipGetLastError();
}

hipError_t launch_rnn_cell(const RnnArgs& a, int k, hipStream_t st) {
  if (a.R == 0) return hipSuccess;
  const dim3 grid((a.R + 15) / 16, (a.rank + 15) / 16);
  if (a.w_bf16) hipLaunchKernelGGL((k_rnn_cell<uint16_t>), grid, dim3(256), 0, st, a, k);
  else hipLaunchKernelGGL((k_rnn_cell<float>), grid, dim3(256), 0, st, a, k);
  return hipGetLastError();
}

}  // namespace dspark
