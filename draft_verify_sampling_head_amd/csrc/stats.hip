// stats.hip -- per-chunk statistics of logit rows on gfx950.
//
// Every sampler and every normaliser of the round works on per-chunk
// summaries of a vocabulary row (kChunk = 128 consecutive entries):
//   SAMPLE : (M_c, S_c) = (max_{v in c} x_v, sum_{v in c} exp((x_v - M_c)/T)),
//            x the raw score; the chunk log-mass is M_c/T + log S_c
//   GREEDY : (M_c, -) and I_c = the lowest argmax
//   RESID  : (0, sum_{v in c} max(0, p_t(v) - p_d(v)))   (residual mass)
// Two producers:
//   k_row_stats   : streams rows that need no bias (rank-0 draft rows, target
//                   rows of the verify batch).  16-byte loads, a chunk spans
//                   16 lanes (bf16) or 32 lanes (fp32); reductions use DPP row
//                   moves.  HBM-bound.
//   k_markov_mfma : draft / residual rows with the Markov transition bias
//                   W1[x_{k-1}] W2 (DSpark summary page, Method details, Markov
//                   head).  The bias block of 32 vocabulary entries x 32 rows
//                   is one v_mfma_f32_32x32x16_bf16 chain over the rank; the
//                   accumulator is seeded with U so the bias add is free; the
//                   vocabulary is the MFMA M dimension, arranged so each lane
//                   ends with 16 consecutive entries of one row.
//   k_markov_valu : the same with float32 weights on the vector ALU.
#include "launch.hpp"
#include "sampling.hpp"

namespace dspark {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// ===================================================================== rows
template <typename T>
__device__ __forceinline__ void load_vec(const T* p, float* out);
template <>
__device__ __forceinline__ void load_vec<uint16_t>(const uint16_t* p, float* out) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  out[0] = bf16_lo(u.x); out[1] = bf16_hi(u.x); out[2] = bf16_lo(u.y); out[3] = bf16_hi(u.y);
  out[4] = bf16_lo(u.z); out[5] = bf16_hi(u.z); out[6] = bf16_lo(u.w); out[7] = bf16_hi(u.w);
}
template <>
__device__ __forceinline__ void load_vec<float>(const float* p, float* out) {
  const float4 u = *reinterpret_cast<const float4*>(p);
  out[0] = u.x; out[1] = u.y; out[2] = u.z; out[3] = u.w;
}

template <int LPC>
__device__ __forceinline__ float chunk_max(float v) {
  v = row16_max(v);
  if (LPC == 32) v = fmaxf(v, __shfl_xor(v, 16));
  return v;
}
template <int LPC>
__device__ __forceinline__ float chunk_sum(float v) {
  v = row16_sum(v);
  if (LPC == 32) v += __shfl_xor(v, 16);
  return v;
}
template <int LPC>
__device__ __forceinline__ void chunk_argmax(float& v, int& i) {
  row16_argmax(v, i);
  if (LPC == 32) argmax_merge(v, i, __shfl_xor(v, 16), __shfl_xor(i, 16));
}

// One wave: chunks [c0, c1) of one row.
template <typename T, bool GREEDY>
__device__ __forceinline__ void row_segment(const T* row, int V, int c0, int c1, float scale2,
                                            bool vec_ok, float2* L, int* I, uint32_t* status) {
  constexpr int VPL = 16 / sizeof(T);       // values per lane per 16-byte load
  constexpr int LPC = kChunk / VPL;         // lanes per chunk
  constexpr int CPI = 64 / LPC;             // chunks per wave-wide load
  constexpr int UNR = 4;                    // loads in flight per lane
  const int lane = threadIdx.x & 63;
  const int sub = lane % LPC;
  const int cl = lane / LPC;
  for (int cb = c0; cb < c1; cb += CPI * UNR) {
    float x[UNR][VPL];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int c = cb + u * CPI + cl;
      const int v0 = c * kChunk + sub * VPL;
      if (c < c1 && vec_ok && v0 + VPL <= V) {
        load_vec<T>(row + v0, x[u]);
      } else {
#pragma unroll
        for (int e = 0; e < VPL; ++e)
          x[u][e] = (c < c1 && v0 + e < V) ? Elem<T>::get(row, v0 + e) : -INFINITY;
      }
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int c = cb + u * CPI + cl;
      const int v0 = c * kChunk + sub * VPL;
      if (GREEDY) {
        float bv = -INFINITY;
        int bi = 0x7FFFFFFF;
#pragma unroll
        for (int e = 0; e < VPL; ++e)
          if (x[u][e] > bv) { bv = x[u][e]; bi = v0 + e; }
        chunk_argmax<LPC>(bv, bi);
        if (sub == 0 && c < c1) {
          L[c] = make_float2(bv, 0.f);
          I[c] = bi;
          if (!(fabsf(bv) <= 3.0e38f)) set_flag(status, kFlagNonFinite);
        }
      } else {
        float m = -INFINITY;
#pragma unroll
        for (int e = 0; e < VPL; ++e) m = fmaxf(m, x[u][e]);
        m = chunk_max<LPC>(m);
        float s = 0.f;
        if (m != -INFINITY) {
#pragma unroll
          for (int e = 0; e < VPL; ++e) s += __builtin_amdgcn_exp2f((x[u][e] - m) * scale2);
        }
        s = chunk_sum<LPC>(s);
        if (sub == 0 && c < c1) {
          L[c] = make_float2(m, s);
          if (!(s <= 3.0e38f) || m == INFINITY) set_flag(status, kFlagNonFinite);
        }
      }
    }
  }
}

template <typename T, bool GREEDY>
__global__ __launch_bounds__(256) void k_row_stats(RowStatsArgs a) {
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nwaves = gridDim.x * 4;
  if (a.zero_me && blockIdx.x == 0 && threadIdx.x == 0) *a.zero_me = 0u;
  int nrows = a.nrows_cap;
  if (a.kind != kRowsDraft) nrows = min(nrows, a.cu[a.R]);
  const int64_t items = (int64_t)nrows * a.segs;
  for (int64_t it = wave; it < items; it += nwaves) {
    const int q = (int)(it / a.segs);
    const int seg = (int)(it % a.segs);
    int64_t row;
    if (a.kind == kRowsDraft) {
      row = (int64_t)q * a.gamma + (a.k - 1);
    } else if (a.kind == kRowsVerifyPacked) {
      row = q;
    } else {
      int lo = 0, hi = a.R - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.cu[mid] <= q) lo = mid; else hi = mid - 1;
      }
      row = (int64_t)lo * (a.gamma + 1) + (q - a.cu[lo]);
    }
    const T* rp = reinterpret_cast<const T*>(a.base) + row * a.V;
    const int c0 = seg * a.cps, c1 = min(a.nch, c0 + a.cps);
    const int64_t o = (int64_t)q * a.nch;
    row_segment<T, GREEDY>(rp, a.V, c0, c1, a.scale2, a.vec_ok, a.L + o, a.I + o, a.status);
  }
}

// ==================================================================== MFMA
template <typename T>
__device__ __forceinline__ void load16(const T* p, bool vec, int v0, int V, float* out) {
  // 16 consecutive values starting at p[v0]; -inf past V
  if (vec && v0 + 16 <= V) {
    load_vec<T>(p + v0, out);
    load_vec<T>(p + v0 + 16 / sizeof(T) * 1, out + 16 / sizeof(T));
    if (sizeof(T) == 4) {
      load_vec<T>(p + v0 + 8, out + 8);
      load_vec<T>(p + v0 + 12, out + 12);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 16; ++e) out[e] = (v0 + e < V) ? Elem<T>::get(p, v0 + e) : -INFINITY;
  }
}

template <typename UT, int KS, int MODE>
__global__ __launch_bounds__(256) void k_markov_mfma(MarkovArgs a) {
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int b = blockIdx.x;
  const int xcd = b & 7, s = b >> 3;
  const int rtg = s % a.nrtg;
  const int cg = (s / a.nrtg) * 8 + xcd;
  const int rt = rtg * 4 + wv;
  if (cg >= a.ncg || rt >= a.nrt) return;
  int nrows = a.R;
  if (MODE == kModeResid) nrows = *a.rej_count;
  if (rt * 32 >= nrows) return;

  const int n = lane & 31, half = lane >> 5;
  const int row = rt * 32 + n;
  const bool valid = row < nrows;
  int req = 0, kk = a.k, trow = 0, qrow = 0;
  if (valid && MODE == kModeResid) {
    const int4 e = a.rej[row];
    req = e.x; kk = e.y; trow = e.z; qrow = e.w;
  } else if (valid) {
    req = row;
  }
  int prev = 0;
  if (valid) {
    prev = (MODE != kModeResid && kk == 1) ? a.x0[req]
                                           : a.x[(int64_t)req * (a.gamma + 1) + (kk - 1)];
    if (prev < 0 || prev >= a.V) { set_flag(a.status, kFlagBadToken); prev = 0; }
  }
  const UT* urow = reinterpret_cast<const UT*>(a.U) + ((int64_t)req * a.gamma + (kk - 1)) * a.V;
  const UT* tptr = reinterpret_cast<const UT*>(a.target) + (int64_t)trow * a.V;
  float mt = 0.f, lrt2 = 0.f, lse_d = 0.f;
  if (MODE == kModeResid && valid) {
    const float2 nt = a.lse_t[qrow];
    mt = nt.x;
    lrt2 = nt.y * kLog2e;
    lse_d = a.lse_d[(int64_t)req * a.gamma + (kk - 1)];
  }
  const float invT = a.scale2 * kLn2;

  // B operand: the gathered embedding rows, held for the whole wave
  const int nks = a.rank >> 4;
  bf16x8_t Bf[KS];
  const uint16_t* erow = a.W1 + (int64_t)prev * a.rank + half * 8;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    bf16x8_t z = {};
    Bf[ks] = (valid && ks < nks) ? *reinterpret_cast<const bf16x8_t*>(erow + ks * 16) : z;
  }
  // A operand row of this lane: vocabulary offset inside a 32-entry tile such
  // that accumulator j of lane (n, half) is entry 16*half + j.
  const int m = lane & 31;
  const int voff = 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3);

  const int c0 = cg * a.cg, c1 = min(a.nch, c0 + a.cg);
  for (int c = c0; c < c1; ++c) {
    f32x16_t acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float u[16];
      const int vb = c * kChunk + t * 32 + 16 * half;
      if (valid) load16<UT>(urow, a.u_vec_ok, vb, a.V, u);
      else {
#pragma unroll
        for (int e = 0; e < 16; ++e) u[e] = -INFINITY;
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[t][e] = u[e];
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int va = c * kChunk + t * 32 + voff;
      const uint16_t* arow = a.W2t + (int64_t)va * a.rank + half * 8;
      const bool ok = va < a.V;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks < nks) {
          bf16x8_t z = {};
          const bf16x8_t A = ok ? *reinterpret_cast<const bf16x8_t*>(arow + ks * 16) : z;
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, Bf[ks], acc[t], 0, 0, 0);
        }
      }
    }
    // ---- epilogue: lane (n, half) holds entries c*128 + 32t + 16*half + j of row n
    const int64_t o = (int64_t)row * a.nch + c;
    if (MODE == kModeGreedy) {
      float bv = -INFINITY;
      int bi = 0x7FFFFFFF;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (acc[t][j] > bv) { bv = acc[t][j]; bi = c * kChunk + t * 32 + 16 * half + j; }
      argmax_merge(bv, bi, __shfl_xor(bv, 32), __shfl_xor(bi, 32));
      if (half == 0 && valid) {
        a.L[o] = make_float2(bv, 0.f);
        a.I[o] = bi;
        if (!(fabsf(bv) <= 3.0e38f)) set_flag(a.status, kFlagNonFinite);
      }
    } else if (MODE == kModeSample) {
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, acc[t][j]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      float sm = 0.f;
      if (mx != -INFINITY) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int j = 0; j < 16; ++j) sm += __builtin_amdgcn_exp2f((acc[t][j] - mx) * a.scale2);
      }
      sm += __shfl_xor(sm, 32);
      if (half == 0 && valid) {
        a.L[o] = make_float2(mx, sm);
        if (!(sm <= 3.0e38f) || mx == INFINITY) set_flag(a.status, kFlagNonFinite);
      }
    } else {  // residual mass max(0, p_t - p_d) per chunk
      float sm = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        float tv[16];
        const int vb = c * kChunk + t * 32 + 16 * half;
        if (valid) load16<UT>(tptr, a.u_vec_ok, vb, a.V, tv);
        else {
#pragma unroll
          for (int e = 0; e < 16; ++e) tv[e] = -INFINITY;
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float pt = __builtin_amdgcn_exp2f((tv[j] - mt) * a.scale2 - lrt2);
          const float pd = __builtin_amdgcn_exp2f((acc[t][j] * invT - lse_d) * kLog2e);
          sm += fmaxf(pt - pd, 0.f);
        }
      }
      sm += __shfl_xor(sm, 32);
      if (half == 0 && valid) {
        a.L[o] = make_float2(0.f, sm);
        if (!(sm <= 3.0e38f)) set_flag(a.status, kFlagNonFinite);
      }
    }
  }
}

// ==================================================================== VALU
// Float32 weights: one wave per (row, chunk); lane l owns entries c*128 + l
// and c*128 + 64 + l.
template <typename UT, typename WT, int MODE>
__global__ __launch_bounds__(256) void k_markov_valu(MarkovArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nwaves = gridDim.x * 4;
  int nrows = a.R;
  if (MODE == kModeResid) nrows = *a.rej_count;
  const int64_t items = (int64_t)nrows * a.nch;
  const WT* W1 = reinterpret_cast<const WT*>(a.W1v);
  const WT* W2t = reinterpret_cast<const WT*>(a.W2tv);
  for (int64_t it = wave; it < items; it += nwaves) {
    const int row = (int)(it / a.nch);
    const int c = (int)(it % a.nch);
    int req = row, kk = a.k, trow = 0, qrow = 0;
    if (MODE == kModeResid) {
      const int4 e = a.rej[row];
      req = e.x; kk = e.y; trow = e.z; qrow = e.w;
    }
    int prev = (MODE != kModeResid && kk == 1) ? a.x0[req]
                                               : a.x[(int64_t)req * (a.gamma + 1) + (kk - 1)];
    if (prev < 0 || prev >= a.V) { set_flag(a.status, kFlagBadToken); prev = 0; }
    const UT* urow = reinterpret_cast<const UT*>(a.U) + ((int64_t)req * a.gamma + (kk - 1)) * a.V;
    const WT* erow = W1 + (int64_t)prev * a.rank;
    float sv[2];
    int vv[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int v = c * kChunk + h * 64 + lane;
      vv[h] = v;
      sv[h] = -INFINITY;
      if (v < a.V) {
        const float bias = a.rank > 0 ? markov_bias(erow, W2t, a.rank, v) : 0.f;
        sv[h] = Elem<UT>::get(urow, v) + bias;
      }
    }
    const int64_t o = (int64_t)row * a.nch + c;
    if (MODE == kModeGreedy) {
      float bv = sv[0];
      int bi = sv[0] == -INFINITY ? 0x7FFFFFFF : vv[0];
      argmax_merge(bv, bi, sv[1], sv[1] == -INFINITY ? 0x7FFFFFFF : vv[1]);
      wave_argmax(bv, bi);
      if (lane == 0) { a.L[o] = make_float2(bv, 0.f); a.I[o] = bi; }
    } else if (MODE == kModeSample) {
      const float mx = wave_max(fmaxf(sv[0], sv[1]));
      float sm = 0.f;
      if (mx != -INFINITY)
        sm = __builtin_amdgcn_exp2f((sv[0] - mx) * a.scale2) +
             __builtin_amdgcn_exp2f((sv[1] - mx) * a.scale2);
      sm = wave_sum(sm);
      if (lane == 0) {
        a.L[o] = make_float2(mx, sm);
        if (!(sm <= 3.0e38f) || mx == INFINITY) set_flag(a.status, kFlagNonFinite);
      }
    } else {
      const UT* tptr = reinterpret_cast<const UT*>(a.target) + (int64_t)trow * a.V;
      const float2 nt = a.lse_t[qrow];
      const float lse_d = a.lse_d[(int64_t)req * a.gamma + (kk - 1)];
      const float invT = a.scale2 * kLn2;
      float sm = 0.f;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (vv[h] < a.V) {
          const float pt = __builtin_amdgcn_exp2f((Elem<UT>::get(tptr, vv[h]) - nt.x) * a.scale2
                                                  - nt.y * kLog2e);
          const float pd = __builtin_amdgcn_exp2f((sv[h] * invT - lse_d) * kLog2e);
          sm += fmaxf(pt - pd, 0.f);
        }
      }
      sm = wave_sum(sm);
      if (lane == 0) a.L[o] = make_float2(0.f, sm);
    }
  }
}

// ================================================================ launches
static int grid_for(int64_t waves) {
  int64_t b = (waves + 3) / 4;
  if (b > 4096) b = 4096;
  if (b < 1) b = 1;
  return (int)b;
}

hipError_t launch_row_stats(const RowStatsArgs& a0, bool bf16, bool greedy, hipStream_t st) {
  RowStatsArgs a = a0;
  const int vpl = bf16 ? 8 : 4;
  (void)vpl;
  a.cps = 16;
  a.segs = (a.nch + a.cps - 1) / a.cps;
  const int grid = grid_for((int64_t)a.nrows_cap * a.segs);
  if (bf16) {
    if (greedy) hipLaunchKernelGGL((k_row_stats<uint16_t, true>), dim3(grid), dim3(256), 0, st, a);
    else hipLaunchKernelGGL((k_row_stats<uint16_t, false>), dim3(grid), dim3(256), 0, st, a);
  } else {
    if (greedy) hipLaunchKernelGGL((k_row_stats<float, true>), dim3(grid), dim3(256), 0, st, a);
    else hipLaunchKernelGGL((k_row_stats<float, false>), dim3(grid), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

template <typename UT, int MODE>
static void launch_mfma_ks(MarkovArgs& a, int grid, hipStream_t st) {
  const int nks = a.rank / 16;
  if (nks <= 4) hipLaunchKernelGGL((k_markov_mfma<UT, 4, MODE>), dim3(grid), dim3(256), 0, st, a);
  else if (nks <= 8) hipLaunchKernelGGL((k_markov_mfma<UT, 8, MODE>), dim3(grid), dim3(256), 0, st, a);
  else if (nks <= 16) hipLaunchKernelGGL((k_markov_mfma<UT, 16, MODE>), dim3(grid), dim3(256), 0, st, a);
  else hipLaunchKernelGGL((k_markov_mfma<UT, 32, MODE>), dim3(grid), dim3(256), 0, st, a);
}

hipError_t launch_markov_stats(const MarkovArgs& a0, bool u_bf16, bool w_bf16, int mode,
                               hipStream_t st) {
  MarkovArgs a = a0;
  if (w_bf16) {
    a.W1 = reinterpret_cast<const uint16_t*>(a.W1v);
    a.W2t = reinterpret_cast<const uint16_t*>(a.W2tv);
    a.nrt = (a.nrows_cap + 31) / 32;
    a.nrtg = (a.nrt + 3) / 4;
    // chunks per wave: aim at about four waves per SIMD across the chip
    const int64_t target_waves = 4096;
    int cgw = (int)(((int64_t)a.nrt * a.nch + target_waves - 1) / target_waves);
    if (cgw < 1) cgw = 1;
    a.cg = cgw;
    a.ncg = (a.nch + cgw - 1) / cgw;
    const int grid = a.nrtg * ((a.ncg + 7) / 8) * 8;
    if (u_bf16) {
      if (mode == kModeSample) launch_mfma_ks<uint16_t, kModeSample>(a, grid, st);
      else if (mode == kModeGreedy) launch_mfma_ks<uint16_t, kModeGreedy>(a, grid, st);
      else launch_mfma_ks<uint16_t, kModeResid>(a, grid, st);
    } else {
      if (mode == kModeSample) launch_mfma_ks<float, kModeSample>(a, grid, st);
      else if (mode == kModeGreedy) launch_mfma_ks<float, kModeGreedy>(a, grid, st);
      else launch_mfma_ks<float, kModeResid>(a, grid, st);
    }
  } else {
    const int grid = grid_for((int64_t)a.nrows_cap * a.nch);
#define DSPARK_VALU(UT_, M_) \
    hipLaunchKernelGGL((k_markov_valu<UT_, float, M_>), dim3(grid), dim3(256), 0, st, a)
    if (u_bf16) {
      if (mode == kModeSample) DSPARK_VALU(uint16_t, kModeSample);
      else if (mode == kModeGreedy) DSPARK_VALU(uint16_t, kModeGreedy);
      else DSPARK_VALU(uint16_t, kModeResid);
    } else {
      if (mode == kModeSample) DSPARK_VALU(float, kModeSample);
      else if (mode == kModeGreedy) DSPARK_VALU(float, kModeGreedy);
      else DSPARK_VALU(float, kModeResid);
    }
#undef DSPARK_VALU
  }
  return hipGetLastError();
}

}  // namespace dspark
