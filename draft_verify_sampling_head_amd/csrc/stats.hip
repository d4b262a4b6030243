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
#include <type_traits>

#include "launch.hpp"
#include "sampling.hpp"

namespace dspark {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Row of the bias-feature table that multiplies W2 for (request req, block
// position kk).  Markov head: W1[x_{kk-1}] (x_0 the anchor, read from x0 when
// use_x0 is set and kk == 1; a token outside the vocabulary is flagged and
// replaced by 0).  With feat_rows the table is the per-position feature tensor
// [R][gamma][rank] of the RNN head and the row is req * gamma + kk - 1.
__device__ __forceinline__ int bias_row_index(const MarkovArgs& a, int req, int kk, bool use_x0) {
  if (a.feat_rows) return req * a.gamma + (kk - 1);
  int prev = (use_x0 && kk == 1) ? a.x0[req] : a.x[(int64_t)req * (a.gamma + 1) + (kk - 1)];
  if (prev < 0 || prev >= a.V) { set_flag(a.status, kFlagBadToken); prev = 0; }
  return prev;
}

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

constexpr int kCuLds = 2048;               // verify offsets staged in LDS up to this many

template <typename T, bool GREEDY>
__global__ __launch_bounds__(256) void k_row_stats(RowStatsArgs a) {
  __shared__ int cus[kCuLds];
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nwaves = gridDim.x * 4;
  if (a.zero_me && blockIdx.x == 0 && threadIdx.x == 0) *a.zero_me = 0u;
  int nrows = a.nrows_cap;
  if (a.kind != kRowsDraft && a.kind != kRowsAll) nrows = min(nrows, a.cu[a.R]);
  // dense verify rows: the row of packed index q is found by binary search
  // over the offsets, staged in LDS when they fit
  const bool lds_cu = a.kind == kRowsVerifyDense && a.R + 1 <= kCuLds;
  if (lds_cu) {
    for (int t = threadIdx.x; t <= a.R; t += 256) cus[t] = a.cu[t];
    __syncthreads();
  }
  // (the two offset arrays are read on separate paths: a pointer that may
  // point at either LDS or global memory would turn every read into a flat load)
  const int64_t items = (int64_t)nrows * a.segs;
  for (int64_t it = wave; it < items; it += nwaves) {
    const int q = (int)(it / a.segs);
    const int seg = (int)(it % a.segs);
    int64_t row;
    if (a.kind == kRowsDraft) {
      row = (int64_t)q * a.gamma + (a.k - 1);
    } else if (a.kind == kRowsVerifyPacked || a.kind == kRowsAll) {
      row = q;
    } else {
      int lo = 0, hi = a.R - 1, base;
      if (lds_cu) {
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (cus[mid] <= q) lo = mid; else hi = mid - 1;
        }
        base = cus[lo];
      } else {
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (a.cu[mid] <= q) lo = mid; else hi = mid - 1;
        }
        base = a.cu[lo];
      }
      row = (int64_t)lo * (a.gamma + 1) + (q - base);
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

// 16 consecutive logits of one row kept as raw words until they seed an
// accumulator (bf16: 8 dwords, fp32: 16 dwords); -inf past the vocabulary.
template <typename UT> struct URaw;
template <> struct URaw<uint16_t> {
  uint4 w[2];
  __device__ __forceinline__ void fetch(const uint16_t* p, int v0, int V, bool vec, bool valid) {
    if (valid && vec && v0 + 16 <= V) {
      w[0] = *reinterpret_cast<const uint4*>(p + v0);
      w[1] = *reinterpret_cast<const uint4*>(p + v0 + 8);
    } else {
      uint32_t d[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t lo = (valid && v0 + 2 * e < V) ? p[v0 + 2 * e] : 0xFF80u;
        const uint32_t hi = (valid && v0 + 2 * e + 1 < V) ? p[v0 + 2 * e + 1] : 0xFF80u;
        d[e] = lo | (hi << 16);
      }
      w[0] = make_uint4(d[0], d[1], d[2], d[3]);
      w[1] = make_uint4(d[4], d[5], d[6], d[7]);
    }
  }
  __device__ __forceinline__ void unpack(f32x16_t& acc) const {
    const uint32_t d[8] = {w[0].x, w[0].y, w[0].z, w[0].w, w[1].x, w[1].y, w[1].z, w[1].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc[2 * e] = bf16_lo(d[e]);
      acc[2 * e + 1] = bf16_hi(d[e]);
    }
  }
};
template <> struct URaw<float> {
  float4 w[4];
  __device__ __forceinline__ void fetch(const float* p, int v0, int V, bool vec, bool valid) {
    if (valid && vec && v0 + 16 <= V) {
#pragma unroll
      for (int q = 0; q < 4; ++q) w[q] = *reinterpret_cast<const float4*>(p + v0 + 4 * q);
    } else {
      float d[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) d[e] = (valid && v0 + e < V) ? p[v0 + e] : -INFINITY;
#pragma unroll
      for (int q = 0; q < 4; ++q) w[q] = make_float4(d[4 * q], d[4 * q + 1], d[4 * q + 2], d[4 * q + 3]);
    }
  }
  __device__ __forceinline__ void unpack(f32x16_t& acc) const {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[4 * q] = w[q].x; acc[4 * q + 1] = w[q].y; acc[4 * q + 2] = w[q].z; acc[4 * q + 3] = w[q].w;
    }
  }
};

// LDS slot swizzle of a W2t tile row: spreads the 16-byte segments read by one
// ds_read_b128 over distinct banks for the MFMA A-operand row order below.
__device__ __forceinline__ int seg_swizzle(int r) { return (r & 7) | (((r >> 4) & 1) << 3); }

// Markov statistics kernel.  One workgroup = 4 waves = 256 rows (each wave 64
// rows as two 32-row MFMA column tiles, their gathered W1 rows held as B
// operands for the whole kernel) x a contiguous range of vocabulary chunks.
// The W2t tile (32 vocabulary rows x rank) of each step is loaded once per
// workgroup into a double-buffered LDS ring (loads two tiles ahead) and read
// by every wave as MFMA A operands; U is prefetched two tiles ahead and seeds
// the accumulators; the epilogue of tile t-1 is issued after the MFMAs of
// tile t so the vector ALU work overlaps the matrix pipe.
template <typename UT, int KS, int MODE>
__global__ __launch_bounds__(256) void k_markov_mfma_reg(MarkovArgs a) {
  constexpr int SEGMAX = 2 * KS;                    // 16-byte segments per W2t row
  constexpr int NLD = (32 * SEGMAX + 255) / 256;    // staging loads per thread per tile
  __shared__ u32x4_t lds[2][32 * SEGMAX];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int b = blockIdx.x;
  const int xcd = b & 7, sb = b >> 3;
  const int rg = sb % a.nrg;
  const int cg = (sb / a.nrg) * 8 + xcd;
  if (cg >= a.ncg) return;
  int nrows = a.R;
  if (MODE == kModeResid) nrows = *a.rej_count;
  if (rg * 256 >= nrows) return;
  const int c0 = cg * a.cg, c1 = min(a.nch, c0 + a.cg);
  const int T = (c1 - c0) * 4;
  const int vbase = c0 * kChunk;
  const int nseg = a.rank >> 3, nks = a.rank >> 4;   // nks <= KS
  const int smask = ((nseg & (nseg - 1)) == 0) ? min(nseg, 16) - 1 : 0;
  const bool wave_active = rg * 256 + wv * 64 < nrows;

  // ---- the two rows of this lane (column n of each 32-row tile)
  const int n = lane & 31, half = lane >> 5;
  bool valid[2];
  const UT* urow[2];
  const UT* trow[2];
  int prevs[2];
  float mt[2], lrt2[2], lse_d[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int row = rg * 256 + wv * 64 + nt * 32 + n;
    valid[nt] = row < nrows;
    int req = 0, kk = a.k, tr = 0, qr = 0;
    if (valid[nt]) {
      if (MODE == kModeResid) {
        const int4 e = a.rej[row];
        req = e.x; kk = e.y; tr = e.z; qr = e.w;
      } else {
        req = row;
      }
    }
    int prev = 0;
    if (valid[nt]) prev = bias_row_index(a, req, kk, MODE != kModeResid);
    prevs[nt] = prev;
    urow[nt] = reinterpret_cast<const UT*>(a.U) + ((int64_t)req * a.gamma + (kk - 1)) * a.V;
    trow[nt] = reinterpret_cast<const UT*>(a.target) + (int64_t)tr * a.V;
    mt[nt] = 0.f; lrt2[nt] = 0.f; lse_d[nt] = 0.f;
    if (MODE == kModeResid && valid[nt]) {
      const float2 nrm = a.lse_t[qr];
      mt[nt] = nrm.x;
      lrt2[nt] = nrm.y * kLog2e;
      lse_d[nt] = a.lse_d[(int64_t)req * a.gamma + (kk - 1)];
    }
  }
  // ---- B operands: gathered W1 rows for both column tiles, whole kernel
  bf16x8_t Bf[2][KS];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const uint16_t* erow = a.W1 + (int64_t)prevs[nt] * a.rank + half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8_t z = {};
      Bf[nt][ks] = (valid[nt] && ks < nks) ? *reinterpret_cast<const bf16x8_t*>(erow + ks * 16) : z;
    }
  }
  // A operand row of this lane inside a 32-entry tile, ordered so that
  // accumulator j of lane (n, half) is vocabulary entry 16*half + j.
  const int m = lane & 31;
  const int arow = 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3);
  const int aswz = seg_swizzle(arow) & smask;

  // ---- staging of W2t tiles: thread tid owns segments tid + 256*i
  u32x4_t st[2][NLD];
  const int tile_segs = 32 * nseg;
  // every staging load is unconditional (clamped address) so that the staged
  // values stay in registers and their waits can be deferred to the LDS store
  auto stage_load = [&](u32x4_t (&dst)[NLD], int t) __attribute__((always_inline)) {
    const int vb = vbase + t * 32;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int j = min(tid + 256 * i, tile_segs - 1);
      const int r = j / nseg, p = j - r * nseg;
      const int q = p ^ (seg_swizzle(r) & smask);
      const int v = min(vb + r, a.V - 1);
      dst[i] = *reinterpret_cast<const u32x4_t*>(a.W2t + (int64_t)v * a.rank + q * 8);
    }
  };
  auto stage_store = [&](const u32x4_t (&src)[NLD], int P) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int j = tid + 256 * i;
      if (j < tile_segs) {
        const int r = j / nseg;
        lds[P][r * SEGMAX + (j - r * nseg)] = src[i];
      }
    }
  };
  // a rank below 16*KS leaves segments [nseg, SEGMAX) of every LDS row unused:
  // zero them once so the padded MFMA steps (B is zero there too) add nothing
  if (nseg < SEGMAX) {
    const u32x4_t z = {0u, 0u, 0u, 0u};
    for (int j = tid; j < 2 * 32 * SEGMAX; j += 256) {
      const int r = j / SEGMAX;
      if (j - r * SEGMAX >= nseg) lds[r >> 5][(r & 31) * SEGMAX + (j - r * SEGMAX)] = z;
    }
  }

  // ---- epilogue state
  float Mr[2], Sr[2], Ms2[2];   // sample: running max, sum relative to Ms2, max * scale2 (rounded)
  int Ir[2];                    // greedy argmax
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) { Mr[nt] = -INFINITY; Sr[nt] = 0.f; Ms2[nt] = -INFINITY; Ir[nt] = 0x7FFFFFFF; }
  const float s2 = a.scale2;
  const float invT = s2 * kLn2;

  auto epilogue = [&](f32x16_t (&acc)[2], int t) __attribute__((always_inline)) {
    const int vt = vbase + t * 32 + 16 * half;   // entry of accumulator 0
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      if (MODE == kModeGreedy) {
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (acc[nt][j] > Mr[nt]) { Mr[nt] = acc[nt][j]; Ir[nt] = vt + j; }
      } else if (MODE == kModeSample) {
        float tm = acc[nt][0];
#pragma unroll
        for (int j = 1; j < 16; ++j) tm = fmaxf(tm, acc[nt][j]);
        if (tm != -INFINITY) {
          if (tm > Mr[nt]) {
            const float nms2 = tm * s2;
            Sr[nt] *= __builtin_amdgcn_exp2f(Ms2[nt] - nms2);   // keeps a NaN sum NaN
            Mr[nt] = tm;
            Ms2[nt] = nms2;
          }
          float acc_s = 0.f;
#pragma unroll
          for (int j = 0; j < 16; ++j) acc_s += __builtin_amdgcn_exp2f(fmaf(acc[nt][j], s2, -Ms2[nt]));
          Sr[nt] += acc_s;
        }
      } else {
        float tv[16];
        load16<UT>(trow[nt], a.u_vec_ok && valid[nt], vt, valid[nt] ? a.V : 0, tv);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float pt = __builtin_amdgcn_exp2f((tv[j] - mt[nt]) * s2 - lrt2[nt]);
          const float pd = __builtin_amdgcn_exp2f((acc[nt][j] * invT - lse_d[nt]) * kLog2e);
          Sr[nt] += a.overlap ? fminf(pt, pd) : fmaxf(pt - pd, 0.f);
        }
      }
    }
    if ((t & 3) == 3) {   // chunk complete: combine the two half-rows and write
      const int c = c0 + (t >> 2);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int row = rg * 256 + wv * 64 + nt * 32 + n;
        const int64_t o = (int64_t)row * a.nch + c;
        if (MODE == kModeGreedy) {
          float bv = Mr[nt];
          int bi = Ir[nt];
          argmax_merge(bv, bi, __shfl_xor(bv, 32), __shfl_xor(bi, 32));
          if (half == 0 && valid[nt]) {
            a.L[o] = make_float2(bv, 0.f);
            a.I[o] = bi;
            if (nonfinite(bv)) set_flag(a.status, kFlagNonFinite);
          }
          Mr[nt] = -INFINITY; Ir[nt] = 0x7FFFFFFF;
        } else if (MODE == kModeSample) {
          // sums were taken relative to Ms2 = round(M * s2): undo that rounding
          if (valid[nt] && nonfinite(Sr[nt])) set_flag(a.status, kFlagNonFinite);
          float S = Sr[nt];
          if (S > 0.f) S *= __builtin_amdgcn_exp2f(-fmaf(Mr[nt], s2, -Ms2[nt]));
          const float Mo = __shfl_xor(Mr[nt], 32);
          const float So = __shfl_xor(S, 32);
          const float Mn = fmaxf(Mr[nt], Mo);
          float St = 0.f;
          if (Mn != -INFINITY) {
            if (S > 0.f) St += S * __builtin_amdgcn_exp2f((Mr[nt] - Mn) * s2);
            if (So > 0.f) St += So * __builtin_amdgcn_exp2f((Mo - Mn) * s2);
          }
          if (half == 0 && valid[nt]) {
            a.L[o] = make_float2(Mn, St);
            if (nonfinite(St) || Mn == INFINITY) set_flag(a.status, kFlagNonFinite);
          }
          Mr[nt] = -INFINITY; Sr[nt] = 0.f; Ms2[nt] = -INFINITY;
        } else {
          const float St = Sr[nt] + __shfl_xor(Sr[nt], 32);
          if (half == 0 && valid[nt]) {
            a.L[o] = make_float2(0.f, St);
            if (nonfinite(St)) set_flag(a.status, kFlagNonFinite);
          }
          Sr[nt] = 0.f;
        }
      }
    }
  };

  URaw<UT> ub[2][2];
  f32x16_t acc[2][2];
  // ---- prologue: W2t tiles 0 and 1, U of tiles 0 and 1
  stage_load(st[0], 0);
  stage_load(st[1], 1);
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    ub[0][nt].fetch(urow[nt], vbase + 16 * half, a.V, a.u_vec_ok, valid[nt]);
    ub[1][nt].fetch(urow[nt], vbase + 32 + 16 * half, a.V, a.u_vec_ok, valid[nt]);
  }

  auto step = [&](auto Pc, int t) __attribute__((always_inline)) {
    constexpr int P = decltype(Pc)::value;
    stage_store(st[P], P);
    // prefetch two tiles ahead (the last two prefetches repeat the final tile)
    const int tp = min(t + 2, T - 1);
    stage_load(st[P], tp);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) ub[P][nt].unpack(acc[P][nt]);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
      ub[P][nt].fetch(urow[nt], vbase + tp * 32 + 16 * half, a.V, a.u_vec_ok, valid[nt]);
    __syncthreads();
    if (wave_active) {
      const u32x4_t* tile = lds[P] + arow * SEGMAX;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4_t w = tile[(2 * ks + half) ^ aswz];
        const bf16x8_t A = __builtin_bit_cast(bf16x8_t, w);
        acc[P][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, Bf[0][ks], acc[P][0], 0, 0, 0);
        acc[P][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, Bf[1][ks], acc[P][1], 0, 0, 0);
      }
      if (t >= 1) epilogue(acc[1 - P], t - 1);
    }
  };
  for (int t = 0; t < T; t += 2) {
    step(std::integral_constant<int, 0>{}, t);
    if (t + 1 < T) step(std::integral_constant<int, 1>{}, t + 1);
  }
  // T is a multiple of 4 (four tiles per chunk): the last tile used buffer 1
  if (wave_active) epilogue(acc[1], T - 1);
}

// ------------------------------------------------ MFMA, LDS-DMA pipeline
// Same contraction and epilogue as k_markov_mfma_reg, with both operands that
// stream (the W2t tile and the 256 x 32 slab of U) moved by direct-to-LDS loads
// (global_load_lds_dwordx4) into an NBUF-deep LDS ring: tile t+NBUF-1 is in
// flight while tile t is computed, at no register cost.  Requirements: rank a
// multiple of 64 (KS >= 4), U rows 16-byte aligned and V a multiple of the
// elements per 16 bytes; other shapes use k_markov_mfma_reg.
typedef __attribute__((address_space(1))) void gvoid_t;
typedef __attribute__((address_space(3))) void lvoid_t;

__device__ __forceinline__ int u_swizzle(int rr) { return (rr >> 1) ^ (rr >> 3); }

// gfx9 s_waitcnt immediate: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] |
// vmcnt_hi[15:14].  Waits until at most N vector-memory operations of this
// wave are outstanding and all of its LDS operations are done.
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
}

template <typename UT, int KS, int MODE, int NBUF, int NWV>
__global__ __launch_bounds__(64 * NWV) void k_markov_mfma(MarkovArgs a) {
  constexpr int NT = 64 * NWV;                            // threads
  constexpr int NTW = 256 / (32 * NWV);                   // 32-row tiles per wave
  constexpr int SEGMAX = 2 * KS;                          // W2t row segments
  constexpr int EPL = 16 / (int)sizeof(UT);               // U elements per segment
  constexpr int SPR = 32 / EPL;                           // U segments per row of a tile
  constexpr int USEG = 16 / EPL;                          // U segments read per lane (16 values)
  constexpr int W2_SEGS = 32 * SEGMAX;
  constexpr int SLOT = W2_SEGS + 256 * SPR;               // 16-byte units per ring slot
  constexpr int NW = KS / NWV;                            // W2 DMA ops per wave per tile
  constexpr int NU = 4 * SPR / NWV;                       // U DMA ops per wave per tile
  constexpr int OPS = NW + NU;
  static_assert(KS >= 4 && KS % 4 == 0, "DMA path needs rank >= 64");
  static_assert((NWV == 4 || NWV == 8) && KS % NWV == 0 && (4 * SPR) % NWV == 0, "waves");
  static_assert(NBUF == 4, "ring depth");
  __shared__ u32x4_t ring[NBUF * SLOT];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int b = blockIdx.x;
  const int xcd = b & 7, sb = b >> 3;
  const int rg = sb % a.nrg;
  const int cg = (sb / a.nrg) * 8 + xcd;
  if (cg >= a.ncg) return;
  int nrows = a.R;
  if (MODE == kModeResid) nrows = *a.rej_count;
  if (rg * 256 >= nrows) return;
  const int c0 = cg * a.cg, c1 = min(a.nch, c0 + a.cg);
  const int T = (c1 - c0) * 4;
  const int vbase = c0 * kChunk;
  const int nseg = a.rank >> 3;
  const int smask = ((nseg & (nseg - 1)) == 0) ? min(nseg, 16) - 1 : 0;
  const bool wave_active = rg * 256 + wv * 32 * NTW < nrows;

  // ---- rows computed by this lane: column n of the wave's two 32-row tiles
  const int n = lane & 31, half = lane >> 5;
  bool valid[NTW];
  const UT* trow[NTW];
  int prevs[NTW];
  float mt[NTW], lrt2[NTW], lse_d[NTW];
  auto row_info = [&](int row, int& req, int& kk, int& tr, int& qr) __attribute__((always_inline)) {
    req = 0; kk = a.k; tr = 0; qr = 0;
    if (row < nrows) {
      if (MODE == kModeResid) {
        const int4 e = a.rej[row];
        req = e.x; kk = e.y; tr = e.z; qr = e.w;
      } else {
        req = row;
      }
    }
  };
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const int row = rg * 256 + wv * 32 * NTW + nt * 32 + n;
    valid[nt] = row < nrows;
    int req, kk, tr, qr;
    row_info(row, req, kk, tr, qr);
    int prev = 0;
    if (valid[nt]) prev = bias_row_index(a, req, kk, MODE != kModeResid);
    prevs[nt] = prev;
    trow[nt] = reinterpret_cast<const UT*>(a.target) + (int64_t)tr * a.V;
    mt[nt] = 0.f; lrt2[nt] = 0.f; lse_d[nt] = 0.f;
    if (MODE == kModeResid && valid[nt]) {
      const float2 nrm = a.lse_t[qr];
      mt[nt] = nrm.x;
      lrt2[nt] = nrm.y * kLog2e;
      lse_d[nt] = a.lse_d[(int64_t)req * a.gamma + (kk - 1)];
    }
  }
  bf16x8_t Bf[NTW][KS];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const uint16_t* erow = a.W1 + (int64_t)prevs[nt] * a.rank + half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8_t z = {};
      Bf[nt][ks] = (valid[nt] && ks * 16 < a.rank) ? *reinterpret_cast<const bf16x8_t*>(erow + ks * 16) : z;
    }
  }
  const int m = lane & 31;
  const int arow = 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3);
  const int aswz = seg_swizzle(arow) & smask;

  // ---- DMA descriptors of this thread (fixed across tiles)
  int w2_off[NW];
  int w2_row[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int idx = (wv + NWV * i) * 64 + lane;
    const int r = idx / SEGMAX, p = idx - r * SEGMAX;
    w2_row[i] = r;
    w2_off[i] = (p < nseg) ? (p ^ (seg_swizzle(r) & smask)) * 8 : -1;
  }
  const UT* u_ptr[NU];
  int u_seg[NU];
#pragma unroll
  for (int i = 0; i < NU; ++i) {
    const int idx = (wv + NWV * i) * 64 + lane;
    const int rr = idx / SPR, sp = idx - rr * SPR;
    u_seg[i] = (sp ^ (u_swizzle(rr) & (SPR - 1))) * EPL;
    int req, kk, tr, qr;
    const int row = rg * 256 + rr;
    row_info(row < nrows ? row : rg * 256, req, kk, tr, qr);
    u_ptr[i] = reinterpret_cast<const UT*>(a.U) + ((int64_t)req * a.gamma + (kk - 1)) * a.V;
  }
  const int vmax_seg = a.V - EPL;     // last in-range segment start (V % EPL == 0)
  auto issue = [&](auto Sc, int t) __attribute__((always_inline)) {
    constexpr int S = decltype(Sc)::value;
    const int vb = vbase + min(t, T - 1) * 32;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const int g = wv + NWV * i;
      if (w2_off[i] >= 0) {
        const int v = min(vb + w2_row[i], a.V - 1);
        __builtin_amdgcn_global_load_lds(
            (gvoid_t*)(a.W2t + (int64_t)v * a.rank + w2_off[i]),
            (lvoid_t*)(ring + S * SLOT + g * 64), 16, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const int g = wv + NWV * i;
      const int v = min(vb + u_seg[i], vmax_seg);
      __builtin_amdgcn_global_load_lds((gvoid_t*)(u_ptr[i] + v),
                                       (lvoid_t*)(ring + S * SLOT + W2_SEGS + g * 64), 16, 0, 0);
    }
  };
  if (nseg < SEGMAX) {
    const u32x4_t z = {0u, 0u, 0u, 0u};
    for (int j = tid; j < NBUF * W2_SEGS; j += NT) {
      const int sl = j / W2_SEGS, u = j - sl * W2_SEGS;
      if (u % SEGMAX >= nseg) ring[sl * SLOT + u] = z;
    }
  }
  // A tile whose last entries lie past V: the U slots of those entries hold
  // clamped (wrong) data; overwrite them with -inf after the DMA has landed.
  auto mask_tail = [&](auto Sc, int t) __attribute__((always_inline)) {
    constexpr int S = decltype(Sc)::value;
    const int vb = vbase + t * 32;
    if (vb + 32 > a.V) {
      const uint32_t ninf = (EPL == 8) ? 0xFF80FF80u : 0xFF800000u;
      const u32x4_t w = {ninf, ninf, ninf, ninf};
      for (int j = tid; j < 256 * SPR; j += NT) {
        const int rr = j / SPR, sp = j - rr * SPR;
        const int seg = sp ^ (u_swizzle(rr) & (SPR - 1));
        if (vb + seg * EPL >= a.V) ring[S * SLOT + W2_SEGS + j] = w;
      }
      // LDS writes done (lgkmcnt 0), no wait on vector memory (vmcnt 63)
      __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
      __builtin_amdgcn_s_barrier();
    }
  };

  // ---- epilogue state
  float Mr[NTW], Sr[NTW], Ms2[NTW];
  int Ir[NTW];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) { Mr[nt] = -INFINITY; Sr[nt] = 0.f; Ms2[nt] = -INFINITY; Ir[nt] = 0x7FFFFFFF; }
  const float s2 = a.scale2;
  const float invT = s2 * kLn2;

  // straight-line part of the epilogue of one tile: x = acc + U, then the
  // running (max, sum) or argmax update, branch-free
  auto epi_hot = [&](f32x16_t (&acc)[NTW], const u32x4_t (&uw)[NTW][USEG], int t) __attribute__((always_inline)) {
    const int vt = vbase + t * 32 + 16 * half;
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      float x[16];
#pragma unroll
      for (int e = 0; e < USEG; ++e) {
        if (EPL == 8) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            x[8 * e + 2 * q] = acc[nt][8 * e + 2 * q] + bf16_lo(uw[nt][e][q]);
            x[8 * e + 2 * q + 1] = acc[nt][8 * e + 2 * q + 1] + bf16_hi(uw[nt][e][q]);
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) x[4 * e + q] = acc[nt][4 * e + q] + __uint_as_float(uw[nt][e][q]);
        }
      }
      if (MODE == kModeGreedy) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const bool gt = x[j] > Mr[nt];
          Mr[nt] = gt ? x[j] : Mr[nt];
          Ir[nt] = gt ? vt + j : Ir[nt];
        }
      } else if (MODE == kModeSample) {
        float tm = fmaxf(x[0], x[1]);
#pragma unroll
        for (int j = 2; j < 16; ++j) tm = fmaxf(tm, x[j]);
        const float nM = fmaxf(Mr[nt], tm);
        const float nMs2 = nM * s2;
        float sum = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) sum += __builtin_amdgcn_exp2f(fmaf(x[j], s2, -nMs2));
        // rescale the running sum to the new maximum (exp2(-inf) = 0 while empty);
        // a NaN sum stays NaN; an all -inf tile leaves the state unchanged
        const float newS = Sr[nt] * __builtin_amdgcn_exp2f(Ms2[nt] - nMs2) + sum;
        const bool empty = nM == -INFINITY;
        Sr[nt] = empty ? Sr[nt] : newS;
        Ms2[nt] = empty ? Ms2[nt] : nMs2;
        Mr[nt] = nM;
      } else {
        float tv[16];
        load16<UT>(trow[nt], a.u_vec_ok && valid[nt], vt, valid[nt] ? a.V : 0, tv);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float pt = __builtin_amdgcn_exp2f((tv[j] - mt[nt]) * s2 - lrt2[nt]);
          const float pd = __builtin_amdgcn_exp2f((x[j] * invT - lse_d[nt]) * kLog2e);
          Sr[nt] += a.overlap ? fminf(pt, pd) : fmaxf(pt - pd, 0.f);
        }
      }
    }
  };
  // chunk completion after tile t: combine the two half-rows and write
  auto epi_chunk = [&](int t) __attribute__((always_inline)) {
    if ((t & 3) != 3) return;
    const int c = c0 + (t >> 2);
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      const int row = rg * 256 + wv * 32 * NTW + nt * 32 + n;
      const int64_t o = (int64_t)row * a.nch + c;
      if (MODE == kModeGreedy) {
        float bv = Mr[nt];
        int bi = Ir[nt];
        argmax_merge(bv, bi, __shfl_xor(bv, 32), __shfl_xor(bi, 32));
        if (half == 0 && valid[nt]) {
          a.L[o] = make_float2(bv, 0.f);
          a.I[o] = bi;
          if (nonfinite(bv)) set_flag(a.status, kFlagNonFinite);
        }
        Mr[nt] = -INFINITY; Ir[nt] = 0x7FFFFFFF;
      } else if (MODE == kModeSample) {
        if (valid[nt] && nonfinite(Sr[nt])) set_flag(a.status, kFlagNonFinite);
        float S = Sr[nt];
        // sums were taken relative to Ms2 = round(M * s2): undo that rounding
        if (S > 0.f) S *= __builtin_amdgcn_exp2f(-fmaf(Mr[nt], s2, -Ms2[nt]));
        const float Mo = __shfl_xor(Mr[nt], 32);
        const float So = __shfl_xor(S, 32);
        const float Mn = fmaxf(Mr[nt], Mo);
        float St = 0.f;
        if (Mn != -INFINITY) {
          if (S > 0.f) St += S * __builtin_amdgcn_exp2f((Mr[nt] - Mn) * s2);
          if (So > 0.f) St += So * __builtin_amdgcn_exp2f((Mo - Mn) * s2);
        }
        if (half == 0 && valid[nt]) {
          a.L[o] = make_float2(Mn, St);
          if (nonfinite(St) || Mn == INFINITY) set_flag(a.status, kFlagNonFinite);
        }
        Mr[nt] = -INFINITY; Sr[nt] = 0.f; Ms2[nt] = -INFINITY;
      } else {
        const float St = Sr[nt] + __shfl_xor(Sr[nt], 32);
        if (half == 0 && valid[nt]) {
          a.L[o] = make_float2(0.f, St);
          if (nonfinite(St)) set_flag(a.status, kFlagNonFinite);
        }
        Sr[nt] = 0.f;
      }
    }
  };
  auto read_u = [&](auto Sc, u32x4_t (&uw)[NTW][USEG]) __attribute__((always_inline)) {
    constexpr int S = decltype(Sc)::value;
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      const int rr = wv * 32 * NTW + nt * 32 + n;
      const u32x4_t* ul = ring + S * SLOT + W2_SEGS + rr * SPR;
      const int usw = u_swizzle(rr) & (SPR - 1);
#pragma unroll
      for (int e = 0; e < USEG; ++e) uw[nt][e] = ul[(USEG * half + e) ^ usw];
    }
  };

  f32x16_t acc[2][NTW];
  // Schedule of tile t (ring slot t % 4, accumulator buffer t % 2):
  //   wait for tile t's DMA, barrier, DMA of tile t+2 into the slot of t-2,
  //   then the MFMAs of tile t interleaved with the epilogue of tile t-1
  //   (whose U values are still in slot (t-1) % 4).
  auto step = [&](auto Sc, int t, bool with_epi) __attribute__((always_inline)) {
    constexpr int S = decltype(Sc)::value;
    constexpr int P = S & 1;
    constexpr int SP = (S + 3) & 3;                 // slot of tile t-1
    constexpr int SN = (S + 2) & 3;                 // slot of tile t+2 (= t-2)
    wait_vm_lgkm0<OPS>();                           // tile t+1 may still be in flight
    __builtin_amdgcn_s_barrier();
    mask_tail(Sc, t);
    issue(std::integral_constant<int, SN>{}, t + 2);
    if (wave_active) {
      const u32x4_t* tile = ring + S * SLOT + arow * SEGMAX;
      // A operands: all k-steps up front with two 32-row tiles per wave; with
      // one (eight waves, two per SIMD, half the registers) a rolling window
      // three k-steps deep, each loaded two MFMAs before its use
      constexpr int AW_AHEAD = NTW == 1 ? 2 : KS;
      u32x4_t aw[KS];
#pragma unroll
      for (int ks = 0; ks < AW_AHEAD && ks < KS; ++ks) aw[ks] = tile[(2 * ks + half) ^ aswz];
      u32x4_t uw[NTW][USEG];
      if (with_epi) read_u(std::integral_constant<int, SP>{}, uw);
      __builtin_amdgcn_sched_barrier(0);
      const f32x16_t zero = {};
      // the epilogue of tile t-1 is cut into 2*KS slices, one after each MFMA:
      // first half = x = acc + U with the running max (or argmax), second half
      // = the exp sums relative to the new maximum
      constexpr int NSL = NTW * KS;
      constexpr int HALF_SL = NSL / 2;
      constexpr int PER_A = (16 * NTW + HALF_SL - 1) / HALF_SL;
      float x[NTW][16];
      float tmx[NTW], ssum[NTW];
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) { tmx[nt] = -INFINITY; ssum[nt] = 0.f; }
      float nM[NTW], nMs2[NTW];
      const int vt = vbase + (t - 1) * 32 + 16 * half;
#pragma unroll
      for (int i = 0; i < NSL; ++i) {
        const int ks = i / NTW, ntm = i % NTW;
        if (NTW == 1 && ntm == 0 && ks + AW_AHEAD < KS)
          aw[ks + AW_AHEAD] = tile[(2 * (ks + AW_AHEAD) + half) ^ aswz];
        const bf16x8_t A = __builtin_bit_cast(bf16x8_t, aw[ks]);
        acc[P][ntm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, Bf[ntm][ks], ks ? acc[P][ntm] : zero, 0, 0, 0);
        if (with_epi && MODE != kModeResid) {
          if (i < HALF_SL) {
#pragma unroll
            for (int q = 0; q < PER_A; ++q) {
              const int e = i * PER_A + q;
              if (e < 16 * NTW) {
                const int nt = e >> 4, j = e & 15;
                const uint32_t wd = uw[nt][j / EPL][(j % EPL) / (EPL / 4)];
                const float u = (EPL == 8) ? ((j & 1) ? bf16_hi(wd) : bf16_lo(wd)) : __uint_as_float(wd);
                x[nt][j] = acc[1 - P][nt][j] + u;
                if (MODE == kModeGreedy) {
                  const bool gt = x[nt][j] > Mr[nt];
                  Mr[nt] = gt ? x[nt][j] : Mr[nt];
                  Ir[nt] = gt ? vt + j : Ir[nt];
                  asm volatile("" : "+v"(Mr[nt]), "+v"(Ir[nt]));
                } else {
                  tmx[nt] = fmaxf(tmx[nt], x[nt][j]);
                  // keep this slice's work here (IR passes would sink it)
                  asm volatile("" : "+v"(x[nt][j]), "+v"(tmx[nt]));
                }
              }
            }
          } else if (MODE == kModeSample) {
            if (i == HALF_SL) {
#pragma unroll
              for (int nt = 0; nt < NTW; ++nt) {
                nM[nt] = fmaxf(Mr[nt], tmx[nt]);
                nMs2[nt] = nM[nt] * s2;
              }
            }
#pragma unroll
            for (int q = 0; q < PER_A; ++q) {
              const int e = (i - HALF_SL) * PER_A + q;
              if (e < 16 * NTW) {
                const int nt = e >> 4, j = e & 15;
                ssum[nt] += __builtin_amdgcn_exp2f(fmaf(x[nt][j], s2, -nMs2[nt]));
                asm volatile("" : "+v"(ssum[nt]));
              }
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (with_epi) {
        if (MODE == kModeSample) {
#pragma unroll
          for (int nt = 0; nt < NTW; ++nt) {
            // rescale the running sum to the new maximum; an all -inf tile
            // leaves the state unchanged; a NaN sum stays NaN
            const float newS = Sr[nt] * __builtin_amdgcn_exp2f(Ms2[nt] - nMs2[nt]) + ssum[nt];
            const bool empty = nM[nt] == -INFINITY;
            Sr[nt] = empty ? Sr[nt] : newS;
            Ms2[nt] = empty ? Ms2[nt] : nMs2[nt];
            Mr[nt] = nM[nt];
          }
        } else if (MODE == kModeResid) {
          epi_hot(acc[1 - P], uw, t - 1);
        }
      }
    }
    if (with_epi && wave_active) epi_chunk(t - 1);
  };
  // prologue: tiles 0 and 1 in flight, then step 0 (no epilogue yet)
  issue(std::integral_constant<int, 0>{}, 0);
  issue(std::integral_constant<int, 1>{}, 1);
  step(std::integral_constant<int, 0>{}, 0, false);
  int t = 1;
  for (; t + 3 < T; t += 4) {
    step(std::integral_constant<int, 1>{}, t, true);
    step(std::integral_constant<int, 2>{}, t + 1, true);
    step(std::integral_constant<int, 3>{}, t + 2, true);
    step(std::integral_constant<int, 0>{}, t + 3, true);
  }
  // T is a multiple of 4, so three steps remain (slots 1, 2, 3)
  step(std::integral_constant<int, 1>{}, t, true);
  step(std::integral_constant<int, 2>{}, t + 1, true);
  step(std::integral_constant<int, 3>{}, t + 2, true);
  // epilogue of the last tile (T-1, slot 3, accumulator buffer 1)
  wait_vm_lgkm0<0>();
  if (wave_active) {
    u32x4_t uw[NTW][USEG];
    read_u(std::integral_constant<int, 3>{}, uw);
    epi_hot(acc[1], uw, T - 1);
    epi_chunk(T - 1);
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
    const int prev = bias_row_index(a, req, kk, MODE != kModeResid);
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
        if (nonfinite(sm) || mx == INFINITY) set_flag(a.status, kFlagNonFinite);
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
          sm += a.overlap ? fminf(pt, pd) : fmaxf(pt - pd, 0.f);
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
  a.cps = 32;
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
static void launch_mfma_ks(MarkovArgs& a, int grid, hipStream_t st, bool dma) {
  const int nks = a.rank / 16;
  if (dma && nks >= 4) {
    // ring depth: four slots when they fit in LDS, else two
    constexpr int SPR = 32 * (int)sizeof(UT) / 16;
#define DSPARK_DMA(KS_)                                                                          \
    {                                                                                             \
      constexpr int SLOTB = (32 * 2 * KS_ + 256 * SPR) * 16;                                      \
      constexpr int KSD = 4 * SLOTB <= 160 * 1024 ? KS_ : 4;                                      \
      if (4 * SLOTB <= 160 * 1024) {                                                              \
        if (KSD >= 8 && MODE != kModeResid)                                                       \
          hipLaunchKernelGGL((k_markov_mfma<UT, KSD, MODE, 4, (KSD >= 8 ? 8 : 4)>), dim3(grid),   \
                             dim3(512), 0, st, a);                                                \
        else                                                                                      \
          hipLaunchKernelGGL((k_markov_mfma<UT, KSD, MODE, 4, 4>), dim3(grid), dim3(256), 0, st,  \
                             a);                                                                  \
        return;                                                                                   \
      }                                                                                           \
    }
    if (nks <= 4) DSPARK_DMA(4)
    else if (nks <= 8) DSPARK_DMA(8)
    else if (nks <= 16) DSPARK_DMA(16)
    else DSPARK_DMA(32)
#undef DSPARK_DMA
    // ring does not fit in LDS: register-staged kernel below
  }
  if (nks <= 1) hipLaunchKernelGGL((k_markov_mfma_reg<UT, 1, MODE>), dim3(grid), dim3(256), 0, st, a);
  else if (nks <= 2) hipLaunchKernelGGL((k_markov_mfma_reg<UT, 2, MODE>), dim3(grid), dim3(256), 0, st, a);
  else if (nks <= 4) hipLaunchKernelGGL((k_markov_mfma_reg<UT, 4, MODE>), dim3(grid), dim3(256), 0, st, a);
  else if (nks <= 8) hipLaunchKernelGGL((k_markov_mfma_reg<UT, 8, MODE>), dim3(grid), dim3(256), 0, st, a);
  else if (nks <= 16) hipLaunchKernelGGL((k_markov_mfma_reg<UT, 16, MODE>), dim3(grid), dim3(256), 0, st, a);
  else hipLaunchKernelGGL((k_markov_mfma_reg<UT, 32, MODE>), dim3(grid), dim3(256), 0, st, a);
}

hipError_t launch_markov_stats(const MarkovArgs& a0, bool u_bf16, bool w_bf16, int mode,
                               hipStream_t st) {
  MarkovArgs a = a0;
  if (w_bf16) {
    a.W1 = reinterpret_cast<const uint16_t*>(a.W1v);
    a.W2t = reinterpret_cast<const uint16_t*>(a.W2tv);
    a.nrg = (a.nrows_cap + 255) / 256;
    // chunks per workgroup: about one workgroup per compute unit
    int cgw = (int)(((int64_t)a.nrg * a.nch + 255) / 256);
    if (cgw < 1) cgw = 1;
    a.cg = cgw;
    a.ncg = (a.nch + cgw - 1) / cgw;
    const int grid = a.nrg * ((a.ncg + 7) / 8) * 8;
    // the LDS-DMA pipeline needs 16-byte aligned U rows (and target rows in
    // residual mode) with V a multiple of the elements per 16 bytes
    const int epl = u_bf16 ? 8 : 4;
    const bool dma = a.u_vec_ok && (a.V % epl) == 0 && a.V >= epl;
    if (u_bf16) {
      if (mode == kModeSample) launch_mfma_ks<uint16_t, kModeSample>(a, grid, st, dma);
      else if (mode == kModeGreedy) launch_mfma_ks<uint16_t, kModeGreedy>(a, grid, st, dma);
      else launch_mfma_ks<uint16_t, kModeResid>(a, grid, st, dma);
    } else {
      if (mode == kModeSample) launch_mfma_ks<float, kModeSample>(a, grid, st, dma);
      else if (mode == kModeGreedy) launch_mfma_ks<float, kModeGreedy>(a, grid, st, dma);
      else launch_mfma_ks<float, kModeResid>(a, grid, st, dma);
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
