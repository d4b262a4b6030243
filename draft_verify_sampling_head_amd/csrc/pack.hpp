// pack.hpp -- ragged pack by one 1024-thread workgroup (DSpark summary page,
// Supplementary details, variable-length routing; CSDN DSpark article,
// section 3.3, flatten + marker tensors): row r contributes its first len(r)
// tokens, flattened back to back with offsets and (owning request, position)
// markers; the total may be padded to a captured-graph tier (DeepSpec
// analysis page, section 5.4).  Shared by the stand-alone pack kernel
// (lengths read from memory) and the scheduler (the lengths it has just
// decided, still in LDS).
#pragma once
#include "launch.hpp"

namespace dspark {

constexpr int kPackThreads = 1024;
constexpr int kPackLds = 40;               // ints of LDS the scan needs

// Exclusive scan of one value per thread over the 1024-thread workgroup;
// returns the thread's prefix and writes the workgroup total to *total.
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

// Row of packed slot q: the largest r with cu[r] <= q (rows of length zero
// share their offset with the next row, which is the one that holds q).
__device__ __forceinline__ int pack_row_of(const int* cu, int R, int q) {
  int lo = 0, hi = R - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= q) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Tokens of kPackSlots packed slots per thread and pass: every load of a pass
// is issued before its stores (the output buffers are written through other
// pointers than the rows, so the compiler could not reorder them).
constexpr int kPackSlots = 4;

__device__ __forceinline__ void pack_copy_slots(const int32_t* __restrict__ rows,
                                                int32_t* __restrict__ flat,
                                                int32_t* __restrict__ marker_req,
                                                int32_t* __restrict__ marker_pos,
                                                const int* cu_l, int R, int width, int N) {
  for (int q0 = threadIdx.x; q0 < N; q0 += kPackSlots * kPackThreads) {
    int r[kPackSlots], j[kPackSlots], tok[kPackSlots];
#pragma unroll
    for (int u = 0; u < kPackSlots; ++u) {
      const int q = q0 + u * kPackThreads;
      r[u] = q < N ? pack_row_of(cu_l, R, q) : 0;
      j[u] = q - cu_l[r[u]];
    }
#pragma unroll
    for (int u = 0; u < kPackSlots; ++u)
      tok[u] = (q0 + u * kPackThreads < N) ? rows[(int64_t)r[u] * width + j[u]] : 0;
#pragma unroll
    for (int u = 0; u < kPackSlots; ++u) {
      const int q = q0 + u * kPackThreads;
      if (q < N) {
        flat[q] = tok[u];
        if (marker_req) marker_req[q] = r[u];
        if (marker_pos) marker_pos[q] = j[u];
      }
    }
  }
}

// The pack of a.rows with the effective length of row r given by len_of(r)
// (a.len and a.len_offset are not read).  A length outside [0, width] is
// clamped and flagged.  The offsets are kept in cu_l (LDS, cu_cap ints) when
// R + 1 fit; the tokens are then copied slot by slot by all threads at once,
// else row by row.
template <typename LenOf>
__device__ inline void pack_rows_block(const PackArgs& a, LenOf len_of, int* lds, int* cu_l,
                                       int cu_cap) {
  const int tid = threadIdx.x;
  const bool by_slot = a.R + 1 <= cu_cap;
  int carry = 0;
  for (int base = 0; base < a.R; base += kPackThreads) {
    const int r = base + tid;
    int l = 0;
    if (r < a.R) {
      l = len_of(r);
      if (l < 0 || l > a.width) {
        set_flag(a.status, kFlagBadLen);
        l = l < 0 ? 0 : a.width;
      }
    }
    int tot;
    const int pos = carry + block_exclusive_scan(l, lds, &tot);
    if (r < a.R) {
      a.cu[r] = pos;
      if (by_slot) {
        cu_l[r] = pos;
      } else {
        const int32_t* src = a.rows + (int64_t)r * a.width;
        for (int j = 0; j < l; ++j) {
          a.flat[pos + j] = src[j];
          if (a.marker_req) a.marker_req[pos + j] = r;
          if (a.marker_pos) a.marker_pos[pos + j] = j;
        }
      }
    }
    carry += tot;
  }
  if (by_slot) {
    if (tid == 0) cu_l[a.R] = carry;
    __syncthreads();
    pack_copy_slots(a.rows, a.flat, a.marker_req, a.marker_pos, cu_l, a.R, a.width, carry);
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
  for (int64_t q = carry + tid; q < a.slots; q += kPackThreads) {
    a.flat[q] = q < npad ? a.pad_token : -1;
    if (a.marker_req) a.marker_req[q] = -1;
    if (a.marker_pos) a.marker_pos[q] = -1;
  }
}

}  // namespace dspark
