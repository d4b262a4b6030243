// sampling.hpp -- wave-level pieces of the chunked Gumbel-max sampler.
//
// Exact categorical sampling from softmax(score) over a vocabulary split into
// chunks of kChunk consecutive entries: pick a chunk c by Gumbel-max over the
// chunk log-masses L_c = ln sum_{v in c} exp(score_v), then an entry inside c
// by Gumbel-max over score_v.  P(c) * P(v | c) = softmax(score)(v) (the
// Gumbel-max theorem applied at both levels), so only ceil(V/kChunk) + kChunk
// uniforms are drawn instead of V.  Keys are float32 sums; ties go to the
// lower index.  With a single chunk no chunk-level uniform is drawn.
#pragma once
#include "device_common.hpp"

namespace dspark {

struct PickResult {
  int idx;       // winner (-1 if nothing had mass)
  float key;     // its key
  float gap;     // best minus second-best key (only when asked for)
};

// Reductions over one chunk's lanes when a wave-wide 16-byte load covers
// 64 / LPC chunks (LPC = 16 lanes for bf16 rows, 32 for fp32).
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

// One wave: chunks [c0, c1) of one row.  UNR 16-byte loads per lane are in
// flight at once (64 UNR / LPC chunks per batch); the data stays as raw
// words until it is used.
template <typename T, bool GREEDY, int UNR = 8>
__device__ __forceinline__ void row_segment(const T* row, int V, int c0, int c1, float scale2,
                                            bool vec_ok, float2* L, int* I, uint32_t* status) {
  constexpr int VPL = 16 / sizeof(T);       // values per lane per 16-byte load
  constexpr int LPC = kChunk / VPL;         // lanes per chunk
  constexpr int CPI = 64 / LPC;             // chunks per wave-wide load
  const int lane = threadIdx.x & 63;
  const int sub = lane % LPC;
  const int cl = lane / LPC;
  for (int cb = c0; cb < c1; cb += CPI * UNR) {
    uint4 raw[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int c = cb + u * CPI + cl;
      const int v0 = c * kChunk + sub * VPL;
      if (c < c1 && vec_ok && v0 + VPL <= V) {
        raw[u] = *reinterpret_cast<const uint4*>(row + v0);
      } else {
        // ragged tail: element loads, -inf past the segment or the vocabulary
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (sizeof(T) == 2) {
            const uint32_t lo = (c < c1 && v0 + 2 * q < V) ? reinterpret_cast<const uint16_t*>(row)[v0 + 2 * q] : 0xFF80u;
            const uint32_t hi = (c < c1 && v0 + 2 * q + 1 < V) ? reinterpret_cast<const uint16_t*>(row)[v0 + 2 * q + 1] : 0xFF80u;
            w[q] = lo | (hi << 16);
          } else {
            w[q] = (c < c1 && v0 + q < V) ? __float_as_uint(reinterpret_cast<const float*>(row)[v0 + q])
                                          : __float_as_uint(-INFINITY);
          }
        }
        raw[u] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int c = cb + u * CPI + cl;
      const int v0 = c * kChunk + sub * VPL;
      float x[VPL];
      {
        const uint32_t w[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
#pragma unroll
        for (int e = 0; e < VPL; ++e)
          x[e] = (sizeof(T) == 2) ? ((e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1])) : __uint_as_float(w[e]);
      }
      if (GREEDY) {
        float bv = -INFINITY;
        int bi = 0x7FFFFFFF;
#pragma unroll
        for (int e = 0; e < VPL; ++e)
          if (x[e] > bv) { bv = x[e]; bi = v0 + e; }
        chunk_argmax<LPC>(bv, bi);
        if (sub == 0 && c < c1) {
          L[c] = make_float2(bv, 0.f);
          I[c] = bi;
          if (nonfinite(bv)) set_flag(status, kFlagNonFinite);
        }
      } else {
        float m = -INFINITY;
#pragma unroll
        for (int e = 0; e < VPL; ++e) m = fmaxf(m, x[e]);
        m = chunk_max<LPC>(m);
        float s = 0.f;
        if (m != -INFINITY) {
#pragma unroll
          for (int e = 0; e < VPL; ++e) s += __builtin_amdgcn_exp2f((x[e] - m) * scale2);
        }
        s = chunk_sum<LPC>(s);
        if (sub == 0 && c < c1) {
          L[c] = make_float2(m, s);
          if (nonfinite(s) || m == INFINITY) set_flag(status, kFlagNonFinite);
        }
      }
    }
  }
}

// Per-chunk statistics are (M_c, S_c): M_c the raw maximum of the row's scores
// x over chunk c (before the temperature), S_c = sum_{v in c} exp((x_v - M_c)/T).
// Chunk log-mass L_c = M_c/T + log S_c.  Everything below is kept relative to
// the row maximum m, so log-probabilities stay accurate when x/T is large.
struct RowNorm {
  float m;        // raw row maximum (-inf: no mass)
  float lse_rel;  // log sum_c S_c exp((M_c - m)/T)   (normaliser = m/T + lse_rel)
};

// One wave; the chunk statistics are read 16 per lane at a time, all loads of
// a batch in flight together.
__device__ inline RowNorm row_norm(const float2* st, int nch, float invT) {
  constexpr int B = 16;
  const int lane = threadIdx.x & 63;
  float m = -INFINITY;
  for (int c0 = 0; c0 < nch; c0 += 64 * B) {
    float x[B];
#pragma unroll
    for (int t = 0; t < B; ++t) {
      const int c = c0 + lane + 64 * t;
      x[t] = c < nch ? st[c].x : -INFINITY;
    }
#pragma unroll
    for (int t = 0; t < B; ++t) m = fmaxf(m, x[t]);
  }
  m = wave_max(m);
  if (m == -INFINITY) return RowNorm{-INFINITY, -INFINITY};
  float s = 0.f;
  for (int c0 = 0; c0 < nch; c0 += 64 * B) {
    float2 v[B];
#pragma unroll
    for (int t = 0; t < B; ++t) {
      const int c = c0 + lane + 64 * t;
      v[t] = c < nch ? st[c] : make_float2(-INFINITY, 0.f);
    }
#pragma unroll
    for (int t = 0; t < B; ++t)
      if (v[t].y > 0.f) s += v[t].y * expf((v[t].x - m) * invT);
  }
  s = wave_sum(s);
  return RowNorm{m, s > 0.f ? logf(s) : -INFINITY};
}

// Chunk-level Gumbel pick: key_c = (M_c - m)/T + log S_c + G_c (chunks with
// S_c == 0 carry no mass).  One wave; lane l handles chunk blocks of four,
// one Philox block per four chunks.
__device__ inline PickResult pick_chunk(const float2* st, int nch, float m, float invT,
                                        uint64_t seed, uint64_t round, uint32_t tag, uint32_t req,
                                        uint32_t k, bool want_gap) {
  const int lane = threadIdx.x & 63;
  PickResult r{-1, -INFINITY, INFINITY};
  if (nch == 1) {
    const float2 v = st[0];
    r.idx = (v.y > 0.f) ? 0 : -1;
    r.key = (v.y > 0.f) ? (v.x - m) * invT + logf(v.y) : -INFINITY;
    return r;
  }
  float best = -INFINITY;
  int bi = 0x7FFFFFFF;
  for (int b = lane; b * 4 < nch; b += 64) {
    const uint4 blk = stream_block(seed, round, tag, req, k, (uint32_t)b);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int c = b * 4 + w;
      if (c < nch) {
        const float2 v = st[c];
        if (v.y > 0.f) {
          const float key = (v.x - m) * invT + logf(v.y) + gumbel_of(word_of(blk, (uint32_t)w));
          argmax_merge(best, bi, key, c);
        }
      }
    }
  }
  wave_argmax(best, bi);
  r.idx = (best == -INFINITY) ? -1 : bi;
  r.key = best;
  if (want_gap && r.idx >= 0) {
    float second = -INFINITY;
    for (int b = lane; b * 4 < nch; b += 64) {
      const uint4 blk = stream_block(seed, round, tag, req, k, (uint32_t)b);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int c = b * 4 + w;
        if (c < nch && c != r.idx) {
          const float2 v = st[c];
          if (v.y > 0.f)
            second = fmaxf(second, (v.x - m) * invT + logf(v.y) + gumbel_of(word_of(blk, (uint32_t)w)));
        }
      }
    }
    r.gap = best - wave_max(second);
  }
  return r;
}

// In-chunk Gumbel pick: lane l holds the scores of entries base+l and
// base+64+l (-inf = excluded / outside the vocabulary).
__device__ inline PickResult pick_in_chunk(float s0, float s1, int base, uint64_t seed,
                                           uint64_t round, uint32_t tag, uint32_t req,
                                           uint32_t k, bool want_gap) {
  const int lane = threadIdx.x & 63;
  const int v0 = base + lane, v1 = base + 64 + lane;
  const uint4 b0 = stream_block(seed, round, tag, req, k, (uint32_t)v0 >> 2);
  const uint4 b1 = stream_block(seed, round, tag, req, k, (uint32_t)v1 >> 2);
  const float k0 = (s0 == -INFINITY) ? -INFINITY : s0 + gumbel_of(word_of(b0, (uint32_t)v0 & 3u));
  const float k1 = (s1 == -INFINITY) ? -INFINITY : s1 + gumbel_of(word_of(b1, (uint32_t)v1 & 3u));
  float best = k0;
  int bi = v0;
  argmax_merge(best, bi, k1, v1);
  if (best == -INFINITY) bi = 0x7FFFFFFF;
  wave_argmax(best, bi);
  PickResult r{best == -INFINITY ? -1 : bi, best, INFINITY};
  if (want_gap && r.idx >= 0) {
    float second = -INFINITY;
    if (v0 != r.idx) second = fmaxf(second, k0);
    if (v1 != r.idx) second = fmaxf(second, k1);
    r.gap = best - wave_max(second);
  }
  return r;
}

// Lowest-index argmax over per-chunk maxima (st[c].x) / argmaxes I (greedy).
__device__ inline void argmax_chunks(const float2* st, const int* I, int nch, float& v, int& idx) {
  constexpr int B = 16;
  const int lane = threadIdx.x & 63;
  v = -INFINITY;
  idx = 0x7FFFFFFF;
  for (int c0 = 0; c0 < nch; c0 += 64 * B) {
    float x[B];
    int ix[B];
#pragma unroll
    for (int t = 0; t < B; ++t) {
      const int c = c0 + lane + 64 * t;
      x[t] = c < nch ? st[c].x : -INFINITY;
      ix[t] = c < nch ? I[c] : 0x7FFFFFFF;
    }
#pragma unroll
    for (int t = 0; t < B; ++t) argmax_merge(v, idx, x[t], ix[t]);
  }
  wave_argmax(v, idx);
}

// Markov bias W1[prev] . W2t[v] for one vocabulary entry: float32 FMA chain in
// ascending i.  e is the gathered W1 row (the same address in every lane);
// rank is a multiple of 16 and rows are 16-byte aligned.
__device__ inline float markov_bias(const uint16_t* e, const uint16_t* W2t, int rank, int v) {
  const uint4* w = reinterpret_cast<const uint4*>(W2t + (int64_t)v * rank);
  const uint4* ev = reinterpret_cast<const uint4*>(e);
  float b = 0.f;
  for (int q = 0; q < rank / 8; ++q) {
    const uint4 u = w[q];
    const uint4 x = ev[q];
    b = fmaf(bf16_lo(x.x), bf16_lo(u.x), b);
    b = fmaf(bf16_hi(x.x), bf16_hi(u.x), b);
    b = fmaf(bf16_lo(x.y), bf16_lo(u.y), b);
    b = fmaf(bf16_hi(x.y), bf16_hi(u.y), b);
    b = fmaf(bf16_lo(x.z), bf16_lo(u.z), b);
    b = fmaf(bf16_hi(x.z), bf16_hi(u.z), b);
    b = fmaf(bf16_lo(x.w), bf16_lo(u.w), b);
    b = fmaf(bf16_hi(x.w), bf16_hi(u.w), b);
  }
  return b;
}
__device__ inline float markov_bias(const float* e, const float* W2t, int rank, int v) {
  const float4* w = reinterpret_cast<const float4*>(W2t + (int64_t)v * rank);
  const float4* ev = reinterpret_cast<const float4*>(e);
  float b = 0.f;
  for (int q = 0; q < rank / 4; ++q) {
    const float4 u = w[q];
    const float4 x = ev[q];
    b = fmaf(x.x, u.x, b);
    b = fmaf(x.y, u.y, b);
    b = fmaf(x.z, u.z, b);
    b = fmaf(x.w, u.w, b);
  }
  return b;
}

// ------------------------------------------------------------ block-level
// Reductions across the NT/64 waves of an NT-thread block (NT <= 1024) through
// LDS; every thread of the block must call them (they contain barriers).
template <int NW>
struct BlockScratchN {
  float f[NW];
  int i[NW];
  float g[NW];
};
using BlockScratch = BlockScratchN<8>;       // blocks of up to 512 threads
using BlockScratch16 = BlockScratchN<16>;    // blocks of up to 1024 threads

template <int NT = 256, typename S = BlockScratch>
__device__ inline float block_max(float v, S& sh) {
  constexpr int NWV = NT / 64;
  const int wv = threadIdx.x >> 6;
  v = wave_max(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh.f[wv] = v;
  __syncthreads();
  float r = sh.f[0];
#pragma unroll
  for (int q = 1; q < NWV; ++q) r = fmaxf(r, sh.f[q]);
  return r;
}
template <int NT = 256, typename S = BlockScratch>
__device__ inline float block_sum(float v, S& sh) {
  constexpr int NWV = NT / 64;
  const int wv = threadIdx.x >> 6;
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh.f[wv] = v;
  __syncthreads();
  // pairwise, in wave order
  float r[NWV];
#pragma unroll
  for (int q = 0; q < NWV; ++q) r[q] = sh.f[q];
#pragma unroll
  for (int w = 1; w < NWV; w *= 2)
#pragma unroll
    for (int q = 0; q + w < NWV; q += 2 * w) r[q] += r[q + w];
  return r[0];
}
template <int NT = 256, typename S = BlockScratch>
__device__ inline void block_argmax(float& v, int& idx, S& sh) {
  constexpr int NWV = NT / 64;
  const int wv = threadIdx.x >> 6;
  wave_argmax(v, idx);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) { sh.f[wv] = v; sh.i[wv] = idx; }
  __syncthreads();
  v = sh.f[0];
  idx = sh.i[0];
#pragma unroll
  for (int q = 1; q < NWV; ++q) argmax_merge(v, idx, sh.f[q], sh.i[q]);
}

// Chunk-level Gumbel pick by an NT-thread block: thread t scans chunk blocks
// t, t+NT, ... (four chunks per Philox block).  Returns the chunk and,
// through *sum_rel when it is not null, sum_c S_c exp((M_c - m)/T) (the row
// normaliser above m).
// COH: the statistics were written by other workgroups of the same launch
// (device-coherent loads).
template <int NT = 256, bool COH = false, typename S = BlockScratch>
__device__ inline PickResult block_pick_chunk(const float2* st, int nch, float m, float invT,
                                              uint64_t seed, uint64_t round, uint32_t tag,
                                              uint32_t req, uint32_t k, bool want_gap,
                                              float* sum_rel, S& sh) {
  float best = -INFINITY, ssum = 0.f;
  int bi = 0x7FFFFFFF;
  const bool draw = nch > 1;
  for (int b = threadIdx.x; b * 4 < nch; b += NT) {
    uint4 blk = make_uint4(0, 0, 0, 0);
    if (draw) blk = stream_block(seed, round, tag, req, k, (uint32_t)b);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int c = b * 4 + w;
      if (c < nch) {
        const float2 v = COH ? ld_coh2(st + c) : st[c];
        if (v.y > 0.f) {
          const float rel = (v.x - m) * invT;
          ssum += v.y * expf(rel);
          const float key = rel + logf(v.y) + (draw ? gumbel_of(word_of(blk, (uint32_t)w)) : 0.f);
          argmax_merge(best, bi, key, c);
        }
      }
    }
  }
  if (sum_rel) *sum_rel = block_sum<NT>(ssum, sh);
  block_argmax<NT>(best, bi, sh);
  PickResult r{best == -INFINITY ? -1 : bi, best, INFINITY};
  if (want_gap && r.idx >= 0 && draw) {
    float second = -INFINITY;
    for (int b = threadIdx.x; b * 4 < nch; b += NT) {
      const uint4 blk = stream_block(seed, round, tag, req, k, (uint32_t)b);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int c = b * 4 + w;
        if (c < nch && c != r.idx) {
          const float2 v = COH ? ld_coh2(st + c) : st[c];
          if (v.y > 0.f)
            second = fmaxf(second, (v.x - m) * invT + logf(v.y) + gumbel_of(word_of(blk, (uint32_t)w)));
        }
      }
    }
    r.gap = best - block_max<NT>(second, sh);
  }
  return r;
}

// In-chunk Gumbel pick by an NT-thread block: NT/128 consecutive threads share
// one entry; the first of them holds the score of entry base + t/(NT/128)
// (-inf = excluded).
template <int NT = 256, typename S = BlockScratch>
__device__ inline PickResult block_pick_in_chunk(float s, int base, uint64_t seed, uint64_t round,
                                                 uint32_t tag, uint32_t req, uint32_t k,
                                                 bool want_gap, S& sh) {
  constexpr int TPE = NT / kChunk;
  const int t = threadIdx.x;
  const int v = base + t / TPE;
  float key = -INFINITY;
  int bi = 0x7FFFFFFF;
  if ((t % TPE) == 0 && s != -INFINITY) {
    const uint4 blk = stream_block(seed, round, tag, req, k, (uint32_t)v >> 2);
    key = s + gumbel_of(word_of(blk, (uint32_t)v & 3u));
    bi = v;
  }
  float best = key;
  int bidx = bi;
  block_argmax<NT>(best, bidx, sh);
  PickResult r{best == -INFINITY ? -1 : bidx, best, INFINITY};
  if (want_gap && r.idx >= 0) {
    const float second = block_max<NT>((bi == r.idx) ? -INFINITY : key, sh);
    r.gap = best - second;
  }
  return r;
}

// Part h of nparts of the Markov bias dot product W1[prev] . W2t[v]: entries
// [h*rank/nparts, (h+1)*rank/nparts), float32 FMA chain in ascending order.
template <int UNR = 8>
__device__ inline float markov_bias_half(const uint16_t* e, const uint16_t* W2t, int rank, int v,
                                         int h, int nparts = 2) {
  const int nq = rank / (8 * nparts);            // 8-value groups per part
  const uint4* w = reinterpret_cast<const uint4*>(W2t + (int64_t)v * rank) + h * nq;
  const uint4* ev = reinterpret_cast<const uint4*>(e) + h * nq;
  float b = 0.f;
#pragma unroll UNR
  for (int q = 0; q < nq; ++q) {
    const uint4 u = w[q];
    const uint4 x = ev[q];
    b = fmaf(bf16_lo(x.x), bf16_lo(u.x), b);
    b = fmaf(bf16_hi(x.x), bf16_hi(u.x), b);
    b = fmaf(bf16_lo(x.y), bf16_lo(u.y), b);
    b = fmaf(bf16_hi(x.y), bf16_hi(u.y), b);
    b = fmaf(bf16_lo(x.z), bf16_lo(u.z), b);
    b = fmaf(bf16_hi(x.z), bf16_hi(u.z), b);
    b = fmaf(bf16_lo(x.w), bf16_lo(u.w), b);
    b = fmaf(bf16_hi(x.w), bf16_hi(u.w), b);
  }
  return b;
}
template <int UNR = 8>
__device__ inline float markov_bias_half(const float* e, const float* W2t, int rank, int v, int h,
                                         int nparts = 2) {
  const int nq = rank / (4 * nparts);            // 4-value groups per part
  const float4* w = reinterpret_cast<const float4*>(W2t + (int64_t)v * rank) + h * nq;
  const float4* ev = reinterpret_cast<const float4*>(e) + h * nq;
  float b = 0.f;
#pragma unroll UNR
  for (int q = 0; q < nq; ++q) {
    const float4 u = w[q];
    const float4 x = ev[q];
    b = fmaf(x.x, u.x, b);
    b = fmaf(x.y, u.y, b);
    b = fmaf(x.z, u.z, b);
    b = fmaf(x.w, u.w, b);
  }
  return b;
}

}  // namespace dspark
