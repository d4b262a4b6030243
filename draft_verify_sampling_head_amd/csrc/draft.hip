// draft.hip -- Markov draft head: the gamma-step sequential chain.
//
// DSpark summary page, Method details (causal block distribution, Markov
// head): p_k(v | x_0, x_<k) = softmax(U_k + W1[x_{k-1}] W2)(v), sampled left to
// right.  Every step k has two phases:
//   A. per-chunk statistics of s = (U_k + bias)/T for every request (the bias
//      contraction on MFMA);
//   B. the pick, one workgroup per request: the row normaliser from the chunk
//      statistics, the chunk-level Gumbel pick, then the in-chunk pick after
//      rebuilding the 128 scores of the chosen chunk (bias by FMA chain).
// Two schedules of the same phases:
//   persistent : one co-resident launch for all gamma steps (k_draft_persistent).
//                Each workgroup owns a 512-entry vocabulary slice and keeps its
//                W2 slice in registers as MFMA operands for the whole round, so
//                W2 is read from memory once per round instead of once per
//                step; U_k is streamed once; the W1 rows of the requests sit in
//                LDS.  Phases are separated by grid barriers.
//   steps      : two launches per step (stats.hip, then k_draft_pick); stream
//                order is the only synchronisation.  Used for shapes the
//                persistent kernel does not take (float32 data, rank other than
//                64/128/256, vocabularies beyond 512 entries per compute unit).
// Nothing returns to the host in either schedule.
#include <atomic>
#include <cfloat>
#include <cstdlib>
#include <cstring>

#include "launch.hpp"
#include "persist_common.hpp"
#include "sampling.hpp"
#include "workspace.hpp"

namespace dspark {


// Pick of position k for request i by an NT-thread block (NT in {256, 512});
// lrow is the row of the chunk statistics.
template <typename UT, typename WT, bool GREEDY, int NT>
__device__ __forceinline__ void pick_row(const DraftPickArgs& a, int i, int k, int64_t lrow,
                                         BlockScratch& sh) {
  constexpr int TPE = NT / kChunk;          // threads per rebuilt entry
  const int tid = threadIdx.x;
  const int64_t xo = (int64_t)i * (a.gamma + 1);
  const int prev = a.rank == 0 ? 0 : (k == 1) ? a.x0[i] : a.x[xo + k - 1];
  const float2* Lr = a.L + lrow * a.nch;
  int xk;
  float logp, lse, gap = INFINITY;
  if (GREEDY) {
    float v = -INFINITY;
    int idx = 0x7FFFFFFF;
    const int* Ir = a.I + lrow * a.nch;
    for (int c = tid; c < a.nch; c += NT) argmax_merge(v, idx, Lr[c].x, Ir[c]);
    block_argmax<NT>(v, idx, sh);
    xk = idx;
    lse = v;
    logp = 0.f;
    if (xk < 0 || xk >= a.V) { set_flag(a.status, kFlagNonFinite); xk = 0; }
  } else {
    float m = -INFINITY;
    for (int c = tid; c < a.nch; c += NT) m = fmaxf(m, Lr[c].x);
    m = block_max<NT>(m, sh);
    const bool want_gap = a.margin != nullptr;
    float srel;
    const PickResult pc = block_pick_chunk<NT>(Lr, a.nch, m, a.invT, a.seed, a.round,
                                               kTagDraftChunk, (uint32_t)i, (uint32_t)k, want_gap,
                                               &srel, sh);
    const float lse_rel = logf(srel);
    // the absolute normaliser is assembled in double: m / T can be large at a
    // low temperature, where a float product would cost several ulps
    lse = (float)((double)m / (double)a.T + (double)lse_rel);
    int c = pc.idx;
    if (c < 0) { set_flag(a.status, kFlagNonFinite); c = 0; }
    const int base = c * kChunk;
    // rebuild the 128 scores of the chosen chunk: TPE threads per entry, each
    // a 1/TPE part of the rank
    const int v = base + tid / TPE, h = tid % TPE;
    const bool in = v < a.V;
    float b = 0.f;
    if (a.rank > 0 && in) {
      const int pv = (prev >= 0 && prev < a.V) ? prev : 0;
      const WT* erow = a.feat ? reinterpret_cast<const WT*>(a.feat) + ((int64_t)i * a.gamma + (k - 1)) * a.rank
                              : reinterpret_cast<const WT*>(a.W1) + (int64_t)pv * a.rank;
      b = markov_bias_half<(NT > 256 ? 2 : 8)>(erow, reinterpret_cast<const WT*>(a.W2t), a.rank, v, h, TPE);
    }
#pragma unroll
    for (int o = 1; o < TPE; o *= 2) b += __shfl_xor(b, o);
    const UT* urow = reinterpret_cast<const UT*>(a.U) + ((int64_t)i * a.gamma + (k - 1)) * a.V;
    const float s = in ? (Elem<UT>::get(urow, v) + b - m) / a.T : -INFINITY;
    const PickResult pe = block_pick_in_chunk<NT>(s, base, a.seed, a.round, kTagDraftElem,
                                                  (uint32_t)i, (uint32_t)k, want_gap, sh);
    xk = pe.idx;
    if (xk < 0) { set_flag(a.status, kFlagNonFinite); xk = base; }
    // the winner's score: held by thread TPE * (xk - base)
    __syncthreads();
    if (tid == TPE * (xk - base)) sh.g[0] = s;
    __syncthreads();
    logp = sh.g[0] - lse_rel;
    gap = fminf(pc.gap, pe.gap);
  }
  if (tid == 0) {
    if (k == 1) a.x[xo] = a.x0[i];
    a.x[xo + k] = xk;
    const int64_t o = (int64_t)i * a.gamma + (k - 1);
    a.logp_d[o] = logp;
    a.lse_d[o] = lse;
    if (a.margin) a.margin[o] = gap;
  }
  __syncthreads();                          // sh is reused by the next call
}

// One 256-thread block per request (step a.k), or per (request, position)
// when all positions are independent (rank 0, all_pos).
template <typename UT, typename WT, bool GREEDY>
__global__ __launch_bounds__(256) void k_draft_pick(DraftPickArgs a) {
  __shared__ BlockScratch sh;
  if (a.all_pos)
    pick_row<UT, WT, GREEDY, 256>(a, blockIdx.x / a.gamma, blockIdx.x % a.gamma + 1, blockIdx.x, sh);
  else
    pick_row<UT, WT, GREEDY, 256>(a, blockIdx.x, a.k, blockIdx.x, sh);
}

struct PersistArgs {
  DraftPickArgs p;                          // pick view (k set per step)
  float scale2;                             // log2(e)/T; 1 when greedy
  int nslice;                               // vocabulary slices = ceil(V / 512)
  uint32_t* bar;                            // grid-barrier counter, zero at launch
  uint32_t spin_limit;                      // bounded wait per barrier
  // RNN head: the recurrent cell runs inside the launch before each step
  const float* rP;                          // [R*gamma][3 rank] h part of the projection
  float* rstate;                            // [R][gamma][rank] s_1 .. s_gamma
  uint16_t* rfeat;                          // [R][gamma][rank] e_1 .. e_gamma (bf16)
  const uint16_t* rWr;                      // [3 rank][2 rank + d]
  int rd;                                   // d
};


// Pick of step a.k for request i by the 512-thread workgroup of the persistent
// launch.  Thread t keeps the statistics of chunks 4t..4t+3 in registers.
// Sampling: the row maximum m, then one reduction gives both the chunk-level
// Gumbel winner of (M_c - m)/T + ln S_c + G_c and the normaliser
// sum_c S_c exp((M_c - m)/T); the chosen chunk's 128 scores are rebuilt by
// four threads per entry (all W2t loads issued at once, the entry noise
// computed while they are in flight), and the thread holding the in-chunk
// winner writes the outputs.
//
// known_prev >= 0: x_{k-1} as the caller already holds it (the persistent
// launch keeps each workgroup's last pick in LDS), with its W1 row already in
// pl.E when e_loaded; the token then goes to *last_out too.  At the end only
// LDS is synchronised: the stores need not have completed (other workgroups
// poll for the token; a grid barrier waits for its workgroup's own stores).
template <int KS, bool GREEDY>
__device__ __forceinline__ void pick_row_p(const DraftPickArgs& a, int i, float s2, BlockScratch& sh,
                                           PickLds<2 * KS>& pl, const uint16_t* feat,
                                           int known_prev = -1, bool e_loaded = false,
                                           int* last_out = nullptr) {
  constexpr int NT = kPThreads, TPE = NT / kChunk;
  constexpr int SEG = 2 * KS, NQ = SEG / TPE;   // 16-byte pieces of the rank per thread
  static_assert(kPMaxChunks <= 4 * NT, "four chunks per thread");
  const int tid = threadIdx.x;
  const int k = a.k;
  const int64_t xo = (int64_t)i * (a.gamma + 1);
  int prev = known_prev;
  if (prev < 0 && !GREEDY) prev = (k == 1) ? a.x0[i] : ld_coh(a.x + xo + k - 1);
  if (prev < 0 || prev >= a.V) prev = 0;        // flagged when phase A read it
  const float2* Lr = a.L + (int64_t)i * a.nch;
  // chunk statistics of this thread's four chunks (all loads in flight)
  float2 Lv[4];
  int Iv[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int c = 4 * tid + w;
    Lv[w] = make_float2(-INFINITY, 0.f);
    Iv[w] = 0x7FFFFFFF;
    if (c < a.nch) {
      Lv[w] = ld_coh2(Lr + c);
      if (GREEDY) Iv[w] = ld_coh(a.I + (int64_t)i * a.nch + c);
    }
  }
  if (!GREEDY && tid < SEG && !e_loaded)
    pl.E[tid] = feat ? ld_coh16(feat + ((int64_t)i * a.gamma + (k - 1)) * a.rank + 8 * tid)
                     : *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.W1) +
                                                       (int64_t)prev * a.rank + 8 * tid);
  const int64_t o = (int64_t)i * a.gamma + (k - 1);
  if (GREEDY) {
    float v = -INFINITY;
    int idx = 0x7FFFFFFF;
#pragma unroll
    for (int w = 0; w < 4; ++w) argmax_merge(v, idx, Lv[w].x, Iv[w]);
    block_argmax_v(v, idx, pl.farg, pl.iarg);
    int xk = idx;
    if (xk < 0 || xk >= a.V) { set_flag(a.status, kFlagNonFinite); xk = 0; }
    if (tid == 0) {
      if (k == 1) st_coh(a.x + xo, a.x0[i]);
      st_coh(a.x + xo + k, xk);
      a.logp_d[o] = 0.f;
      a.lse_d[o] = v;
      if (a.margin) a.margin[o] = INFINITY;
      if (last_out) *last_out = xk;
    }
  } else {
    // the chunk noise while the statistics are in flight
    float g[4];
    chunk_noise(a, i, k, g);
    // scores are kept relative to the raw row maximum m (accuracy at low T)
    float mloc = fmaxf(fmaxf(Lv[0].x, Lv[1].x), fmaxf(Lv[2].x, Lv[3].x));
    const float m = block_max_v(mloc, pl.fmax);
    PickRed pr{-INFINITY, 0x7FFFFFFF, 0.f};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float2 v = Lv[w];
      if (v.y > 0.f) {
        pr.s += v.y * __builtin_amdgcn_exp2f((v.x - m) * s2);
        const float key = (v.x - m) * a.invT + __builtin_amdgcn_logf(v.y) * kLn2 + g[w];
        argmax_merge(pr.key, pr.idx, key, 4 * tid + w);
      }
    }
    const PickRed rr = block_pick_reduce(pr, pl.red);
    const float lse_rel = logf(rr.s);
    const float lse = (float)((double)m / (double)a.T + (double)lse_rel);
    int c = rr.key == -INFINITY ? -1 : rr.idx;
    if (c < 0) { if (tid == 0) set_flag(a.status, kFlagNonFinite); c = 0; }
    // in-chunk: entry base + tid / TPE, part tid % TPE of the rank
    const int base = c * kChunk;
    const int v = base + tid / TPE, h = tid % TPE;
    const bool in = v < a.V;
    uint4 wq[NQ];
    float u = 0.f;
    if (in) {
      const uint4* wr = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.W2t) +
                                                       (int64_t)v * a.rank) + h * NQ;
#pragma unroll
      for (int q = 0; q < NQ; ++q) wq[q] = wr[q];
      u = bf16_at(reinterpret_cast<const uint16_t*>(a.U), ((int64_t)i * a.gamma + (k - 1)) * a.V + v);
    }
    // the entry's noise while the loads are in flight
    float gel = 0.f;
    if (h == 0 && in) {
      const uint4 blk = stream_block(a.seed, a.round, kTagDraftElem, (uint32_t)i, (uint32_t)k, (uint32_t)v >> 2);
      gel = gumbel_of(word_of(blk, (uint32_t)v & 3u));
    }
    float bsum = 0.f;
    if (in) {
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const uint4 x = pl.E[h * NQ + q];
        const uint4 w = wq[q];
        bsum = fmaf(bf16_lo(x.x), bf16_lo(w.x), bsum);
        bsum = fmaf(bf16_hi(x.x), bf16_hi(w.x), bsum);
        bsum = fmaf(bf16_lo(x.y), bf16_lo(w.y), bsum);
        bsum = fmaf(bf16_hi(x.y), bf16_hi(w.y), bsum);
        bsum = fmaf(bf16_lo(x.z), bf16_lo(w.z), bsum);
        bsum = fmaf(bf16_hi(x.z), bf16_hi(w.z), bsum);
        bsum = fmaf(bf16_lo(x.w), bf16_lo(w.w), bsum);
        bsum = fmaf(bf16_hi(x.w), bf16_hi(w.w), bsum);
      }
    }
    static_assert(TPE == 4, "four threads per entry");
    bsum += dpp_f<kDppXor1>(bsum);
    bsum += dpp_f<kDppXor2>(bsum);
    const float sv = in ? (u + bsum - m) / a.T : -INFINITY;      // score of entry v, minus m/T
    float key = -INFINITY;
    int kid = 0x7FFFFFFF;
    if (h == 0 && in) {
      key = sv + gel;
      kid = v;
    }
    float best = key;
    int bidx = kid;
    block_argmax_v(best, bidx, pl.farg, pl.iarg);
    int xk = best == -INFINITY ? -1 : bidx;
    float gap = INFINITY;
    if (a.margin != nullptr) {
      // second-best keys (debug output only)
      float second = -INFINITY;
      if (a.nch > 1) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float2 lv = Lv[w];
          if (4 * tid + w != c && lv.y > 0.f)
            second = fmaxf(second, (lv.x - m) * a.invT + __builtin_amdgcn_logf(lv.y) * kLn2 + g[w]);
        }
      }
      const float cgap = (a.nch > 1) ? rr.key - block_max<NT>(second, sh) : INFINITY;
      const float egap = (xk >= 0) ? best - block_max<NT>(kid == xk ? -INFINITY : key, sh) : INFINITY;
      gap = fminf(cgap, egap);
    }
    if (xk < 0) {
      if (tid == 0) set_flag(a.status, kFlagNonFinite);
      xk = base;
    }
    // the thread holding the winner writes the outputs
    if (tid == TPE * (xk - base)) {
      if (k == 1) st_coh(a.x + xo, a.x0[i]);
      st_coh(a.x + xo + k, xk);
      a.logp_d[o] = sv - lse_rel;
      a.lse_d[o] = lse;
      if (a.margin) a.margin[o] = gap;
      if (last_out) *last_out = xk;
    }
  }
  lds_sync();                               // LDS slots and the W1 row are reused
}

// The persistent launch's pick as a launch of its own for the per-step
// schedule (bf16 data and weights, rank 64/128/256): one 512-thread workgroup
// per request, step a.k.
template <int KS, bool GREEDY>
__global__ __launch_bounds__(kPThreads) void k_draft_pick_p(DraftPickArgs a, float s2) {
  __shared__ BlockScratch sh;
  __shared__ PickLds<2 * KS> pl;
  pick_row_p<KS, GREEDY>(a, blockIdx.x, s2, sh, pl, reinterpret_cast<const uint16_t*>(a.feat));
}

// ---- RNN head inside the persistent launch
// Feature rows e_k of requests row0 .. row0 + rows - 1 into LDS rows of ROWP
// 16-byte pieces (the layout of gather_w1_rows).  They were written by other
// workgroups in this launch, so they are read with device-coherent loads,
// eight pieces per thread in flight at once.
template <int SEG, int ROWP>
__device__ __forceinline__ void gather_feat_rows(uint4* E, int row0, int rows, int k, int gamma,
                                                 const uint16_t* feat, int rank) {
  const int npieces = rows * ROWP;
  for (int p0 = threadIdx.x; p0 < npieces; p0 += 8 * kPThreads) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int p = min(p0 + u * kPThreads, npieces - 1);
      const int rl = p / ROWP, sp = p % ROWP;
      v[u] = ld_coh16(feat + ((int64_t)(row0 + rl) * gamma + (k - 1)) * rank + 8 * (sp < SEG ? sp : 0));
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (p0 + u * kPThreads < npieces) E[p0 + u * kPThreads] = v[u];
  }
}

// float32 -> bf16 bits, round to nearest, ties to even (finite values)
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// bf16 parts hi + mid + lo of eight fp32 values (24 significant bits: the
// products with bf16 weights are exact in fp32)
__device__ __forceinline__ void split3_bf16(const float (&v)[8], bf16x8_t& hi, bf16x8_t& mid,
                                            bf16x8_t& lo) {
  uint16_t h[8], m[8], l[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    h[t] = (uint16_t)bf16_bits(v[t]);
    const float r1 = v[t] - __uint_as_float((uint32_t)h[t] << 16);
    m[t] = (uint16_t)bf16_bits(r1);
    const float r2 = r1 - __uint_as_float((uint32_t)m[t] << 16);
    l[t] = (uint16_t)bf16_bits(r2);
  }
  hi = __builtin_bit_cast(bf16x8_t, h);
  mid = __builtin_bit_cast(bf16x8_t, m);
  lo = __builtin_bit_cast(bf16x8_t, l);
}

// The cell of step k (DSpark summary page, Method details, RNN head):
// g = sigmoid(Wr_g z), s_k = g s_{k-1} + (1 - g) tanh(Wr_c z), e_k = tanh(Wr_o z)
// with z = [s_{k-1} ; W1[x_{k-1}] ; h_k], the h part precomputed in rP.  Tile
// (rt, jt) = requests 16 rt + [0, 16) x state entries 16 jt + [0, 16) with
// their gate, candidate and output rows; workgroup b takes tiles b, b + grid,
// ...  Wave w computes k-step w (32 columns) of the recurrent product on
// MFMA, the state half as three exact bf16 parts; red (LDS, 24 KB) adds the
// eight waves' partial results, then waves 0-3 finish request rows 4 g + w.
// s_{k-1} and the tokens x_{k-1} come from other workgroups (device-coherent
// loads; tokens waited for), and s_k, e_k go out with device-coherent stores.
__device__ __forceinline__ void rnn_cell_tiles_p(const PersistArgs& P, int k, float* red) {
  const DraftPickArgs& a = P.p;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = a.rank, ldw = 2 * r + P.rd, nks = r / 32;   // r in {64, 128, 256}
  const int ntj = r / 16, ntiles = ((a.R + 15) / 16) * ntj;
  const int m = lane & 15, kg = lane >> 4;
  const uint16_t* W1 = reinterpret_cast<const uint16_t*>(a.W1);
  const bool has_s = k >= 2;
  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int req0 = (tile / ntj) * 16, j0 = (tile % ntj) * 16;
    f32x4_t acc[3];
#pragma unroll
    for (int q = 0; q < 3; ++q) acc[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (w < nks) {
      const int reqA = req0 + m;
      const bool okA = reqA < a.R;
      int prev = 0;
      if (okA) {
        prev = (k == 1) ? a.x0[reqA]
                        : wait_token(a.x + (int64_t)reqA * (a.gamma + 1) + (k - 1), P.spin_limit,
                                     a.status);
        if (prev >= a.V || (k == 1 && prev < 0)) set_flag(a.status, kFlagBadToken);
        if (prev < 0 || prev >= a.V) prev = 0;
      }
      const int c = 32 * w + 8 * kg;
      const bf16x8_t zero = {};
      const bf16x8_t ev = okA ? *reinterpret_cast<const bf16x8_t*>(W1 + (int64_t)prev * r + c) : zero;
      bf16x8_t ws[3], we[3];
#pragma unroll
      for (int q = 0; q < 3; ++q) {
        const uint16_t* wrow = P.rWr + (int64_t)(q * r + j0 + m) * ldw;
        ws[q] = *reinterpret_cast<const bf16x8_t*>(wrow + c);
        we[q] = *reinterpret_cast<const bf16x8_t*>(wrow + r + c);
      }
      if (has_s) {
        float sv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (okA) {
          const float* srow = P.rstate + ((int64_t)reqA * a.gamma + (k - 2)) * r + c;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float2 v = ld_coh2(reinterpret_cast<const float2*>(srow) + t);
            sv[2 * t] = v.x;
            sv[2 * t + 1] = v.y;
          }
        }
        bf16x8_t hi, mid, lo;
        split3_bf16(sv, hi, mid, lo);
#pragma unroll
        for (int q = 0; q < 3; ++q) {
          acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, ws[q], acc[q], 0, 0, 0);
          acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mid, ws[q], acc[q], 0, 0, 0);
          acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, ws[q], acc[q], 0, 0, 0);
        }
      }
#pragma unroll
      for (int q = 0; q < 3; ++q)
        acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ev, we[q], acc[q], 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < 3; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[((q * kPWaves + w) * 64 + lane) * 4 + i] = acc[q][i];
    __syncthreads();
    if (w < 4) {
      float pre[3];
#pragma unroll
      for (int q = 0; q < 3; ++q) {
        float t = 0.f;
#pragma unroll
        for (int ww = 0; ww < kPWaves; ++ww) t += red[((q * kPWaves + ww) * 64 + lane) * 4 + w];
        pre[q] = t;
      }
      const int req = req0 + 4 * kg + w, j = j0 + m;
      float e = 0.f;
      if (req < a.R) {
        const int64_t pos = (int64_t)req * a.gamma + (k - 1);
        const float* Pr = P.rP + pos * 3 * r;
        const float pg = pre[0] + Pr[j], pc = pre[1] + Pr[r + j], po = pre[2] + Pr[2 * r + j];
        float sp = 0.f;
        if (has_s)
          sp = __hip_atomic_load(P.rstate + (pos - 1) * r + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const float g = 1.f / (1.f + expf(-pg));
        const float sn = g * sp + (1.f - g) * tanhf(pc);
        e = tanhf(po);
        if (!isfinite(pg) || !isfinite(pc) || !isfinite(po)) set_flag(a.status, kFlagNonFinite);
        __hip_atomic_store(P.rstate + pos * r + j, sn, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      // entries j, j + 1 share a 32-bit word of the feature row
      const uint32_t eb = bf16_bits(e);
      const uint32_t other = (uint32_t)__shfl_xor((int)eb, 1);
      if (req < a.R && (m & 1) == 0) {
        const int64_t pos = (int64_t)req * a.gamma + (k - 1);
        st_coh(reinterpret_cast<int*>(P.rfeat + pos * r + j), (int)(eb | (other << 16)));
      }
    }
    __syncthreads();                        // red is reused by the next tile
  }
}

// Picks per workgroup whose last token stays in LDS (further picks, R above
// this many times the grid, read it from x).
constexpr int kLastPicks = 16;

template <int KS, bool GREEDY, bool FEAT>
__global__ __launch_bounds__(kPThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_draft_persistent(PersistArgs P) {
  constexpr int SEG = 2 * KS;               // 16-byte segments per W1 row (rank / 8)
  static_assert(KS % 2 == 0, "rank must be a multiple of 32");
  constexpr int ROWP = SEG + 1;             // padded LDS row: rows start 16 bytes apart in the
                                            // bank space, so the 16 lanes of a ds_read_b128
                                            // phase (16 rows, same segment) never collide
  // LDS: the group's W1 rows, the phase-A statistics per (row, wave), the
  // group's tokens and the pick's slots
  __shared__ uint4 E[kPRows * ROWP];
  __shared__ float2 HS[kPRows * kPWaves];   // [row][wave]
  __shared__ int PV[kPRows];
  __shared__ BlockScratch sh;
  __shared__ PickLds<SEG> pl;
  __shared__ int lastx[kLastPicks];         // x_{k-1} of this workgroup's first picks

  DraftPickArgs a = P.p;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int b = blockIdx.x;
  const int V = a.V, R = a.R;
  const int wslice = b * kPSlice + 64 * wv;
  const bool slice_active = b < P.nslice;
  const bool wave_active = slice_active && wslice < V;
  const float s2 = P.scale2;
  const uint16_t* U = reinterpret_cast<const uint16_t*>(a.U);
  const uint16_t* W1 = reinterpret_cast<const uint16_t*>(a.W1);
  const uint16_t* W2t = reinterpret_cast<const uint16_t*>(a.W2t);

  // ---- W2 slice of this wave, resident for the whole launch
  constexpr int KT = KS / 2;                // k-steps of 32
  bf16x8_t Af[4][KT];
  load_w2_slice<KT>(Af, W2t, a.rank, wslice, V, wave_active);
  // this lane's 16 entries: two 8-entry pieces of U, inside V or not
  const int lg = lane >> 4;
  bool uok[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) uok[q] = wave_active && wslice + slice_entry(lg, 8 * q) + 8 <= V;
  const bool wave_full = wave_active && wslice + 64 <= V;

  // the anchors of the requests this workgroup picks (i = b + j grid); its
  // picks then keep them current, so a pick reads x_{k-1} from here
  if (tid < kLastPicks) {
    const int i = b + tid * (int)gridDim.x;
    const int x0 = (i < R) ? a.x0[i] : 0;
    lastx[tid] = (x0 < 0 || x0 >= V) ? 0 : x0;   // flagged when phase A reads it
  }
  __syncthreads();
  uint32_t epoch = 0;
  const int ngroups = (R + kPRows - 1) / kPRows;
  for (int k = 1; k <= a.gamma; ++k) {
    a.k = k;
    if constexpr (FEAT) {
      // ================= RNN cell of step k: e_k and s_k of every request,
      // visible to every workgroup after the barrier
      rnn_cell_tiles_p(P, k, reinterpret_cast<float*>(E));
      grid_barrier(P.bar, ++epoch, P.spin_limit, a.status);
    }
    // ================= phase A: chunk statistics of step k for every request
    for (int g = 0; g < ngroups; ++g) {
      const int row0 = g * kPRows;
      const int rows = min(kPRows, R - row0);
      // U of the group's first two tiles does not depend on the tokens: its
      // loads are in flight while the tokens and W1 rows arrive
      UStream us;
      us.init(U + (int64_t)(k - 1) * V, (int64_t)a.gamma * V, row0, rows, wslice, uok, wave_full);
      uint4 ua[2], ub[2];
      if (wave_active) {
        us.load(ua, 0);
        us.load(ub, 1);
      }
      if (slice_active) {
        // tokens x_{k-1} of the group (staged in LDS), then their W1 rows.
        // x_{k-1} is written by the picks of step k-1: waiting for each
        // token to appear is the only synchronisation with them
        if constexpr (FEAT) {
          // the group's feature rows e_k (written by the cell phase)
          gather_feat_rows<SEG, ROWP>(E, row0, rows, k, a.gamma, P.rfeat, a.rank);
        } else {
          for (int rl = tid; rl < rows; rl += kPThreads) {
            const int row = row0 + rl;
            int prev = (k == 1) ? a.x0[row]
                                : wait_token(a.x + (int64_t)row * (a.gamma + 1) + (k - 1), P.spin_limit,
                                             a.status);
            if (prev >= V || (k == 1 && prev < 0)) set_flag(a.status, kFlagBadToken);
            if (prev < 0 || prev >= V) prev = 0;
            PV[rl] = prev;
          }
          __syncthreads();
          gather_w1_rows<SEG, ROWP>(E, PV, rows, W1, a.rank);
        }
      }
      wait_vm_zero();
      __syncthreads();
      if (wave_active) {
        if (wave_full)
          slice_tiles<KT, ROWP, GREEDY, false>(Af, E, HS, us, ua, ub, wslice, uok, s2);
        else
          slice_tiles<KT, ROWP, GREEDY, true>(Af, E, HS, us, ua, ub, wslice, uok, s2);
      } else {
        // no entries in this wave's slice: empty statistics
        const float2 empty = make_float2(-INFINITY, GREEDY ? __int_as_float(0x7FFFFFFF) : 0.f);
        for (int rl = lane; rl < rows; rl += 64) HS[rl * kPWaves + wv] = empty;
      }
      // LDS-only barriers around the merge: the tile loop's last U prefetches
      // may still be in flight and need not be waited for here
      lds_sync();
      // merge the two halves (waves 2c, 2c+1) of each of the slice's four
      // chunks and store the chunk statistics: S relative to the raw maximum
      if (slice_active) {
        for (int t = tid; t < rows * 4; t += kPThreads) {
          const int rl = t >> 2, c = t & 3;
          const int chunk = 4 * b + c;
          if (chunk >= a.nch) continue;
          const int row = row0 + rl;
          const float2 h0 = HS[rl * kPWaves + 2 * c], h1 = HS[rl * kPWaves + 2 * c + 1];
          float2* Lo = const_cast<float2*>(a.L) + (int64_t)row * a.nch + chunk;
          if (GREEDY) {
            float bv = h0.x;
            int bi = __float_as_int(h0.y);
            argmax_merge(bv, bi, h1.x, __float_as_int(h1.y));
            st_coh2(Lo, make_float2(bv, 0.f));
            st_coh(const_cast<int*>(a.I) + (int64_t)row * a.nch + chunk, bi);
            if (nonfinite(bv)) set_flag(a.status, kFlagNonFinite);
          } else {
            // half h holds S_h relative to scaled_ref(M_h): refer it to Mr s2
            // exactly (one rounding)
            const float Mn = fmaxf(h0.x, h1.x);
            const float Mr = (Mn == -INFINITY) ? 0.f : Mn;
            const float St = h0.y * __builtin_amdgcn_exp2f(fmaf(-Mr, s2, scaled_ref(h0.x, s2))) +
                             h1.y * __builtin_amdgcn_exp2f(fmaf(-Mr, s2, scaled_ref(h1.x, s2)));
            st_coh2(Lo, make_float2(Mn, St));
            if (nonfinite(St) || Mn == INFINITY) set_flag(a.status, kFlagNonFinite);
          }
        }
      }
      lds_sync();                           // E, PV and HS are rewritten by the next group
    }
    // the W1 row of x_{k-1} for this workgroup's first pick: a direct-to-LDS
    // load issued now completes with the barrier's own wait for the stores
    const bool e_pre = !GREEDY && !FEAT && b < R;
    if (e_pre && wv == 0 && lane < SEG) lds_dma16(W1 + (int64_t)lastx[0] * a.rank + 8 * lane, pl.E);
    grid_barrier(P.bar, ++epoch, P.spin_limit, a.status);
    // ================= phase B: the pick of step k, one request per workgroup.
    // No barrier follows: phase A of step k+1 waits for the tokens it reads,
    // and a token is written after its pick has read the chunk statistics
    // that phase A of step k+1 overwrites.
    for (int i = b, j = 0; i < R; i += gridDim.x, ++j) {
      const bool known = !FEAT && j < kLastPicks;
      pick_row_p<KS, GREEDY>(a, i, s2, sh, pl, FEAT ? P.rfeat : nullptr, known ? lastx[j] : -1,
                             e_pre && j == 0, known ? &lastx[j] : nullptr);
    }
  }
}

// ================================================= residual statistics
// Per-chunk residual mass sum_{v in c} max(0, p_t(v) - p_d(v)) of the rows in
// the verify's residual work list (DSpark: resample the first rejected
// position from norm(max(0, p_t - p_d))), or with OVERLAP the overlap mass
// sum_{v in c} min(p_t(v), p_d(v)) (the acceptance rate c* of a position).  p_d is rebuilt exactly as the draft
// computed it: U + W1[x_{k-1}] W2 over the whole vocabulary.  Same layout as
// the persistent draft's phase A: workgroup b loads its 512-entry W2 slice
// into registers once and computes every listed row in 16-row tiles, so W2 is
// streamed once per call whatever the number of rejections.
struct ResidArgs {
  int R, gamma, V, rank, nch, nslice;
  float scale2;                             // log2(e)/T
  const uint16_t* U;
  const uint16_t* W1;
  const uint16_t* W2t;
  const uint16_t* target;
  const int32_t* x;
  const int32_t* rej_count;
  const int4* rej;                          // (request, position k, target row, verify row)
  const float2* lse_t;                      // [verify row] (raw max, log-normaliser above it)
  const float* lse_d;
  float2* L;                                // out [slot][nch] (0, residual mass)
  uint32_t* status;
  bool feat_rows;                           // W1 holds per-position features [R][gamma][rank]
};

template <int KS, bool OVERLAP>
__global__ __launch_bounds__(kPThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_resid_stats(ResidArgs A) {
  constexpr int SEG = 2 * KS, ROWP = SEG + 1, KT = KS / 2;
  __shared__ uint4 E[kPRows * ROWP];
  __shared__ float HS[kPRows * kPWaves];
  __shared__ int PV[kPRows];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int b = blockIdx.x;
  const int nrows = min(*A.rej_count, A.R);
  if (nrows <= 0) return;
  const int V = A.V;
  const int wslice = b * kPSlice + 64 * wv;
  const bool wave_active = wslice < V;
  bf16x8_t Af[4][KT];
  load_w2_slice<KT>(Af, A.W2t, A.rank, wslice, V, wave_active);
  const int ln = lane & 15, lg = lane >> 4;
  bool uok[2];
  int uoff[2];                              // value j of the lane: entry uoff[j >> 3] + (j & 7)
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int e = wslice + slice_entry(lg, 8 * q);
    uok[q] = wave_active && e + 8 <= V;
    uoff[q] = uok[q] ? e : 0;
  }
  const float s2 = A.scale2, invT = s2 * kLn2;
  for (int row0 = 0; row0 < nrows; row0 += kPRows) {
    const int rows = min(kPRows, nrows - row0);
    for (int rl = tid; rl < rows; rl += kPThreads) {
      const int4 e = A.rej[row0 + rl];
      int prev;
      if (A.feat_rows) {
        prev = e.x * A.gamma + (e.y - 1);
      } else {
        prev = A.x[(int64_t)e.x * (A.gamma + 1) + (e.y - 1)];
        if (prev < 0 || prev >= V) { set_flag(A.status, kFlagBadToken); prev = 0; }
      }
      PV[rl] = prev;
    }
    __syncthreads();
    gather_w1_rows<SEG, ROWP>(E, PV, rows, A.W1, A.rank);
    __syncthreads();
    if (wave_active) {
      const int ntiles = (rows + 15) / 16;
      // per tile, this lane's row: its U and target pieces and normalisers
      struct RowIn { uint4 u[2], t[2]; float2 nt; float ld; };
      auto load_row = [&](RowIn& d, int i) __attribute__((always_inline)) {
        const int4 e = A.rej[row0 + min(16 * i + ln, rows - 1)];
        const uint16_t* up = A.U + ((int64_t)e.x * A.gamma + (e.y - 1)) * V;
        const uint16_t* tp = A.target + (int64_t)e.z * V;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          d.u[q] = *reinterpret_cast<const uint4*>(up + uoff[q]);
          d.t[q] = *reinterpret_cast<const uint4*>(tp + uoff[q]);
        }
        d.nt = A.lse_t[e.w];
        d.ld = A.lse_d[(int64_t)e.x * A.gamma + (e.y - 1)];
      };
      RowIn cur, nxt;
      load_row(nxt, 0);
      for (int i = 0; i < ntiles; ++i) {
        cur = nxt;
        if (i + 1 < ntiles) load_row(nxt, i + 1);
        f32x4_t acc[4];
        zero_acc(acc);
        const int rl = 16 * i + ln;
        tile_mfma<KT>(acc, Af, E + rl * ROWP + lg);
        // x = fl(U + bias): the base logits join the bias in one rounding
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[j >> 2][j & 3] += u_piece(cur.u[j >> 3], j & 7);
        const float lrt2 = cur.nt.y * kLog2e;
        float S = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          if (uok[j >> 3]) {
            const uint32_t w = (j & 8) ? ((j & 4) ? ((j & 2) ? cur.t[1].w : cur.t[1].z)
                                                  : ((j & 2) ? cur.t[1].y : cur.t[1].x))
                                       : ((j & 4) ? ((j & 2) ? cur.t[0].w : cur.t[0].z)
                                                  : ((j & 2) ? cur.t[0].y : cur.t[0].x));
            const float tv = (j & 1) ? bf16_hi(w) : bf16_lo(w);
            const float pt = __builtin_amdgcn_exp2f((tv - cur.nt.x) * s2 - lrt2);
            const float pd = __builtin_amdgcn_exp2f((acc[j >> 2][j & 3] * invT - cur.ld) * kLog2e);
            S += OVERLAP ? fminf(pt, pd) : fmaxf(pt - pd, 0.f);
          }
        }
        S += __shfl_xor(S, 16);
        S += __shfl_xor(S, 32);
        if (lg == 0 && rl < rows) HS[rl * kPWaves + wv] = S;
      }
    } else {
      for (int rl = lane; rl < rows; rl += 64) HS[rl * kPWaves + wv] = 0.f;
    }
    __syncthreads();
    for (int t = tid; t < rows * 4; t += kPThreads) {
      const int rl = t >> 2, c = t & 3;
      const int chunk = 4 * b + c;
      if (chunk >= A.nch) continue;
      const float St = HS[rl * kPWaves + 2 * c] + HS[rl * kPWaves + 2 * c + 1];
      A.L[(int64_t)(row0 + rl) * A.nch + chunk] = make_float2(0.f, St);
      if (nonfinite(St)) set_flag(A.status, kFlagNonFinite);
    }
    __syncthreads();
  }
}

// Residual statistics on the W2-slice layout when the shape allows it
// (bf16 data and weights, rank 64/128/256, 16-byte aligned rows, V a multiple
// of 8); returns false to let the caller use the per-tile kernel.
bool launch_resid_slices(int R, int gamma, int V, int rank, float T, const void* U,
                         const void* W1, const void* W2t, const void* target, const int32_t* x,
                         const int32_t* rej_count, const int4* rej, const float2* lse_t,
                         const float* lse_d, float2* L, uint32_t* status, hipStream_t st,
                         hipError_t* err, bool overlap, bool feat_rows) {
  if (switches().force_per_step) return false;
  if ((V % 8) != 0 || (rank != 64 && rank != 128 && rank != 256)) return false;
  for (const void* p : {U, W1, W2t, target})
    if (reinterpret_cast<uintptr_t>(p) & 15) return false;
  ResidArgs A{};
  A.R = R; A.gamma = gamma; A.V = V; A.rank = rank; A.nch = (V + kChunk - 1) / kChunk;
  A.nslice = (V + kPSlice - 1) / kPSlice;
  A.scale2 = kLog2e / T;
  A.U = reinterpret_cast<const uint16_t*>(U);
  A.W1 = reinterpret_cast<const uint16_t*>(W1);
  A.W2t = reinterpret_cast<const uint16_t*>(W2t);
  A.target = reinterpret_cast<const uint16_t*>(target);
  A.x = x; A.rej_count = rej_count; A.rej = rej; A.lse_t = lse_t; A.lse_d = lse_d; A.L = L;
  A.status = status;
  A.feat_rows = feat_rows;
#define DSPARK_RS(KS_, OV_) hipLaunchKernelGGL((k_resid_stats<KS_, OV_>), dim3(A.nslice), dim3(kPThreads), 0, st, A)
  if (overlap) {
    if (rank == 64) DSPARK_RS(4, true); else if (rank == 128) DSPARK_RS(8, true); else DSPARK_RS(16, true);
  } else {
    if (rank == 64) DSPARK_RS(4, false); else if (rank == 128) DSPARK_RS(8, false); else DSPARK_RS(16, false);
  }
#undef DSPARK_RS
  *err = hipGetLastError();
  return true;
}

// Per-device facts for the persistent schedule (compute units; whether one
// workgroup of each instance fits per compute unit).
struct PersistInfo {
  // filled on first use; calls from several host threads may race to fill
  // an entry, all with the same value (atomic, relaxed)
  std::atomic<int> cus{-1};
  std::atomic<int> fits[3][2][2];
  PersistInfo() {
    for (auto& a : fits)
      for (auto& b : a)
        for (auto& c : b) c.store(-1, std::memory_order_relaxed);
  }
};
static PersistInfo g_pinfo[64];

template <int KS, bool G, bool F>
static bool persist_fits(PersistInfo& pi, int ki) {
  int f = pi.fits[ki][G][F].load(std::memory_order_relaxed);
  if (f < 0) {
    int nb = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &nb, reinterpret_cast<const void*>(k_draft_persistent<KS, G, F>), kPThreads, 0);
    f = (e == hipSuccess && nb >= 1) ? 1 : 0;
    (void)hipGetLastError();
    pi.fits[ki][G][F].store(f, std::memory_order_relaxed);
  }
  return f == 1;
}

template <int KS, bool G, bool F>
static hipError_t launch_persist_ks(PersistArgs& P, int grid, hipStream_t st) {
  void* args[] = {&P};
  return launch_coresident(reinterpret_cast<const void*>(k_draft_persistent<KS, G, F>), dim3(grid),
                           dim3(kPThreads), args, 0, st);
}

// The persistent schedule takes bf16 U and weights, rank 64/128/256, rows and
// weight tables 16-byte aligned, V a multiple of 8 with at most 512 entries per
// compute unit, and 16 request rows of U (16 gamma V entries) within 2 GiB (the
// U loads use 32-bit lane offsets).  DSPARK_DRAFT_KERNEL=steps in the
// environment selects the per-step schedule for every shape.
static int persistent_grid(int gamma, int V, int rank, bool u_bf16, bool w_bf16, bool u_vec,
                           const void* W1, const void* W2t, bool greedy, bool feat) {
  if (switches().force_per_step) return 0;
  if (!u_bf16 || !w_bf16 || !u_vec || (V % 8) != 0) return 0;
  if ((int64_t)32 * gamma * V >= ((int64_t)1 << 31)) return 0;
  if (rank != 64 && rank != 128 && rank != 256) return 0;
  if ((reinterpret_cast<uintptr_t>(W1) & 15) || (reinterpret_cast<uintptr_t>(W2t) & 15)) return 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  PersistInfo& pi = g_pinfo[dev];
  int cus = pi.cus.load(std::memory_order_relaxed);
  if (cus < 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 0;
    pi.cus.store(cus, std::memory_order_relaxed);
  }
  const int nslice = (V + kPSlice - 1) / kPSlice;
  if (cus < 1 || cus > kMaxGrid || nslice > cus || (V + kChunk - 1) / kChunk > kPMaxChunks)
    return 0;
  bool fits;
#define DSPARK_FITS(KS_, KI_, F_) \
  (greedy ? persist_fits<KS_, true, F_>(pi, KI_) : persist_fits<KS_, false, F_>(pi, KI_))
  if (feat) {
    if (rank == 64) fits = DSPARK_FITS(4, 0, true);
    else if (rank == 128) fits = DSPARK_FITS(8, 1, true);
    else fits = DSPARK_FITS(16, 2, true);
  } else {
    if (rank == 64) fits = DSPARK_FITS(4, 0, false);
    else if (rank == 128) fits = DSPARK_FITS(8, 1, false);
    else fits = DSPARK_FITS(16, 2, false);
  }
#undef DSPARK_FITS
  return fits ? cus : 0;
}

__global__ void k_zero_words(uint32_t* p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0u;
}

// Before the persistent launch: barrier flags to zero, drafted positions
// x[i][1..gamma] to -1 (not yet written), x[i][0] to the anchor.
__global__ void k_draft_prep(uint32_t* flags, int nflags, int32_t* x, const int32_t* x0, int R, int gamma) {
  const int t0 = blockIdx.x * blockDim.x + threadIdx.x, nt = gridDim.x * blockDim.x;
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < nflags; i += blockDim.x) flags[i] = 0u;
  const int64_t n = (int64_t)R * (gamma + 1);
  for (int64_t q = t0; q < n; q += nt) {
    const int64_t i = q / (gamma + 1);
    const int j = (int)(q - i * (gamma + 1));
    x[q] = (j == 0) ? x0[i] : -1;
  }
}

hipError_t launch_draft(int R, int gamma, int V, int rank, float T, uint64_t seed, uint64_t round,
                        const void* U, bool u_bf16, const void* W1, const void* W2t, bool w_bf16,
                        const int32_t* x0, int32_t* x, float* logp_d, float* lse_d, float* margin,
                        const DraftWs& ws, hipStream_t st, hipEvent_t* ev_begin, hipEvent_t* ev_end,
                        int* n_timed, const RnnArgs* rnn) {
  uint32_t* status = ws.status;
  float2* Lc = reinterpret_cast<float2*>(ws.draft_l);
  int* Ic = reinterpret_cast<int*>(ws.draft_i);
  const int nch = (V + kChunk - 1) / kChunk;
  const bool greedy = (T == 0.f);
  const float scale2 = greedy ? 1.f : kLog2e / T;
  const size_t usz = u_bf16 ? 2 : 4;
  const bool u_vec = ((reinterpret_cast<uintptr_t>(U) & 15) == 0) && (((size_t)V * usz) % 16 == 0);

  DraftPickArgs p{};
  p.R = R; p.gamma = gamma; p.k = 1; p.V = V; p.rank = rank; p.nch = nch;
  p.invT = greedy ? 1.f : 1.f / T; p.T = greedy ? 1.f : T; p.seed = seed; p.round = round;
  p.U = U; p.W1 = W1; p.W2t = W2t; p.x0 = x0; p.x = x; p.logp_d = logp_d; p.lse_d = lse_d;
  p.margin = margin; p.L = Lc; p.I = Ic; p.status = status;

  // RNN head: the features e_k come from the recurrent cell, run inside the
  // persistent launch before each step (its h part precomputed), or launched
  // before each step of the per-step schedule.  The fused form also needs
  // bf16 h / Wr with 16-byte aligned rows and a 16-byte aligned feature tensor.
  const void* feat = rnn ? rnn->feat : nullptr;
  p.feat = feat;
  const Switches sw = switches();
  const bool rnn_fused_ok =
      rnn && rnn->w_bf16 && rnn->h_bf16 && !sw.rnn_cell_valu &&
      ((reinterpret_cast<uintptr_t>(rnn->Wr) | reinterpret_cast<uintptr_t>(rnn->feat)) & 15) == 0 &&
      ((2 * rank + rnn->d) % 8) == 0;
  const int grid = (rnn && !rnn_fused_ok)
                       ? 0
                       : persistent_grid(gamma, V, rank, u_bf16, w_bf16, u_vec, W1, W2t, greedy,
                                         rnn != nullptr);
  // the Markov head with the pipelined kernel (request groups pipelined
  // across the steps, no grid barrier) when that switch selects it; else,
  // and for the debug margin output and the RNN head, one grid barrier per
  // step
  if (grid > 0 && !rnn && margin == nullptr && sw.draft_kernel == 1) {
    hipError_t e = hipSuccess;
    if (launch_draft_pipe(p, greedy, scale2, grid, sw.barrier_spins ? sw.barrier_spins : kBarrierSpins,
                          ws, st, ev_begin, ev_end, n_timed, &e))
      return e;
  }
  if (grid > 0) {
    PersistArgs P{};
    P.p = p;
    P.scale2 = scale2;
    P.nslice = (V + kPSlice - 1) / kPSlice;
    P.bar = ws.bar;
    P.spin_limit = sw.barrier_spins ? sw.barrier_spins : kBarrierSpins;
    const int prep_blocks = (int)std::min<int64_t>(64, ((int64_t)R * (gamma + 1) + 255) / 256);
    hipError_t e;
    if (rnn) {
      P.rP = rnn->P;
      P.rstate = rnn->state;
      P.rfeat = reinterpret_cast<uint16_t*>(rnn->feat);
      P.rWr = reinterpret_cast<const uint16_t*>(rnn->Wr);
      P.rd = rnn->d;
      if ((e = launch_rnn_hproj(*rnn, st)) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_draft_prep, dim3(prep_blocks), dim3(256), 0, st, P.bar, kMaxGrid, x, x0, R,
                       gamma);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (ev_begin && (e = hipEventRecord(ev_begin[0], st)) != hipSuccess) return e;
#define DSPARK_LP(KS_, F_) \
    (greedy ? launch_persist_ks<KS_, true, F_>(P, grid, st) : launch_persist_ks<KS_, false, F_>(P, grid, st))
    if (rnn) {
      if (rank == 64) e = DSPARK_LP(4, true);
      else if (rank == 128) e = DSPARK_LP(8, true);
      else e = DSPARK_LP(16, true);
    } else {
      if (rank == 64) e = DSPARK_LP(4, false);
      else if (rank == 128) e = DSPARK_LP(8, false);
      else e = DSPARK_LP(16, false);
    }
#undef DSPARK_LP
    if (e != hipSuccess) return e;
    if (ev_end && (e = hipEventRecord(ev_end[0], st)) != hipSuccess) return e;
    if (n_timed) *n_timed = 1;
    return hipSuccess;
  }

#define DSPARK_PICK(UT_, WT_, G_, NB_) \
    hipLaunchKernelGGL((k_draft_pick<UT_, WT_, G_>), dim3(NB_), dim3(256), 0, st, p)
#define DSPARK_PICK_ALL(NB_)                                                                          \
    if (u_bf16 && w_bf16) { if (greedy) DSPARK_PICK(uint16_t, uint16_t, true, NB_); else DSPARK_PICK(uint16_t, uint16_t, false, NB_); } \
    else if (u_bf16)      { if (greedy) DSPARK_PICK(uint16_t, float, true, NB_);    else DSPARK_PICK(uint16_t, float, false, NB_); }    \
    else if (w_bf16)      { if (greedy) DSPARK_PICK(float, uint16_t, true, NB_);    else DSPARK_PICK(float, uint16_t, false, NB_); }    \
    else                  { if (greedy) DSPARK_PICK(float, float, true, NB_);       else DSPARK_PICK(float, float, false, NB_); }
  if (rank == 0 && !rnn && ws.rows_l != nullptr) {
    // rank 0 (no transition bias): the positions are independent, so the
    // statistics of all R gamma rows of U are one launch (into the target-row
    // statistics region, unused until the verify) and the picks another
    RowStatsArgs a{};
    a.base = U; a.kind = kRowsAll; a.R = R; a.gamma = gamma; a.k = 0; a.V = V; a.nch = nch;
    a.nrows_cap = R * gamma; a.scale2 = scale2; a.vec_ok = u_vec;
    a.L = reinterpret_cast<float2*>(ws.rows_l); a.I = reinterpret_cast<int*>(ws.rows_i);
    a.status = status;
    hipError_t e;
    if (ev_begin && (e = hipEventRecord(ev_begin[0], st)) != hipSuccess) return e;
    if ((e = launch_row_stats(a, u_bf16, greedy, st)) != hipSuccess) return e;
    if (ev_end && (e = hipEventRecord(ev_end[0], st)) != hipSuccess) return e;
    p.all_pos = true;
    p.L = a.L;
    p.I = a.I;
    DSPARK_PICK_ALL(R * gamma)
    if (n_timed) *n_timed = 1;
    return hipGetLastError();
  }
  if (rnn) {
    const hipError_t e = launch_rnn_hproj(*rnn, st);
    if (e != hipSuccess) return e;
  }
  // the 512-thread pick of the persistent launch where its shape limits hold
  const bool fast_pick = u_bf16 && w_bf16 && (rank == 64 || rank == 128 || rank == 256) &&
                         nch <= kPMaxChunks;
  for (int k = 1; k <= gamma; ++k) {
    hipError_t e;
    if (rnn && (e = launch_rnn_cell(*rnn, k, st)) != hipSuccess) return e;
    if (ev_begin && (e = hipEventRecord(ev_begin[k - 1], st)) != hipSuccess) return e;
    if (rank == 0) {
      RowStatsArgs a{};
      a.base = U; a.kind = kRowsDraft; a.R = R; a.gamma = gamma; a.k = k; a.V = V; a.nch = nch;
      a.nrows_cap = R; a.scale2 = scale2; a.vec_ok = u_vec; a.L = Lc; a.I = Ic;
      a.status = status;
      e = launch_row_stats(a, u_bf16, greedy, st);
    } else {
      MarkovArgs a{};
      a.R = R; a.gamma = gamma; a.k = k; a.V = V; a.rank = rank; a.nch = nch; a.nrows_cap = R;
      a.U = U; a.W1v = feat ? feat : W1; a.W2tv = W2t; a.x0 = x0; a.x = x; a.feat_rows = feat != nullptr;
      a.scale2 = scale2; a.u_vec_ok = u_vec;
      a.L = Lc; a.I = Ic; a.status = status;
      e = launch_markov_stats(a, u_bf16, w_bf16, greedy ? kModeGreedy : kModeSample, st);
    }
    if (e != hipSuccess) return e;
    if (ev_end && (e = hipEventRecord(ev_end[k - 1], st)) != hipSuccess) return e;
    p.k = k;
    if (fast_pick) {
#define DSPARK_PICKP(KS_)                                                                     \
      if (greedy) hipLaunchKernelGGL((k_draft_pick_p<KS_, true>), dim3(R), dim3(kPThreads), 0, st, p, scale2); \
      else hipLaunchKernelGGL((k_draft_pick_p<KS_, false>), dim3(R), dim3(kPThreads), 0, st, p, scale2)
      if (rank == 64) { DSPARK_PICKP(4); }
      else if (rank == 128) { DSPARK_PICKP(8); }
      else { DSPARK_PICKP(16); }
#undef DSPARK_PICKP
    } else {
      DSPARK_PICK_ALL(R)
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
#undef DSPARK_PICK_ALL
#undef DSPARK_PICK
  if (n_timed) *n_timed = gamma;
  return hipSuccess;
}

}  // namespace dspark
