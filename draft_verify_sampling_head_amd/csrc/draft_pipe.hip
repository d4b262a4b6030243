// draft_pipe.hip -- the Markov draft head with request groups pipelined
// across the gamma sequential steps (one co-resident launch for the block).
//
// DSpark summary page, Method details (causal block distribution, Markov
// head): p_k(v | x_0, x_<k) = softmax(U_k + W1[x_{k-1}] W2)(v), sampled left to
// right.  Request i's step k depends only on request i's token x_{k-1}, so the
// requests are independent chains; the one-grid-barrier-per-step schedule
// (draft.hip) makes every chain wait for the slowest pick of the step.  Here
// the requests are split into groups of kGR rows and every workgroup streams
// the groups of all steps back to back, (k, g) in order:
//
//   tiles     workgroup b owns the vocabulary slice [512 b, 512 b + 512) with
//             its W2 slice in registers (the tile loop of persist_common.hpp);
//             for every row of the group it merges its four chunks into one
//             record: the chunk-level Gumbel winner of the slice (key
//             L_c + G_c, L_c = log sum_{v in c} exp(s(v))) and the slice's
//             log-mass, tagged with the launch and the step.
//   pick      request i is picked by workgroup i mod grid while the NEXT
//             group's tiles run, at service points between tiles: it reads
//             the slice records of i (all slices, tags checked), takes the
//             chunk winner c* and the normaliser, stages W1[x_{k-1}], the 128
//             W2t rows of c* and the U values of c* in LDS with direct-to-LDS
//             loads, and at a later service point rebuilds the 128 scores,
//             draws the in-chunk Gumbel winner and publishes x_k.
//   gather    the W1 rows of the group after the next are fetched into the
//             other LDS buffer as soon as its tokens are published.
//
// Nothing synchronises the grid: records carry tags, tokens start at -1 (set
// before the launch), and every cross-workgroup wait is bounded (past the
// spin limit it sets DSPARK_FLAG_BARRIER and every later wait returns at
// once, so the launch always ends).  A workgroup waiting for tokens keeps
// advancing its own pending pick, so the chains cannot deadlock: all tiles of
// step k need only the tokens of step k-1, and every pick of step k needs only
// the tiles of step k.
#include <atomic>
#include <cfloat>

#include "launch.hpp"
#include "persist_common.hpp"
#include "sampling.hpp"
#include "workspace.hpp"

namespace dspark {

constexpr int kGR = 128;                    // rows per request group
constexpr int kStagePad = 64;               // LDS pieces past a buffer (DMA tails, pick staging)
constexpr int kPipeMaxPicks = 8;            // requests per workgroup (R <= 8 grid)
constexpr uint32_t kSentinel = 0xFFFFFFFFu; // LDS word not yet written by a direct-to-LDS load

struct PipeArgs {
  DraftPickArgs p;                          // shapes, sampling constants, inputs and outputs
  float scale2;                             // log2(e)/T; 1 when greedy
  int nslice;                               // vocabulary slices = ceil(V / 512)
  int ngroups;                              // ceil(R / kGR)
  uint32_t spin_limit;                      // bounded wait
  uint64_t* rec;                            // [2][R][nslice] records, two words each
  const uint32_t* epoch_word;               // launch counter (advanced before the launch)
};

// Record words: (tag << 32) | payload.  Word A: the slice's chunk winner key
// (sampling) or maximum (greedy), tag = epoch << 8 | k << 2 | local chunk.
// Word B: the slice's log-mass (sampling) or first argmax (greedy), tag =
// epoch << 8 | k << 2.
__device__ __forceinline__ uint32_t rec_tag(uint32_t epoch, int k) {
  return (epoch << 8) | ((uint32_t)k << 2);
}
__device__ __forceinline__ uint64_t ld_coh64(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ int tid_here() { return tid_opaque(); }

// All LDS operations of this wave done (no wait on vector memory).
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Direct-to-LDS loads are not ordered with this wave's other vector-memory
// operations, so a count-based wait does not prove they have landed.  Every
// LDS slot such a load will write is first set to a sentinel by the same
// lane (wait_lgkm0 orders that store before the load is issued); the reader
// validates the contents (record tags, tokens >= 0, no sentinel words) and
// only falls back to a full vmcnt(0) wait when something is still missing.
__device__ __forceinline__ bool has_sentinel(const uint4& q) {
  return q.x == kSentinel || q.y == kSentinel || q.z == kSentinel || q.w == kSentinel;
}

// Direct-to-LDS gather of `rows` table rows (row rl starts at rowptr(rl), SEG
// 16-byte segments) into LDS rows of ROWP pieces (the pad piece re-reads
// segment 0; the pieces of the last wave instruction past the last row
// re-read it and land in the buffer's pad).  Issued only: the caller waits.
template <int SEG, int ROWP, typename F>
__device__ __forceinline__ void dma_rows(uint4* E, int rows, F rowptr) {
  const int tix = tid_here(), lane = tix & 63, wv = tix >> 6;
  const int npieces = rows * ROWP;
  for (int p0 = wv * 64; p0 < npieces; p0 += kPThreads) {
    const int p = p0 + lane;
    const int rl = min(p / ROWP, rows - 1), sp = p % ROWP;
    lds_dma16(rowptr(rl) + 8 * (sp < SEG ? sp : 0), E + p0);
  }
}
// The same, with every slot first set to the sentinel by the lane that loads it.
template <int SEG, int ROWP, typename F>
__device__ __forceinline__ void dma_rows_marked(uint4* E, int rows, F rowptr) {
  const int tix = tid_here(), lane = tix & 63, wv = tix >> 6;
  const int npieces = rows * ROWP;
  const uint4 sent = make_uint4(kSentinel, kSentinel, kSentinel, kSentinel);
  for (int p0 = wv * 64; p0 < npieces; p0 += kPThreads) E[p0 + lane] = sent;
  wait_lgkm0();
  for (int p0 = wv * 64; p0 < npieces; p0 += kPThreads) {
    const int p = p0 + lane;
    const int rl = min(p / ROWP, rows - 1), sp = p % ROWP;
    lds_dma16(rowptr(rl) + 8 * (sp < SEG ? sp : 0), E + p0);
  }
}

// Waits until at most N (0, 2 or 4) vector-memory operations of this wave are
// outstanding.  Vector-memory operations complete in issue order, so with
// `after` operations issued since a direct-to-LDS load, waiting for at most
// min(after, 4) (rounded down to even) outstanding completes that load.
__device__ __forceinline__ void wait_vm_after(int after) {
  if (after >= 4) __builtin_amdgcn_s_waitcnt(0x0F74);
  else if (after >= 2) __builtin_amdgcn_s_waitcnt(0x0F72);
  else __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Bounded polling helper: true once the launch has given up waiting.
__device__ __forceinline__ bool gave_up(const uint32_t* status) {
  return (__hip_atomic_load(const_cast<uint32_t*>(status), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) &
          kFlagBarrier) != 0;
}

// Coherent direct-to-LDS loads (device-scope, sc1: they see values other
// workgroups stored with device-coherent stores in this launch): 16 or 4
// bytes per lane from gptr to lds_wave_base + size * lane.  Issued from inline
// assembly, like lds_dma16, so that the compiler does not fence later LDS
// accesses behind them; the caller waits explicitly.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16_coh(const void* gptr, const void* lds_wave_base) {
  const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_wave_base);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off sc1"
               :: "s"(l), "v"(gptr) : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4_coh(const void* gptr, const void* lds_wave_base) {
  const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_wave_base);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off sc1"
               :: "s"(l), "v"(gptr) : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ float unif(float v) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

template <int KS>
struct PipeLds {
  static constexpr int SEG = 2 * KS, ROWP = SEG + 1;
  static constexpr int BUF = kGR * ROWP + kStagePad;   // pieces per buffer
  uint4 E[2][BUF];                 // W1 rows of a group; the idle buffer stages a pick
  float2 HS[kGR * kPWaves];        // per (row, wave) statistics of the group
  uint4 recs[256];                 // the pending pick's slice records (coherent loads)
  int tok[kGR];                    // tokens of the group being gathered (coherent loads)
  int lastx[kPipeMaxPicks];        // last token of each request this workgroup picks
  float fmax[kPWaves];
  float farg[kPWaves];
  int iarg[kPWaves];
  PickRed red[kPWaves];
  int vote[2][kPWaves];             // block votes, two alternating slot sets
};

// Service state.  Every wave runs the same state machine on the same inputs
// (block reductions and LDS contents read after barriers), so the state is
// identical in every wave; readfirstlane keeps it in scalar registers.
//   pick: 0 records not requested; 1 records requested (coherent DMA); 2
//         chunk staged (DMA of W2t rows, W1[x_{k-1}] and U values issued)
//   gath: 0 tokens not requested; 1 tokens requested; 2 W1 rows requested
template <int KS, bool GREEDY>
struct PipeCtx {
  const PipeArgs& P;
  PipeLds<KS>& L;
  uint32_t epoch;
  int req, pk, pstage;             // pending pick: request (-1 none), step, stage
  int chunk, prev;                 // c* and x_{k-1} (stage 2)
  float lse_hi, lse_lo;            // normaliser (stage 2), a double as two floats
  int gG, gstage;                  // gather: stream group, stage
  uint32_t spins;
  int vset;                        // slot set of the next block vote

  __device__ __forceinline__ PipeCtx(const PipeArgs& P_, PipeLds<KS>& L_, uint32_t e)
      : P(P_), L(L_), epoch(e) {
    req = -1; pk = 0; pstage = 0; chunk = 0; prev = 0; lse_hi = 0.f; lse_lo = 0.f;
    gG = -1; gstage = 0; spins = 0; vset = 0;
  }

  __device__ __forceinline__ int group_rows(int g) const { return min(kGR, P.p.R - g * kGR); }

  // Block-wide any(pred) (one barrier, LDS only: the library's vote reads the
  // workgroup size with vector-memory loads, whose wait would drain the U
  // prefetch).  Two slot sets alternate: a wave writes set s again only after
  // the barrier of the vote in between, which every wave reaches after
  // reading set s.
  __device__ __forceinline__ bool vote_any(bool pred) {
    const uint64_t m = __ballot(pred);
    const int wv = threadIdx.x >> 6, s = vset;
    if ((threadIdx.x & 63) == 0) L.vote[s][wv] = m != 0;
    lds_sync();
    int r = 0;
#pragma unroll
    for (int w = 0; w < kPWaves; ++w) r |= L.vote[s][w];
    vset = s ^ 1;
    return uni(r) != 0;
  }
  __device__ __forceinline__ bool vote_all(bool pred) { return !vote_any(!pred); }

  // bounded-wait bookkeeping (uniform): true when waiting must stop
  __device__ __forceinline__ bool spin_out() {
    const int stop = vote_any(threadIdx.x == 0 && gave_up(P.p.status));
    if (stop) return true;
    // each poll here waits for coherent loads (about a microsecond), so the
    // bound is the spin limit over 64
    if (++spins >= max(1u, P.spin_limit >> 6)) {
      if (threadIdx.x == 0) atomicOr(P.p.status, kFlagBarrier);
      return true;
    }
    __builtin_amdgcn_s_sleep(1);
    return false;
  }

  // ------------------------------------------------------------- picks
  // Outcome of a poll of data requested with coherent direct-to-LDS loads.
  static constexpr int kNotLanded = 0, kStale = 1, kReady = 2;

  // Coherent loads of the records of (req, pk) into L.recs (every slot first
  // set to the sentinel by the lane that loads it).
  __device__ __forceinline__ void records_request() {
    const DraftPickArgs& a = P.p;
    const int t = tid_here(), wv = t >> 6;
    if (wv < 4) {
      L.recs[t] = make_uint4(kSentinel, kSentinel, kSentinel, kSentinel);
      wait_lgkm0();
      const int sl = min(t, P.nslice - 1);
      lds_dma16_coh(P.rec + (((int64_t)(pk & 1) * a.R + req) * P.nslice + sl) * 2, L.recs + 64 * wv);
    }
    pstage = 1;
  }

  // Records of (req, pk) in L.recs: not landed yet, landed but some slice had
  // not published (stale tags), or all present.  A tag is never the
  // sentinel (its low byte is 4 k + chunk < 132).
  __device__ __forceinline__ int records_poll() {
    const int t = tid_here();
    const uint32_t tagB = rec_tag(epoch, pk);
    int landed = 1, valid = 1;
    if (t < P.nslice) {
      const uint4 r = L.recs[t];
      landed = !has_sentinel(r);
      valid = landed && ((r.y & ~3u) == tagB) && (r.w == tagB);
    }
    if (!vote_all(landed)) return kNotLanded;
    return vote_all(valid) ? kReady : kStale;
  }

  // All records present: the chunk-level winner and the normaliser; greedy:
  // the token.  Sampling: the chunk is staged in S (W2t rows of c*, W1[x_{k-1}],
  // the U values of c*; sentinel-marked direct-to-LDS loads).
  __device__ __forceinline__ void records_reduce(uint4* S) {
    const DraftPickArgs& a = P.p;
    const int t = tid_here(), i = req, k = pk;
    float key = -INFINITY, lb = -INFINITY;
    int idx = 0x7FFFFFFF;
    if (t < P.nslice) {
      const uint4 r = L.recs[t];
      key = __uint_as_float(r.x);
      if (GREEDY) {
        idx = (int)r.z;                       // first argmax of the slice
      } else {
        idx = 4 * t + (int)(r.y & 3u);        // chunk of the slice's winner
        lb = __uint_as_float(r.z);
      }
    }
    const int64_t o = (int64_t)i * a.gamma + (k - 1);
    if (GREEDY) {
      float v = key;
      block_argmax_v(v, idx, L.farg, L.iarg);
      int xk = idx;
      if (v == -INFINITY || xk < 0 || xk >= a.V) {
        if (t == 0) set_flag(a.status, kFlagNonFinite);
        xk = 0;
      }
      if (t == 0) {
        st_coh(a.x + (int64_t)i * (a.gamma + 1) + k, xk);
        a.logp_d[o] = 0.f;
        a.lse_d[o] = v;
        L.lastx[i / gridDim.x] = xk;
      }
      req = -1;
      pstage = 0;
      lds_sync();                               // reduction slots are reused
      return;
    }
    // normaliser over the slices' log-masses, and the chunk-level winner
    const float m = block_max_v(lb, L.fmax);
    PickRed pr{key, idx, (lb == -INFINITY) ? 0.f : __expf(lb - m)};
    const PickRed rr = block_pick_reduce(pr, L.red);
    const double lse = (double)m + log((double)rr.s);
    int c = rr.key == -INFINITY ? -1 : rr.idx;
    if (c < 0 || c >= a.nch || !(rr.s > 0.f) || nonfinite(m)) {
      if (t == 0) set_flag(a.status, kFlagNonFinite);
      if (c < 0 || c >= a.nch) c = 0;
    }
    chunk = uni(c);
    prev = uni(L.lastx[i / gridDim.x]);
    lse_hi = unif((float)lse);
    lse_lo = unif((float)(lse - (double)lse_hi));
    constexpr int SEG = PipeLds<KS>::SEG, ROWP = PipeLds<KS>::ROWP;
    const uint16_t* W2t = reinterpret_cast<const uint16_t*>(a.W2t);
    const uint16_t* W1 = reinterpret_cast<const uint16_t*>(a.W1);
    const uint16_t* U = reinterpret_cast<const uint16_t*>(a.U);
    const int base = chunk * kChunk;
    dma_rows_marked<SEG, ROWP>(S, kChunk,
                               [&](int rl) { return W2t + (int64_t)min(base + rl, a.V - 1) * a.rank; });
    if ((t >> 6) == 0) {
      const int lane = t & 63;
      const uint16_t* src;
      if (lane < SEG) {
        src = W1 + (int64_t)prev * a.rank + 8 * lane;
      } else {
        const int q = min(lane - SEG, 15);
        src = U + o * a.V + min(base + 8 * q, a.V - 8);
      }
      S[kChunk * ROWP + lane] = make_uint4(kSentinel, kSentinel, kSentinel, kSentinel);
      wait_lgkm0();
      lds_dma16(src, S + kChunk * ROWP);
    }
    pstage = 2;
    lds_sync();                               // reduction slots are reused
  }

  // The staged chunk: rebuild its 128 scores (four threads per entry), draw
  // the in-chunk Gumbel winner, publish x_k, log p_d and lse_d.  Returns
  // false, having written nothing, while some staged piece has not landed
  // (force: every load is known to have landed; the data read stands).
  __device__ __forceinline__ bool pick_compute(const uint4* S, bool force) {
    const DraftPickArgs& a = P.p;
    constexpr int SEG = PipeLds<KS>::SEG, ROWP = PipeLds<KS>::ROWP;
    constexpr int TPE = kPThreads / kChunk, NQ = SEG / TPE;
    static_assert(TPE == 4, "four threads per entry");
    const int t = tid_here(), i = req, k = pk;
    const int base = chunk * kChunk;
    const int e = t / TPE, h = t % TPE;
    const int v = base + e;
    const bool in = v < a.V;
    const uint4* wrow = S + e * ROWP + h * NQ;
    const uint4* erow = S + kChunk * ROWP + h * NQ;
    bool miss = false;
    float bsum = 0.f;
    // two pieces at a time: fully unrolled, every load would be hoisted and
    // the extra live registers spill in the tile loop around the call
#pragma unroll 2
    for (int q = 0; q < NQ; ++q) {
      const uint4 x = erow[q], w = wrow[q];
      miss |= has_sentinel(x) | has_sentinel(w);
      bsum = fmaf(bf16_lo(x.x), bf16_lo(w.x), bsum);
      bsum = fmaf(bf16_hi(x.x), bf16_hi(w.x), bsum);
      bsum = fmaf(bf16_lo(x.y), bf16_lo(w.y), bsum);
      bsum = fmaf(bf16_hi(x.y), bf16_hi(w.y), bsum);
      bsum = fmaf(bf16_lo(x.z), bf16_lo(w.z), bsum);
      bsum = fmaf(bf16_hi(x.z), bf16_hi(w.z), bsum);
      bsum = fmaf(bf16_lo(x.w), bf16_lo(w.w), bsum);
      bsum = fmaf(bf16_hi(x.w), bf16_hi(w.w), bsum);
    }
    const uint4 up = S[kChunk * ROWP + SEG + (e >> 3)];
    miss |= has_sentinel(up);
    if (vote_any(miss) && !force) return false;
    bsum += dpp_f<kDppXor1>(bsum);
    bsum += dpp_f<kDppXor2>(bsum);
    const float u = u_piece(up, e & 7);
    const float sv = in ? (u + bsum) / a.T : -INFINITY;
    float key = -INFINITY;
    int kid = 0x7FFFFFFF;
    if (h == 0 && in) {
      const uint4 blk = stream_block(a.seed, a.round, kTagDraftElem, (uint32_t)i, (uint32_t)k, (uint32_t)v >> 2);
      key = sv + gumbel_of(word_of(blk, (uint32_t)v & 3u));
      kid = v;
    }
    float best = key;
    int bidx = kid;
    block_argmax_v(best, bidx, L.farg, L.iarg);
    int xk = best == -INFINITY ? -1 : bidx;
    if (xk < 0) {
      if (t == 0) set_flag(a.status, kFlagNonFinite);
      xk = base;
    }
    if (in && nonfinite(sv)) set_flag(a.status, kFlagNonFinite);
    if (t == TPE * (xk - base)) {
      const int64_t o = (int64_t)i * a.gamma + (k - 1);
      const double lse = (double)lse_hi + (double)lse_lo;
      a.logp_d[o] = (float)((double)sv - lse);
      a.lse_d[o] = (float)lse;
      st_coh(a.x + (int64_t)i * (a.gamma + 1) + k, xk);
      L.lastx[i / gridDim.x] = xk;
    }
    req = -1;
    pstage = 0;
    lds_sync();                               // staging and slots are reused
    return true;
  }

  // One stage of the pending pick at a service point; nothing waits here.
  __device__ __forceinline__ void pick_step(uint4* S) {
    if (pstage == 0) {
      records_request();
    } else if (pstage == 1) {
      const int r = records_poll();
      if (r == kReady) records_reduce(S);
      else if (r == kStale) records_request();
    } else {
      pick_compute(S, false);
    }
  }

  // Blocking (bounded) completion of the pending pick: after a full wait
  // every requested load has landed, so each poll decides.
  __device__ __forceinline__ void pick_finish(uint4* S) {
    spins = 0;
    while (req >= 0) {
      if (pstage == 0) records_request();
      wait_vm_after(0);
      __syncthreads();
      if (pstage == 1) {
        if (records_poll() == kReady) {
          records_reduce(S);
          continue;
        }
        if (spin_out()) {
          // gave up (DSPARK_FLAG_BARRIER is set): a placeholder draw keeps the
          // outputs in range; they are invalid, as the flag says
          if (threadIdx.x == 0) {
            const DraftPickArgs& a = P.p;
            const int64_t o = (int64_t)req * a.gamma + (pk - 1);
            a.logp_d[o] = 0.f;
            a.lse_d[o] = 0.f;
            st_coh(a.x + (int64_t)req * (a.gamma + 1) + pk, 0);
            L.lastx[req / gridDim.x] = 0;
          }
          req = -1;
          pstage = 0;
          __syncthreads();
          break;
        }
        records_request();
      } else {
        pick_compute(S, true);
      }
    }
  }

  // At the end of stream group G (k, g): the pending pick (registered at the
  // end of G-1) is completed, then the pick of group (k, g) is registered if
  // this workgroup picks one of its rows (request i is picked by workgroup
  // i mod grid; grid >= kGR, so a group holds at most one request of a
  // workgroup).  With a single group per step the next group needs that
  // pick's token at once, so it is completed here too.
  __device__ __forceinline__ void pick_settle(int G, int k, int g) {
    int todo = -1;
    {
      const int row0 = g * kGR, rows = group_rows(g);
      const int NB = gridDim.x, b = blockIdx.x;
      const int i = (row0 <= b) ? b : b + ((row0 - b + NB - 1) / NB) * NB;
      if (i >= row0 && i < row0 + rows) todo = i;
    }
    if (req >= 0) pick_finish(L.E[(G + 1) & 1]);
    if (todo >= 0) {
      req = uni(todo);
      pk = uni(k);
      pstage = 0;
      if (P.ngroups == 1) pick_finish(L.E[(G + 1) & 1]);
    }
  }

  // ------------------------------------------------------------- gathers
  // The tokens x_{k-1} of group (k, g) into L.tok by coherent direct-to-LDS
  // loads into slots set to -2 first: the anchors (k == 1, an input; a -2
  // there is an invalid token and times out as unpublished), else the tokens
  // other workgroups published (>= 0; unpublished ones read -1).  No plain
  // load: its wait would also drain the U prefetch.
  __device__ __forceinline__ void tokens_request(int k, int g) {
    const DraftPickArgs& a = P.p;
    const int t = tid_here(), wv = t >> 6;
    if (wv < kGR / 64) {
      const int row = g * kGR + min(t, group_rows(g) - 1);
      L.tok[t] = -2;
      wait_lgkm0();
      const int32_t* src = (k == 1) ? a.x0 + row : a.x + (int64_t)row * (a.gamma + 1) + (k - 1);
      lds_dma4_coh(src, L.tok + 64 * wv);
    }
    gstage = 1;
  }
  __device__ __forceinline__ int tokens_poll(int k, int g) {
    const int t = tid_here(), rows = group_rows(g);
    int landed = 1, valid = 1;
    if (t < rows) {
      const int v = L.tok[t];
      landed = v != -2;
      valid = k == 1 || v >= 0;
    }
    if (!vote_all(landed)) return kNotLanded;
    return vote_all(valid) ? kReady : kStale;
  }
  // The W1 rows of the tokens in L.tok into Ebuf (issued, not waited for).
  __device__ __forceinline__ void tokens_gather(int k, int g, uint4* Ebuf) {
    const DraftPickArgs& a = P.p;
    const int t = tid_here(), rows = group_rows(g);
    if (t < rows) {
      const int pv = L.tok[t];
      if (pv >= a.V || (k == 1 && pv < 0)) set_flag(a.status, kFlagBadToken);
    }
    constexpr int SEG = PipeLds<KS>::SEG, ROWP = PipeLds<KS>::ROWP;
    const uint16_t* W1 = reinterpret_cast<const uint16_t*>(a.W1);
    dma_rows<SEG, ROWP>(Ebuf, rows, [&](int rl) {
      const int pv = L.tok[rl];
      return W1 + (int64_t)((pv < 0 || pv >= a.V) ? 0 : pv) * a.rank;
    });
    gstage = 2;
  }

  // Service point inside the tile loop of stream group G: one stage of the
  // pending pick (of group G-1) and one stage of the gather of group G+1.
  // Both use the buffer group G does not: the pick stages there first, the
  // W1 rows go there once it is done (the tokens are requested and polled
  // meanwhile).  Nothing waits: polls find data not yet landed and look
  // again later.
  __device__ __forceinline__ void service(int G) {
    uint4* S = L.E[(G + 1) & 1];
    if (req >= 0) pick_step(S);
    const int G1 = G + 1, k1 = G1 / P.ngroups + 1, g1 = G1 % P.ngroups;
    if (k1 > P.p.gamma || gG == G1) return;
    if (gstage == 0) {
      tokens_request(k1, g1);
    } else {
      const int r = tokens_poll(k1, g1);
      if (r == kReady) {
        if (req < 0) {
          tokens_gather(k1, g1, S);
          gG = uni(G1);
        }
      } else if (r == kStale) {
        tokens_request(k1, g1);
      }
    }
  }

  // The W1 rows of stream group G in its buffer.  Normally a service point of
  // group G-1 issued the gather, and the full wait after that group's tile
  // loop completed it.  Otherwise: the tokens (polls after full waits), the
  // gather and the wait for its loads.  The picks that publish these tokens
  // (group G - ngroups) are complete: each workgroup finishes a pick at the
  // end of the group after the one that registered it, or at once when a
  // step has a single group.
  __device__ __forceinline__ void ensure_gather(int G) {
    if (gG != G) {
      const int k = G / P.ngroups + 1, g = G % P.ngroups;
      uint4* Ebuf = L.E[G & 1];
      spins = 0;
      if (gstage != 1) tokens_request(k, g);
      for (;;) {
        wait_vm_after(0);
        __syncthreads();
        if (tokens_poll(k, g) == kReady) break;
        if (spin_out()) {
          // give up (flag set): row 0 for the missing tokens
          if (threadIdx.x < kGR && L.tok[threadIdx.x] < 0) L.tok[threadIdx.x] = 0;
          __syncthreads();
          break;
        }
        tokens_request(k, g);
      }
      tokens_gather(k, g, Ebuf);
      gG = uni(G);
      wait_vm_after(0);
      __syncthreads();
    }
    gstage = 0;
  }
};

// U of one wave as one stream of 16-row tiles over the whole launch.  A step
// has T = ceil(R / 16) row tiles, padded to an even count Tp (an extra tile
// re-reads the step's last tile; its rows past R are computed and never
// merged), so that every group, kGR rows = 8 tiles or the step's padded
// remainder, has an even tile count and its two U register sets keep their
// roles from group to group (a swap would read registers whose loads are in
// flight, i.e. wait for them).  Stream tile t is padded tile t mod Tp of step
// t / Tp + 1: a group's loads two tiles ahead run on into the next group, so
// that group's first tiles are in flight while this one ends; past the
// launch's last tile the stream re-reads that tile.  Lane offsets are 32-bit
// (16 rows of U fit in 2 GiB, checked on the host).
struct PipeUStream {
  const char* base;                           // U, row 0 of step 1
  int64_t rbytes;                             // bytes per 16 rows (all steps)
  int64_t kbytes;                             // bytes per step within a row
  uint32_t v0, v1, l0, l1;                    // lane offsets: full tiles, a step's last tile
  int T, Tp, nsteps;                          // tiles per step, padded, steps
  int k0, rt0;                                // tile 0 of the current group: step - 1, row tile
  __device__ __forceinline__ void init(const uint16_t* U, int R, int V, int gamma, int wslice,
                                       const bool (&uok)[2], bool full) {
    const int lane = threadIdx.x & 63, ln = lane & 15, lg = lane >> 4;
    const int64_t rstride = (int64_t)gamma * V;
    T = (R + 15) / 16;
    Tp = 2 * ((R + 31) / 32);
    nsteps = gamma;
    const int e0 = (full || uok[0]) ? wslice + slice_entry(lg, 0) : 0;
    const int e1 = (full || uok[1]) ? wslice + slice_entry(lg, 8) : 0;
    const int lrow_last = min(16 * (T - 1) + ln, R - 1) - 16 * (T - 1);
    v0 = (uint32_t)(2 * ((int64_t)ln * rstride + e0));
    v1 = (uint32_t)(2 * ((int64_t)ln * rstride + e1));
    l0 = (uint32_t)(2 * ((int64_t)lrow_last * rstride + e0));
    l1 = (uint32_t)(2 * ((int64_t)lrow_last * rstride + e1));
    base = reinterpret_cast<const char*>(U);
    rbytes = 32 * rstride;
    kbytes = 2 * (int64_t)V;
    k0 = 0;
    rt0 = 0;
  }
  // tiles of row group g (kGR rows; the last group of a step may be partial)
  static __device__ __forceinline__ int group_tiles_of(int rows) { return 2 * ((rows + 31) / 32); }
  __device__ __forceinline__ void group(int k, int g) {   // k: step (1-based), g: row group
    k0 = k - 1;
    rt0 = g * (kGR / 16);
  }
  // tile i of the current group (i may run past the group); i is wave-uniform
  __device__ __forceinline__ void load(uint4 (&dst)[2], int i) const {
    int kk = k0, rt = rt0 + i;
    while (rt >= Tp) {
      rt -= Tp;
      ++kk;
    }
    if (kk >= nsteps) {                       // past the launch: its last tile again
      kk = nsteps - 1;
      rt = T - 1;
    }
    rt = min(rt, T - 1);
    const bool last = rt == T - 1;
    const char* p = base + kk * kbytes + rt * rbytes;
    dst[0] = ld_stream16(p + (last ? l0 : v0));
    dst[1] = ld_stream16(p + (last ? l1 : v1));
  }
};

// The tile loop of one group (persist_common.hpp's pipeline) with a service
// point before each step after the first: sp(j) runs between the epilogue of
// tile j-1 and the step that draws tile j+1.  Every tile's epilogue refills
// its U registers with the tile two ahead (into the next group at the end);
// ntiles is even, so on return ua and ub hold the next group's tiles 0 and 1.
// Every wave calls sp the same number of times.
template <int KT, int ROWP, bool GREEDY, bool MASK, typename SP>
__device__ __forceinline__ void group_tiles(const bf16x8_t (&Af)[4][KT], const uint4* E, float2* HS,
                                            const PipeUStream& us, int ntiles, uint4 (&ua)[2],
                                            uint4 (&ub)[2], int wslice, const bool (&uok)[2], float s2,
                                            SP&& sp) {
  // lane-derived offsets are recomputed at each use (from the opaque thread
  // index): kept live across the loop they would be spilled, and a reload
  // from scratch waits for the U loads in flight
  auto store = [&](int i, const EpiState& st) __attribute__((always_inline)) {
    const int t = tid_opaque(), ln = t & 15, lg = (t >> 4) & 3, wv = t >> 6;
    if (lg == 0) HS[(16 * i + ln) * kPWaves + wv] = make_float2(st.m, GREEDY ? __int_as_float(st.bi) : st.s0);
  };
  auto fresh = [&]() __attribute__((always_inline)) {
    EpiState st;
    st.m = -INFINITY; st.s0 = 0.f; st.s1 = 0.f; st.m2 = -FLT_MAX; st.bi = 0x7FFFFFFF;
    return st;
  };
  auto step2 = [&](f32x4_t (&acc_cur)[4], f32x4_t (&acc_next)[4], uint4 (&un)[2], int i)
      __attribute__((always_inline)) {
    const int t = tid_opaque(), ln = t & 15, lg = (t >> 4) & 3;
    zero_acc(acc_next);
    EpiState st = fresh();
    mfma_with_epilogue<KT, GREEDY, MASK>(acc_next, Af, E + (16 * (i + 1) + ln) * ROWP + lg, acc_cur, un,
                                         us, i + 2, uok, s2, wslice + 8 * lg, st);
    store(i, st);
  };
  auto last = [&](f32x4_t (&acc)[4], uint4 (&un)[2], int i) __attribute__((always_inline)) {
    const int t = tid_opaque(), lg = (t >> 4) & 3;
    EpiState st = fresh();
    epilogue_all<GREEDY, MASK>(st, acc, un, uok, s2, wslice + 8 * lg);
    us.load(un, i + 2);
    store(i, st);
  };
  f32x4_t accA[4], accB[4];
  zero_acc(accA);
  {
    const int t = tid_opaque();
    tile_mfma<KT>(accA, Af, E + (t & 15) * ROWP + ((t >> 4) & 3));
  }
  for (int i = 0;; i += 2) {                  // pairs of tiles (ntiles is even)
    if (i > 0) sp(i);
    step2(accA, accB, ua, i);
    sp(i + 1);
    if (i + 2 == ntiles) {
      last(accB, ub, i + 1);
      break;
    }
    step2(accB, accA, ub, i + 1);
  }
}

template <int KS, bool GREEDY>
__global__ __launch_bounds__(kPThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_draft_pipe(PipeArgs P) {
  constexpr int SEG = 2 * KS, ROWP = SEG + 1, KT = KS / 2;
  static_assert(KS % 2 == 0, "rank must be a multiple of 32");
  __shared__ PipeLds<KS> L;
  const DraftPickArgs& a = P.p;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int b = blockIdx.x;
  const int V = a.V, R = a.R;
  const int wslice = b * kPSlice + 64 * wv;
  const bool slice_active = b < P.nslice;
  const bool wave_active = slice_active && wslice < V;
  const float s2 = P.scale2;
  const uint16_t* U = reinterpret_cast<const uint16_t*>(a.U);
  const uint16_t* W2t = reinterpret_cast<const uint16_t*>(a.W2t);

  bf16x8_t Af[4][KT];
  load_w2_slice<KT>(Af, W2t, a.rank, wslice, V, wave_active);
  const int lg = lane >> 4;
  bool uok[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) uok[q] = wave_active && wslice + slice_entry(lg, 8 * q) + 8 <= V;
  const bool wave_full = wave_active && wslice + 64 <= V;

  PipeCtx<KS, GREEDY> cx(P, L, *P.epoch_word);
  // x_0 of the requests this workgroup picks (then each pick's own token)
  if (tid < kPipeMaxPicks) {
    const int i = b + tid * (int)gridDim.x;
    int x0 = (i < R) ? a.x0[i] : 0;
    if (i < R && (x0 < 0 || x0 >= V)) set_flag(a.status, kFlagBadToken);
    L.lastx[tid] = (x0 < 0 || x0 >= V) ? 0 : x0;
  }
  __syncthreads();
  PipeUStream us;
  us.init(U, R, V, a.gamma, wslice, uok, wave_full);
  uint4 ua[2], ub[2];
  if (wave_active) {                          // tiles 0 and 1 of the first group
    us.load(ua, 0);
    us.load(ub, 1);
  }
  const int NG = P.ngroups, NS = a.gamma * NG;
  for (int G = 0; G < NS; ++G) {
    const int k = G / NG + 1, g = G % NG;
    const int row0 = g * kGR, rows = min(kGR, R - row0);
    const int ntiles = PipeUStream::group_tiles_of(rows);   // even
    // ---- W1 rows of this group in E[G & 1]
    cx.ensure_gather(G);
    const uint4* E = L.E[G & 1];
    us.group(k, g);
    auto sp = [&](int j) __attribute__((always_inline)) { (void)j; cx.service(G); };
    if (wave_active) {
      // one (masked) expansion for every slice keeps the kernel small
      group_tiles<KT, ROWP, GREEDY, true>(Af, E, L.HS, us, ntiles, ua, ub, wslice, uok, s2, sp);
    } else {
      const float2 empty = make_float2(-INFINITY, GREEDY ? __int_as_float(0x7FFFFFFF) : 0.f);
      for (int rl = lane; rl < rows; rl += 64) L.HS[rl * kPWaves + wv] = empty;
      for (int j = 1; j < ntiles; ++j) sp(j);
    }
    // completes what service points issued (a gather or staging) and the
    // next group's first U tiles, issued during this group's last two tiles
    wait_vm_after(0);
    __syncthreads();
    // ---- the slice's record of every row of the group: four threads per row
    if (slice_active) {
      const uint32_t tag = rec_tag(cx.epoch, k);
      const int t = tid;                      // rows * 4 <= 512
      const int rl = t >> 2, c = t & 3;
      const int chunk = 4 * b + c;
      const bool valid_row = rl < rows;
      if (valid_row) {
        const int row = row0 + rl;
        const float2 h0 = L.HS[rl * kPWaves + 2 * c], h1 = L.HS[rl * kPWaves + 2 * c + 1];
        uint64_t* q = P.rec + (((int64_t)(k & 1) * R + row) * P.nslice + b) * 2;
        if (GREEDY) {
          float bv = h0.x;
          int bi = __float_as_int(h0.y);
          argmax_merge(bv, bi, h1.x, __float_as_int(h1.y));
          if (chunk >= a.nch) { bv = -INFINITY; bi = 0x7FFFFFFF; }
          if (nonfinite(bv) && chunk < a.nch) set_flag(a.status, kFlagNonFinite);
          // first argmax over the quad (ties: lower entry)
#pragma unroll
          for (int o = 1; o <= 2; o <<= 1) {
            const float vo = __shfl_xor(bv, o);
            const int io = __shfl_xor(bi, o);
            argmax_merge(bv, bi, vo, io);
          }
          if (c == 0) {
            st_coh64(q, ((uint64_t)tag << 32) | __float_as_uint(bv));
            st_coh64(q + 1, ((uint64_t)tag << 32) | (uint32_t)bi);
          }
        } else {
          const float Mn = fmaxf(h0.x, h1.x);
          const float Mr = (Mn == -INFINITY) ? 0.f : Mn;
          const float St = h0.y * __builtin_amdgcn_exp2f(fmaf(-Mr, s2, scaled_ref(h0.x, s2))) +
                           h1.y * __builtin_amdgcn_exp2f(fmaf(-Mr, s2, scaled_ref(h1.x, s2)));
          const bool valid = chunk < a.nch && St > 0.f && Mn != -INFINITY;
          if (chunk < a.nch && (nonfinite(St) || Mn == INFINITY)) set_flag(a.status, kFlagNonFinite);
          // chunk log-mass L_c = M/T + ln S (natural units)
          const float Lc = valid ? Mn / a.T + __logf(St) : -INFINITY;
          float key = Lc;
          if (a.nch > 1) {
            const uint4 blk = stream_block(a.seed, a.round, kTagDraftChunk, (uint32_t)row, (uint32_t)k,
                                           (uint32_t)b);
            key = valid ? Lc + gumbel_of(word_of(blk, (uint32_t)c)) : -INFINITY;
          }
          // quad: winner (ties: lower chunk) and log-sum-exp of the four masses
          int ci = c;
          float mx = Lc;
#pragma unroll
          for (int o = 1; o <= 2; o <<= 1) {
            const float ko = __shfl_xor(key, o);
            const int co = __shfl_xor(ci, o);
            argmax_merge(key, ci, ko, co);
            mx = fmaxf(mx, __shfl_xor(mx, o));
          }
          float se = (Lc == -INFINITY) ? 0.f : __expf(Lc - mx);
          se += __shfl_xor(se, 1);
          se += __shfl_xor(se, 2);
          const float Lb = (mx == -INFINITY) ? -INFINITY : mx + __logf(se);
          if (c == 0) {
            st_coh64(q, ((uint64_t)(tag | (uint32_t)(ci & 3)) << 32) | __float_as_uint(key));
            st_coh64(q + 1, ((uint64_t)tag << 32) | __float_as_uint(Lb));
          }
        }
      }
    }
    // ---- the pick of the previous group must be done before this group's
    // own is registered (it normally finished at a service point)
    cx.pick_settle(G, k, g);
    lds_sync();                               // HS is rewritten by the next group
  }
  if (cx.req >= 0) cx.pick_finish(L.E[NS & 1]);   // the last group's pick
}

// ----------------------------------------------------------------- launch
__global__ void k_pipe_prep(uint32_t* epoch_word, int32_t* x, const int32_t* x0, int R, int gamma) {
  const int t0 = blockIdx.x * blockDim.x + threadIdx.x, nt = gridDim.x * blockDim.x;
  if (t0 == 0) *epoch_word += 1u;
  const int64_t n = (int64_t)R * (gamma + 1);
  for (int64_t q = t0; q < n; q += nt) {
    const int64_t i = q / (gamma + 1);
    const int j = (int)(q - i * (gamma + 1));
    x[q] = (j == 0) ? x0[i] : -1;
  }
}

struct PipeInfo {
  // filled on first use (atomic, relaxed: racing fills store the same value)
  std::atomic<int> fits[3][2];
  PipeInfo() {
    for (auto& a : fits)
      for (auto& c : a) c.store(-1, std::memory_order_relaxed);
  }
};
static PipeInfo g_pipe[64];

template <int KS, bool G>
static bool pipe_fits(int dev, int ki) {
  int f = g_pipe[dev].fits[ki][G].load(std::memory_order_relaxed);
  if (f < 0) {
    int nb = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &nb, reinterpret_cast<const void*>(k_draft_pipe<KS, G>), kPThreads, 0);
    f = (e == hipSuccess && nb >= 1) ? 1 : 0;
    (void)hipGetLastError();
    g_pipe[dev].fits[ki][G].store(f, std::memory_order_relaxed);
  }
  return f == 1;
}

template <int KS, bool G>
static hipError_t launch_pipe_ks(PipeArgs& P, int grid, hipStream_t st) {
  void* args[] = {&P};
  return launch_coresident(reinterpret_cast<const void*>(k_draft_pipe<KS, G>), dim3(grid),
                           dim3(kPThreads), args, 0, st);
}

// Launches the pipelined draft (the caller has checked the persistent
// schedule's shape limits and that `grid` workgroups, one per compute unit,
// cover the vocabulary slices).  Returns false, launching nothing, when the
// kernel does not fit one workgroup per compute unit or the grid is smaller
// than a request group.
bool launch_draft_pipe(const DraftPickArgs& p, bool greedy, float scale2, int grid,
                       uint32_t spin_limit, const DraftWs& ws, hipStream_t st, hipEvent_t* ev_begin,
                       hipEvent_t* ev_end, int* n_timed, hipError_t* err) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
  if (grid < kGR || grid > 1024 || ws.rec == nullptr) return false;
  if ((int64_t)p.R > (int64_t)kPipeMaxPicks * grid) return false;
  const int ki = p.rank == 64 ? 0 : p.rank == 128 ? 1 : 2;
  bool fits;
  if (p.rank == 64) fits = greedy ? pipe_fits<4, true>(dev, ki) : pipe_fits<4, false>(dev, ki);
  else if (p.rank == 128) fits = greedy ? pipe_fits<8, true>(dev, ki) : pipe_fits<8, false>(dev, ki);
  else fits = greedy ? pipe_fits<16, true>(dev, ki) : pipe_fits<16, false>(dev, ki);
  if (!fits) return false;
  PipeArgs P{};
  P.p = p;
  P.scale2 = scale2;
  P.nslice = (p.V + kPSlice - 1) / kPSlice;
  P.ngroups = (p.R + kGR - 1) / kGR;
  P.spin_limit = spin_limit;
  P.rec = reinterpret_cast<uint64_t*>(ws.rec);
  P.epoch_word = ws.status + 2;
  const int prep_blocks = (int)std::min<int64_t>(64, ((int64_t)p.R * (p.gamma + 1) + 255) / 256);
  hipLaunchKernelGGL(k_pipe_prep, dim3(prep_blocks), dim3(256), 0, st, ws.status + 2, p.x, p.x0, p.R,
                     p.gamma);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && ev_begin) e = hipEventRecord(ev_begin[0], st);
  if (e == hipSuccess) {
    if (p.rank == 64) e = greedy ? launch_pipe_ks<4, true>(P, grid, st) : launch_pipe_ks<4, false>(P, grid, st);
    else if (p.rank == 128) e = greedy ? launch_pipe_ks<8, true>(P, grid, st) : launch_pipe_ks<8, false>(P, grid, st);
    else e = greedy ? launch_pipe_ks<16, true>(P, grid, st) : launch_pipe_ks<16, false>(P, grid, st);
  }
  if (e == hipSuccess && ev_end) e = hipEventRecord(ev_end[0], st);
  if (e == hipSuccess && n_timed) *n_timed = 1;
  *err = e;
  return true;
}

}  // namespace dspark

