// persist_common.hpp -- device pieces shared by the persistent draft kernels
// (draft.hip: one grid barrier per step; draft_pipe.hip: request groups
// pipelined across steps): the register-resident W2 slice, the software-
// pipelined MFMA tile loop with its statistics epilogue, cross-workgroup
// coherent accesses and the block reductions of the 512-thread pick.
#pragma once
#include <cfloat>

#include "launch.hpp"
#include "sampling.hpp"

namespace dspark {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// A streamed 16-byte load (non-temporal: U is read once per step, so it is
// not kept in the caches in place of W2t and W1 rows, which the picks and
// gathers read again).
__device__ __forceinline__ uint4 ld_stream16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

struct DraftPickArgs {
  int R, gamma, k, V, rank, nch;
  float invT;               // 1/T (sampling)
  float T;                  // T (sampling; 1 when greedy)
  uint64_t seed, round;
  const void* U;
  const void* W1;
  const void* W2t;
  const void* feat;         // nullable: per-position bias features [R][gamma][rank] (RNN head)
  bool all_pos;             // rank 0: block b picks position b % gamma + 1 of request b / gamma,
                            // statistics row b (all positions in one launch)
  const int32_t* x0;
  int32_t* x;
  float* logp_d;
  float* lse_d;
  float* margin;
  const float2* L;          // [R][nch] chunk (max, scaled sum) or (max, -) when greedy
  const int* I;             // [R][nch] chunk argmax (greedy)
  uint32_t* status;
};

// ============================================================= persistent
// Workgroup b (512 threads, eight waves) owns vocabulary slice [512 b, 512 b +
// 512): wave w holds entries 512 b + 64 w + [0, 64) of W2 as the A operands of
// v_mfma_f32_16x16x32_bf16 (four 16-entry M tiles x rank/32 k-steps, loaded
// once).  The requests are the N dimension: 16-row tiles whose B operands
// (W1[x_{k-1}] rows) are read from LDS, and U seeds the accumulators.  Entry
// order inside a wave (slice_entry): lane (n, g) of a 16x16 result holds two
// runs of 8 consecutive entries of request row n, 8 g + [0, 8) and 32 + 8 g +
// [0, 8), so the 16 rows x 4 lane groups of one U load instruction read 64
// contiguous bytes per row.  Each lane keeps its own partial statistics (no
// cross-lane work in the tile loop); a row's 8 partials per 128-entry chunk
// are merged once the whole group is done.
constexpr int kPThreads = 512;
constexpr int kPWaves = 8;
constexpr int kPSlice = 512;                // vocabulary entries per workgroup
constexpr int kPRows = 256;                 // requests per row group (LDS-resident W1 rows)
constexpr int kPMaxChunks = 2048;           // chunk statistics per pick (four per thread)

// Grid-wide barrier number `epoch` (1-based) over gridDim.x co-resident
// workgroups, as a flag array: workgroup b stores `epoch` in its own word
// flags[b] and polls all gridDim.x words until every one has reached `epoch`.
// No word takes more than one store per barrier, so nothing serialises on a
// shared counter.  Before the flag store every wave waits for its own memory
// operations to complete; flags are written and read with relaxed
// device-scope atomics.  The wait is bounded: past spin_limit polls the
// workgroup sets kFlagBarrier and stops waiting, and every later barrier of
// the launch returns at once, so the kernel always runs to its end.
constexpr int kMaxGrid = 1024;              // flag words in the workspace

// s_waitcnt vmcnt(0) (gfx9 encoding: expcnt and lgkmcnt fields at their
// maxima).  Placed where no useful load is in flight, it clears the
// compiler's record of possibly pending loads, which otherwise merges across
// the step loop into a full wait at the first LDS store of every tile.
__device__ __forceinline__ void wait_vm_zero() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Arrival: every wave first waits until its own stores have completed (the
// workgroup barrier alone does not wait for them), then the workgroup barrier,
// then the workgroup's flag is raised.  The data the flag publishes is
// written with device-coherent stores, so completion makes it visible to
// every workgroup that later sees the flag.
__device__ __forceinline__ void grid_arrive(uint32_t* flags, uint32_t epoch) {
  wait_vm_zero();
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_store(flags + blockIdx.x, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every workgroup has arrived at barrier `epoch` (bounded).  Every
// decision to stop waiting is taken from a workgroup-barrier reduction, so all
// waves of the workgroup take it together (a wave that left early would pair
// its later barriers with the wrong ones of the others).
__device__ __forceinline__ void grid_wait(uint32_t* flags, uint32_t epoch, uint32_t spin_limit,
                                          uint32_t* status) {
  // a barrier of this launch already gave up: do not wait
  const int brk = threadIdx.x == 0 &&
      (__hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & kFlagBarrier) != 0;
  if (!__syncthreads_or(brk)) {
    for (uint32_t spins = 0;; ++spins) {
      int ok = 1;
      for (uint32_t t = threadIdx.x; t < gridDim.x; t += blockDim.x)
        ok &= __hip_atomic_load(flags + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= epoch;
      if (__syncthreads_and(ok)) break;
      if (spins + 1 >= spin_limit) {
        if (threadIdx.x == 0) atomicOr(status, kFlagBarrier);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
}
__device__ __forceinline__ void grid_barrier(uint32_t* flags, uint32_t epoch, uint32_t spin_limit,
                                             uint32_t* status) {
  grid_arrive(flags, epoch);
  grid_wait(flags, epoch, spin_limit, status);
}

// Token written by another workgroup's pick in this launch: x is -1 until
// then (set before the launch).  Polled with relaxed device-scope loads; the
// wait is bounded like the grid barrier's (past spin_limit polls, or once a
// wait of this launch has given up, it returns -1 and kFlagBarrier is set).
__device__ __forceinline__ int wait_token(const int* p, uint32_t spin_limit, uint32_t* status) {
  int v = __hip_atomic_load(const_cast<int*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (v >= 0) return v;
  if (__hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & kFlagBarrier) return -1;
  for (uint32_t spins = 1;; ++spins) {
    __builtin_amdgcn_s_sleep(1);
    v = __hip_atomic_load(const_cast<int*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (v >= 0) return v;
    if (spins >= spin_limit) {
      atomicOr(status, kFlagBarrier);
      return -1;
    }
  }
}


// One direct-to-LDS load per lane: 16 bytes from gptr to lds_wave_base + 16 *
// lane (global_load_lds_dwordx4; M0 holds the wave's LDS base).  A scalar
// write of M0 needs one wait state before an LDS DMA reads it (s_nop 0): the
// compiler's hazard check does not look inside inline assembly.  Issued from
// inline assembly so that the compiler, which does not see it, does not fence
// every later LDS access of the kernel behind outstanding vector-memory loads;
// the caller waits for it explicitly (wait_vm_zero) before the data is used.
// Nothing else in this kernel uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(const void* gptr, const void* lds_wave_base) {
  const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_wave_base);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(l), "v"(gptr) : "memory", "m0");
}
#pragma clang diagnostic pop

// Entry of the wave's 64-entry slice held by lane group lg (= lane / 16) in
// value j of its 16 results (acc[j >> 2][j & 3], C-matrix row 4 lg + (j & 3)
// of M tile j >> 2): values 0-7 and 8-15 are two runs of 8 consecutive
// entries, so each run is one 16-byte piece of a U row and the four lane
// groups of a row together read 64 contiguous bytes per load instruction.
__device__ __forceinline__ constexpr int slice_entry(int lg, int j) {
  return 32 * (j >> 3) + 8 * lg + (j & 7);
}

// The wave's 64-entry W2 slice as A operands of v_mfma_f32_16x16x32_bf16:
// lane (m, kg) of M tile mt holds entry slice_entry(m >> 2, 4 mt + (m & 3)) of
// the slice (C row m of M tile mt), k-values 32 kt + 8 kg + [0, 8).  Entries
// past V re-read entry V-1.
template <int KT>
__device__ __forceinline__ void load_w2_slice(bf16x8_t (&Af)[4][KT], const uint16_t* W2t, int rank,
                                              int wslice, int V, bool active) {
  const int lane = threadIdx.x & 63;
  const int m = lane & 15, kg = lane >> 4;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    int voc = wslice + slice_entry(m >> 2, 4 * mt + (m & 3));
    voc = active ? min(voc, V - 1) : 0;
    const uint16_t* wr = W2t + (int64_t)voc * rank + 8 * kg;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) Af[mt][kt] = *reinterpret_cast<const bf16x8_t*>(wr + 32 * kt);
  }
}

// W1 rows of the tokens PV[0, rows) into LDS rows of ROWP 16-byte pieces:
// piece p is segment p % ROWP of row p / ROWP (the pad piece of a row
// re-reads its segment 0; pieces past the last row re-read it).  Direct-to-LDS
// loads, one 1 KB run per wave instruction, waited for before returning.
template <int SEG, int ROWP>
__device__ __forceinline__ void gather_w1_rows(uint4* E, const int* PV, int rows, const uint16_t* W1,
                                               int rank) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int npieces = rows * ROWP;
  for (int p0 = wv * 64; p0 < npieces; p0 += (int)blockDim.x) {
    const int p = p0 + lane;
    const int rl = min(p / ROWP, rows - 1), sp = p % ROWP;
    lds_dma16(W1 + (int64_t)PV[rl] * rank + 8 * (sp < SEG ? sp : 0), E + p0);
  }
  wait_vm_zero();
}

// MFMA chain of one 16-row tile: acc[mt] (seeded by the caller) += the wave's
// W2 slice x the W1 rows of tile rows.  erow points at segment lg of the
// lane's row; B operands pass through a three-deep register ring (the LDS
// read of k-step kt+2 is issued before the MFMAs of kt).
template <int KT>
__device__ __forceinline__ void tile_mfma(f32x4_t (&acc)[4], const bf16x8_t (&Af)[4][KT],
                                          const uint4* erow) {
  bf16x8_t Bq[3];
  Bq[0] = __builtin_bit_cast(bf16x8_t, erow[0]);
  if (KT > 1) Bq[1] = __builtin_bit_cast(bf16x8_t, erow[4]);
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + 2 < KT) Bq[(kt + 2) % 3] = __builtin_bit_cast(bf16x8_t, erow[4 * (kt + 2)]);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Af[mt][kt], Bq[kt % 3], acc[mt], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Cross-lane exchanges on the VALU (gfx950 v_permlane16_swap /
// v_permlane32_swap with both operands the same register): afterwards every
// lane holds {its own value, the value of lane ^ 16 (resp. ^ 32)} in some
// order, so a merge that is symmetric in the pair gives the same bits on both
// lanes.
template <int X>
__device__ __forceinline__ void xswap(float v, float& a, float& b) {
  const auto r = (X == 16)
      ? __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false)
      : __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
template <int X>
__device__ __forceinline__ void iswap(int v, int& a, int& b) {
  const auto r = (X == 16) ? __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false)
                           : __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
  a = (int)r[0];
  b = (int)r[1];
}

// Scaled reference of a partial with raw maximum m: fl(m s2), or -FLT_MAX
// when the partial is empty (m = -inf), so that differences of references
// are never NaN.
__device__ __forceinline__ float scaled_ref(float m, float s2) {
  return (m == -INFINITY) ? -FLT_MAX : m * s2;
}

// Statistics of one 16-row tile: every lane first reduces its 16 values of
// one request row, then the four lanes of the row (xor 16, xor 32) merge.
// The work is split into 8 units so that it can be interleaved with the MFMAs
// of the next tile (unit u runs after the MFMAs of the k-step that owns it).
//   sampling: raw maximum M, scaled reference m2 = scaled_ref(M), and
//             S = sum_j exp2(x_j s2 - m2).  Merging two partials keeps the
//             larger reference: S = S_big + S_small exp2(m2_small - m2_big)
//             (one exponential, never above 1), and since fl(m s2) is
//             monotone in m the merged m2 is again scaled_ref(merged M).
//             Units 0-1 the maximum, 2-5 the exponentials (two partial
//             sums), 6 the xor-16 merge, 7 the xor-32 merge.
//   greedy:   the maximum and the lowest entry holding it (0x7FFFFFFF when
//             the maximum is -inf).  Units 0-1 the maximum, 2-3 the index
//             scan from j = 15 down, 4-5 the merges.
// MASK: the lane's pieces past V (uok false) count as -inf.
struct EpiState {
  float m, s0, s1, m2;
  int bi;
};
template <int X>
__device__ __forceinline__ void merge_sample(EpiState& st) {
  float m_a, m_b, r_a, r_b, s_a, s_b;
  xswap<X>(st.m, m_a, m_b);
  xswap<X>(st.m2, r_a, r_b);
  xswap<X>(st.s0, s_a, s_b);
  const bool a_big = r_a >= r_b;
  const float hi = fmaxf(r_a, r_b), lo = fminf(r_a, r_b);
  const float e = __builtin_amdgcn_exp2f(lo - hi);
  st.s0 = fmaf(a_big ? s_b : s_a, e, a_big ? s_a : s_b);
  st.m = fmaxf(m_a, m_b);
  st.m2 = hi;
}
template <int X>
__device__ __forceinline__ void merge_greedy(EpiState& st) {
  float v0, v1;
  int i0, i1;
  xswap<X>(st.m, v0, v1);
  iswap<X>(st.bi, i0, i1);
  argmax_merge(v0, i0, v1, i1);
  st.m = v0;
  st.bi = i0;
}
// U value e (0-7) of a 16-byte piece of eight bf16 entries
__device__ __forceinline__ float u_piece(const uint4& q, int e) {
  const uint32_t w = (e >> 1) == 0 ? q.x : (e >> 1) == 1 ? q.y : (e >> 1) == 2 ? q.z : q.w;
  return (e & 1) ? bf16_hi(w) : bf16_lo(w);
}
// Units 0 and 1 first add the lane's U values to the accumulators: the bias
// contraction accumulates from zero (its terms are small), and the base
// logits join it in one rounding, x = fl(U + bias).  Seeding the
// accumulators with U instead would round a large value after every k-step.
template <bool GREEDY, bool MASK>
__device__ __forceinline__ void epi_unit(int u, EpiState& st, f32x4_t (&acc)[4], const uint4 (&un)[2],
                                         const bool (&uok)[2], float s2, int gbase) {
  // a masked piece becomes -inf once, when U is added
  auto xv = [&](int j) __attribute__((always_inline)) { return acc[j >> 2][j & 3]; };
  if (u == 0 || u == 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = 8 * u + e;
      const float x = acc[j >> 2][j & 3] + u_piece(un[u], e);
      acc[j >> 2][j & 3] = (!MASK || uok[u]) ? x : -INFINITY;
    }
  }
  if (u == 0) {
    float m = fmaxf(fmaxf(xv(0), xv(1)), xv(2));
    m = fmaxf(fmaxf(m, xv(3)), xv(4));
    m = fmaxf(fmaxf(m, xv(5)), xv(6));
    st.m = fmaxf(m, xv(7));
  } else if (u == 1) {
    float m = fmaxf(fmaxf(st.m, xv(8)), xv(9));
    m = fmaxf(fmaxf(m, xv(10)), xv(11));
    m = fmaxf(fmaxf(m, xv(12)), xv(13));
    m = fmaxf(fmaxf(m, xv(14)), xv(15));
    st.m = m;
    if (!GREEDY) st.m2 = scaled_ref(m, s2);
  } else if (GREEDY) {
    if (u == 2 || u == 3) {
      int bl = (u == 2) ? 16 : st.bi;
#pragma unroll
      for (int q = 7; q >= 0; --q) {
        const int j = 8 * (3 - u) + q;
        bl = (xv(j) == st.m) ? j : bl;
      }
      st.bi = bl;
      if (u == 3)
        st.bi = (st.m == -INFINITY || bl == 16) ? 0x7FFFFFFF : gbase + 32 * (bl >> 3) + (bl & 7);
    } else if (u == 4) {
      merge_greedy<16>(st);
    } else if (u == 5) {
      merge_greedy<32>(st);
    }
  } else if (u >= 2 && u <= 5) {
    const int j0 = 4 * (u - 2);
    st.s0 += __builtin_amdgcn_exp2f(fmaf(xv(j0), s2, -st.m2));
    st.s1 += __builtin_amdgcn_exp2f(fmaf(xv(j0 + 1), s2, -st.m2));
    st.s0 += __builtin_amdgcn_exp2f(fmaf(xv(j0 + 2), s2, -st.m2));
    st.s1 += __builtin_amdgcn_exp2f(fmaf(xv(j0 + 3), s2, -st.m2));
  } else if (u == 6) {
    st.s0 += st.s1;
    merge_sample<16>(st);
  } else if (u == 7) {
    merge_sample<32>(st);
  }
}

__device__ __forceinline__ void zero_acc(f32x4_t (&acc)[4]) {
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
}

// One pipelined tile step: the MFMA chain of the next tile (acc_next, zeroed)
// interleaved k-step by k-step with the epilogue units of the current tile
// (acc_cur, whose U values are in un).  Once units 0 and 1 have consumed un,
// the U pieces of tile `reload` are loaded into it.  B operands come through
// a three-deep register ring.
template <int KT, bool GREEDY, bool MASK, typename US>
__device__ __forceinline__ void mfma_with_epilogue(f32x4_t (&acc_next)[4], const bf16x8_t (&Af)[4][KT],
                                                   const uint4* erow, f32x4_t (&acc_cur)[4],
                                                   uint4 (&un)[2], const US& us, int reload,
                                                   const bool (&uok)[2], float s2, int gbase,
                                                   EpiState& st) {
  constexpr int NU = 8;                     // epilogue units
  constexpr int KT_RELOAD = KT / NU;        // the k-step whose units include unit 1
  bf16x8_t Bq[3];
  Bq[0] = __builtin_bit_cast(bf16x8_t, erow[0]);
  if (KT > 1) Bq[1] = __builtin_bit_cast(bf16x8_t, erow[4]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + 2 < KT) Bq[(kt + 2) % 3] = __builtin_bit_cast(bf16x8_t, erow[4 * (kt + 2)]);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      acc_next[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Af[mt][kt], Bq[kt % 3], acc_next[mt], 0, 0, 0);
#pragma unroll
    for (int u = kt * NU / KT; u < (kt + 1) * NU / KT; ++u)
      epi_unit<GREEDY, MASK>(u, st, acc_cur, un, uok, s2, gbase);
    if (kt == KT_RELOAD) us.load(un, reload);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The whole epilogue of a tile without MFMAs (last tile of a group).
template <bool GREEDY, bool MASK>
__device__ __forceinline__ void epilogue_all(EpiState& st, f32x4_t (&acc)[4], const uint4 (&un)[2],
                                             const bool (&uok)[2], float s2, int gbase) {
#pragma unroll
  for (int u = 0; u < 8; ++u) epi_unit<GREEDY, MASK>(u, st, acc, un, uok, s2, gbase);
}

// U pieces of one wave for one row group, tile by tile.  The lane's two 8-entry
// pieces (a piece past V re-reads the row's entry 0) are addressed as a
// wave-uniform tile base plus a 32-bit lane offset (16 rows of U fit in 2 GiB,
// checked on the host); lanes past the last row of a ragged last tile re-read
// that row.
struct UStream {
  const char* tbase;
  int64_t tstep;                              // bytes per 16 rows
  uint32_t v0, v1, l0, l1;                    // lane offsets: full tiles, last tile
  int ntiles;
  __device__ __forceinline__ void init(const uint16_t* ustep, int64_t rstride, int row0, int rows,
                                       int wslice, const bool (&uok)[2], bool full) {
    const int lane = threadIdx.x & 63, ln = lane & 15, lg = lane >> 4;
    ntiles = (rows + 15) / 16;
    const int e0 = (full || uok[0]) ? wslice + slice_entry(lg, 0) : 0;
    const int e1 = (full || uok[1]) ? wslice + slice_entry(lg, 8) : 0;
    const int lrow_last = min(16 * (ntiles - 1) + ln, rows - 1) - 16 * (ntiles - 1);
    v0 = (uint32_t)(2 * ((int64_t)ln * rstride + e0));
    v1 = (uint32_t)(2 * ((int64_t)ln * rstride + e1));
    l0 = (uint32_t)(2 * ((int64_t)lrow_last * rstride + e0));
    l1 = (uint32_t)(2 * ((int64_t)lrow_last * rstride + e1));
    tbase = reinterpret_cast<const char*>(ustep + (int64_t)row0 * rstride);
    tstep = 32 * rstride;
  }
  // tile i (past the last tile: the last one); i is wave-uniform
  __device__ __forceinline__ void load(uint4 (&dst)[2], int i) const {
    const int t = min(i, ntiles - 1);
    const bool last = t == ntiles - 1;
    const char* p = tbase + t * tstep;
    dst[0] = ld_stream16(p + (last ? l0 : v0));
    dst[1] = ld_stream16(p + (last ? l1 : v1));
  }
};

// Phase A of one wave for one row group: 16-row tiles, software-pipelined so
// that while the MFMAs of tile i+1 run, the vector ALU works on the epilogue
// of tile i (which adds U to the bias).  U is prefetched about two tiles
// ahead; the caller has already issued the loads of tiles 0 and 1 (ua, ub).
// The statistics of every tile row over the wave's 64 entries go to
// HS[row][wave] (rows past `rows`, in the ragged last tile, are never read).
template <int KT, int ROWP, bool GREEDY, bool MASK>
__device__ __forceinline__ void slice_tiles(const bf16x8_t (&Af)[4][KT], const uint4* E, float2* HS,
                                            const UStream& us, uint4 (&ua)[2], uint4 (&ub)[2], int wslice,
                                            const bool (&uok)[2], float s2) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int ln = lane & 15, lg = lane >> 4;
  const int ntiles = us.ntiles;
  // after the merges every lane of a row holds the row's statistics over the
  // wave's 64 entries; lane group 0 stores them (HS[row][wave])
  float2* hs = HS + ln * kPWaves + wv;
  const int gbase = wslice + 8 * lg;
  auto store = [&](int i, const EpiState& st) __attribute__((always_inline)) {
    if (lg == 0) hs[16 * kPWaves * i] = make_float2(st.m, GREEDY ? __int_as_float(st.bi) : st.s0);
  };
  auto fresh = [&]() __attribute__((always_inline)) {
    EpiState st;
    st.m = -INFINITY; st.s0 = 0.f; st.s1 = 0.f; st.m2 = -FLT_MAX; st.bi = 0x7FFFFFFF;
    return st;
  };
  // epilogue of tile i (acc_cur, its U values in un, which is then refilled
  // with tile i+2) with the MFMAs of tile i+1 (acc_next, from zero)
  auto step2 = [&](f32x4_t (&acc_cur)[4], f32x4_t (&acc_next)[4], uint4 (&un)[2], int i)
      __attribute__((always_inline)) {
    zero_acc(acc_next);
    EpiState st = fresh();
    mfma_with_epilogue<KT, GREEDY, MASK>(acc_next, Af, E + (16 * (i + 1) + ln) * ROWP + lg, acc_cur, un,
                                         us, i + 2, uok, s2, gbase, st);
    store(i, st);
  };
  auto last = [&](f32x4_t (&acc)[4], const uint4 (&un)[2], int i) __attribute__((always_inline)) {
    EpiState st = fresh();
    epilogue_all<GREEDY, MASK>(st, acc, un, uok, s2, gbase);
    store(i, st);
  };
  f32x4_t accA[4], accB[4];
  zero_acc(accA);                             // tile 0 (U(0) in ua, U(1) in ub)
  tile_mfma<KT>(accA, Af, E + ln * ROWP + lg);
  int i = 0;
  for (; i + 2 < ntiles; i += 2) {
    step2(accA, accB, ua, i);                 // epilogue i (U in ua), MFMA i+1
    step2(accB, accA, ub, i + 1);             // epilogue i+1 (U in ub), MFMA i+2
  }
  if (i + 1 < ntiles) {
    step2(accA, accB, ua, i);
    last(accB, ub, i + 1);
  } else {
    last(accA, ua, i);
  }
}

// Wave-wide reductions on the VALU alone: DPP steps inside rows of 16 lanes,
// then the xor-16 and xor-32 swaps; every lane ends with the result, and each
// combine is symmetric, so all lanes hold the same bits.
__device__ __forceinline__ float wave_max_v(float v) {
  v = row16_max(v);
  float a, b;
  xswap<16>(v, a, b);
  v = fmaxf(a, b);
  xswap<32>(v, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float wave_sum_v(float v) {
  v = row16_sum(v);
  float a, b;
  xswap<16>(v, a, b);
  v = a + b;
  xswap<32>(v, a, b);
  return a + b;
}
template <int X>
__device__ __forceinline__ void argmax_swap(float& v, int& i) {
  float v0, v1;
  int i0, i1;
  xswap<X>(v, v0, v1);
  iswap<X>(i, i0, i1);
  argmax_merge(v0, i0, v1, i1);
  v = v0;
  i = i0;
}
__device__ __forceinline__ void wave_argmax_v(float& v, int& i) {
  row16_argmax(v, i);
  argmax_swap<16>(v, i);
  argmax_swap<32>(v, i);
}

// (key, index) argmax with the lower index winning ties, and a sum.
struct PickRed {
  float key;
  int idx;
  float s;
};
// The thread index, opaque to the optimiser: what is derived from it is
// computed where it is used, not hoisted out of an enclosing loop (a value
// kept live across a register-bound tile loop gets spilled, and each reload
// from scratch is a vector-memory wait).
__device__ __forceinline__ int tid_opaque() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// Workgroup barrier for LDS traffic only: this wave's LDS operations are
// done, then s_barrier.  Unlike __syncthreads it releases no global memory,
// so it does not wait for this wave's outstanding vector-memory operations
// (prefetches in flight, stores).  The "memory" clobber keeps the compiler
// from moving memory accesses across it.
__device__ __forceinline__ void lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Block-wide reductions over the 512 threads: wave results go through LDS
// slots owned by one reduction each (so no barrier is needed before the
// stores) and are combined in wave order.
__device__ __forceinline__ float block_max_v(float v, float* slot) {
  v = wave_max_v(v);
  const int t = tid_opaque();
  if ((t & 63) == 0) slot[t >> 6] = v;
  lds_sync();
  float r = slot[0];
#pragma unroll
  for (int q = 1; q < kPWaves; ++q) r = fmaxf(r, slot[q]);
  return r;
}
__device__ __forceinline__ PickRed block_pick_reduce(PickRed v, PickRed* slot) {
  wave_argmax_v(v.key, v.idx);
  v.s = wave_sum_v(v.s);
  const int t = tid_opaque();
  if ((t & 63) == 0) slot[t >> 6] = v;
  lds_sync();
  PickRed r = slot[0];
#pragma unroll
  for (int q = 1; q < kPWaves; ++q) {
    argmax_merge(r.key, r.idx, slot[q].key, slot[q].idx);
    r.s += slot[q].s;
  }
  return r;
}
__device__ __forceinline__ void block_argmax_v(float& v, int& idx, float* fslot, int* islot) {
  wave_argmax_v(v, idx);
  const int t = tid_opaque();
  if ((t & 63) == 0) { fslot[t >> 6] = v; islot[t >> 6] = idx; }
  lds_sync();
  v = fslot[0];
  idx = islot[0];
#pragma unroll
  for (int q = 1; q < kPWaves; ++q) argmax_merge(v, idx, fslot[q], islot[q]);
}

// Gumbel noise of the chunk-level draw for request i at step k: thread t owns
// chunks 4t..4t+3 (one Philox block).  Independent of the data, so it is
// computed while the chunk statistics are being loaded.
__device__ __forceinline__ void chunk_noise(const DraftPickArgs& a, int i, int k, float (&g)[4]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int w = 0; w < 4; ++w) g[w] = 0.f;
  if (a.nch > 1 && 4 * t < a.nch) {
    const uint4 blk = stream_block(a.seed, a.round, kTagDraftChunk, (uint32_t)i, (uint32_t)k, (uint32_t)t);
#pragma unroll
    for (int w = 0; w < 4; ++w) g[w] = gumbel_of(word_of(blk, (uint32_t)w));
  }
}

// LDS of the persistent pick: reduction slots and the W1 row of x_{k-1}.
template <int SEG>
struct PickLds {
  float fmax[kPWaves];
  float farg[kPWaves];
  int iarg[kPWaves];
  PickRed red[kPWaves];
  uint4 E[SEG];
};

}  // namespace dspark
