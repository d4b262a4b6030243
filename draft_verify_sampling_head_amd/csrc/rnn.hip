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
//                      accumulation (bf16 products are exact in fp32),
//                      128 x 96 tiles fed by direct-to-LDS loads three
//                      stages ahead.
//   k_rnn_hproj_valu : the same for float32 operands or unaligned rows.
//   k_rnn_cell_mfma  : per step, the recurrent part [s_{k-1} ; W1[x_{k-1}]]
//                      (2r inputs) on MFMA with the fp32 state split into
//                      three exact bf16 parts, plus P, then the gates, s_k and
//                      e_k.  A workgroup owns 16 requests x 16 state entries
//                      with their gate, candidate and output rows, so the cell
//                      completes locally.
//   k_rnn_cell       : the same cell in fp32 on the vector ALU (float32
//                      weights, rows that are not 16-byte aligned).
// The cell kernels serve the per-step schedule.  When the shape fits the
// persistent draft launch (draft.hip), that launch runs the same cell, tile by
// tile, as a phase of every step, and only k_rnn_hproj_mfma runs before it.
#include <algorithm>
#include <cstdlib>
#include <type_traits>

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
// Workgroup tile kBM x kBN = 128 x 96 (at 4096 x 768 that is 256 workgroups,
// one per compute unit) with eight waves of 32 x 48 (2 x 3 tiles of
// v_mfma_f32_16x16x32_bf16, fp32 accumulation), two waves per SIMD.  The
// tile's rows of h and of Wr stream through a kNB-deep LDS ring in stages of
// kBK columns, moved by direct-to-LDS loads (global_load_lds_dwordx4: no
// registers, no LDS write instructions) issued three stages before they are
// due, from a wave-uniform base plus 32-bit lane offsets.  LDS layout of a
// stage: row-major 16-byte pieces, eight per row (64 bf16 columns), the piece
// index XORed with the row's low three bits, so the rows one ds_read_b128
// touches at one column spread over the banks (the bank-conflict counter reads
// zero); a DMA instruction fills 64 consecutive pieces, each lane fetching
// the global piece that belongs in its slot.  Workgroups b, b + 8, ... run on
// one XCD: each XCD takes a contiguous run of tiles, N fastest, so tiles that
// share rows of h share that XCD's L2.  Measured at 4096 x 768 x 4096: 39.6 us
// (0.65 PFLOP/s) against 56 us for 64 x 96 tiles with register-staged loads;
// four waves of 64 x 48 (fewer LDS bytes per MFMA, one wave per SIMD) took
// 49 us, and reading h from L2 instead of HBM changed nothing.
constexpr int kBM = 128, kBN = 96, kBK = 64;
constexpr int kNB = 5;                       // LDS ring depth, in stages
constexpr int kAPc = kBM * (kBK / 8);        // 16-byte pieces of h per stage (1024)
constexpr int kBPc = kBN * (kBK / 8);        // and of Wr (768)
constexpr int kSlotP = kAPc + kBPc;          // pieces per ring slot (28 KB)
constexpr int kIA = kAPc / 64, kIB = kBPc / 64;   // DMA instructions per stage (16 + 12)
constexpr int kXcds = 8;                     // XCDs of an MI355X
constexpr int kHprojWaves = 8;

typedef __attribute__((address_space(1))) void hp_gvoid_t;
typedef __attribute__((address_space(3))) void hp_lvoid_t;

__device__ __forceinline__ int hp_slot(int row, int p) { return row * 8 + (p ^ (row & 7)); }

// s_waitcnt: at most N vector-memory operations of this wave outstanding, and
// none of its LDS operations (gfx9 encoding: vmcnt[3:0], expcnt[6:4],
// lgkmcnt[11:8], vmcnt[15:14])
template <int N>
__device__ __forceinline__ void hp_wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
}

// NW waves: 4 (wave tile 64 x 48, waves 2 x 2) or 8 (32 x 48, waves 4 x 2).
// Wave wv issues the stage's h instructions wv + NW i and, if wv < kBW, the
// Wr instructions wv + kBW i.
template <int NW>
__global__ __launch_bounds__(64 * NW, 1) void k_rnn_hproj_mfma(const uint16_t* __restrict__ h,
                                                                const uint16_t* __restrict__ Wr,
                                                                int M, int N, int d, int ldw,
                                                                int wcol, float* __restrict__ P) {
  constexpr int NT = 64 * NW;
  constexpr int WNN = 2, WNM = NW / WNN;       // waves along N and along M
  constexpr int kWM = kBM / WNM, kWN = kBN / WNN;
  constexpr int kTM = kWM / 16, kTN = kWN / 16;
  constexpr int NA = kIA / NW;                 // h instructions per wave and stage
  constexpr int kBW = 4, NBI = kIB / kBW;      // waves that load Wr, and their instructions
  static_assert(kIA % NW == 0 && kIB % kBW == 0 && kBW <= NW, "whole DMA instructions per wave");
  __shared__ uint4 ring[kNB * kSlotP];
  // the wave index as a scalar: the per-wave choice of loads and waits below
  // is then a scalar branch, not two exec-masked paths
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nN = (N + kBN - 1) / kBN, tiles = ((M + kBM - 1) / kBM) * nN;
  const int per_xcd = (tiles + kXcds - 1) / kXcds;
  const int t = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (t >= tiles) return;
  const int m0 = (t / nN) * kBM, n0 = (t % nN) * kBN;
  const int nst = (d + kBK - 1) / kBK;
  const bool bw = wv < kBW;
  // this lane's DMA pieces: slot -> (row, piece) through the XOR swizzle,
  // addressed as a wave-uniform stage base plus a 32-bit byte offset (the host
  // checks that h and the Wr rows span less than 4 GiB), so a stage's loads
  // need no per-lane address arithmetic.  The last stage has offsets of its
  // own: its columns past d re-read column d - 8 (a valid address) and are
  // zeroed in LDS once they have landed.
  const int lastc = (nst - 1) * kBK;
  uint32_t oa[NA], oal[NA], ob[NBI], obl[NBI];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int q = (wv + NW * i) * 64 + lane, row = q >> 3, p = (q & 7) ^ (row & 7);
    const uint32_t rb = (uint32_t)min(m0 + row, M - 1) * (uint32_t)d;
    oa[i] = 2u * (rb + 8u * p);
    oal[i] = 2u * (rb + (uint32_t)min(lastc + 8 * p, d - 8)) - 2u * lastc;
  }
#pragma unroll
  for (int i = 0; i < NBI; ++i) {
    const int q = ((bw ? wv : 0) + kBW * i) * 64 + lane, row = q >> 3, p = (q & 7) ^ (row & 7);
    const uint32_t rb = (uint32_t)min(n0 + row, N - 1) * (uint32_t)ldw + (uint32_t)wcol;
    ob[i] = 2u * (rb + 8u * p);
    obl[i] = 2u * (rb + (uint32_t)min(lastc + 8 * p, d - 8)) - 2u * lastc;
  }
  const char* hb = reinterpret_cast<const char*>(h);
  const char* wb = reinterpret_cast<const char*>(Wr);
  // stage st into ring slot st % kNB; stages past the last re-read the last
  // one into a slot that is not read again, so every wave always has the
  // same number of loads in flight
  auto issue = [&](int st) __attribute__((always_inline)) {
    const bool last = st >= nst - 1;
    const int64_t sb = 2 * (int64_t)(last ? lastc : st * kBK);
    uint4* slot = ring + (st % kNB) * kSlotP;
#pragma unroll
    for (int i = 0; i < NA; ++i)
      __builtin_amdgcn_global_load_lds((hp_gvoid_t*)(hb + sb + (last ? oal[i] : oa[i])),
                                       (hp_lvoid_t*)(slot + (wv + NW * i) * 64), 16, 0, 0);
    if (bw) {
#pragma unroll
      for (int i = 0; i < NBI; ++i)
        __builtin_amdgcn_global_load_lds((hp_gvoid_t*)(wb + sb + (last ? obl[i] : ob[i])),
                                         (hp_lvoid_t*)(slot + kAPc + (wv + kBW * i) * 64), 16, 0, 0);
    }
  };
  f32x4_t acc[kTM][kTN];
#pragma unroll
  for (int a = 0; a < kTM; ++a)
#pragma unroll
    for (int b = 0; b < kTN; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int rl = lane & 15, kg = lane >> 4;
  const int wm = kWM * (wv / WNN), wn = kWN * (wv % WNN);
  // stage s is due: this wave's pieces of it have landed (the loads of the
  // AHEAD stages issued after it may still be in flight), then every wave's
  // (barrier); a partial last stage has its columns past d zeroed
  auto arrive = [&](auto ahead, int s) __attribute__((always_inline)) {
    constexpr int AH = decltype(ahead)::value;
    if (bw) hp_wait_vm_lgkm0<AH * (NA + NBI)>();
    else hp_wait_vm_lgkm0<AH * NA>();
    __builtin_amdgcn_s_barrier();
    if (s == nst - 1 && d - s * kBK < kBK) {
      const int cols = d - s * kBK;
      uint4* w = ring + (s % kNB) * kSlotP;
      for (int q = tid; q < kSlotP; q += NT) {
        const int row = (q < kAPc ? q : q - kAPc) >> 3, p = (q & 7) ^ (row & 7);
        if (8 * p >= cols) w[q] = make_uint4(0u, 0u, 0u, 0u);
      }
      hp_wait_vm_lgkm0<0>();
      __builtin_amdgcn_s_barrier();
    }
  };
  auto frags = [&](int s, int sub, bf16x8_t (&Af)[kTM], bf16x8_t (&Bf)[kTN])
      __attribute__((always_inline)) {
    const uint4* slot = ring + (s % kNB) * kSlotP;
    const int p = 4 * sub + kg;
#pragma unroll
    for (int i = 0; i < kTM; ++i)
      Af[i] = __builtin_bit_cast(bf16x8_t, slot[hp_slot(wm + 16 * i + rl, p)]);
#pragma unroll
    for (int j = 0; j < kTN; ++j)
      Bf[j] = __builtin_bit_cast(bf16x8_t, slot[kAPc + hp_slot(wn + 16 * j + rl, p)]);
  };
  auto mfmas = [&](const bf16x8_t (&Af)[kTM], const bf16x8_t (&Bf)[kTN])
      __attribute__((always_inline)) {
#pragma unroll
    for (int a = 0; a < kTM; ++a)
#pragma unroll
      for (int b = 0; b < kTN; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Af[a], Bf[b], acc[a][b], 0, 0, 0);
  };
  // Software pipeline over the two 32-column halves of each stage: the LDS
  // reads of one half are in flight during the other half's MFMAs, across
  // stage boundaries too.  The DMA of stage s is issued three stages before
  // s is due; the slot it fills was last read a full stage earlier, before
  // the barrier of the stage that precedes the issue.
  for (int s = 0; s < kNB - 1; ++s) issue(s);
  arrive(std::integral_constant<int, kNB - 2>{}, 0);
  bf16x8_t A0[kTM], B0[kTN], A1[kTM], B1[kTN];
  frags(0, 0, A0, B0);
  for (int st = 0; st < nst; ++st) {
    frags(st, 1, A1, B1);
    mfmas(A0, B0);
    if (st + 1 < nst) {
      arrive(std::integral_constant<int, kNB - 3>{}, st + 1);
      issue(st + kNB - 1);
      frags(st + 1, 0, A0, B0);
    }
    mfmas(A1, B1);
  }
  // the trailing loads (of stages past the last) complete before the stores
  hp_wait_vm_lgkm0<0>();
#pragma unroll
  for (int a = 0; a < kTM; ++a)
#pragma unroll
    for (int b = 0; b < kTN; ++b) {
      const int n = n0 + wn + 16 * b + rl;
      if (n >= N) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + wm + 16 * a + 4 * kg + i;
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
// entry against its request's recurrent input over the 2r columns.  Those
// columns go through LDS (as fp32) in chunks of kKC: every load of a chunk is
// issued at once (16-byte weight pieces when the rows allow), and the next
// chunk's loads are in flight while the current one is consumed.
constexpr int kKC = 128;
constexpr int kKP = kKC + 4;                 // padded LDS row (float4 reads stay conflict-light)

template <typename WT, bool VEC>
__global__ __launch_bounds__(256) void k_rnn_cell(RnnArgs a, int k) {
  constexpr int EPP = VEC ? 16 / (int)sizeof(WT) : 1;   // weight elements per load
  constexpr int PPR = kKC / EPP;                         // loads per weight row and chunk
  constexpr int NWP = 48 * PPR / 256;                    // weight loads per thread and chunk
  constexpr int NZ = 16 * kKC / 256;                     // input values per thread and chunk
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
  using Raw = typename std::conditional<VEC, uint4, float>::type;
  Raw wraw[NWP];
  float zraw[NZ];
  auto load = [&](int q0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NWP; ++i) {
      const int p = tid + 256 * i, row = p / PPR, q = q0 + (p % PPR) * EPP;
      const WT* src = Wr + (int64_t)((row >> 4) * r + j0 + (row & 15)) * ldw + q;
      if constexpr (VEC) wraw[i] = q < nin ? *reinterpret_cast<const uint4*>(src) : uint4{0u, 0u, 0u, 0u};
      else wraw[i] = q < nin ? ld_f(src, 0) : 0.f;
    }
#pragma unroll
    for (int i = 0; i < NZ; ++i) {
      const int idx = tid + 256 * i, row = idx / kKC, q = q0 + idx % kKC;
      const int req = req0 + row;
      float v = 0.f;
      if (req < a.R && q < nin) {
        if (q < r) v = (k == 1) ? 0.f : a.state[((int64_t)req * a.gamma + (k - 2)) * r + q];
        else v = ld_f(W1, (int64_t)PV[row] * r + (q - r));
      }
      zraw[i] = v;
    }
  };
  auto store = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NWP; ++i) {
      const int p = tid + 256 * i, row = p / PPR, c = (p % PPR) * EPP;
      float* dst = W + row * kKP + c;
      if constexpr (VEC && sizeof(WT) == 2) {
        const uint4 u = wraw[i];
        *reinterpret_cast<float4*>(dst) = make_float4(bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y));
        *reinterpret_cast<float4*>(dst + 4) = make_float4(bf16_lo(u.z), bf16_hi(u.z), bf16_lo(u.w), bf16_hi(u.w));
      } else if constexpr (VEC) {
        *reinterpret_cast<uint4*>(dst) = wraw[i];
      } else {
        dst[0] = wraw[i];
      }
    }
#pragma unroll
    for (int i = 0; i < NZ; ++i) {
      const int idx = tid + 256 * i;
      Z[(idx / kKC) * kKP + idx % kKC] = zraw[i];
    }
  };
  float pg = 0.f, pc = 0.f, po = 0.f;
  load(0);
  for (int q0 = 0; q0 < nin; q0 += kKC) {
    store();
    __syncthreads();
    if (q0 + kKC < nin) load(q0 + kKC);      // in flight while this chunk is consumed
    const float4* zr = reinterpret_cast<const float4*>(Z + rr * kKP);
    const float4* gr = reinterpret_cast<const float4*>(W + jj * kKP);
    const float4* cr = reinterpret_cast<const float4*>(W + (16 + jj) * kKP);
    const float4* orw = reinterpret_cast<const float4*>(W + (32 + jj) * kKP);
#pragma unroll 8
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

// The cell on MFMA (bf16 weights with 16-byte aligned rows).  Workgroup
// (rt, jt) owns requests 16 rt + [0, 16) and state entries 16 jt + [0, 16):
// three 16 x 16 results (gate, candidate and output rows of those entries)
// over the 2r recurrent columns, as v_mfma_f32_16x16x32_bf16 with the
// requests as M and the weight rows as N.  The embedding half of z is bf16
// already; the fp32 state is split into three bf16 parts s = hi + mid + lo
// (together its 24 significant bits), so every product is exact in fp32 and
// the accumulation is fp32, as on the vector ALU.  Wave w takes the k-steps
// w, w + 4, ... of both halves (all its loads issued at once) and the four
// partial results are added through LDS; wave w then finishes request row
// 4 g + w of every lane group g.
__device__ __forceinline__ void split3(const float4& a, const float4& b, bf16x8_t& hi,
                                       bf16x8_t& mid, bf16x8_t& lo) {
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint16_t h[8], m[8], l[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    h[t] = f32_to_bf16(v[t]);
    const float r1 = v[t] - __uint_as_float((uint32_t)h[t] << 16);
    m[t] = f32_to_bf16(r1);
    const float r2 = r1 - __uint_as_float((uint32_t)m[t] << 16);
    l[t] = f32_to_bf16(r2);
  }
  hi = __builtin_bit_cast(bf16x8_t, h);
  mid = __builtin_bit_cast(bf16x8_t, m);
  lo = __builtin_bit_cast(bf16x8_t, l);
}

constexpr int kCellIt = 4;                   // k-steps per wave and half: r <= 4 * 4 * 32 = 512

__global__ __launch_bounds__(256) void k_rnn_cell_mfma(RnnArgs a, int k) {
  __shared__ float red[3][4][64][4];          // [part][wave][lane][row]
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = a.rank, ldw = 2 * r + a.d, nks = (r + 31) / 32;
  const int req0 = blockIdx.x * 16, j0 = blockIdx.y * 16;
  const int m = lane & 15, kg = lane >> 4;
  const uint16_t* W1 = reinterpret_cast<const uint16_t*>(a.W1);
  const uint16_t* Wr = reinterpret_cast<const uint16_t*>(a.Wr);
  // operand rows of this lane: request req0 + m (A), weight row j0 + m of each part (B)
  const int reqA = req0 + m;
  const bool okA = reqA < a.R;
  int prev = 0;
  if (okA) {
    prev = (k == 1) ? a.x0[reqA] : a.x[(int64_t)reqA * (a.gamma + 1) + (k - 1)];
    if (prev < 0 || prev >= a.V) { if (w == 0) set_flag(a.status, kFlagBadToken); prev = 0; }
  }
  const bool has_s = k >= 2;                  // s_0 = 0: no state half at the first step
  const float* srow = a.state + ((int64_t)(okA ? reqA : 0) * a.gamma + (has_s ? k - 2 : 0)) * r;
  const uint16_t* erow = W1 + (int64_t)prev * r;
  const uint16_t* wrow[3];
#pragma unroll
  for (int p = 0; p < 3; ++p) wrow[p] = Wr + (int64_t)(p * r + j0 + m) * ldw;
  const bf16x8_t zero = {};
  const float4 fz = make_float4(0.f, 0.f, 0.f, 0.f);
  float4 sv[kCellIt][2];
  bf16x8_t ev[kCellIt], ws[kCellIt][3], we[kCellIt][3];
#pragma unroll
  for (int it = 0; it < kCellIt; ++it) {
    const int c = 32 * (w + 4 * it) + 8 * kg;
    const bool in = c < r;                     // r % 16 == 0: a group is all in or all out
    const bool sin = in && has_s && okA;
    sv[it][0] = sin ? *reinterpret_cast<const float4*>(srow + c) : fz;
    sv[it][1] = sin ? *reinterpret_cast<const float4*>(srow + c + 4) : fz;
    ev[it] = (in && okA) ? *reinterpret_cast<const bf16x8_t*>(erow + c) : zero;
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      ws[it][p] = (in && has_s) ? *reinterpret_cast<const bf16x8_t*>(wrow[p] + c) : zero;
      we[it][p] = in ? *reinterpret_cast<const bf16x8_t*>(wrow[p] + r + c) : zero;
    }
  }
  f32x4_t acc[3];
#pragma unroll
  for (int p = 0; p < 3; ++p) acc[p] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int it = 0; it < kCellIt; ++it) {
    if (w + 4 * it >= nks) break;              // wave-uniform
    if (has_s) {
      bf16x8_t hi, mid, lo;
      split3(sv[it][0], sv[it][1], hi, mid, lo);
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        acc[p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, ws[it][p], acc[p], 0, 0, 0);
        acc[p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mid, ws[it][p], acc[p], 0, 0, 0);
        acc[p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, ws[it][p], acc[p], 0, 0, 0);
      }
    }
#pragma unroll
    for (int p = 0; p < 3; ++p)
      acc[p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ev[it], we[it][p], acc[p], 0, 0, 0);
  }
#pragma unroll
  for (int p = 0; p < 3; ++p)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[p][w][lane][i] = acc[p][i];
  __syncthreads();
  // lane (n, g) of wave w: request req0 + 4 g + w, entry j0 + n
  float pre[3];
#pragma unroll
  for (int p = 0; p < 3; ++p)
    pre[p] = red[p][0][lane][w] + red[p][1][lane][w] + red[p][2][lane][w] + red[p][3][lane][w];
  const int req = req0 + 4 * kg + w, j = j0 + m;
  if (req >= a.R) return;
  const int64_t pos = (int64_t)req * a.gamma + (k - 1);
  const float* Pr = a.P + pos * 3 * r;
  const float pg = pre[0] + Pr[j], pc = pre[1] + Pr[r + j], po = pre[2] + Pr[2 * r + j];
  const float sp = has_s ? a.state[(pos - 1) * r + j] : 0.f;
  const float g = 1.f / (1.f + expf(-pg));
  const float s = g * sp + (1.f - g) * tanhf(pc);
  const float e = tanhf(po);
  if (!isfinite(pg) || !isfinite(pc) || !isfinite(po)) set_flag(a.status, kFlagNonFinite);
  a.state[pos * r + j] = s;
  reinterpret_cast<uint16_t*>(a.feat)[pos * r + j] = f32_to_bf16(e);
}

}  // namespace

hipError_t launch_rnn_hproj(const RnnArgs& a, hipStream_t st) {
  const int M = a.R * a.gamma, N = 3 * a.rank, ldw = 2 * a.rank + a.d, wcol = 2 * a.rank;
  if (M == 0) return hipSuccess;
  const bool aligned = ((reinterpret_cast<uintptr_t>(a.h) | reinterpret_cast<uintptr_t>(a.Wr)) & 15) == 0;
  // the MFMA kernel addresses h and Wr with 32-bit byte offsets
  const bool span_ok = (int64_t)M * a.d * 2 < ((int64_t)1 << 32) &&
                       (int64_t)N * ldw * 2 < ((int64_t)1 << 32);
  if (a.h_bf16 && a.w_bf16 && aligned && (a.d % 8) == 0 && span_ok) {
    const int tiles = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
    hipLaunchKernelGGL(k_rnn_hproj_mfma<kHprojWaves>, dim3(kXcds * ((tiles + kXcds - 1) / kXcds)),
                       dim3(64 * kHprojWaves), 0, st, reinterpret_cast<const uint16_t*>(a.h),
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
  const size_t es = a.w_bf16 ? 2 : 4;
  const bool vec = (reinterpret_cast<uintptr_t>(a.Wr) & 15) == 0 &&
                   ((size_t)(2 * a.rank + a.d) * es) % 16 == 0;
  const bool mfma_ok = a.w_bf16 && vec && a.rank <= 4 * kCellIt * 32 &&
                       (reinterpret_cast<uintptr_t>(a.W1) & 15) == 0 &&
                       !switches().rnn_cell_valu;
  if (mfma_ok) {
    hipLaunchKernelGGL(k_rnn_cell_mfma, grid, dim3(256), 0, st, a, k);
  } else if (a.w_bf16) {
    if (vec) hipLaunchKernelGGL((k_rnn_cell<uint16_t, true>), grid, dim3(256), 0, st, a, k);
    else hipLaunchKernelGGL((k_rnn_cell<uint16_t, false>), grid, dim3(256), 0, st, a, k);
  } else {
    if (vec) hipLaunchKernelGGL((k_rnn_cell<float, true>), grid, dim3(256), 0, st, a, k);
    else hipLaunchKernelGGL((k_rnn_cell<float, false>), grid, dim3(256), 0, st, a, k);
  }
  return hipGetLastError();
}

}  // namespace dspark
