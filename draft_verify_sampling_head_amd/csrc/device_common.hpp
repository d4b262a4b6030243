// device_common.hpp -- device helpers shared by the libdspark kernels (gfx950).
//
// Random stream: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11, "Parallel
// Random Numbers: As Easy as 1, 2, 3"): ten rounds of two 32x32->64 products
// whose halves are cross-xored with the other counter words and the round key,
// the key bumped by the two Weyl constants between rounds.  Key = the 64-bit
// seed, counter = (idx/4, k | tag<<16, request, lo32 round), word = idx % 4.
// A word y maps to u = (y + 1/2) 2^-32 and to a standard Gumbel -log(-log u);
// for u > 1/2 the inner log is taken as log1p(-(1-u)) with 1-u = (~y + 1/2) 2^-32,
// which keeps full float precision where u rounds towards 1.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dspark {

constexpr int kChunk = 128;        // vocabulary entries per Gumbel chunk
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963407f;

enum : uint32_t {
  kTagDraftChunk = 1, kTagDraftElem = 2, kTagAccept = 3,
  kTagResidChunk = 4, kTagResidElem = 5, kTagBonusChunk = 6, kTagBonusElem = 7
};

enum : uint32_t { kFlagNonFinite = 1u, kFlagBadLen = 2u, kFlagBadToken = 4u, kFlagBarrier = 8u,
                  kFlagTier = 16u };

// ------------------------------------------------------------------ Philox
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    const uint32_t hi0 = __umulhi(0xD2511F53u, c.x);
    const uint32_t lo0 = 0xD2511F53u * c.x;
    const uint32_t hi1 = __umulhi(0xCD9E8D57u, c.z);
    const uint32_t lo1 = 0xCD9E8D57u * c.z;
    c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

// The four words of counter block idx4 (= idx / 4) of one stream.
__device__ __forceinline__ uint4 stream_block(uint64_t seed, uint64_t round, uint32_t tag,
                                              uint32_t req, uint32_t k, uint32_t idx4) {
  return philox4x32_10(make_uint4(idx4, k | (tag << 16), req, (uint32_t)round),
                       (uint32_t)seed, (uint32_t)(seed >> 32));
}

__device__ __forceinline__ uint32_t word_of(uint4 b, uint32_t lane4) {
  return lane4 == 0 ? b.x : lane4 == 1 ? b.y : lane4 == 2 ? b.z : b.w;
}

// log(u) for u = (y + 1/2) 2^-32, accurate for every word y.
__device__ __forceinline__ float log_uniform(uint32_t y) {
  if (y < 0x80000000u) {
    return logf(fmaf((float)y, 0x1p-32f, 0x1p-33f));
  }
  return log1pf(-fmaf((float)(~y), 0x1p-32f, 0x1p-33f));
}

// Standard Gumbel -ln(-ln u), u = (y + 1/2) 2^-32, from the hardware base-2
// logarithm (v_log_f32, about one ulp) instead of the library logf/log1pf.
// For u >= 1/2, -ln u = -log1p(x) with x = u - 1 taken exactly from y, and
// log1p(x) = ln(1 + x) x / ((1 + x) - 1) (Goldberg's formula: the rounding of
// 1 + x cancels), so small |x| keeps its relative accuracy.  Branch-free: both
// halves are evaluated and one is selected.
__device__ __forceinline__ float gumbel_of(uint32_t y) {
  const float ulo = fmaf((float)y, 0x1p-32f, 0x1p-33f);            // u, for y < 2^31
  const float nlo = -__builtin_amdgcn_logf(ulo) * kLn2;
  const float x = -fmaf((float)(~y), 0x1p-32f, 0x1p-33f);          // u - 1, for y >= 2^31
  const float u1 = 1.f + x;
  const float r = __builtin_amdgcn_logf(u1) * kLn2 * __builtin_amdgcn_rcpf(u1 - 1.f);
  const float nhi = (u1 == 1.f) ? -x : -(r * x);
  const float nl = (y < 0x80000000u) ? nlo : nhi;                   // -ln u > 0
  return -__builtin_amdgcn_logf(nl) * kLn2;
}

// ------------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_at(const uint16_t* p, int64_t i) {
  return __uint_as_float(((uint32_t)p[i]) << 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float get(const float* p, int64_t i) { return p[i]; }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float get(const uint16_t* p, int64_t i) { return bf16_at(p, i); }
};

// ------------------------------------------------------------ reductions
// DPP moves inside a row of 16 lanes (quad_perm xor1 / xor2, half-mirror,
// mirror): four steps leave every lane of the row with the row's result.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f<kDppMirror>(v));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  v += dpp_f<kDppMirror>(v);
  return v;
}
// (value, index) max with the lower index winning ties.
__device__ __forceinline__ void argmax_merge(float& v, int& i, float vo, int io) {
  if (vo > v || (vo == v && io < i)) { v = vo; i = io; }
}
template <int CTRL>
__device__ __forceinline__ void row16_argmax_step(float& v, int& i) {
  const float vo = dpp_f<CTRL>(v);
  const int io = dpp_i<CTRL>(i);
  argmax_merge(v, i, vo, io);
}
__device__ __forceinline__ void row16_argmax(float& v, int& i) {
  row16_argmax_step<kDppXor1>(v, i);
  row16_argmax_step<kDppXor2>(v, i);
  row16_argmax_step<kDppHalfMirror>(v, i);
  row16_argmax_step<kDppMirror>(v, i);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float vo = __shfl_xor(v, o);
    const int io = __shfl_xor(i, o);
    argmax_merge(v, i, vo, io);
  }
}

// ln(sum exp) combine of (max, sum-of-exp2-relative-to-max) pairs in log2 units.
__device__ __forceinline__ void lse2_merge(float& m, float& s, float mo, float so) {
  const float mn = fmaxf(m, mo);
  if (mn == -INFINITY) return;
  s = s * exp2f(m - mn) + so * exp2f(mo - mn);
  m = mn;
}

// True for +-inf and NaN (exponent bits all ones); an integer test, so no
// floating-point assumption can fold it away.
__device__ __forceinline__ bool nonfinite(float x) {
  return (__float_as_uint(x) & 0x7F800000u) == 0x7F800000u;
}

__device__ __forceinline__ void set_flag(uint32_t* status, uint32_t f) {
  if (status) atomicOr(status, f);
}

// Values that cross workgroups inside one launch (chunk statistics, chunk
// argmaxes, drafted tokens, row normalisers) are stored and loaded with
// device-scope relaxed atomics.  Those accesses are coherent across the
// XCDs' L2 caches by themselves, so a grid barrier or a completion counter
// only has to order them: no L2 write-back or invalidation (XCD-wide
// operations) is needed.
__device__ __forceinline__ int ld_coh(const int* p) {
  return __hip_atomic_load(const_cast<int*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 ld_coh2(const float2* p) {
  const uint64_t u = __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float2*>(p)),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float((uint32_t)u), __uint_as_float((uint32_t)(u >> 32)));
}
// 16 bytes written by another workgroup in this launch: two device-coherent
// 64-bit loads (p 16-byte aligned).
__device__ __forceinline__ uint4 ld_coh16(const void* p) {
  uint64_t* q = reinterpret_cast<uint64_t*>(const_cast<void*>(p));
  const uint64_t lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_uint4((uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32));
}
__device__ __forceinline__ void st_coh2(float2* p, float2 v) {
  const uint64_t u = (uint64_t)__float_as_uint(v.x) | ((uint64_t)__float_as_uint(v.y) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace dspark
