// sv_device.hpp -- device-side helpers shared by the verify-step kernels (gfx950).
//
// bf16 storage, MFMA operand types, wavefront reductions, and the Philox4x64-10
// counter-based generator (Salmon, Moraes, Dror, Shaw, "Parallel random numbers:
// as easy as 1, 2, 3", SC'11) that keys every random draw of the sampling rule by
// (seed, sequence, absolute position, purpose) -- the per-position independent
// randomness that [Self-spec] section 3.3 requires.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

typedef uint16_t bf16_t;                                              // bf16 bit pattern
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));             // MFMA A/B operand
typedef float f32x4 __attribute__((ext_vector_type(4)));               // 16x16 MFMA accumulator
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));        // 16-byte load

constexpr int WAVE = 64;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_to_f32(bf16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// float32 -> bf16, round to nearest even (inputs are finite here; NaN maps to a quiet NaN).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return bf16_t(0x7fc0);
  u += 0x7fffu + ((u >> 16) & 1u);
  return bf16_t(u >> 16);
}

// 16-byte global load that bypasses cache retention (streamed weights).
__device__ __forceinline__ u32x4 load_stream16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Device-coherent word stores for data one workgroup hands to another inside the
// same kernel.  The eight XCDs have separate L2 caches; these relaxed agent-scope
// atomic stores write through to the coherent memory side, so the writer needs no
// L2 write-back fence (see last_workgroup in sv_accept.hpp).
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<unsigned*>(p), __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Row statistics partial: running max, sum of exp((l - max) / T), argmax.
// The argmax keeps the lowest index on ties.
struct alignas(16) RowPart {
  float m;
  float s;
  int a;
  int pad;
};

__device__ __forceinline__ void store_part(RowPart* p, float m, float s, int a) {
  const unsigned long long ms = (static_cast<unsigned long long>(__float_as_uint(s)) << 32) | __float_as_uint(m);
  __hip_atomic_store(reinterpret_cast<unsigned long long*>(p), ms, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  store_coherent(&p->a, a);
}



// Merge (m2, s2, a2) into (m, s, a); c = log2(e) / T (0 when sums are not needed).
// The identity element is (-inf, 0, INT_MAX); rescaling is skipped for empty sums so
// that two identities never form inf - inf.
__device__ __forceinline__ void merge_stat(float& m, float& s, int& a, float m2, float s2, int a2, float c) {
  if (m2 > m || (m2 == m && a2 < a)) {
    if (c != 0.0f) s = (s != 0.0f ? s * exp2f((m - m2) * c) : 0.0f) + s2;
    m = m2;
    a = a2;
  } else if (c != 0.0f && s2 != 0.0f) {
    s = s + s2 * exp2f((m2 - m) * c);
  }
}

__device__ __forceinline__ void wave_merge_stat(float& m, float& s, int& a, float c, int width = WAVE) {
  for (int o = width / 2; o > 0; o >>= 1) {
    float m2 = __shfl_xor(m, o);
    float s2 = __shfl_xor(s, o);
    int a2 = __shfl_xor(a, o);
    merge_stat(m, s, a, m2, s2, a2, c);
  }
}

// DPP lane exchanges within rows of 16 lanes: xor 1, xor 2 (quad permutes), the
// mirror of each half row and of the whole row.  After xor 1 and xor 2 every quad
// holds one value, so the two mirrors complete a 16-lane butterfly; xor 16 and
// xor 32 then go through the LDS crossbar.
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140;

template <int CTRL>
__device__ __forceinline__ int dpp(int v) { return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true); }
template <int CTRL>
__device__ __forceinline__ float dpp(float v) { return __int_as_float(dpp<CTRL>(__float_as_int(v))); }

template <int CTRL>
__device__ __forceinline__ void dpp_merge_stat(float& m, float& s, int& a, float c) {
  merge_stat(m, s, a, dpp<CTRL>(m), dpp<CTRL>(s), dpp<CTRL>(a), c);
}
__device__ __forceinline__ void xor_merge_stat(float& m, float& s, int& a, float c, int o) {
  merge_stat(m, s, a, __shfl_xor(m, o), __shfl_xor(s, o), __shfl_xor(a, o), c);
}

// Butterfly all-reduce of (max, sum, argmax) over the wavefront; every lane ends with
// the same bits (each step merges the same two operands on both sides).
__device__ __forceinline__ void wave_allmerge_stat(float& m, float& s, int& a, float c) {
  dpp_merge_stat<DPP_XOR1>(m, s, a, c);
  dpp_merge_stat<DPP_XOR2>(m, s, a, c);
  dpp_merge_stat<DPP_HALF_MIRROR>(m, s, a, c);
  dpp_merge_stat<DPP_MIRROR>(m, s, a, c);
  xor_merge_stat(m, s, a, c, 16);
  xor_merge_stat(m, s, a, c, 32);
}

// Butterfly all-reduces over the wavefront (DPP within rows of 16, then xor 16 and 32).
__device__ __forceinline__ float wave_allmax(float v) {
  v = fmaxf(v, dpp<DPP_XOR1>(v));
  v = fmaxf(v, dpp<DPP_XOR2>(v));
  v = fmaxf(v, dpp<DPP_HALF_MIRROR>(v));
  v = fmaxf(v, dpp<DPP_MIRROR>(v));
  v = fmaxf(v, __shfl_xor(v, 16));
  return fmaxf(v, __shfl_xor(v, 32));
}
__device__ __forceinline__ float wave_allsum(float v) {
  v += dpp<DPP_XOR1>(v);
  v += dpp<DPP_XOR2>(v);
  v += dpp<DPP_HALF_MIRROR>(v);
  v += dpp<DPP_MIRROR>(v);
  v += __shfl_xor(v, 16);
  return v + __shfl_xor(v, 32);
}
// The same within each row of 16 lanes.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp<DPP_XOR1>(v));
  v = fmaxf(v, dpp<DPP_XOR2>(v));
  v = fmaxf(v, dpp<DPP_HALF_MIRROR>(v));
  return fmaxf(v, dpp<DPP_MIRROR>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<DPP_XOR1>(v);
  v += dpp<DPP_XOR2>(v);
  v += dpp<DPP_HALF_MIRROR>(v);
  return v + dpp<DPP_MIRROR>(v);
}

// (score, index) argmax with lowest index on ties.
__device__ __forceinline__ void merge_best(float& s, int& i, float s2, int i2) {
  if (s2 > s || (s2 == s && i2 < i)) { s = s2; i = i2; }
}

template <int CTRL>
__device__ __forceinline__ void dpp_merge_best(float& s, int& i) { merge_best(s, i, dpp<CTRL>(s), dpp<CTRL>(i)); }

__device__ __forceinline__ void wave_allmerge_best(float& s, int& i) {
  dpp_merge_best<DPP_XOR1>(s, i);
  dpp_merge_best<DPP_XOR2>(s, i);
  dpp_merge_best<DPP_HALF_MIRROR>(s, i);
  dpp_merge_best<DPP_MIRROR>(s, i);
  merge_best(s, i, __shfl_xor(s, 16), __shfl_xor(i, 16));
  merge_best(s, i, __shfl_xor(s, 32), __shfl_xor(i, 32));
}

__device__ __forceinline__ void wave_merge_best(float& s, int& i) {
  for (int o = WAVE / 2; o > 0; o >>= 1) {
    float s2 = __shfl_xor(s, o);
    int i2 = __shfl_xor(i, o);
    merge_best(s, i, s2, i2);
  }
}

// ---------------------------------------------------------------------------
// Philox4x64-10.  State: four 64-bit counter words; key: two 64-bit words.  Each
// round forms the 128-bit products of counter words 0 and 2 with two fixed odd
// multipliers, then sets (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0); the key is
// advanced by two Weyl constants between rounds.  Constants as published with the
// generator.
struct Philox4 {
  uint64_t w[4];
};

// 128-bit product a * b from four 32 x 32 -> 64-bit partial products (schoolbook; each
// step is one v_mad_u64_u32, and no intermediate sum overflows 64 bits).
__device__ __forceinline__ void mul_wide64(uint64_t a, uint64_t b, uint64_t& hi, uint64_t& lo) {
  const uint32_t al = uint32_t(a), ah = uint32_t(a >> 32), bl = uint32_t(b), bh = uint32_t(b >> 32);
  const uint64_t p0 = uint64_t(al) * bl;
  const uint64_t t = uint64_t(al) * bh + (p0 >> 32);
  const uint64_t u = uint64_t(ah) * bl + uint32_t(t);
  lo = (u << 32) | uint32_t(p0);
  hi = uint64_t(ah) * bh + ((t >> 32) + (u >> 32));
}

__device__ __forceinline__ Philox4 philox4x64_10(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3,
                                                 uint64_t k0, uint64_t k1) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += W0; k1 += W1; }
    uint64_t hi0, lo0, hi1, lo1;
    mul_wide64(M0, c0, hi0, lo0);
    mul_wide64(M1, c2, hi1, lo1);
    uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
  }
  Philox4 o;
  o.w[0] = c0; o.w[1] = c1; o.w[2] = c2; o.w[3] = c3;
  return o;
}

constexpr uint64_t TAG_ACCEPT = 0;
constexpr uint64_t TAG_GUMBEL = 1;
constexpr uint64_t TAG_DRAFT = 2;    // the drafter's Gumbel noise (laid out as tag 1)

// Acceptance uniform of the token at absolute position ``pos`` of sequence ``seq``:
// 24 random bits, exact in float32.
__device__ __forceinline__ float accept_uniform(uint64_t seed, uint64_t seq, uint64_t pos) {
  Philox4 r = philox4x64_10(0, pos, seq, TAG_ACCEPT, seed, 0);
  return float(uint32_t(r.w[0] >> 40)) * 5.9604644775390625e-08f;   // 2^-24
}

// Uniform in (0, 1) with 23 random bits from one Philox word.
__device__ __forceinline__ float gumbel_uniform_from_word(uint64_t w) {
  return (float(uint32_t(w >> 41)) + 0.5f) * 1.1920928955078125e-07f;  // 2^-23
}

}  // namespace sv
