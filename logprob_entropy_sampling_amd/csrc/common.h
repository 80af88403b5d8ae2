// Device helpers shared by the scoring kernels (gfx950 only).
//
// Online reduction state.  A row's logits are folded tile by tile into
//   m = max_v u_v,  s = sum_v 2^(u_v - m),  a = sum_v 2^(u_v - m) (u_v - m)
// with u = z * log2(e) = x * (log2(e) / tau): base-2 units, so every
// exponential is one v_exp_f32.  From the merged state:
//   LSE     = ln2 * (m + log2 s)
//   entropy = ln2 * (log2 s - a / s)            (= -sum p ln p)
//   logprob = ln2 * (u_y - m - log2 s)
// (xorl issue #71 section 1: log-sum-exp, then the selected logprob;
//  SkyRL PR #2004: entropy from the same exponentials.)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vs {

constexpr float kLog2e = 1.4426950408889634f;
// log2(e) rounded to 16 significant bits (see scale16): the base-2 scale of
// the bf16 inputs of the softmax L1, which takes no temperature.
constexpr float kLog2eBf16 = 1.44268798828125f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();
// Exponent floor: 2^-256 is 0 in fp32, and keeps e * d finite when d = -inf.
constexpr float kDFloor = -256.0f;

constexpr uint8_t kRowEmpty = 0x01;
constexpr uint8_t kRowOutside = 0x02;
constexpr uint8_t kRowBad = 0x04;
constexpr uint8_t kRowFallback = 0x08;
constexpr uint8_t kRowTruncated = 0x10;

struct Part {
  float m, s, a;
};

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// The base-2 scale c = log2(e) / tau rounded to 16 significant bits (nearest,
// ties away from zero).  Its product with a bf16 value (8 significant bits)
// is exact in fp32, so for bf16 logits the fused form fma(x, c, -m), with m
// the product of the running maximum and c, is exactly 0 at the maximum and
// one rounding of the exact difference elsewhere - at any magnitude.  (With
// c unrounded, fma(x_max, c, -round(x_max * c)) is the product's rounding
// error, about |u| * 2^-24, which at |u| near 2^127 is itself huge.)  The
// rounding moves 1/tau by at most 2^-17 relative.
__device__ __forceinline__ float scale16(float c) {
  return __uint_as_float((__float_as_uint(c) + 0x80u) & 0xFFFFFF00u);
}
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }

// Streaming 16-byte loads (non-temporal): for data read once, or whose
// re-read is not served by the caches anyway.  On gfx950 they sustain about
// 7 TB/s of HBM reads where plain loads stop near 5.4 TB/s.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 stream_load(const uint4* p) {
  u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 stream_load(const float4* p) {
  f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}

// bf16 halves of a packed 32-bit word -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// NaN-preserving floor: a NaN difference stays NaN (and poisons s), -inf
// becomes kDFloor (weight 0, zero entropy contribution).
__device__ __forceinline__ float floor_d(float d) { return d < kDFloor ? kDFloor : d; }

// Fold one more value (already in base-2 units, relative to a fixed m) into s, a.
__device__ __forceinline__ void fold(float d, float& s, float& a) {
  d = floor_d(d);
  float e = exp2_hw(d);
  s += e;
  a = __builtin_fmaf(e, d, a);
}

// Merge two partial states.  Commutative bit for bit (the larger max is
// always the base; on equal maxima both sums are plain commutative adds), so
// any fixed tree gives reproducible results.
__device__ __forceinline__ Part merge(Part p, Part q) {
  if (p.m < q.m) {
    Part t = p;
    p = q;
    q = t;
  }
  if (q.m == kNegInf && q.s == 0.0f) return p;  // q holds no mass (a NaN s still propagates)
  float d = q.m - p.m;           // <= 0, NaN if p.m = +inf
  float f = exp2_hw(d);
  Part r;
  r.m = p.m;
  r.s = p.s + q.s * f;
  // f = 0 (q's maximum far below p's): q adds nothing; q.s * d may
  // overflow to -inf there, and 0 * -inf would be NaN
  r.a = f == 0.0f ? p.a : p.a + f * __builtin_fmaf(q.s, d, q.a);
  return r;
}

// fmaxf drops NaN, so a block whose max is -inf may still hold a NaN: the
// state then carries s = NaN (the row becomes BAD) instead of "empty".
template <int N>
__device__ __forceinline__ float empty_block_s(const float* v) {
  bool nan = false;
#pragma unroll
  for (int i = 0; i < N; ++i) nan |= (v[i] != v[i]);
  return nan ? __builtin_nanf("") : 0.0f;
}

__device__ __forceinline__ bool tau_ok(float tau) { return tau > 0.0f && tau < __builtin_inff(); }

__device__ __forceinline__ float shfl_xor_f(float v, int mask) { return __shfl_xor(v, mask, 64); }
__device__ __forceinline__ float shfl_down_f(float v, int d) { return __shfl_down(v, d, 64); }

// Tree merge across the 64 lanes of a wave; the result is valid in lane 0.
__device__ __forceinline__ Part wave_merge_to_lane0(Part p) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    Part q;
    q.m = shfl_down_f(p.m, off);
    q.s = shfl_down_f(p.s, off);
    q.a = shfl_down_f(p.a, off);
    if ((threadIdx.x & 63 & ((off << 1) - 1)) == 0) p = merge(p, q);
  }
  return p;
}

}  // namespace vs
