// Device-side building blocks for the MonarchAttention kernels (gfx950).
//
// Everything here is written for CDNA4 wave64: one 16x16 MFMA tile per wave
// instruction, fp32 accumulation, and the accumulator layout in which lane l
// holds rows 4*(l/16)+r (r = 0..3) of column l%16.  The kernels compute every
// score tile transposed (keys on the MFMA M dimension, queries on N), so a
// lane owns one query and the four lanes l, l^16, l^32, l^48 share it: row
// reductions over keys are register-local plus two cross-lane steps.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ma {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;
constexpr int WAVES = 4;              // waves per workgroup
constexpr int THREADS = WAVE * WAVES;
constexpr int KT = 64;                // keys per streamed tile
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// MFMA traits: KPL = k-values each lane supplies per instruction (the lane
// group g = lane/16 supplies the g-th run of KPL consecutive k of a step of
// 4*KPL).  Only the consistency of this mapping between the A and B operands
// matters for the result, and both operands are built with it.
template <typename T> struct Mfma;

template <> struct Mfma<bf16> {
  static constexpr int KPL = 8;
  typedef bf16x8 frag;
  __device__ static inline f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mfma<float> {
  static constexpr int KPL = 1;
  typedef float frag;
  __device__ static inline f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

__device__ inline float to_f32(float x) { return x; }
__device__ inline float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ inline T from_f32(float x);
template <> __device__ inline float from_f32<float>(float x) { return x; }
template <> __device__ inline bf16 from_f32<bf16>(float x) { return (bf16)x; }

// 16-byte vector of T: 8 bf16 or 4 floats.
template <typename T> struct Vec16;
template <> struct Vec16<bf16> { typedef bf16x8 type; static constexpr int N = 8; };
template <> struct Vec16<float> { typedef f32x4 type; static constexpr int N = 4; };

// Reductions over the lanes l, l^16, l^32, l^48 with the gfx950 lane-swap
// VALU instructions (no LDS round trip).  permlane16_swap(v, v) returns
// {v of the even 16-lane row of each pair, v of the odd row} in every lane
// of the pair; permlane32_swap(v, v) does the same for the two 32-lane
// halves.  Combining the two results gives op(v[l], v[l^16]) and then
// op(v[l], v[l^32]); operand order differs by lane, which fp max and fp add
// do not see (both are commutative).
__device__ inline float xor16_pair(float v, float& w) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  w = __uint_as_float(r[1]);
  return __uint_as_float(r[0]);
}
__device__ inline float xor32_pair(float v, float& w) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  w = __uint_as_float(r[1]);
  return __uint_as_float(r[0]);
}
__device__ inline float wave_max_x16x32(float v) {
  float w;
  float a = xor16_pair(v, w);
  v = fmaxf(a, w);
  a = xor32_pair(v, w);
  return fmaxf(a, w);
}
__device__ inline float wave_sum_x16x32(float v) {
  float w;
  float a = xor16_pair(v, w);
  v = a + w;
  a = xor32_pair(v, w);
  return a + w;
}

// Store 4 consecutive values (one accumulator column run) to global memory.
__device__ inline void store4(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }
__device__ inline void store4(bf16* p, f32x4 v) {
  bf16x4 b;
  b[0] = (bf16)v[0]; b[1] = (bf16)v[1]; b[2] = (bf16)v[2]; b[3] = (bf16)v[3];
  *reinterpret_cast<bf16x4*>(p) = b;
}

// Tokens along one grid axis: token(r) = base + (r / m) * s1 + (r % m) * s2,
// or base + r * s2 when m == 0 (uniform over a workgroup).  In a padded flat
// sequence the grid positions whose token falls outside [0, hi] are padding:
// at() clamps them to a real token, so every load through it stays in
// bounds, and valid() tells them apart (stores must check it).
struct AxisMap {
  int64_t base;
  int m, s1, s2;
  int64_t hi;           // last real token
  __device__ inline int64_t raw(int r) const {
    if (m == 0) return base + (int64_t)r * s2;
    const int a = r / m;
    return base + (int64_t)a * s1 + (int64_t)(r - a * m) * s2;
  }
  // tokens fit 32 bits (the grid is limited to 2^26 positions)
  __device__ inline int64_t at(int r) const {
    return min(max((int)raw(r), 0), (int)hi);      // one v_med3_i32
  }
  __device__ inline bool valid(int r) const {
    const int t = (int)raw(r);
    return t >= 0 && t <= (int)hi;
  }
};

// ---------------------------------------------------------------------------
// Token order <-> grid position (l, i): the flat reshape and the six aligned
// video layouts of an f x h x w latent (row-major tokens).
// ---------------------------------------------------------------------------
struct GridMap {
  int kind;          // ma_layout
  int b1, b2;
  int h, w, hw;
  int pre;           // padding positions before the first token (flat only)
  int n;             // real tokens; n < b1*b2 for a padded flat sequence

  // Padding (flat layout only): the grid holds b1*b2 >= n positions; with
  // `pre` leading padding positions, position l*b2 + i holds token
  // l*b2 + i - pre, and positions outside [0, n) are padding (MonarchAttention,
  // OpenReview author response on block sizes: m = ceil(N/b), pre- or
  // post-padding).
  __device__ inline bool padded() const { return n != b1 * b2; }

  // Token at grid position (l, i), clamped to a real token at padding
  // positions (loads only; see valid()).
  __device__ inline int64_t token(int l, int i) const {
    return min(max((int)raw_token(l, i), 0), n - 1);
  }
  __device__ inline bool valid(int l, int i) const {
    const int t = (int)raw_token(l, i);
    return t >= 0 && t < n;
  }
  // Number of real rows l in [l0, l1) of column i.
  __device__ inline int real_rows(int i, int l0, int l1) const {
    if (kind != 0) return l1 - l0;
    // token l*b2 + i - pre in [0, n)  <=>  l in [lo, hi)
    const int a = pre - i, c = n + pre - i;                // l*b2 >= a, l*b2 < c
    const int lo = a <= 0 ? 0 : (a + b2 - 1) / b2;
    const int hi = c <= 0 ? 0 : (c + b2 - 1) / b2;
    return max(0, min(hi, l1) - max(lo, l0));
  }
  // Real keys of block k: positions j in [key_lo(k), key_hi(k)).
  __device__ inline int key_lo(int k) const {
    return kind == 0 ? min(max(pre - k * b2, 0), b2) : 0;
  }
  __device__ inline int key_hi(int k) const {
    return kind == 0 ? min(max(n + pre - k * b2, 0), b2) : b2;
  }

  // PAD = false: an unpadded grid (no leading padding to subtract)
  template <bool PAD = true>
  __device__ inline int64_t raw_token(int l, int i) const {
    switch (kind) {
      case 2:  // (w, fh): l = w, i = f*h + h
      case 4:  // (hw, f): l = h*w + w, i = f
        return (int64_t)i * b1 + l;
      case 5: {  // (fw, h): l = f*w + w_, i = h_
        int fi = l / w, wi = l - fi * w;
        return (int64_t)fi * hw + (int64_t)i * w + wi;
      }
      case 6: {  // (h, fw): l = h_, i = f*w + w_
        int fi = i / w, wi = i - fi * w;
        return (int64_t)fi * hw + (int64_t)l * w + wi;
      }
      default:  // flat, (fh, w), (f, hw): row-major reshape
        return (int64_t)l * b2 + i - (PAD ? pre : 0);
    }
  }

  // token(l, i) as a function of i (row l of the grid)
  template <bool PAD = true>
  __device__ inline AxisMap row_axis(int l) const {
    const int64_t hi = n - 1;
    switch (kind) {
      case 2:
      case 4: return AxisMap{l, 0, 0, b1, hi};
      case 5: { const int fi = l / w; return AxisMap{(int64_t)fi * hw + (l - fi * w), 0, 0, w, hi}; }
      case 6: return AxisMap{(int64_t)l * w, w, hw, 1, hi};
      default: return AxisMap{(int64_t)l * b2 - (PAD ? pre : 0), 0, 0, 1, hi};
    }
  }
  // token(l, i) as a function of l (column i of the grid)
  template <bool PAD = true>
  __device__ inline AxisMap col_axis(int i) const {
    const int64_t hi = n - 1;
    switch (kind) {
      case 2:
      case 4: return AxisMap{(int64_t)i * b1, 0, 0, 1, hi};
      case 5: return AxisMap{(int64_t)i * w, w, hw, 1, hi};
      case 6: { const int fi = i / w; return AxisMap{(int64_t)fi * hw + (i - fi * w), 0, 0, w, hi}; }
      default: return AxisMap{(int64_t)i - (PAD ? pre : 0), 0, 0, b2, hi};
    }
  }
};

// Map a linear workgroup id so that consecutive logical ids run on the same
// XCD (the dispatcher deals workgroups to the 8 XCDs round-robin), which lets
// neighbours that read the same tiles share one L2.  Exact bijection on
// [0, n) for any n.
__device__ inline uint32_t xcd_swizzle(uint32_t id, uint32_t n) {
  constexpr uint32_t X = 8;
  uint32_t q = n / X, r = n % X;
  uint32_t xcd = id % X, pos = id / X;
  // XCDs below r own q+1 workgroups, the others q
  uint32_t base = xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q;
  return base + pos;
}

}  // namespace ma
