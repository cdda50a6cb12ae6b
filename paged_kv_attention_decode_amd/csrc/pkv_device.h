// Device-side helpers shared by the decode, append and prefill kernels:
// element formats, the page-chunk layout, wave-level reductions, operand
// conversions and MFMA wrappers for gfx950.  Included by the .hip sources only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_internal.h"

namespace pkv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Element width in bits; elem_t is the storage word of one element (int4: a
// byte holding two, the even element in the low nibble).
template <int KVT> struct Kv;
template <> struct Kv<KV_F32> { static constexpr int BITS = 32; typedef uint32_t elem_t; };
template <> struct Kv<KV_BF16> { static constexpr int BITS = 16; typedef uint16_t elem_t; };
template <> struct Kv<KV_FP8> { static constexpr int BITS = 8; typedef uint8_t elem_t; };
template <> struct Kv<KV_INT8> { static constexpr int BITS = 8; typedef uint8_t elem_t; };
template <> struct Kv<KV_INT4> { static constexpr int BITS = 4; typedef uint8_t elem_t; };
// Byte offset of element index x (element indices of int4 chunks are even
// wherever a whole byte is addressed).
template <int KVT>
__device__ __forceinline__ size_t elem_byte(size_t x) { return x * Kv<KVT>::BITS / 8; }
// Element x of an array of stored elements, as its code (int4: the nibble).
template <int KVT>
__device__ __forceinline__ uint32_t get_code(const void* base, size_t x) {
  typedef typename Kv<KVT>::elem_t T;
  if constexpr (Kv<KVT>::BITS == 4)
    return ((uint32_t)static_cast<const uint8_t*>(base)[x >> 1] >> (4 * (x & 1))) & 0xFu;
  else
    return static_cast<const T*>(base)[x];
}
// Store element x (int4: read-modify-write of its byte; no other thread may
// write the same byte concurrently).
template <int KVT>
__device__ __forceinline__ void put_code(void* base, size_t x, uint32_t c) {
  typedef typename Kv<KVT>::elem_t T;
  if constexpr (Kv<KVT>::BITS == 4) {
    uint8_t* p = static_cast<uint8_t*>(base) + (x >> 1);
    const int sh = 4 * (int)(x & 1);
    *p = (uint8_t)((*p & ~(0xF << sh)) | ((c & 0xFu) << sh));
  } else {
    static_cast<T*>(base)[x] = (T)c;
  }
}

// ---------------------------------------------------------------------------
// Chunk addressing shared by every kernel.  A (page, kv head) chunk holds P
// tokens x D elements; E = 16 / element bytes; V blocks hold TB = 4E tokens.
// ---------------------------------------------------------------------------
template <int E>
__device__ __forceinline__ int k_elem(int j, int d, int P) {
  return ((d / E) * P + j) * E + (d % E);
}
template <int E>
__device__ __forceinline__ int v_elem(int j, int d, int D) {
  constexpr int TB = 4 * E;
  const int blk = j / TB, r = j % TB;
  const int c = (r & 15) >> 2, e = 4 * (r >> 4) + (r & 3);
  return blk * TB * D + (c * D + d) * E + e;
}
__device__ __forceinline__ size_t chunk_elem(int page, int g, int Hkv, int P, int D) {
  return ((size_t)page * (size_t)Hkv + (size_t)g) * (size_t)P * (size_t)D;
}

// ---------------------------------------------------------------------------
// Wave-level helpers (64 lanes)
// ---------------------------------------------------------------------------
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int x = __shfl_up(v, o);
    if (lane >= o) v += x;
  }
  return v;
}
typedef const int32_t __attribute__((address_space(4)))* const_i32_ptr;
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ float fbits(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t ubits(float f) { return __builtin_bit_cast(uint32_t, f); }

// Round-to-nearest-even fp32 -> bf16 bits (NaN stays NaN).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = ubits(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) & 0x8000u) | 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
// Upper halves of two fp32 words packed as (lo, hi) bf16 pair = truncation.
__device__ __forceinline__ uint32_t pack_hi16(float lo, float hi) {
  return __builtin_amdgcn_perm(ubits(hi), ubits(lo), 0x07060302u);
}
// p = hi + lo with hi, lo bf16 (truncated): ~16 significant bits of p.
__device__ __forceinline__ u32x2_t split_pair(float a, float b) {
  const float ra = a - fbits(ubits(a) & 0xffff0000u);
  const float rb = b - fbits(ubits(b) & 0xffff0000u);
  return u32x2_t{pack_hi16(a, b), pack_hi16(ra, rb)};
}
// Probabilities of two 16-token tiles (8 per lane) as hi and lo bf16x8 operands.
__device__ __forceinline__ void split_probs(const float (&x)[4], const float (&y)[4], float mul,
                                           u32x4_t& hi, u32x4_t& lo) {
  const u32x2_t a = split_pair(x[0] * mul, x[1] * mul), b = split_pair(x[2] * mul, x[3] * mul);
  const u32x2_t c = split_pair(y[0] * mul, y[1] * mul), d = split_pair(y[2] * mul, y[3] * mul);
  hi = u32x4_t{a.x, b.x, c.x, d.x};
  lo = u32x4_t{a.y, b.y, c.y, d.y};
}
// Two fp32 -> packed bf16 pair (round to nearest even), element a low.
__device__ __forceinline__ uint32_t pack_bf16_rne(float a, float b) {
  const bf16x2_t r = __builtin_convertvector(f32x2_t{a, b}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, r);
}
// v *= a element by element, each product written back into its own register
// (a plain multiply inside a rarely taken branch makes the compiler give the
// products new registers and copy every accumulator on the common path).
__device__ __forceinline__ void scale_in_place(f32x4_t& v, float a) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float x = v[i];
    asm("v_mul_f32 %0, %1, %0" : "+v"(x) : "v"(a));
    v[i] = x;
  }
}

// Maximum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one MFMA column):
// the 16-lane row swap pairs rows 0-1 and 2-3, the 32-lane swap the halves.
__device__ __forceinline__ float colmax4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(ubits(x), ubits(x), false, false);
  const float y = fmaxf(fbits(a[0]), fbits(a[1]));
  const auto c = __builtin_amdgcn_permlane32_swap(ubits(y), ubits(y), false, false);
  return fmaxf(fbits(c[0]), fbits(c[1]));
}

// Four fp8 e4m3 bytes -> four bf16 (exact: every e4m3 value is a bf16 value),
// two at a time by the hardware fp8 -> bf16 conversion with scale 1.
__device__ __forceinline__ u32x2_t fp8x4_to_bf16x4(uint32_t w) {
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, false);   // bytes 0, 1
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, true);    // bytes 2, 3
  return u32x2_t{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
}
// Four int8 bytes -> four bf16 (exact: |v| <= 128 has at most 8 significant
// bits).  Each signed-byte conversion is one instruction (a sign-extending byte
// select on the int -> float convert).
__device__ __forceinline__ u32x2_t i8x4_to_bf16x4(uint32_t w) {
  const float a = (float)(int8_t)w, b = (float)(int8_t)(w >> 8);
  const float c = (float)(int8_t)(w >> 16), d = (float)((int32_t)w >> 24);
  return u32x2_t{pack_hi16(a, b), pack_hi16(c, d)};
}
// Eight int4 codes (one word, element k in nibble k: element 2i in the low
// nibble of byte i) -> a bf16x8 operand holding 136 + n for each code n in
// [-8, 7]: with u = n + 8 (the code with its top bit flipped), the bf16 pattern
// 0x4300 | u is exactly 128 + u.  Nibbles i and 4 + i lie 16 bits apart, so
// one shift and one and-xor (which also flips the top bits) give both: slot
// order (e0, e4, e1, e5, e2, e6, e3, e7).  The other operand of each product
// is laid out in that order, and products carry 136 * (sum of the other
// operand), which callers subtract.
__device__ __forceinline__ u32x4_t nib8_to_bf16x8(uint32_t w) {
  u32x4_t r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = ((w >> (4 * i)) & 0x000F000Fu) ^ 0x43084308u;
  return r;
}
// Eight bf16 values (natural order) reordered to the slot order above.
__device__ __forceinline__ u32x4_t zip_halves(u32x4_t x) {
  return u32x4_t{__builtin_amdgcn_perm(x[2], x[0], 0x05040100u), __builtin_amdgcn_perm(x[2], x[0], 0x07060302u),
                 __builtin_amdgcn_perm(x[3], x[1], 0x05040100u), __builtin_amdgcn_perm(x[3], x[1], 0x07060302u)};
}
constexpr float INT4_BIAS = 136.f;
// The same codes as fp16 operands: 0x6400 | u is 1024 + u, so a code n
// (u = n + 8) becomes 1032 + n, in the slot order of nib8_to_bf16x8.
__device__ __forceinline__ u32x4_t nib8_to_f16x8(uint32_t w) {
  u32x4_t r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = ((w >> (4 * i)) & 0x000F000Fu) ^ 0x64086408u;
  return r;
}
constexpr float INT4_F16_BIAS = 1032.f;
// Four int8 bytes -> four fp16 values 1152 + b (bytes in order): with
// u = b + 128 (the sign bit flipped), 0x6400 | u is 1024 + u, so one xor and
// two byte permutes (each placing two bytes under the 0x64 exponent byte)
// widen four values exactly.
__device__ __forceinline__ u32x2_t i8x4_to_f16x4_biased(uint32_t w) {
  const uint32_t u = w ^ 0x80808080u;
  return u32x2_t{__builtin_amdgcn_perm(0x64646464u, u, 0x04010400u),
                 __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u)};
}
constexpr float INT8_F16_BIAS = 1152.f;
// Two fp32 -> packed fp16 pair (round to nearest even), element a low.
__device__ __forceinline__ uint32_t pack_f16_rne(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, f16x2_t));
}

// Eight one-byte cache elements (fp8 e4m3 or int8) -> a bf16x8 MFMA operand.
template <int KVT>
__device__ __forceinline__ u32x4_t byte8_to_bf16x8(uint32_t w0, uint32_t w1) {
  const u32x2_t a = KVT == KV_FP8 ? fp8x4_to_bf16x4(w0) : i8x4_to_bf16x4(w0);
  const u32x2_t b = KVT == KV_FP8 ? fp8x4_to_bf16x4(w1) : i8x4_to_bf16x4(w1);
  return u32x4_t{a.x, a.y, b.x, b.y};
}

__device__ __forceinline__ f32x4_t mfma_bf16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_f16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_f32(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ u32x4_t ld16(const uint8_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}
// Streaming load for K/V: each byte is read exactly once per call, so mark it
// nontemporal and keep it from displacing other lines in L2 and the MALL.
__device__ __forceinline__ u32x4_t ld16_stream(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

// ---------------------------------------------------------------------------
// Work split.  Units are (b, g, range) in b-major, then g, then range order;
// range r of (b, g) covers tokens [r*PT, min(L_b, (r+1)*PT)).  In front of the
// ranges of each (b, g) sit SWITCH_UNITS cost-only units that stand for what a
// wave pays to start a new (b, g) (its query, page id and first tile arrive
// one round trip after another): a wave whose share begins on them starts at
// the pair's first range, one whose share ends on them stops before the pair.
// With T units (cost units included) and at most Wmax waves,
// k = ceil(T / Wmax) and W = ceil(T / k) waves get work.  The waves of
// workgroup i run on XCD i mod 8 (round-robin dispatch), and the waves of the
// odd XCDs stream 8-10 % slower than those of the even ones (per-wave
// timestamps of the decode, on every box measured), so when every share holds
// at least 3 units (k >= 5) the shares are weighted (odd : even = 56 : 64,
// the best of 64 down to 44 in same-box timings of four workloads, with three
// switch units per (b, g), the best of 0 to 6): wave w owns units
// [T * C(w) / C(W), T * C(w + 1) / C(W)), C(w) = sum of the weights of waves
// 0 .. w - 1 (even XCD: WEIGHT_EVEN, odd: WEIGHT_ODD); otherwise
// [w * T / W, (w + 1) * T / W).
// ---------------------------------------------------------------------------
#ifndef PKV_WEIGHT_ODD
#define PKV_WEIGHT_ODD 56
#endif
#ifndef PKV_SWITCH_UNITS
#define PKV_SWITCH_UNITS 3
#endif
constexpr int WEIGHT_EVEN = 64, WEIGHT_ODD = PKV_WEIGHT_ODD;
constexpr int SWITCH_UNITS = PKV_SWITCH_UNITS;
struct Split {
  int64_t T;
  int64_t W;
  int64_t CW;      // C(W) when weighted, else 0
};
// C(w): sum of the share weights of waves 0 .. w - 1 (32 waves = 8 workgroups
// = one round of the 8 XCDs).
__device__ __forceinline__ int64_t share_weight_sum(int64_t w) {
  constexpr int64_t ROUND = 16 * WEIGHT_EVEN + 16 * WEIGHT_ODD;
  const int r = (int)(w & 31), grp = r >> 2;
  const int64_t c = (w >> 5) * ROUND + 4 * (((grp + 1) >> 1) * WEIGHT_EVEN + (grp >> 1) * WEIGHT_ODD);
  return c + (r & 3) * ((grp & 1) ? WEIGHT_ODD : WEIGHT_EVEN);
}
__device__ __forceinline__ Split make_split(int64_t T, int Wmax) {
  Split s;
  s.T = T;
  const int64_t k = (T + Wmax - 1) / Wmax;
  s.W = T > 0 ? (T + k - 1) / k : 0;
  s.CW = (k >= 5 && WEIGHT_ODD != WEIGHT_EVEN) ? share_weight_sum(s.W) : 0;
  return s;
}
__device__ __forceinline__ int64_t range_begin(const Split& s, int64_t w) {
  return s.CW ? s.T * share_weight_sum(w) / s.CW : w * s.T / s.W;
}
// The wave whose range contains unit idx: the last w with range_begin(w) <= idx.
__device__ __forceinline__ int64_t wave_of(const Split& s, int64_t idx) {
  if (!s.CW) return ((idx + 1) * s.W - 1) / s.T;
  // range_begin(w) <= idx  <=>  T * C(w) < (idx + 1) * C(W)
  int64_t lo = 0, hi = s.W - 1;
  const int64_t lim = (idx + 1) * s.CW;
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) >> 1;
    if (s.T * share_weight_sum(mid) < lim) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}
__device__ __forceinline__ int ranges_of(int L, int PT) { return L > 0 ? (L + PT - 1) / PT : 0; }
// Units of one (b, g) in the split: its ranges plus the switch-cost units
// (which count only where a range is one tile, PT = tile size TS).
__device__ __forceinline__ int units_of(int L, int PT, int A) { return L > 0 ? (L + PT - 1) / PT + A : 0; }

// Store 4 consecutive outputs.
template <bool OUT_BF16>
__device__ __forceinline__ void store_out4(void* out_, size_t idx, f32x4_t v) {
  if (OUT_BF16) {
    u32x2_t p;
    p.x = bf16_rne(v[0]) | (bf16_rne(v[1]) << 16);
    p.y = bf16_rne(v[2]) | (bf16_rne(v[3]) << 16);
    *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(out_) + idx) = p;
  } else {
    *reinterpret_cast<f32x4_t*>(static_cast<float*>(out_) + idx) = v;
  }
}

}  // namespace pkv
