// HIP kernels for paged KV-cache decode attention on CDNA4 (gfx950).
//
// Operations (first page, TensorRT-LLM concept page): the cache is kept in
// fixed-size pages reached through a per-sequence page table ("key mechanisms");
// a page-table lookup precedes every cache read and write ("compile-time graph
// optimization"); each decode iteration's attention reads the pages and the
// new token is stored into them ("runtime execution model").  The attention is
// softmax(scale * q K^T) V per query head; long caches are split into ranges
// combined by log-sum-exp, the rule FlashAttention-style kernels (named on the
// first page's "compile-time graph optimization" section and the fourth page)
// use to merge partial softmax results.
//
// Design for gfx950
// -----------------
// * One wavefront owns a contiguous, equal share of all (sequence, kv head,
//   range) work units, so every wave streams the same number of bytes and the
//   grid drains together; the share is derived on the device from seq_lens.
// * A kv page chunk is read once per kv head: the G query heads of the group are
//   the N columns of 16x16 MFMA tiles (padded to 16).
// * The page layout puts each 16-byte group where a lane needs it as an MFMA
//   operand: K groups hold E consecutive dims of one token (QK^T A operand,
//   tokens = M), V groups hold E tokens of one dim (PV A operand, dims = M), so
//   K and V go from HBM straight into operand registers with 256-byte
//   contiguous runs per 16 lanes and no LDS round trip.
// * The QK^T output layout (lane = head column, 4 token rows per lane) is
//   exactly the PV B-operand layout, so probabilities never cross lanes.
// * Online softmax in the log2 domain against a lazy reference: it grows only
//   when a tile's max passes it by more than 8, so the common tile needs no
//   cross-lane step; the running sum stays lane-local until the end.
// * Probabilities enter the bf16 MFMA as a hi + lo bf16 pair (~16 bits);
//   the int4 and int8 caches' value products run on fp16 operands, one
//   fp16 each.
// * fp8 e4m3 is widened exactly to bf16 in registers; the K scale multiplies
//   the logits, the V scale the probabilities (int4, int8: each tile's
//   products).

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "pkv_internal.h"
#include "pkv_device.h"

namespace pkv {

// Cache stores of the append paths are nontemporal: the decode that reads the
// cache next ran 5-14 us slower while the new tokens' lines sat dirty in L2
// (whole-line stores made no difference; streaming stores did).
template <typename T>
__device__ __forceinline__ void store_nt(T* p, T v) { __builtin_nontemporal_store(v, p); }
// The new token's V codes of a lane (NPL dims, element indexes x[i]; each
// in its own 16-byte group).  int4 codes share their byte with a neighbouring
// token, so the old bytes are loaded first, all of them before any store (a
// load after a store would wait for the store as well).
template <int KVT, int NPL>
__device__ __forceinline__ void put_row_codes_nt(void* base, const size_t (&x)[NPL], const uint32_t (&c)[NPL]) {
  if constexpr (Kv<KVT>::BITS == 4) {
    uint8_t* b = static_cast<uint8_t*>(base);
    uint8_t old[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) old[i] = b[x[i] >> 1];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int sh = 4 * (int)(x[i] & 1);
      store_nt(b + (x[i] >> 1), (uint8_t)((old[i] & ~(0xF << sh)) | ((c[i] & 0xFu) << sh)));
    }
  } else {
    typedef typename Kv<KVT>::elem_t T;
#pragma unroll
    for (int i = 0; i < NPL; ++i) store_nt(static_cast<T*>(base) + x[i], (T)c[i]);
  }
}

template <int KVT>
__device__ __forceinline__ void put_code_nt(void* base, size_t x, uint32_t c) {
  typedef typename Kv<KVT>::elem_t T;
  if constexpr (Kv<KVT>::BITS == 4) {
    uint8_t* p = static_cast<uint8_t*>(base) + (x >> 1);
    const int sh = 4 * (int)(x & 1);
    store_nt(p, (uint8_t)((*p & ~(0xF << sh)) | ((c & 0xFu) << sh)));
  } else {
    store_nt(static_cast<T*>(base) + x, (T)c);
  }
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of the n partial ranges of one (b, g) for 256 of its G*D
// outputs, starting at x0, run by one wave.
// Partial slot layout (floats): O[G][D] unnormalised, then m[G] (log2-domain
// softmax reference), then l[G] (sum of 2^(s - m)).  Contributor i is wave wf + i;
// its slot is slot0 for i = 0 and 2 * (wf + i) otherwise.
//   out = sum_i 2^(m_i - M) O_i / sum_i 2^(m_i - M) l_i,  M = max_i m_i.
// Lanes own 4 consecutive (h, d) outputs; contributors are read 8 at a time so
// their loads are in flight together.
// ---------------------------------------------------------------------------
template <bool OUT_BF16>
__device__ void merge_chunk(const float* __restrict__ partials, int64_t slot0, int64_t wf, int n,
                            void* __restrict__ out_, size_t row0, int G, int D, int x0, int lane) {
  const int stride = G * (D + 2);
  const int total = G * D;
  const float NEG_INF = -__builtin_inff();
  const int x = x0 + 4 * lane;
  if (x >= total) return;
  const int h = x / D;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f, M = NEG_INF;
  bool nan = false;
  for (int s0 = 0; s0 < n; s0 += 8) {
    f32x4_t o[8];
    float ms[8], ls[8];
    // Past the last contributor the last one is re-read (no branch around
    // the loads, so all of them are in flight at once) and then masked out.
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int i = min(s0 + k, n - 1);
      const int64_t slot = i == 0 ? slot0 : 2 * (wf + i);
      const float* ps = partials + slot * stride;
      o[k] = *reinterpret_cast<const f32x4_t*>(ps + x);
      ms[k] = ps[total + h];
      ls[k] = ps[total + G + h];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (s0 + k >= n) {
        o[k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        ms[k] = NEG_INF;
        ls[k] = 0.f;
      }
    }
    float mg = M;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      nan |= ms[k] != ms[k];
      mg = fmaxf(mg, ms[k]);
    }
    const float a = M == NEG_INF ? 0.f : __builtin_amdgcn_exp2f(M - mg);
    acc *= a;
    den *= a;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float f = ms[k] == NEG_INF ? 0.f : __builtin_amdgcn_exp2f(ms[k] - mg);
      acc += f * o[k];
      den += f * ls[k];
    }
    M = mg;
  }
  const float inv = nan ? __builtin_nanf("") : 1.f / den;
  store_out4<OUT_BF16>(out_, row0 + x, acc * inv);
}

// ---------------------------------------------------------------------------
// One-byte appends (fp8 e4m3 or int8) with dynamic page scales (quantise on
// write).  QMAX = 448 (fp8) or 127 (int8); NOCLIP = 464 or 127.5, the largest
// |x| / scale whose encoding is the largest code without clipping.
//
// One wave per (sequence, kv head); K and V each with their own scale:
// a = max |x| of the new row (widened to fp32);
//   slot j == 0 (first token of the page): s = a / QMAX (1 if a == 0);
//   else, s0 = the page's scale: s = s0 if a / s0 <= NOCLIP,
//   otherwise s = a / QMAX and every earlier slot is re-encoded,
//   enc((dec(byte) * s0) / s);
// the new row is stored as enc(x / s) and the page scale becomes s.
// Every division and product is one correctly rounded fp32 operation.
// ---------------------------------------------------------------------------

// fp32 -> e4m3fn: nearest value, ties to the even significand, saturating at
// +-448 (NaN -> 0x7F).  With e = max(exponent(|x|), -6), the e4m3 step at |x|
// is 2^(e-3) (the subnormal step 2^-9 below 2^-6), k = rint(|x| / 2^(e-3)) is
// exact in fp32, and the code is 8 * (e + 6) + k: a carry of k to 16 lands on
// the next binade's first code, and below 2^-6 the code is k itself.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  const uint32_t sign = (ubits(x) >> 24) & 0x80u;
  if (x != x) return 0x7Fu;
  const float a = fminf(fabsf(x), 448.f);
  const int e = max((int)((ubits(a) >> 23) & 0xFFu) - 127, -6);
  const int k = (int)rintf(ldexpf(a, 3 - e));
  return sign | (uint32_t)(8 * (e + 6) + k);
}

// fp32 -> symmetric int8 byte: nearest integer, ties to even, clamped to +-127.
__device__ __forceinline__ uint32_t int8_encode(float x) {
  const float r = fminf(fmaxf(rintf(x), -127.f), 127.f);
  return (uint32_t)(int)r & 0xFFu;
}

template <int KVT> struct ByteFmt;
template <> struct ByteFmt<KV_FP8> {
  static constexpr float QMAX = 448.f, NOCLIP = 464.f;
  __device__ static uint32_t enc(float y) { return e4m3_encode(y); }
  __device__ static void dec4(uint32_t w, float (&v)[4]) {
    const f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    const f32x2_t b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    v[0] = a.x; v[1] = a.y; v[2] = b.x; v[3] = b.y;
  }
};
template <> struct ByteFmt<KV_INT8> {
  static constexpr float QMAX = 127.f, NOCLIP = 127.5f;
  __device__ static uint32_t enc(float y) { return int8_encode(y); }
  __device__ static void dec4(uint32_t w, float (&v)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (float)(int8_t)(uint8_t)(w >> (8 * i));
  }
};
// int4: codes are two's complement nibbles; symmetric, clamped to +-7.
template <> struct ByteFmt<KV_INT4> {
  static constexpr float QMAX = 7.f, NOCLIP = 7.5f;
  __device__ static uint32_t enc(float y) {
    const float r = fminf(fmaxf(rintf(y), -7.f), 7.f);
    return (uint32_t)(int)r & 0xFu;
  }
  __device__ static float dec(uint32_t c) { return (float)(int)((c & 0xFu) ^ 8u) - 8.f; }
};

// One element re-encoded under a new scale: enc((dec(code) * s0) / s), the
// product and the quotient each rounded once.
template <int KVT>
__device__ __forceinline__ uint32_t requant1(float v, float s0, float s) {
  const float real = v * s0;
  return ByteFmt<KVT>::enc(real / s);
}
// Four bytes of a word re-encoded (int4: both nibbles of each byte).
template <int KVT>
__device__ __forceinline__ uint32_t requant4(uint32_t w, float s0, float s) {
  uint32_t r = 0;
  if constexpr (KVT == KV_INT4) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      r |= requant1<KVT>(ByteFmt<KVT>::dec(w >> (4 * i)), s0, s) << (4 * i);
  } else {
    float v[4];
    ByteFmt<KVT>::dec4(w, v);
#pragma unroll
    for (int i = 0; i < 4; ++i) r |= requant1<KVT>(v[i], s0, s) << (8 * i);
  }
  return r;
}

// Scale decision for one row: returns the new scale; sets requant when the
// page's earlier slots must be re-encoded.  A row fits the current scale while
// its largest element encodes to the largest code without clipping:
// |x| / s0 <= NOCLIP (fp8: 464, the midpoint above 448, rounds down to 448;
// int8: 127.5 rounds to 128 and clamps to 127, still within half a step).
template <int KVT>
__device__ __forceinline__ float page_scale(float a, int j, float s0, bool& requant) {
  requant = false;
  if (j == 0) return a > 0.f ? a / ByteFmt<KVT>::QMAX : 1.f;
  if (a / s0 <= ByteFmt<KVT>::NOCLIP) return s0;
  requant = true;
  return a / ByteFmt<KVT>::QMAX;
}

// A re-encode maps each old byte through enc((dec(byte) * s0) / s), a function
// of the byte alone: the wave tabulates it once (4 codes per lane) in LDS and
// then re-encodes by lookup.
__device__ __forceinline__ uint32_t lut4(const uint8_t* lut, uint32_t w) {
  return (uint32_t)lut[w & 0xFFu] | ((uint32_t)lut[(w >> 8) & 0xFFu] << 8) |
         ((uint32_t)lut[(w >> 16) & 0xFFu] << 16) | ((uint32_t)lut[w >> 24] << 24);
}

// Re-encode slots [0, j) of a K chunk.  Token t's dims E c .. E c + E - 1 are
// the 16-byte group at chunk + 16 (c P + t); lane l takes tokens l, l + 64, ...
// (TPL of them per round, all GPT groups of each), so no group index is
// divided, and every load of a round is issued before any conversion.
template <int KVT, int D>
__device__ __forceinline__ void requant_k(uint8_t* pool, int j, int P, const uint8_t* lut, int lane) {
  constexpr int GPT = D * Kv<KVT>::BITS / 128;       // 16-byte groups per token
  constexpr int TPL = 16 / GPT;                      // tokens per lane per round
  for (int t0 = 0; t0 < j; t0 += 64 * TPL) {
    u32x4_t w[TPL][GPT];
#pragma unroll
    for (int a = 0; a < TPL; ++a) {
      const int t = min(t0 + 64 * a + lane, j - 1);    // clamped: in-bounds, stored only if owned
#pragma unroll
      for (int c = 0; c < GPT; ++c) w[a][c] = *reinterpret_cast<const u32x4_t*>(pool + 16 * (c * P + t));
    }
#pragma unroll
    for (int a = 0; a < TPL; ++a) {
      const int t = t0 + 64 * a + lane;
      if (t < j) {
#pragma unroll
        for (int c = 0; c < GPT; ++c) {
          u32x4_t r;
#pragma unroll
          for (int q = 0; q < 4; ++q) r[q] = lut4(lut, w[a][c][q]);
          store_nt(reinterpret_cast<u32x4_t*>(pool + 16 * (c * P + t)), r);
        }
      }
    }
  }
}

// Masks of a run of four consecutive elements of BITS bits starting at bit o
// of a word, whose tokens are k0 .. k0 + 3 places after slot j (k = j - first
// token of the run): elements before j go into lt, the one at j into eq.
template <int BITS>
__device__ __forceinline__ void run_masks(int k, int o, uint32_t& lt, uint32_t& eq) {
  constexpr uint32_t RUN = BITS == 8 ? 0xFFFFFFFFu : 0xFFFFu, EL = (1u << BITS) - 1u;
  const int n = min(max(k, 0), 4);
  lt |= (n == 4 ? RUN : ((1u << (BITS * n)) - 1u)) << o;
  if (k >= 0 && k < 4) eq |= EL << (BITS * k + o);
}

// Re-encode a V chunk for a scale change at slot j: a 16-byte group holds E
// tokens of one dim from one TB = 4E token block; blocks 0 .. j/TB are
// rewritten group by group.  Blocks before j's hold earlier slots only and are
// re-encoded whole; in j's block, tokens < j are re-encoded, token j takes its
// new code (nbj, from LDS) and later slots keep theirs.  A round's 64 * GPL
// groups cover whole blocks (4 D groups each), so the block of a lane's i-th
// group, and with it the choice between the two, is the same on every lane.
template <int KVT, int D>
__device__ __forceinline__ void requant_v(uint8_t* pool, int j, const uint8_t* lut, const uint8_t* nbj,
                                          int lane) {
  constexpr int BITS = Kv<KVT>::BITS, E = 128 / BITS;
  constexpr int GPL = 16, TB = 4 * E;
  constexpr int GPB = 4 * D;    // 16-byte groups per V block (blocks are contiguous)
  static_assert((64 * GPL) % GPB == 0 && GPB % 64 == 0, "a round covers whole blocks");
  const int jb = j / TB;
  const int ngrp = (jb + 1) * GPB;
  for (int base = 0; base < ngrp; base += 64 * GPL) {
    u32x4_t w[GPL];
#pragma unroll
    for (int i = 0; i < GPL; ++i) {
      const int gi = min(base + lane + 64 * i, ngrp - 1);
      w[i] = *reinterpret_cast<const u32x4_t*>(pool + (size_t)gi * 16);   // blocks are contiguous
    }
#pragma unroll
    for (int i = 0; i < GPL; ++i) {
      const int blk = uniform((base + 64 * i) / GPB);
      if (blk > jb) continue;                          // past j's block (uniform)
      const int gi = base + lane + 64 * i;
      u32x4_t r;
      if (blk < jb) {
#pragma unroll
        for (int q = 0; q < 4; ++q) r[q] = lut4(lut, w[i][q]);
      } else {
        // element e of the group holds token 16 (e / 4) + 4c + e % 4 of the
        // block: each word holds runs of four consecutive tokens (one run of
        // bytes, or two runs of nibbles 16 tokens apart), so per word the
        // elements before j, at j and after j are three bit masks
        const int rem = gi - blk * GPB;
        const int c = rem / D, d = rem - c * D;
        const uint32_t fresh = nbj[d] * (BITS == 4 ? 0x11111111u : 0x01010101u);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t lt = 0, eq = 0;
          if constexpr (BITS == 4) {
            run_masks<4>(j - (blk * TB + 32 * q + 4 * c), 0, lt, eq);
            run_masks<4>(j - (blk * TB + 32 * q + 16 + 4 * c), 16, lt, eq);
          } else {
            run_masks<8>(j - (blk * TB + 16 * q + 4 * c), 0, lt, eq);
          }
          r[q] = (lut4(lut, w[i][q]) & lt) | (fresh & eq) | (w[i][q] & ~(lt | eq));
        }
      }
      store_nt(reinterpret_cast<u32x4_t*>(pool + (size_t)gi * 16), r);
    }
  }
}


// New rows of (b, g) for the quantising append: lane l holds dims
// l * D / 64 .. of the K and the V row, widened to fp32 (bf16 or fp32 input).
template <int D>
__device__ __forceinline__ void load_new_rows(const void* k_new, const void* v_new, bool in_bf16, size_t row,
                                              float (&xk)[D / 64], float (&xv)[D / 64]) {
#pragma unroll
  for (int i = 0; i < D / 64; ++i) {
    xk[i] = in_bf16 ? fbits((uint32_t)static_cast<const uint16_t*>(k_new)[row + i] << 16)
                    : static_cast<const float*>(k_new)[row + i];
    xv[i] = in_bf16 ? fbits((uint32_t)static_cast<const uint16_t*>(v_new)[row + i] << 16)
                    : static_cast<const float*>(v_new)[row + i];
  }
}

// Largest |x| of a row held D / 64 elements per lane (wave-uniform result):
// rotations within each 16-lane row (DPP), then across the four rows.
template <int NPL>
__device__ __forceinline__ float row_amax(const float (&x)[NPL]) {
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < NPL; ++i) a = fmaxf(a, fabsf(x[i]));
  a = fmaxf(a, fbits((uint32_t)__builtin_amdgcn_update_dpp(0, (int)ubits(a), 0x128, 0xF, 0xF, false)));  // row_ror:8
  a = fmaxf(a, fbits((uint32_t)__builtin_amdgcn_update_dpp(0, (int)ubits(a), 0x124, 0xF, 0xF, false)));  // row_ror:4
  a = fmaxf(a, fbits((uint32_t)__builtin_amdgcn_update_dpp(0, (int)ubits(a), 0x122, 0xF, 0xF, false)));  // row_ror:2
  a = fmaxf(a, fbits((uint32_t)__builtin_amdgcn_update_dpp(0, (int)ubits(a), 0x121, 0xF, 0xF, false)));  // row_ror:1
  return fbits(uniform((int)ubits(colmax4(a))));
}

// The quantising append of one (b, g) pair of rows into slot j of its page,
// run by one wave (lane l holds dims d0 = l * D / 64 .. of each row): the new
// page scales, the new codes, the re-encode of the page's earlier slots when a
// scale rises, then the new scales.  kp / vp point at the page's K / V chunk,
// si indexes its scales, sk0 / sv0 are their values before this append (read
// by the caller; ignored for slot 0); lut (2 x 64 words) and nb (D bytes) are
// this wave's LDS scratch.  Used by the standalone append and by the
// quantising step.
template <int KVT, int D>
__device__ __forceinline__ void quant_store_row(const float (&xk)[D / 64], const float (&xv)[D / 64], int j,
                                                uint8_t* kp, uint8_t* vp, int P, float* kscales, float* vscales,
                                                size_t si, float sk0, float sv0, uint32_t (*lut)[64], uint8_t* nb,
                                                int lane) {
  constexpr int NPL = D / 64;
  const int d0 = lane * NPL;
  if (j == 0) sk0 = sv0 = 1.f;          // the page's first token: the old scales are not used
  const float ak = row_amax(xk), av = row_amax(xv);
  sk0 = fbits(uniform((int)ubits(sk0)));
  sv0 = fbits(uniform((int)ubits(sv0)));
  bool rk, rv;
  const float sk = page_scale<KVT>(ak, j, sk0, rk);
  const float sv = page_scale<KVT>(av, j, sv0, rv);
  uint32_t nbk[NPL], nbv[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    nbk[i] = ByteFmt<KVT>::enc(xk[i] / sk);
    nbv[i] = ByteFmt<KVT>::enc(xv[i] / sv);
  }
  const uint8_t* lutk = reinterpret_cast<const uint8_t*>(lut[0]);
  const uint8_t* lutv = reinterpret_cast<const uint8_t*>(lut[1]);
  if (rk || rv) {
    const uint32_t codes = (uint32_t)(4 * lane) * 0x01010101u + 0x03020100u;   // 4 codes per lane
    if (rk) lut[0][lane] = requant4<KVT>(codes, sk0, sk);
    if (rv) lut[1][lane] = requant4<KVT>(codes, sv0, sv);
    __builtin_amdgcn_wave_barrier();     // one wave's LDS operations complete in order
  }
  constexpr int E = 128 / Kv<KVT>::BITS;
  if (rk) requant_k<KVT, D>(kp, j, P, lutk, lane);
  // the new K token's dims d0.. are consecutive elements of one group
  // (disjoint from the re-encoded slots): two bytes, or one int4 byte
  uint8_t* kt = kp + elem_byte<KVT>(k_elem<E>(j, d0, P));
  if constexpr (KVT == KV_INT4)
    store_nt(kt, (uint8_t)(nbk[0] | (nbk[NPL - 1] << 4)));
  else if constexpr (NPL == 2)
    store_nt(reinterpret_cast<uint16_t*>(kt), (uint16_t)(nbk[0] | (nbk[NPL - 1] << 8)));
  else
    store_nt(kt, (uint8_t)nbk[0]);
  if (rv) {
#pragma unroll
    for (int i = 0; i < NPL; ++i) nb[d0 + i] = (uint8_t)nbv[i];
    __builtin_amdgcn_wave_barrier();     // one wave's LDS operations complete in order
    requant_v<KVT, D>(vp, j, lutv, nb, lane);
  } else {
    size_t xv[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) xv[i] = v_elem<E>(j, d0 + i, D);
    put_row_codes_nt<KVT, NPL>(vp, xv, nbv);   // own codes
  }
  if (lane == 0) {
    kscales[si] = sk;
    vscales[si] = sv;
  }
}

// One row (K if !IS_V, else V) of the quantising step's append into slot j
// of its page: the row's page scale, its codes, the new scale.  When the
// scale rises, the split kernel has already stored the page as the append
// leaves it (slots [0, j) re-encoded, slot j's new codes), so only the scale
// is written here.  The K and V rows are independent (own scales), so the
// merge kernel gives each its own wave.  pc points at the page's K or V
// chunk, si indexes its scale, s0 is the scale before this append (ignored
// for slot 0).
template <int KVT, int D, bool IS_V>
__device__ __forceinline__ void quant_store_half(const float (&x)[D / 64], int j, uint8_t* pc, int P, float* scales,
                                                 size_t si, float s0, int lane) {
  constexpr int NPL = D / 64, E = 128 / Kv<KVT>::BITS;
  const int d0 = lane * NPL;
  if (j == 0) s0 = 1.f;
  const float a = row_amax(x);
  s0 = fbits(uniform((int)ubits(s0)));
  bool r;
  const float sc = page_scale<KVT>(a, j, s0, r);
  if (!r) {
    uint32_t nbc[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) nbc[i] = ByteFmt<KVT>::enc(x[i] / sc);
    if constexpr (!IS_V) {
      uint8_t* kt = pc + elem_byte<KVT>(k_elem<E>(j, d0, P));
      if constexpr (KVT == KV_INT4)
        store_nt(kt, (uint8_t)(nbc[0] | (nbc[NPL - 1] << 4)));
      else if constexpr (NPL == 2)
        store_nt(reinterpret_cast<uint16_t*>(kt), (uint16_t)(nbc[0] | (nbc[NPL - 1] << 8)));
      else
        store_nt(kt, (uint8_t)nbc[0]);
    } else {
      size_t xv[NPL];
#pragma unroll
      for (int i = 0; i < NPL; ++i) xv[i] = v_elem<E>(j, d0 + i, D);
      put_row_codes_nt<KVT, NPL>(pc, xv, nbc);   // own codes
    }
  }
  if (lane == 0) scales[si] = sc;
}

// ---------------------------------------------------------------------------
// Decode, part 1: each wave streams its unit range.  A (b, g) covered by one
// wave is finished here; otherwise each covering wave leaves a partial and the
// wave holding the first unit of (b, g) leaves a descriptor (first contributing
// wave, number of contributors, slot of the first) for the merge kernel.
// ---------------------------------------------------------------------------
template <int KVT, int D, bool OUT_BF16, bool QNEW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void decode_split_kernel(
    const void* __restrict__ q_, const uint8_t* __restrict__ kpool, const uint8_t* __restrict__ vpool,
    const void* __restrict__ k_new, const void* __restrict__ v_new,
    const float* __restrict__ kscales, const float* __restrict__ vscales,
    const int32_t* __restrict__ bt, const int32_t* __restrict__ seq_lens, void* __restrict__ out_,
    float* __restrict__ partials, int4* __restrict__ descs, int4* __restrict__ qdescs, int B, int MP, int NP,
    int Hq, int Hkv, int G, int P, int PT, int Wmax, float scale_log2, int new_bf16) {
  constexpr int BITS = Kv<KVT>::BITS;
  constexpr int E = 128 / BITS;     // elements per 16-byte group
  constexpr int TS = 4 * E;         // tokens per step (= V block)
  constexpr int NSUB = TS / 16;     // 16-token QK^T tiles per step
  constexpr int NKK = D / (4 * E);  // K groups per lane per 16-token tile
  constexpr int NDT = D / 16;       // 16-dim PV tiles
  constexpr bool I4 = KVT == KV_INT4;
  // int4 and int8: the value products run on fp16 operands, the codes widened
  // to V_BIAS + n and the bias taken back out through LP (see below)
  constexpr bool F16PV = I4 || KVT == KV_INT8;
  constexpr float V_BIAS = I4 ? INT4_F16_BIAS : INT8_F16_BIAS;
  constexpr bool SCALED = BITS <= 8;   // fp8, int8, int4: per-page scales, widened exactly
  constexpr int NCH = I4 ? 4 : SCALED ? 2 : 1;   // bf16x8 operands per 16-byte group
  constexpr int NQ = NCH * NKK;
  static_assert(NKK >= 1, "head_dim too small for this element width");

  constexpr float TH = 8.f;          // softmax reference lag allowed before a rescale (log2 units)
  constexpr float P_SHIFT = 7.f;     // int4: probabilities enter fp16 products as p * 2^7

  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15, c4 = lane >> 4;
  // wave-uniform (the compiler cannot tell that threadIdx.x >> 6 is)
  const int wv = uniform(threadIdx.x >> 6);
  const int w = uniform(blockIdx.x * 4 + wv);
  // per-wave LDS slots: the step entry's new K and V rows, the query operand
  __shared__ __attribute__((aligned(16))) uint8_t s_new[4][2 * D * BITS / 8];
  __shared__ u32x4_t s_q[4][NQ][64];
  // quantising step: per-wave re-encode tables (K, V) of the last page, and
  // the step's raw new K and V rows (bf16 or fp32)
  __shared__ uint32_t s_lut[QNEW ? 4 : 1][2][64];
  __shared__ __attribute__((aligned(16))) uint8_t s_row[QNEW ? 4 : 1][QNEW ? 2 * D * 4 : 16];

  // ---- this wave's unit range -------------------------------------------------
  // seq_lens of the first NC*64 sequences are read once, in one round trip, and
  // kept in registers (prefix counts of ranges); longer batches re-read the rest.
  constexpr int NC = 4;
  const int A = PT == TS ? SWITCH_UNITS : 0;     // switch-cost units per (b, g)
  int Lc[NC], inclc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int bb = c * 64 + lane;
    Lc[c] = bb < B ? seq_lens[bb] : 0;
  }
  int np_sum = 0, n_empty = 0;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    inclc[c] = np_sum;
    if (c * 64 < B) {                     // uniform: skip chunks past the batch
      const int bb = c * 64 + lane;
      const int np = units_of(Lc[c], PT, A);
      const int incl = wave_incl_scan(np, lane);
      inclc[c] = np_sum + incl;
      np_sum = uniform(np_sum + __builtin_amdgcn_readlane(incl, 63));
      n_empty += __builtin_popcountll(__ballot(bb < B && np == 0));
    }
  }
  for (int b0 = NC * 64; b0 < B; b0 += 64) {
    const int bb = b0 + lane;
    const int np = units_of(bb < B ? seq_lens[bb] : 0, PT, A);
    np_sum = uniform(np_sum + wave_sum(np));
    n_empty += __builtin_popcountll(__ballot(bb < B && np == 0));
  }
  n_empty = uniform(n_empty);
  // sequences with no tokens get zero rows (sequence b is cleared by wave b mod Wmax)
  if (n_empty) {
    for (int b0 = 0; b0 < B; b0 += 64) {
      const int bb = b0 + lane;
      const int L = bb < B ? seq_lens[bb] : 0;
      uint64_t mine = __ballot(bb < B && ranges_of(L, PT) == 0 && bb % Wmax == w);
      while (mine) {
        const int be = b0 + __builtin_ctzll(mine);
        mine &= mine - 1;
        for (int x = 4 * lane; x < Hq * D; x += 256)
          store_out4<OUT_BF16>(out_, (size_t)be * Hq * D + x, f32x4_t{0.f, 0.f, 0.f, 0.f});
        // descriptor "nothing to merge or append" for each kv head of the sequence
        for (int gg = lane; gg < Hkv; gg += 64) descs[(size_t)be * Hkv + gg] = make_int4(0, 0, 0, 0);
      }
    }
  }
  const Split sp = make_split((int64_t)np_sum * Hkv, Wmax);
  if (w >= sp.W) return;
  const int64_t u0 = range_begin(sp, w), u1 = range_begin(sp, w + 1);

  // sequence holding unit u0, and the number of units before it
  int b = -1, Lb = 0;
  int64_t base = 0;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (b < 0) {
      const int np = units_of(Lc[c], PT, A);
      const uint64_t hit = __ballot((int64_t)inclc[c] * Hkv > u0);
      if (hit) {
        const int f = uniform(__builtin_ctzll(hit));
        b = c * 64 + f;
        base = (int64_t)__builtin_amdgcn_readlane(inclc[c] - np, f) * Hkv;
        Lb = __builtin_amdgcn_readlane(Lc[c], f);
      }
    }
  }
  if (b < 0) {
    int run = uniform(__builtin_amdgcn_readlane(inclc[NC - 1], 63));
    for (int b0 = NC * 64;; b0 += 64) {
      const int bb = b0 + lane;
      const int L = bb < B ? seq_lens[bb] : 0;
      const int np = units_of(L, PT, A);
      const int incl = run + wave_incl_scan(np, lane);
      const uint64_t hit = __ballot((int64_t)incl * Hkv > u0);
      if (hit) {
        const int f = uniform(__builtin_ctzll(hit));
        b = b0 + f;
        base = (int64_t)__builtin_amdgcn_readlane(incl - np, f) * Hkv;
        Lb = __builtin_amdgcn_readlane(L, f);
        break;
      }
      run = uniform(__builtin_amdgcn_readlane(incl, 63));
    }
  }
  b = uniform(b);
  base = uniform64(base);
  Lb = uniform(Lb);
  int cpb = units_of(Lb, PT, A);     // units of each (b, g) of sequence b

  const float NEG_INF = -__builtin_inff();
  const bool hv = r16 < G;

  // Length of sequence bb: those of the first NC * 64 sequences are in
  // registers (lane bb mod 64 of Lc[bb / 64]); later ones are read.
  static_assert(NC == 4, "len_of reads Lc[0..3]");
  auto len_of = [&](int bb) -> int {
    bb = uniform(bb);
    const int c = bb >> 6, ln = bb & 63;
    int v;
    if (c == 0) v = __builtin_amdgcn_readlane(Lc[0], ln);
    else if (c == 1) v = __builtin_amdgcn_readlane(Lc[1], ln);
    else if (c == 2) v = __builtin_amdgcn_readlane(Lc[2], ln);
    else if (c == 3) v = __builtin_amdgcn_readlane(Lc[3], ln);
    else v = seq_lens[bb];
    return uniform(v);
  };
  // first page id of the next segment, looked up one segment ahead
  bool have_next = false;
  int page_next = 0;

  bool first = true;                 // no segment of this wave finished yet
  for (int64_t u = u0; u < u1;) {
    const int64_t off = u - base;
    const int g = uniform((int)(off / cpb));
    // ranges of (b, g) are units [S, Eu); the A units before S only carry cost
    const int64_t S = base + (int64_t)g * cpb + A, Eu = base + (int64_t)(g + 1) * cpb;
    if (u < S) {
      u = S;
      if (u >= u1) break;
    }
    const int rg = (int)(u - S);
    const int64_t ue = Eu < u1 ? Eu : u1;
    const int tok0 = uniform(rg * PT);
    const int tok1 = uniform(min(Lb, (int)(ue - S) * PT));
    const bool complete = (u == S) && (ue == Eu);
    const int h = g * G + r16;

    // ---- query operand: B matrix of QK^T (K dim = head dims, N = heads) --------
    // Parked in this wave's LDS slot and re-read next to each MFMA, so it holds
    // no registers across the streaming loop.
    // The loads are issued here; the LDS store waits until the segment's first
    // tile loads are also in flight (below), so the two round trips overlap.
    u32x4_t qv_ld[NQ];
    if constexpr (KVT == KV_F32) {
      const float* q = static_cast<const float*>(q_) + ((size_t)b * Hq + h) * D;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
        qv_ld[kk] = hv ? ld16(reinterpret_cast<const uint8_t*>(q + (c4 + 4 * kk) * 4)) : u32x4_t{0, 0, 0, 0};
    } else {
      const uint16_t* q = static_cast<const uint16_t*>(q_) + ((size_t)b * Hq + h) * D;
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
        // group kk covers dims E*(c4+4kk) .. +E, taken 8 at a time (one bf16x8
        // operand per chunk; E = 8 for bf16, 16 for fp8 / int8, 32 for int4).
        const int d0 = E * (c4 + 4 * (i / NCH)) + 8 * (i % NCH);
        qv_ld[i] = hv ? ld16(reinterpret_cast<const uint8_t*>(q + d0)) : u32x4_t{0, 0, 0, 0};
        if constexpr (I4) qv_ld[i] = zip_halves(qv_ld[i]);
      }
    }
    auto qop = [&](int i) -> u32x4_t { return s_q[wv][i][lane]; };

    // step entry: the segment that ends the sequence reads the new token row;
    // it is parked in this wave's LDS slot once the first tile's loads are out.
    const bool has_new = k_new != nullptr && tok1 == Lb;
    constexpr int NEWCH = D * BITS / 128;           // 16-byte chunks per K (or V) row
    u32x4_t new_chunk = {0, 0, 0, 0};
    // Quantising step: k_new / v_new are bf16 or fp32 rows, quantised on write
    // with the page scale rule of the quantising append.  A segment that reads
    // any tile of (b, g)'s last page (the one holding slot Lb - 1) sees that
    // page as the append leaves it: the new scales qsk / qsv, its earlier
    // slots re-encoded when a scale rises (qrk / qrv, through LUTs built in
    // LDS), token Lb - 1 encoded with the new scale.  The merge kernel makes
    // the same decisions from the same values and stores them.
    // The raw rows are loaded here, before the first tile's loads, in 16-byte
    // pieces, and parked in LDS once those loads are out (as the step entry
    // parks its pre-quantised row), so nothing waits on them in the tile loop.
    constexpr int NPL = D / 64;
    const int lp = (Lb - 1) / P;
    const bool qfix = QNEW && k_new != nullptr && tok1 > lp * P;
    const int rowb = D * (new_bf16 ? 2 : 4);        // bytes per raw row
    const int nrch = rowb / 16;                      // 16-byte pieces per row
    float qsk = 1.f, qsv = 1.f;
    bool qrk = false, qrv = false;
    u32x4_t qrow = {0, 0, 0, 0};
    if constexpr (QNEW) {
      if (qfix && lane < 2 * nrch) {
        const size_t off = ((size_t)b * Hkv + g) * (size_t)rowb;
        const uint8_t* src = lane < nrch ? static_cast<const uint8_t*>(k_new) + off + lane * 16
                                         : static_cast<const uint8_t*>(v_new) + off + (lane - nrch) * 16;
        qrow = ld16(src);
      }
    }
    if (!QNEW && has_new && lane < 2 * NEWCH) {
      const size_t nrow = elem_byte<KVT>(((size_t)b * Hkv + g) * D);
      const uint8_t* src = lane < NEWCH ? static_cast<const uint8_t*>(k_new) + nrow
                                        : static_cast<const uint8_t*>(v_new) + nrow - NEWCH * 16;
      new_chunk = ld16(src + lane * 16);
    }

    f32x4_t O[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) O[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m = NEG_INF, l = 0.f;
    // int4: K codes widen to bf16 136 + n (QK^T), V codes to fp16 1032 + n
    // (PV; int8: V bytes to fp16 1152 + b); LP accumulates the V-scaled sum of
    // the probabilities exactly as the PV products see them (a product with an
    // all-ones operand: every entry holds the column's sum), and qsum is the
    // head's sum of query values, so that the biases come back out exactly.
    f32x4_t LP = {0.f, 0.f, 0.f, 0.f};
    float qsum = 0.f;
    if constexpr (I4) {
#pragma unroll
      for (int i = 0; i < NQ; ++i)
#pragma unroll
        for (int x = 0; x < 4; ++x)
          qsum += fbits(qv_ld[i][x] << 16) + fbits(qv_ld[i][x] & 0xffff0000u);
      qsum += __shfl_xor(qsum, 16);
      qsum += __shfl_xor(qsum, 32);
    }
    const float nbias = -INT4_BIAS * qsum;

    // Loop state is wave-uniform; readfirstlane lets the compiler keep it in
    // scalar registers, so page ids come from scalar loads (lgkmcnt) that do
    // not serialise behind the vector K/V loads in flight.
    int pgi = uniform(tok0 / P);
    int j0 = uniform(tok0 - pgi * P);
    // The page table is read through the constant address space: with a uniform
    // index this is a scalar load.
    const const_i32_ptr btrow = (const_i32_ptr)(bt + (size_t)b * MP);
    auto page_of = [&](int idx) -> int {
      idx = uniform(idx);
      const int v = btrow[idx < MP ? idx : MP - 1];
      return idx < MP ? v : -1;
    };
    // An invalid page id marks the segment bad (NaN result); page 0 is read instead.
    // Byte addresses of a lane's 16-byte groups in the page layout, for a tile
    // starting at slot j (a multiple of the V block):
    //   K token j + 16 sub + r16, dims E (c4 + 4 kk) ..:
    //     chunk + 16 j + 64 P kk + 16 (P c4 + r16) + 256 sub
    //   V tokens j + 4 c4 .., dim 16 dt + r16:
    //     chunk + j D BITS / 8 + 16 (D c4 + r16) + 256 dt
    // i.e. a wave-uniform base, one per-lane offset and a constant, which the
    // loads take as a base register pair + immediate offsets.
    u32x4_t kr[NSUB][NKK], vr[NDT];
    const uint32_t k_lane = (uint32_t)(16 * (P * c4 + r16));
    const uint32_t v_lane = (uint32_t)(16 * (D * c4 + r16));
    auto load_k = [&](int pg, int j) {
      const uint8_t* kc = kpool + elem_byte<KVT>(chunk_elem(pg, g, Hkv, P, D)) + 16 * (size_t)j;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const uint8_t* kb = kc + (size_t)(64 * P * kk) + k_lane;
#pragma unroll
        for (int sub = 0; sub < NSUB; ++sub) kr[sub][kk] = ld16_stream(kb + 256 * sub);
      }
    };
    auto load_v = [&](int pg, int j) {
      const uint8_t* vb = vpool + elem_byte<KVT>(chunk_elem(pg, g, Hkv, P, D)) + (size_t)j * (D * BITS / 8) + v_lane;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) vr[dt] = ld16_stream(vb + 256 * dt);
    };
    // the quantising step's stores of a re-encoded tile (same addresses)
    auto store_k = [&](int pg, int j) {
      uint8_t* kc = const_cast<uint8_t*>(kpool) + elem_byte<KVT>(chunk_elem(pg, g, Hkv, P, D)) + 16 * (size_t)j;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        uint8_t* kb = kc + (size_t)(64 * P * kk) + k_lane;
#pragma unroll
        for (int sub = 0; sub < NSUB; ++sub) store_nt(reinterpret_cast<u32x4_t*>(kb + 256 * sub), kr[sub][kk]);
      }
    };
    auto store_v = [&](int pg, int j) {
      uint8_t* vb = const_cast<uint8_t*>(vpool) + elem_byte<KVT>(chunk_elem(pg, g, Hkv, P, D)) +
                    (size_t)j * (D * BITS / 8) + v_lane;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) store_nt(reinterpret_cast<u32x4_t*>(vb + 256 * dt), vr[dt]);
    };
    int page = (have_next && pgi == 0) ? page_next : page_of(pgi);
    // The segment after this one, if the wave has one, starts at token 0 of kv
    // head g + 1 of this sequence or of kv head 0 of the next sequence with
    // tokens.  Its sequence and first page id are found now, so the switch
    // waits only for its K / V loads.
    int nb = b;
    have_next = ue == Eu && Eu + A < u1;    // the next (b, g) starts inside this wave's share
    if (have_next) {
      if (g + 1 == Hkv) {
        do ++nb;
        while (ranges_of(len_of(nb), PT) == 0);
      }
      page_next = uniform(((const_i32_ptr)(bt + (size_t)nb * MP))[0]);
    }
    // step entry: the wave that writes (b, g)'s descriptor also looks up the
    // page of slot Lb - 1, where the merge kernel stores the new token (-1:
    // beyond the table).  Scalar load; it is consumed only at the segment end.
    const int pg_new = (k_new != nullptr && u == S) ? page_of((Lb - 1) / P) : -1;
    bool bad = (unsigned)page >= (unsigned)NP;
    int pg_ld = bad ? 0 : page;
    float ksc = 1.f, vsc = 1.f;
    if constexpr (SCALED) {
      ksc = kscales[(size_t)pg_ld * Hkv + g];
      vsc = vscales[(size_t)pg_ld * Hkv + g];
    }
    load_k(pg_ld, j0);
    load_v(pg_ld, j0);
    __builtin_amdgcn_wave_barrier();      // the previous segment's LDS reads are done
#pragma unroll
    for (int i = 0; i < NQ; ++i) s_q[wv][i][lane] = qv_ld[i];
    if (!QNEW && has_new && lane < 2 * NEWCH) *reinterpret_cast<u32x4_t*>(s_new[wv] + lane * 16) = new_chunk;
    // Quantising step: the last page's old scales are loaded here, with the
    // new rows; the decisions, LUTs and the new token's codes (qprep) wait for
    // the first tile of that page, so these loads overlap the tiles before it.
    float s0k = 1.f, s0v = 1.f;
    int jl = 0, pgl = -1;
    bool qready = false;
    if constexpr (QNEW) {
      if (qfix) {
        if (lane < 2 * nrch) *reinterpret_cast<u32x4_t*>(s_row[wv] + lane * 16) = qrow;
        pgl = page_of(lp);
        jl = Lb - 1 - lp * P;
        const size_t si = (size_t)((unsigned)pgl < (unsigned)NP ? pgl : 0) * Hkv + g;
        if (jl > 0) {
          s0k = kscales[si];
          s0v = vscales[si];
        }
      }
    }
    auto qprep = [&]() {
      if constexpr (QNEW) {
        s0k = fbits(uniform((int)ubits(s0k)));
        s0v = fbits(uniform((int)ubits(s0v)));
        float qxk[NPL], qxv[NPL];
        {
          const int d0 = lane * NPL;
#pragma unroll
          for (int i = 0; i < NPL; ++i) {
            if (new_bf16) {
              const uint16_t* r = reinterpret_cast<const uint16_t*>(s_row[wv]);
              qxk[i] = fbits((uint32_t)r[d0 + i] << 16);
              qxv[i] = fbits((uint32_t)r[D + d0 + i] << 16);
            } else {
              const float* r = reinterpret_cast<const float*>(s_row[wv]);
              qxk[i] = r[d0 + i];
              qxv[i] = r[D + d0 + i];
            }
          }
        }
        qsk = page_scale<KVT>(row_amax(qxk), jl, s0k, qrk);
        qsv = page_scale<KVT>(row_amax(qxv), jl, s0v, qrv);
        // the merge kernel, which stores this append, takes the old scales from here
        if (has_new && lane == 0) qdescs[(size_t)b * Hkv + g] = make_int4((int)ubits(s0k), (int)ubits(s0v), 0, 0);
        if (qrk || qrv) {
          const uint32_t codes = (uint32_t)(4 * lane) * 0x01010101u + 0x03020100u;   // 4 codes per lane
          if (qrk) s_lut[wv][0][lane] = requant4<KVT>(codes, s0k, qsk);
          if (qrv) s_lut[wv][1][lane] = requant4<KVT>(codes, s0v, qsv);
        }
        if (has_new) {        // token Lb - 1's codes, in the row layout the injection reads
          constexpr int RB = D * BITS / 8;            // bytes per row
          const int d0 = lane * NPL;
          uint32_t ck[NPL], cv[NPL];
#pragma unroll
          for (int i = 0; i < NPL; ++i) {
            ck[i] = ByteFmt<KVT>::enc(qxk[i] / qsk);
            cv[i] = ByteFmt<KVT>::enc(qxv[i] / qsv);
          }
          if constexpr (I4) {
            s_new[wv][d0 >> 1] = (uint8_t)(ck[0] | (ck[NPL - 1] << 4));
            s_new[wv][RB + (d0 >> 1)] = (uint8_t)(cv[0] | (cv[NPL - 1] << 4));
          } else {
#pragma unroll
            for (int i = 0; i < NPL; ++i) {
              s_new[wv][d0 + i] = (uint8_t)ck[i];
              s_new[wv][RB + d0 + i] = (uint8_t)cv[i];
            }
          }
        }
        __builtin_amdgcn_wave_barrier();  // one wave's LDS operations complete in order
        qready = true;
      }
    };

    // One tile of TS tokens.  Streaming tiles (LAST = false) always have a next
    // tile: its K loads go out as soon as QK^T has consumed kr and its V loads
    // as soon as PV has consumed vr (rolling pipeline, no stores, no masking).
    // The last tile of a segment (LAST = true) issues no loads; it masks tokens
    // at or past tok1 and, for the step entry, takes in the appended token.
    auto tile = [&](const int t, auto last_tag, auto fix_tag) {
      constexpr bool LAST = decltype(last_tag)::value;
      // streaming tiles of the quantising step's last page (FIX) are their own
      // instance, so the other streaming tiles carry none of its code
      constexpr bool FIX = decltype(fix_tag)::value;
      int pgi_n = pgi, j_n = j0, page_n = page;
      if constexpr (!LAST) {
        j_n = j0 + TS;
        if (j_n == P) {
          j_n = 0;
          ++pgi_n;
        }
        page_n = page_of(pgi_n);
      }
      const bool bad_n = (unsigned)page_n >= (unsigned)NP;
      const int pg_ld_n = bad_n ? 0 : page_n;
      // quantising step: a tile of the last page takes the appended view of it
      const bool fixp = QNEW && (LAST ? qfix && pgi == lp : FIX);
      // slot jl of the last page, relative to this tile's first token: codes of
      // earlier slots are re-encoded, later ones (masked out of the attention)
      // keep their bytes, since a rising scale's tiles are stored back below
      const int jrel = jl - j0;
      if constexpr (QNEW) {
        if (fixp && !qready) qprep();
        if (fixp && qrk) {
          const uint8_t* lut = reinterpret_cast<const uint8_t*>(s_lut[wv][0]);
#pragma unroll
          for (int sub = 0; sub < NSUB; ++sub) {
            const bool before = 16 * sub + r16 < jrel;     // token of the lane's K groups
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
              for (int x = 0; x < 4; ++x) {
                const uint32_t m = lut4(lut, kr[sub][kk][x]);
                kr[sub][kk][x] = before ? m : kr[sub][kk][x];
              }
          }
        }
        if (fixp && qrv) {
          const uint8_t* lut = reinterpret_cast<const uint8_t*>(s_lut[wv][1]);
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int x = 0; x < 4; ++x) {
              // element e of the lane's group holds token 16 (e / 4) + 4 c4 + e % 4
              uint32_t lt = 0, eq = 0;
              if constexpr (I4) {
                run_masks<4>(jrel - (32 * x + 4 * c4), 0, lt, eq);
                run_masks<4>(jrel - (32 * x + 16 + 4 * c4), 16, lt, eq);
              } else {
                run_masks<8>(jrel - (16 * x + 4 * c4), 0, lt, eq);
              }
              vr[dt][x] = (lut4(lut, vr[dt][x]) & lt) | (vr[dt][x] & ~lt);
            }
        }
      }
      const float kmul = scale_log2 * (fixp ? qsk : ksc), vmul = fixp ? qsv : vsc;

      if constexpr (LAST) {
        // ---- fused append (step entry): the tile holding token Lb-1 takes this
        // step's k_new / v_new row (prefetched at segment start) into its
        // registers in place of the slot's old contents.  The row is stored into
        // the page by the merge kernel, so this kernel issues no pool stores.
        if (has_new) {
          const int rel = Lb - 1 - t;
          const int sub_t = rel >> 4, r_t = rel & 15;
          const int c_t = r_t >> 2, e_t = 4 * sub_t + (r_t & 3);
          typedef typename Kv<KVT>::elem_t T;
          // bitwise merge (no data-dependent array index, which would force the
          // tile registers into scratch)
#pragma unroll
          for (int kk = 0; kk < NKK; ++kk) {
            const u32x4_t nv = *reinterpret_cast<const u32x4_t*>(s_new[wv] + (c4 + 4 * kk) * 16);
#pragma unroll
            for (int sub = 0; sub < NSUB; ++sub) {
              const uint32_t m = (r16 == r_t && sub == sub_t) ? 0xffffffffu : 0u;
              kr[sub][kk] = (kr[sub][kk] & ~m) | (nv & m);
            }
          }
          if (c4 == c_t) {
            const int kw = (e_t * BITS) >> 5, sh = (e_t * BITS) & 31;
            const uint32_t msk = (uint32_t)((1ull << BITS) - 1ull) << sh;
            const T* vrow = reinterpret_cast<const T*>(s_new[wv] + NEWCH * 16);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
              const int dd = dt * 16 + r16;
              const uint32_t code = I4 ? ((uint32_t)vrow[dd >> 1] >> (4 * (dd & 1))) & 0xFu : (uint32_t)vrow[dd];
              const uint32_t bits = code << sh;
#pragma unroll
              for (int x = 0; x < 4; ++x) {
                const uint32_t mx = x == kw ? msk : 0u;
                vr[dt][x] = (vr[dt][x] & ~mx) | (bits & mx);
              }
            }
          }
        }
      }

      // quantising step, a scale that rises: this tile of the last page is stored
      // back as the append leaves it (re-encoded slots, the new token, later
      // slots unchanged), so the merge kernel writes only the scale
      if constexpr (QNEW) {
        if (fixp && (qrk || qrv) && (unsigned)pgl < (unsigned)NP) {
          if (qrk) store_k(pgl, j0);
          if (qrv) store_v(pgl, j0);
        }
      }

      // ---- S = K q^T: rows = 16 tokens, columns = heads --------------------------
      float s[NSUB][4];
#pragma unroll
      for (int sub = 0; sub < NSUB; ++sub) {
        // int4: the products start from -136 * (sum of q), which takes the
        // bias of the widened codes out inside the accumulation
        f32x4_t acc = {nbias, nbias, nbias, nbias};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          if constexpr (KVT == KV_F32) {
            {
              const u32x4_t qv = qop(kk);
#pragma unroll
              for (int e = 0; e < 4; ++e) acc = mfma_f32(fbits(kr[sub][kk][e]), fbits(qv[e]), acc);
            }
          } else if constexpr (KVT == KV_BF16) {
            acc = mfma_bf16(kr[sub][kk], qop(kk), acc);
          } else if constexpr (I4) {
#pragma unroll
            for (int c = 0; c < 4; ++c) acc = mfma_bf16(nib8_to_bf16x8(kr[sub][kk][c]), qop(4 * kk + c), acc);
          } else {
            acc = mfma_bf16(byte8_to_bf16x8<KVT>(kr[sub][kk][0], kr[sub][kk][1]), qop(2 * kk), acc);
            acc = mfma_bf16(byte8_to_bf16x8<KVT>(kr[sub][kk][2], kr[sub][kk][3]), qop(2 * kk + 1), acc);
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) s[sub][i] = acc[i] * kmul;
      }
      if constexpr (!LAST) {
        load_k(pg_ld_n, j_n);
        if constexpr (SCALED) {
          ksc = kscales[(size_t)pg_ld_n * Hkv + g];
          vsc = vscales[(size_t)pg_ld_n * Hkv + g];
        }
      }

      // ---- last step: mask logits, zero V of absent tokens -----------------------
      if constexpr (LAST) {
        if (t + TS > tok1) {
#pragma unroll
          for (int sub = 0; sub < NSUB; ++sub)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (t + 16 * sub + 4 * c4 + i >= tok1) s[sub][i] = NEG_INF;
          // per element of the lane's V group (element e holds token
          // 16 * (e / 4) + 4 * c4 + e % 4 of the step)
          u32x4_t keep;
          constexpr int FIELD = BITS < 8 ? BITS : 8;     // mask granularity: bytes, or nibbles
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            uint32_t msk = 0;
#pragma unroll
            for (int f = 0; f < 32 / FIELD; ++f) {
              const int e = (32 * k + FIELD * f) / BITS;
              const int tok = t + 16 * (e >> 2) + 4 * c4 + (e & 3);
              if (tok < tok1) msk |= ((1u << FIELD) - 1u) << (FIELD * f);
            }
            keep[k] = msk;
          }
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) vr[dt] &= keep;
        }
      }

      // ---- online softmax (log2 domain, lazy reference) ---------------------------
      // The reference m of a head column grows only when the column's max passes
      // it by more than TH (so p <= 2^TH).  Each lane tests its own scores; the
      // column max across the four lanes of a column is formed only when one
      // passes, so the common tile has no cross-lane step.  m = -inf (no tile
      // yet) is passed by any finite score.
      float lmax = NEG_INF;
#pragma unroll
      for (int sub = 0; sub < NSUB; ++sub)
#pragma unroll
        for (int i = 0; i < 4; ++i) lmax = fmaxf(lmax, s[sub][i]);
      if (__ballot(lmax > m + TH)) {
        const float cmax = colmax4(lmax);
        const bool grow = cmax > m + TH;
        const float mref = grow ? cmax : m;
        const float alpha = grow ? __builtin_amdgcn_exp2f(m - mref) : 1.f;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) O[dt] *= alpha;
        if constexpr (F16PV) LP *= alpha;
        l *= alpha;
        m = mref;
      }
      // int4 and int8 take the probabilities as p * 2^P_SHIFT (see the value product)
      const float mp = F16PV ? m - P_SHIFT : m;
      float p[NSUB][4];
      float lsum = 0.f;
#pragma unroll
      for (int sub = 0; sub < NSUB; ++sub)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[sub][i] = __builtin_amdgcn_exp2f(s[sub][i] - mp);
          lsum += p[sub][i];
        }
      l += lsum;

      // ---- O^T += V^T P^T: rows = 16 dims, columns = heads -------------------------
      if constexpr (KVT == KV_F32) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) O[dt] = mfma_f32(fbits(vr[dt][i]), p[0][i], O[dt]);
      } else if constexpr (KVT == KV_BF16) {
        u32x4_t ph, pl;
        split_probs(p[0], p[1], 1.f, ph, pl);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          O[dt] = mfma_bf16(vr[dt], ph, O[dt]);
          O[dt] = mfma_bf16(vr[dt], pl, O[dt]);
        }
      } else if constexpr (I4) {
        // fp16 operands: the codes widen to 1032 + n, the probabilities are
        // p * 2^P_SHIFT (at most 2^15 under the lazy reference, and values down
        // to 2^-31 of the reference stay representable), one fp16 each.  The
        // tile's products start from zero and enter O (and LP, the sum of the
        // probabilities as the products see them) times the page's V scale, so
        // no scale of any size meets the fp16 range.
        u32x4_t pf[4];
        const u32x4_t ones = {0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};
        f32x4_t lp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
#pragma unroll
          for (int i = 0; i < 4; ++i) pf[c][i] = pack_f16_rne(p[2 * c][i], p[2 * c + 1][i]);
          lp = mfma_f16(ones, pf[c], lp);
        }
        LP += lp * vmul;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c = 0; c < 4; ++c) acc = mfma_f16(nib8_to_f16x8(vr[dt][c]), pf[c], acc);
          O[dt] += acc * vmul;
        }
      } else if constexpr (KVT == KV_INT8) {
        // as int4: fp16 operands, V bytes widened to 1152 + b, one fp16 per
        // probability (p * 2^P_SHIFT), the tile's products times the V scale
        u32x4_t pf[2];
        const u32x4_t ones = {0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};
        f32x4_t lp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          pf[c] = u32x4_t{pack_f16_rne(p[2 * c][0], p[2 * c][1]), pack_f16_rne(p[2 * c][2], p[2 * c][3]),
                          pack_f16_rne(p[2 * c + 1][0], p[2 * c + 1][1]),
                          pack_f16_rne(p[2 * c + 1][2], p[2 * c + 1][3])};
          lp = mfma_f16(ones, pf[c], lp);
        }
        LP += lp * vmul;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const u32x2_t a = i8x4_to_f16x4_biased(vr[dt][0]), b = i8x4_to_f16x4_biased(vr[dt][1]);
          const u32x2_t c = i8x4_to_f16x4_biased(vr[dt][2]), d = i8x4_to_f16x4_biased(vr[dt][3]);
          f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
          acc = mfma_f16(u32x4_t{a.x, a.y, b.x, b.y}, pf[0], acc);
          acc = mfma_f16(u32x4_t{c.x, c.y, d.x, d.y}, pf[1], acc);
          O[dt] += acc * vmul;
        }
      } else {
        u32x4_t ph[2], pl[2];
        split_probs(p[0], p[1], vmul, ph[0], pl[0]);
        split_probs(p[2], p[3], vmul, ph[1], pl[1]);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const u32x4_t a0 = byte8_to_bf16x8<KVT>(vr[dt][0], vr[dt][1]);
          const u32x4_t a1 = byte8_to_bf16x8<KVT>(vr[dt][2], vr[dt][3]);
          O[dt] = mfma_bf16(a0, ph[0], O[dt]);
          O[dt] = mfma_bf16(a0, pl[0], O[dt]);
          O[dt] = mfma_bf16(a1, ph[1], O[dt]);
          O[dt] = mfma_bf16(a1, pl[1], O[dt]);
        }
      }
      if constexpr (!LAST) {
        load_v(pg_ld_n, j_n);
        bad |= bad_n;
        page = page_n;
        pgi = pgi_n;
        j0 = j_n;
      }
    };

    int t = tok0;
    const int tfix = QNEW && qfix ? lp * P : tok1;      // first token of the tiles that need the appended view
    for (; t + TS < tok1 && t < tfix; t += TS) tile(t, std::false_type{}, std::false_type{});
    if constexpr (QNEW)
      for (; t + TS < tok1; t += TS) tile(t, std::false_type{}, std::true_type{});
    tile(t, std::true_type{}, std::false_type{});

    // ---- finish the segment ------------------------------------------------------
    float lt = l + __shfl_xor(l, 16);
    lt += __shfl_xor(lt, 32);
    if constexpr (F16PV) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) O[dt] -= V_BIAS * LP[0];
    }
    const float qnan = __builtin_nanf("");
    if (complete) {
      if (hv) {
        const float inv = bad ? qnan : 1.f / lt;
        const size_t o = ((size_t)b * Hq + h) * D + 4 * c4;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) store_out4<OUT_BF16>(out_, o + dt * 16, O[dt] * inv);
      }
    } else {
      float* ps = partials + (size_t)(2 * w + (first ? 0 : 1)) * G * (D + 2);
      if (hv) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
          *reinterpret_cast<f32x4_t*>(ps + r16 * D + dt * 16 + 4 * c4) = O[dt];
        if (c4 == 0) {
          ps[G * D + r16] = bad ? qnan : m;
          ps[G * D + G + r16] = lt;
        }
      }
    }
    if (u == S && lane == 0) {
      // descriptor of (b, g): first contributing wave w; 2 * contributors + 1
      // if its partial is in its second slot (slot 2w + 1, else 2w); the page
      // of slot Lb - 1 for the step entry; Lb
      const int64_t wl = wave_of(sp, Eu - 1);
      descs[(size_t)b * Hkv + g] = make_int4((int)w, (int)(2 * (wl - w + 1) + (first ? 0 : 1)), pg_new, Lb);
    }

    // ---- next segment ------------------------------------------------------------
    first = false;
    u = ue;
    if (u < u1 && u == base + (int64_t)cpb * Hkv) {
      base = u;
      b = nb;
      Lb = len_of(b);
      cpb = units_of(Lb, PT, A);
    }
  }
}

// ---------------------------------------------------------------------------
// Decode, part 2: one wave per (b, g) and 256-output chunk of its G*D outputs
// combines the partial ranges of pairs that were split over several waves
// (log-sum-exp merge, see merge_chunk); for the step entry the chunk-0 wave
// also stores this step's token into its page slot.  A chunk per wave keeps
// the dependent memory round trips to two: the descriptor, then the partials
// (and the page id) together.
// ---------------------------------------------------------------------------
template <int KVT, bool OUT_BF16>
__global__ __launch_bounds__(256) void decode_merge_kernel(
    const int4* __restrict__ descs, const float* __restrict__ partials, void* __restrict__ out_, int B,
    int Hq, int Hkv, int G, int D, int nchunk, const void* __restrict__ k_new, const void* __restrict__ v_new,
    void* __restrict__ kpool, void* __restrict__ vpool, int NP, int P) {
  constexpr int E = 128 / Kv<KVT>::BITS;
  // wave-uniform (the compiler cannot tell that threadIdx.x >> 6 is)
  const int wi = uniform(blockIdx.x * 4 + (threadIdx.x >> 6));
  const int bg = wi / nchunk, chunk = wi - bg * nchunk;
  if (bg >= B * Hkv) return;
  const int lane = threadIdx.x & 63;
  const int b = bg / Hkv, g = bg - b * Hkv;
  const bool app = k_new != nullptr && chunk == 0;
  // This step's token row (independent of the descriptor, so issued first).
  // K: its E-element groups are 16-byte units of the layout, one per lane;
  // V: one element per dimension.  Indexes are clamped rather than branched
  // on, so the loads stay in flight across the descriptor load.
  const size_t nrow = ((size_t)b * Hkv + g) * D;
  const int ngrp = D / E;
  u32x4_t kgrp = {0, 0, 0, 0};
  uint32_t vv[2] = {0, 0};                // one element each, kept unpacked
  if (app) {
    kgrp = ld16(static_cast<const uint8_t*>(k_new) + elem_byte<KVT>(nrow + (size_t)min(lane, ngrp - 1) * E));
#pragma unroll
    for (int i = 0; i < 2; ++i) vv[i] = get_code<KVT>(v_new, nrow + min(lane + 64 * i, D - 1));
  }
  // descriptor of (b, g), written by the split kernel in this call: first
  // contributing wave, contributors, slot of the first, sequence length
  // (all zero for an empty sequence).  Everything below depends only on it.
  const int4 d = descs[bg];
  const int L = d.w;
  if (L <= 0) return;                    // empty: rows zeroed by the split kernel, nothing appended
  const int n = d.y >> 1;
  if (n > 1)                             // else finished by one wave
    merge_chunk<OUT_BF16>(partials, 2 * (int64_t)d.x + (d.y & 1), d.x, n, out_,
                          ((size_t)b * Hq + (size_t)g * G) * D, G, D, 256 * chunk, lane);
  // step entry: store the token into slot L-1 of page d.z (the split kernel
  // already attended to it from registers)
  if (app && (unsigned)d.z < (unsigned)NP) {
    const int j = (L - 1) % P;
    const size_t ch = chunk_elem(d.z, g, Hkv, P, D);
    if (lane < ngrp)
      store_nt(reinterpret_cast<u32x4_t*>(static_cast<uint8_t*>(kpool) + elem_byte<KVT>(ch + k_elem<E>(j, lane * E, P))), kgrp);
    if constexpr (Kv<KVT>::BITS == 4) {
      // int4: each code shares its byte with a neighbouring token; both old
      // bytes are loaded before either store (clamped index: in bounds)
      uint8_t* vb = static_cast<uint8_t*>(vpool);
      size_t xv[2];
      uint8_t old[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        xv[i] = ch + v_elem<E>(j, min(lane + 64 * i, D - 1), D);
        old[i] = vb[xv[i] >> 1];
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int sh = 4 * (int)(xv[i] & 1);
        if (lane + 64 * i < D)
          store_nt(vb + (xv[i] >> 1), (uint8_t)((old[i] & ~(0xF << sh)) | ((vv[i] & 0xFu) << sh)));
      }
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) {               // each dim's V element lies in its own byte
        const int dd = lane + 64 * i;
        if (dd < D) put_code_nt<KVT>(vpool, ch + v_elem<E>(j, dd, D), vv[i]);
      }
    }
  }
}

// The quantising step's merge kernel: as decode_merge_kernel, with this
// step's bf16 / fp32 rows quantised on write (quant_store_half) by two extra
// waves per (b, g), one for K and one for V, which make the same scale
// decisions the split kernel made for its view of the last page.
template <int KVT, bool OUT_BF16, int D>
__global__ __launch_bounds__(256) void decode_merge_quant_kernel(
    const int4* __restrict__ descs, const float* __restrict__ partials, void* __restrict__ out_, int B,
    int Hq, int Hkv, int G, int nchunk, const void* __restrict__ k_new, const void* __restrict__ v_new,
    int new_bf16, uint8_t* __restrict__ kpool, uint8_t* __restrict__ vpool, float* __restrict__ kscales,
    float* __restrict__ vscales, const int4* __restrict__ qdescs, int NP, int P) {
  constexpr int NPL = D / 64;
  const int wv = uniform(threadIdx.x >> 6);
  const int wi = uniform(blockIdx.x * 4 + wv);
  // nchunk merging waves and two appending waves (K, V) per (b, g), so the
  // merge's and the append's dependent loads run side by side
  const int bg = wi / (nchunk + 2), chunk = wi - bg * (nchunk + 2);
  if (bg >= B * Hkv) return;
  const int lane = threadIdx.x & 63;
  const int b = bg / Hkv, g = bg - b * Hkv;
  const bool app = chunk >= nchunk, app_v = chunk == nchunk + 1;
  float x[NPL];
  if (app) {   // independent of the descriptor: issued first
    const size_t row = ((size_t)b * Hkv + g) * D + (size_t)(lane * NPL);
    const void* src = app_v ? v_new : k_new;
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      x[i] = new_bf16 ? fbits((uint32_t)static_cast<const uint16_t*>(src)[row + i] << 16)
                      : static_cast<const float*>(src)[row + i];
  }
  const int4 d = descs[bg];
  // the page's scales before this append, as the split kernel read them (in
  // the same round trip as the descriptor)
  const int4 qd = app ? qdescs[bg] : make_int4(0, 0, 0, 0);
  const int L = d.w;
  if (L <= 0) return;
  const int n = d.y >> 1;
  if (!app && n > 1)
    merge_chunk<OUT_BF16>(partials, 2 * (int64_t)d.x + (d.y & 1), d.x, n, out_,
                          ((size_t)b * Hq + (size_t)g * G) * D, G, D, 256 * chunk, lane);
  if (app && (unsigned)d.z < (unsigned)NP) {
    const size_t ch = chunk_elem(d.z, g, Hkv, P, D);
    const size_t si = (size_t)d.z * Hkv + g;
    if (app_v)
      quant_store_half<KVT, D, true>(x, (L - 1) % P, vpool + elem_byte<KVT>(ch), P, vscales, si,
                                     fbits((uint32_t)qd.y), lane);
    else
      quant_store_half<KVT, D, false>(x, (L - 1) % P, kpool + elem_byte<KVT>(ch), P, kscales, si,
                                      fbits((uint32_t)qd.x), lane);
  }
}

// ---------------------------------------------------------------------------
// Append: one workgroup per sequence; element-wise copy through the page table.
// ---------------------------------------------------------------------------
template <int KVT>
__global__ __launch_bounds__(256) void append_kernel(
    const void* __restrict__ k_new, const void* __restrict__ v_new,
    const int32_t* __restrict__ bt, const int32_t* __restrict__ seq_lens,
    void* __restrict__ kpool, void* __restrict__ vpool, int MP, int NP, int Hkv, int D, int P) {
  constexpr int E = 128 / Kv<KVT>::BITS;
  const int b = blockIdx.x;
  const int L = seq_lens[b];
  if (L <= 0) return;
  const int t = L - 1, pgi = t / P, j = t - pgi * P;
  if (pgi >= MP) return;
  const int page = bt[(size_t)b * MP + pgi];
  if ((unsigned)page >= (unsigned)NP) return;
  // Each thread copies a pair of dims (d even): an int4 K pair is one byte of
  // the pool, stored whole from the row's byte; its V elements lie in two
  // different bytes (each shared with another token's nibble, so read,
  // patched and written back), so no byte is written by two threads.
  const size_t row0 = (size_t)b * Hkv * D;
  for (int x = 2 * threadIdx.x; x < Hkv * D; x += 2 * blockDim.x) {
    const int g = x / D, d = x - g * D;
    const size_t ch = chunk_elem(page, g, Hkv, P, D);
    if constexpr (KVT == KV_INT4) {
      store_nt(static_cast<uint8_t*>(kpool) + ((ch + k_elem<E>(j, d, P)) >> 1),
               static_cast<const uint8_t*>(k_new)[(row0 + x) >> 1]);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if constexpr (KVT != KV_INT4)
        put_code_nt<KVT>(kpool, ch + k_elem<E>(j, d + i, P), get_code<KVT>(k_new, row0 + x + i));
      put_code_nt<KVT>(vpool, ch + v_elem<E>(j, d + i, D), get_code<KVT>(v_new, row0 + x + i));
    }
  }
}

template <int KVT, bool IN_BF16, int D>
__global__ __launch_bounds__(256) void append_quant_kernel(
    const void* __restrict__ k_new, const void* __restrict__ v_new,
    const int32_t* __restrict__ bt, const int32_t* __restrict__ seq_lens,
    uint8_t* __restrict__ kpool, uint8_t* __restrict__ vpool,
    float* __restrict__ kscales, float* __restrict__ vscales, int B, int MP, int NP, int Hkv, int P) {
  constexpr int NPL = D / 64;           // new-row elements per lane (consecutive dims)
  __shared__ uint8_t s_nb[4][D];        // the new V row's bytes (V pass of a re-encode)
  __shared__ uint32_t s_lut[4][2][64];  // re-encode tables, K and V (256 codes each)
  const int wv = uniform(threadIdx.x >> 6);
  const int bg = uniform(blockIdx.x * 4 + wv);
  if (bg >= B * Hkv) return;
  const int lane = threadIdx.x & 63;
  const int b = bg / Hkv, g = bg - b * Hkv;
  // the new rows do not depend on the table: their loads go first
  float xk[NPL], xv[NPL];
  load_new_rows<D>(k_new, v_new, IN_BF16, ((size_t)b * Hkv + g) * D + (size_t)(lane * NPL), xk, xv);
  const int L = uniform(((const_i32_ptr)seq_lens)[b]);
  if (L <= 0) return;
  const int t = L - 1, pgi = t / P, j = t - pgi * P;
  if (pgi >= MP) return;
  const int pg = uniform(((const_i32_ptr)bt)[(size_t)b * MP + pgi]);
  if ((unsigned)pg >= (unsigned)NP) return;
  const size_t ch = chunk_elem(pg, g, Hkv, P, D);        // element offset of the chunk
  const size_t si = (size_t)pg * Hkv + g;
  float sk0 = 1.f, sv0 = 1.f;
  if (j > 0) {                           // both scales in one round trip
    sk0 = kscales[si];
    sv0 = vscales[si];
  }
  quant_store_row<KVT, D>(xk, xv, j, kpool + elem_byte<KVT>(ch), vpool + elem_byte<KVT>(ch), P, kscales, vscales,
                          si, sk0, sv0, s_lut[wv], s_nb[wv], lane);
}

// ---------------------------------------------------------------------------
// Debug gather: contiguous copy of each sequence's tokens, same addressing.
// ---------------------------------------------------------------------------
template <int KVT>
__global__ __launch_bounds__(256) void gather_kernel(
    const void* __restrict__ kpool, const void* __restrict__ vpool,
    const int32_t* __restrict__ bt, const int32_t* __restrict__ seq_lens,
    void* __restrict__ k_out, void* __restrict__ v_out, int MP, int NP, int Hkv, int D, int P) {
  constexpr int E = 128 / Kv<KVT>::BITS;
  const int bg = blockIdx.x;
  const int b = bg / Hkv, g = bg - b * Hkv;
  const int L = seq_lens[b];
  if (L <= 0 || L > MP * P) return;
  const int npg = (L + P - 1) / P;
  int ok = 1;
  for (int i = threadIdx.x; i < npg; i += blockDim.x) {
    const int pg = bt[(size_t)b * MP + i];
    if ((unsigned)pg >= (unsigned)NP) ok = 0;
  }
  if (!__syncthreads_and(ok)) return;
  const size_t rows = (size_t)MP * P;
  const size_t o0 = ((size_t)b * Hkv + g) * rows * D;
  // a pair of dims per thread (one output byte for int4)
  for (size_t x = 2 * threadIdx.x; x < (size_t)L * D; x += 2 * blockDim.x) {
    const int t = (int)(x / D), d = (int)(x - (size_t)t * D);
    const int pgi = t / P, j = t - pgi * P;
    const size_t ch = chunk_elem(bt[(size_t)b * MP + pgi], g, Hkv, P, D);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      put_code<KVT>(k_out, o0 + x + i, get_code<KVT>(kpool, ch + k_elem<E>(j, d + i, P)));
      put_code<KVT>(v_out, o0 + x + i, get_code<KVT>(vpool, ch + v_elem<E>(j, d + i, D)));
    }
  }
}

// Workspace of the allocation-free step entry point: a file-scope device
// array, one copy per device.  Host code never passes this name to a kernel
// (on the host it is only a stand-in symbol); it passes the device address
// that static_scratch() looks up.
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
namespace {

struct DevInfo {
  int cus = 0;
  void* scratch = nullptr;   // device address of `scratch` on this device
};
std::mutex g_mu;
DevInfo g_dev[64];

typedef void (*decode_fn_t)(const void*, const uint8_t*, const uint8_t*, const void*, const void*, const float*,
                            const float*, const int32_t*, const int32_t*, void*, float*, int4*, int4*, int, int,
                            int, int, int, int, int, int, int, float, int);

template <int KVT, int D, bool OB, bool QNEW = false>
decode_fn_t decode_fn() {
  return decode_split_kernel<KVT, D, OB, QNEW>;
}

// The quantising step's split kernels (fp8, int8: D 64 or 128; int4: D 128).
decode_fn_t pick_decode_quant(int kvt, int D, bool ob) {
  if (kvt == KV_FP8) {
    if (D == 64) return ob ? decode_fn<KV_FP8, 64, true, true>() : decode_fn<KV_FP8, 64, false, true>();
    return ob ? decode_fn<KV_FP8, 128, true, true>() : decode_fn<KV_FP8, 128, false, true>();
  }
  if (kvt == KV_INT8) {
    if (D == 64) return ob ? decode_fn<KV_INT8, 64, true, true>() : decode_fn<KV_INT8, 64, false, true>();
    return ob ? decode_fn<KV_INT8, 128, true, true>() : decode_fn<KV_INT8, 128, false, true>();
  }
  if (kvt == KV_INT4 && D == 128)
    return ob ? decode_fn<KV_INT4, 128, true, true>() : decode_fn<KV_INT4, 128, false, true>();
  return nullptr;
}

decode_fn_t pick_decode(int kvt, int D, bool ob) {
#define PKV_PICK(K)                                                              \
  if (kvt == K) {                                                                \
    if (D == 64) return ob ? decode_fn<K, 64, true>() : decode_fn<K, 64, false>();  \
    return ob ? decode_fn<K, 128, true>() : decode_fn<K, 128, false>();          \
  }
  PKV_PICK(KV_F32)
  PKV_PICK(KV_BF16)
  PKV_PICK(KV_FP8)
  PKV_PICK(KV_INT8)
#undef PKV_PICK
  // int4: 32-dim groups need D = 128 (one group per lane row)
  if (kvt == KV_INT4 && D == 128) return ob ? decode_fn<KV_INT4, 128, true>() : decode_fn<KV_INT4, 128, false>();
  return nullptr;
}

// Resident decode waves per compute unit for one kernel instantiation (cached).
int waves_per_cu(decode_fn_t fn, int dev) {
  static std::mutex mu;
  static struct {
    decode_fn_t fn;
    int dev;
    int waves;
  } cache[64];
  static int n = 0;
  std::lock_guard<std::mutex> lk(mu);
  for (int i = 0; i < n; ++i)
    if (cache[i].fn == fn && cache[i].dev == dev) return cache[i].waves;
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, reinterpret_cast<const void*>(fn), 256, 0) !=
          hipSuccess ||
      blocks <= 0)
    blocks = 1;
  int waves = blocks * 4;
  if (waves > kMaxWavesPerCU) waves = kMaxWavesPerCU;
  if (n < 64) cache[n++] = {fn, dev, waves};
  return waves;
}

}  // namespace

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_dev[dev].cus <= 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
    g_dev[dev].cus = cus;
  }
  return g_dev[dev].cus;
}

hipError_t static_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_dev[dev].scratch) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // the current device's copy
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_dev[dev].scratch = p;
  }
  *ptr = g_dev[dev].scratch;
  return hipSuccess;
}

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
  if (a.batch <= 0) return hipSuccess;
  dim3 grid(a.batch), block(256);
#define PKV_APPEND(K)                                                                              \
  hipLaunchKernelGGL(append_kernel<K>, grid, block, 0, s, a.k_new, a.v_new, a.block_tables,        \
                     a.seq_lens, a.k_pool, a.v_pool, a.max_pages, a.num_pages, a.num_kv_heads,     \
                     a.head_dim, a.page_size)
  if (a.kvt == KV_F32) PKV_APPEND(KV_F32);
  else if (a.kvt == KV_BF16) PKV_APPEND(KV_BF16);
  else if (a.kvt == KV_INT4) PKV_APPEND(KV_INT4);
  else PKV_APPEND(KV_FP8);          // any one-byte format (fp8, int8): a byte copy
#undef PKV_APPEND
  return hipGetLastError();
}

hipError_t launch_append_quant(const AppendQuantArgs& a, hipStream_t s) {
  if (a.batch <= 0) return hipSuccess;
  dim3 grid((unsigned)(((int64_t)a.batch * a.num_kv_heads + 3) / 4)), block(256);
#define PKV_APPEND_Q(K, BF, DD)                                                                     \
  hipLaunchKernelGGL((append_quant_kernel<K, BF, DD>), grid, block, 0, s, a.k_new, a.v_new,          \
                     a.block_tables, a.seq_lens, static_cast<uint8_t*>(a.k_pool),                    \
                     static_cast<uint8_t*>(a.v_pool), a.k_scales, a.v_scales, a.batch, a.max_pages,  \
                     a.num_pages, a.num_kv_heads, a.page_size)
#define PKV_APPEND_QK(K)                                                                            \
  if (a.new_bf16) {                                                                                 \
    if (a.head_dim == 64) PKV_APPEND_Q(K, true, 64); else PKV_APPEND_Q(K, true, 128);               \
  } else {                                                                                          \
    if (a.head_dim == 64) PKV_APPEND_Q(K, false, 64); else PKV_APPEND_Q(K, false, 128);             \
  }
  if (a.kvt == KV_INT8) {
    PKV_APPEND_QK(KV_INT8)
  } else if (a.kvt == KV_INT4) {
    PKV_APPEND_QK(KV_INT4)
  } else {
    PKV_APPEND_QK(KV_FP8)
  }
#undef PKV_APPEND_QK
#undef PKV_APPEND_Q
  return hipGetLastError();
}

hipError_t launch_gather(const GatherArgs& a, hipStream_t s) {
  if (a.batch <= 0) return hipSuccess;
  dim3 grid(a.batch * a.num_kv_heads), block(256);
#define PKV_GATHER(K)                                                                              \
  hipLaunchKernelGGL(gather_kernel<K>, grid, block, 0, s, a.k_pool, a.v_pool, a.block_tables,      \
                     a.seq_lens, a.k_out, a.v_out, a.max_pages, a.num_pages, a.num_kv_heads,       \
                     a.head_dim, a.page_size)
  if (a.kvt == KV_F32) PKV_GATHER(KV_F32);
  else if (a.kvt == KV_BF16) PKV_GATHER(KV_BF16);
  else if (a.kvt == KV_INT4) PKV_GATHER(KV_INT4);
  else PKV_GATHER(KV_FP8);          // any one-byte format
#undef PKV_GATHER
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  if (a.batch <= 0) return hipSuccess;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const int cus = device_cu_count();
  if (cus <= 0) return hipErrorInvalidDevice;
  decode_fn_t fn = a.new_quant ? pick_decode_quant(a.kvt, a.head_dim, a.out_bf16)
                              : pick_decode(a.kvt, a.head_dim, a.out_bf16);
  if (!fn) return hipErrorInvalidValue;
  // Resident waves: enough for about 64 KB of K/V tiles in flight per CU (a
  // tile is 128 * D bytes in every dtype), i.e. one wave per SIMD at D = 128.
  // More waves than that do not raise the streaming rate: two waves on one
  // SIMD issue in age order, so the second one starts late and finishes last,
  // stretching the tail of the launch.  int4 is the exception: its tile holds
  // the same bytes as a bf16 one but about ten times the vector ALU work
  // (nibble widening, the bias sums), so the second wave on each SIMD hides
  // ALU time rather than adding loads in flight.
  const int tile_waves = a.kvt == KV_INT4 ? 1024 : 512;
  const int Wmax = cus * std::min(waves_per_cu(fn, dev), tile_waves / a.head_dim);
  const int G = a.num_q_heads / a.num_kv_heads;
  const float scale_log2 = a.scale * 1.4426950408889634f;
  dim3 grid((Wmax + 3) / 4), block(256);
  hipLaunchKernelGGL(fn, grid, block, 0, s, a.q, static_cast<const uint8_t*>(a.k_pool),
                     static_cast<const uint8_t*>(a.v_pool), a.k_new, a.v_new, a.k_scales,
                     a.v_scales, a.block_tables,
                     a.seq_lens, a.out, a.partials, a.descs, a.qdescs, a.batch, a.max_pages, a.num_pages,
                     a.num_q_heads, a.num_kv_heads, G, a.page_size, a.partition_tokens, Wmax, scale_log2,
                     a.new_bf16 ? 1 : 0);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int pairs = a.batch * a.num_kv_heads;
  const int nchunk = (G * a.head_dim + 255) / 256;
  dim3 mgrid((unsigned)(((int64_t)pairs * nchunk + 3) / 4));
  void* kp = const_cast<void*>(a.k_pool);
  void* vp = const_cast<void*>(a.v_pool);
  if (a.new_quant) {
    float* ks = const_cast<float*>(a.k_scales);
    float* vs = const_cast<float*>(a.v_scales);
    mgrid = dim3((unsigned)(((int64_t)pairs * (nchunk + 2) + 3) / 4));   // plus two appending waves per pair
#define PKV_MERGE_Q(K, OB, DD)                                                                      \
  hipLaunchKernelGGL((decode_merge_quant_kernel<K, OB, DD>), mgrid, block, 0, s, a.descs, a.partials, a.out, \
                     a.batch, a.num_q_heads, a.num_kv_heads, G, nchunk, a.k_new, a.v_new,                \
                     a.new_bf16 ? 1 : 0, static_cast<uint8_t*>(kp), static_cast<uint8_t*>(vp), ks, vs,    \
                     a.qdescs, a.num_pages, a.page_size)
#define PKV_MERGE_QD(K, OB) \
  if (a.head_dim == 64) PKV_MERGE_Q(K, OB, 64); else PKV_MERGE_Q(K, OB, 128);
    if (a.kvt == KV_FP8) {
      if (a.out_bf16) { PKV_MERGE_QD(KV_FP8, true) } else { PKV_MERGE_QD(KV_FP8, false) }
    } else if (a.kvt == KV_INT8) {
      if (a.out_bf16) { PKV_MERGE_QD(KV_INT8, true) } else { PKV_MERGE_QD(KV_INT8, false) }
    } else {        // int4: D = 128 only
      if (a.out_bf16) PKV_MERGE_Q(KV_INT4, true, 128); else PKV_MERGE_Q(KV_INT4, false, 128);
    }
#undef PKV_MERGE_QD
#undef PKV_MERGE_Q
    return hipGetLastError();
  }
#define PKV_MERGE(K, OB)                                                                           \
  hipLaunchKernelGGL((decode_merge_kernel<K, OB>), mgrid, block, 0, s, a.descs, a.partials, a.out,     \
                     a.batch, a.num_q_heads, a.num_kv_heads, G, a.head_dim, nchunk, a.k_new, a.v_new,  \
                     kp, vp, a.num_pages, a.page_size)
  if (a.kvt == KV_F32) {
    if (a.out_bf16) PKV_MERGE(KV_F32, true); else PKV_MERGE(KV_F32, false);
  } else if (a.kvt == KV_BF16) {
    if (a.out_bf16) PKV_MERGE(KV_BF16, true); else PKV_MERGE(KV_BF16, false);
  } else if (a.kvt == KV_INT4) {
    if (a.out_bf16) PKV_MERGE(KV_INT4, true); else PKV_MERGE(KV_INT4, false);
  } else {            // any one-byte format (the append is a byte copy)
    if (a.out_bf16) PKV_MERGE(KV_FP8, true); else PKV_MERGE(KV_FP8, false);
  }
#undef PKV_MERGE
  return hipGetLastError();
}

}  // namespace pkv
