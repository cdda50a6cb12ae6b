// HIP kernels for causal chunked prefill over the paged KV cache (gfx950).
//
// Operation (first page, TensorRT-LLM concept page): besides the decode
// iterations that read and update the pages ("runtime execution model"),
// context tokens are processed in parallel over the paged cache, the compute
// that sets the first-token latency ("key performance parameters").  Sequence b
// brings C_b tokens whose K/V rows are first written into its pages, so
// seq_lens[b] = L_b counts them; chunk token i sits at position
// p = L_b - C_b + i and attends to cache tokens 0..p.  A position below zero
// (C_b > L_b) attends to nothing and gives zeros.
//
// Design for gfx950
// -----------------
// * Query rows are (chunk token, head of the kv group) pairs.  A workgroup of
//   four waves owns one (sequence, kv head, block of 128/G chunk tokens); each
//   wave holds 32 rows as two 16-column N tiles of the QK^T and PV MFMAs, with
//   its query operand in registers.  A wave needs 168 registers and a
//   workgroup 48 KiB of LDS, so three workgroups share a CU and each SIMD runs
//   three waves: one wave's softmax (VALU, cross-lane exchanges, exp) overlaps
//   the others' MFMAs.  Every tile runs through one body (masking steps are
//   small uniform branches): with a copy of the body per tile kind the
//   compiler kept the output accumulators in two register sets and copied
//   them on every tile.
// * K and V tiles are fetched once per workgroup with direct global -> LDS
//   loads (the page layout puts each 16-byte group where a lane needs it, so a
//   fetching lane's group is exactly some lane's MFMA operand), three buffers
//   deep, two 32-token tiles ahead, and read by all four waves; every K or V
//   operand feeds two MFMAs (one per N tile).  The workgroups of a kv head g are
//   blockIdx = g (mod Hkv), so with eight kv heads all readers of one head's
//   pages run on one XCD and share its L2.
// * Workgroups are dispatched longest sequence first, and within a sequence
//   from its last (longest-range) block to its first: the long ones do not
//   start late and leave a tail, and the blocks of one sequence, which read
//   the same pages, run close together and share them in L2.
// * S^T = K Q^T leaves four tokens of one query row per lane, which is the
//   B-operand layout of O^T += V^T P^T: probabilities never cross lanes.  They
//   enter the MFMA as one bf16 value (round to nearest even); the row sums come
//   from one more MFMA against an all-ones operand, i.e. from the same bf16
//   values the PV products use.
// * Online softmax with a lazy reference: p = 2^(s - m) against a reference m
//   that moves (rescaling O and the row sum) only when a tile's maximum exceeds
//   it by more than 8, so p <= 256 and the rescale, which reads and writes
//   every accumulator, runs a few times per row instead of on most early tiles.
//   The softmax scale (log2 e folded in) enters through one fma per score;
//   a negative scale is folded into the sign of q.
// * Only tiles that reach past a wave's first row position apply the causal
//   mask; V elements of slots at or past the sequence end L (unwritten, may
//   hold anything) are zeroed in LDS by the waves that fetched them, once, when
//   the sequence's last tile arrives.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <type_traits>

#include "pkv_internal.h"
#include "pkv_device.h"

namespace pkv {

typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;
typedef __attribute__((address_space(3))) u32x2_t lds_u32x2_t;

// ---------------------------------------------------------------------------
// Chunk append (f32, fp8, int8 and int4 caches; bf16 below).  Block (b, y)
// copies the chunk tokens of sequence b whose
// position pair t / 2 is y (mod gridDim.y): the two tokens of a pair share
// bytes of an int4 V group, so one block writes both.  Each thread copies a
// pair of dims (one int4 K byte).  A sequence whose chunk does not fit (C > L,
// L beyond its table row, rows outside [0, total)) is skipped, and so is a
// token whose page id is out of range.
// ---------------------------------------------------------------------------
template <int KVT>
__global__ __launch_bounds__(256) void append_chunk_kernel(
    const void* __restrict__ k_new, const void* __restrict__ v_new, const int32_t* __restrict__ cu, int total,
    const int32_t* __restrict__ bt, const int32_t* __restrict__ seq_lens, void* __restrict__ kpool,
    void* __restrict__ vpool, int MP, int NP, int Hkv, int D, int P) {
  constexpr int E = 128 / Kv<KVT>::BITS;
  const int b = blockIdx.x;
  const int r0 = cu[b], r1 = cu[b + 1];
  const int L = seq_lens[b];
  const int C = r1 - r0;
  if (C <= 0 || r0 < 0 || r1 > total || C > L || (int64_t)L > (int64_t)MP * P) return;
  const int t0 = L - C;
  for (int pr = (t0 >> 1) + (int)blockIdx.y; 2 * pr < L; pr += gridDim.y) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int t = 2 * pr + e;
      if (t < t0 || t >= L) continue;
      const int pgi = t / P, j = t - pgi * P;
      const int page = bt[(size_t)b * MP + pgi];
      if ((unsigned)page >= (unsigned)NP) continue;
      const size_t row0 = (size_t)(r0 + t - t0) * Hkv * D;
      for (int x = 2 * threadIdx.x; x < Hkv * D; x += 2 * blockDim.x) {
        const int g = x / D, d = x - g * D;
        const size_t ch = chunk_elem(page, g, Hkv, P, D);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          put_code<KVT>(kpool, ch + k_elem<E>(j, d + i, P), get_code<KVT>(k_new, row0 + x + i));
          put_code<KVT>(vpool, ch + v_elem<E>(j, d + i, D), get_code<KVT>(v_new, row0 + x + i));
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Chunk append, bf16 cache: block (b, y, g) writes kv head g of the 32-token V
// blocks blk = first + y, first + y + gridDim.y, ... of sequence b's chunk (a
// block lies in one page, P being a multiple of 32).  K: each token's 16-byte
// groups of 8 dims are copied whole (tokens adjacent in the layout go to
// adjacent lanes).  V: the block's rows are staged in LDS and each 16-byte
// group of the layout (8 tokens of one dim) is assembled from them and stored
// whole; a block the chunk covers only in part keeps the other tokens' values
// of each group (read from the page first).  Same skip rules as above.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void append_chunk_bf16_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new, const int32_t* __restrict__ cu,
    int total, const int32_t* __restrict__ bt, const int32_t* __restrict__ seq_lens,
    uint16_t* __restrict__ kpool, uint16_t* __restrict__ vpool, int MP, int NP, int Hkv, int P) {
  constexpr int TB = 32;              // tokens per V block
  constexpr int NG = D / 8;           // 16-byte K groups per token row
  constexpr int NIT = TB * NG / 256;  // K groups (and V row pieces) per thread
  static_assert(TB * NG % 256 == 0 && 4 * D % 256 == 0, "D must be 64 or 128");
  __shared__ uint16_t s_v[TB][D + 8];           // V rows of the block (padded rows)
  const int b = blockIdx.x, g = blockIdx.z;
  const int r0 = cu[b], r1 = cu[b + 1];
  const int L = seq_lens[b];
  const int C = r1 - r0;
  if (C <= 0 || r0 < 0 || r1 > total || C > L || (int64_t)L > (int64_t)MP * P) return;
  const int t0 = L - C;
  const int tid = threadIdx.x;
  for (int blk = t0 / TB + (int)blockIdx.y; blk * TB < L; blk += gridDim.y) {
    const int tb0 = blk * TB;
    const int page = bt[(size_t)b * MP + tb0 / P];
    if ((unsigned)page >= (unsigned)NP) continue;          // uniform: the whole block
    const int j0 = tb0 % P;                                // slot of the block's first token
    const size_t ch = chunk_elem(page, g, Hkv, P, D);
    const bool full = tb0 >= t0 && tb0 + TB <= L;
    __syncthreads();                                       // the previous block's LDS reads
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int x = it * 256 + tid;
      const int r = x / NG, c = x % NG;                    // token r of the block, dims 8c ..
      const int tk = tb0 + r;
      if (tk >= t0 && tk < L) {
        const size_t row = ((size_t)(r0 + tk - t0) * Hkv + g) * D + 8 * c;
        const u32x4_t kv = ld16(reinterpret_cast<const uint8_t*>(k_new + row));
        const u32x4_t vv = ld16(reinterpret_cast<const uint8_t*>(v_new + row));
        *reinterpret_cast<u32x4_t*>(kpool + ch + k_elem<8>(j0 + r, 8 * c, P)) = kv;
        *reinterpret_cast<u32x4_t*>(&s_v[r][8 * c]) = vv;
      }
    }
    __syncthreads();
    // V group (cc, d) of the block holds tokens 16 (e / 4) + 4 cc + e % 4, e = 0..7
#pragma unroll
    for (int it = 0; it < 4 * D / 256; ++it) {
      const int x = it * 256 + tid;
      const int cc = x / D, d = x % D;
      uint16_t* dst = vpool + ch + v_elem<8>(j0 + 4 * cc, d, D);
      u32x4_t old = {0, 0, 0, 0};
      if (!full) old = *reinterpret_cast<const u32x4_t*>(dst);
      u32x4_t w;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint32_t h[2];
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          const int e = 2 * k + f;
          const int r = 16 * (e >> 2) + 4 * cc + (e & 3);
          const int tk = tb0 + r;
          const uint32_t o = (old[k] >> (16 * f)) & 0xFFFFu;
          h[f] = (full || (tk >= t0 && tk < L)) ? (uint32_t)s_v[r][d] : o;
        }
        w[k] = h[0] | (h[1] << 16);
      }
      *reinterpret_cast<u32x4_t*>(dst) = w;
    }
  }
}

// ---------------------------------------------------------------------------
// Prefill attention, bf16 cache.  TPW = 128 / G chunk tokens per workgroup;
// row rho (0..127) of a workgroup is chunk token qb * TPW + rho / G and head
// rho % G of kv group g (rows at or past TPW * G are padding).  Wave wv owns
// rows 32 wv .. 32 wv + 31; N tile nt holds rows 32 wv + 16 nt + (0..15).
//
// K/V tiles of 32 tokens are staged in LDS, NBUF buffers deep: a tile is NOP
// operand slices of 64 lanes x 16 bytes (K slice (sub, kk) is what lane l of
// the QK^T MFMA needs as its A operand for 16-token sub-tile sub and k step kk;
// V slice dt the A operand of PV for dims 16 dt ..), each fetched by one wave
// with a direct global -> LDS load (lane l's 16 bytes land at slot l).  Every
// wave then reads the slices as its own operands.  Tiles are fetched NBUF - 1
// ahead, so a fetch has that many tiles of compute to arrive.  One barrier per
// tile: before it each wave waits for its own slices of tile i (its later
// fetches may stay in flight) and for its own LDS reads; after it, tile i is
// complete and no wave still reads buffer (i - 1) mod NBUF, which the fetch of
// tile i + NBUF - 1 then fills.  Every wave runs every iteration (fetches and
// barrier), computing only tiles below its own kv_end.
// ---------------------------------------------------------------------------
template <int KVT, int D, bool OUT_BF16>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(KVT == KV_FP8 ? 2 : 3, 3))) void prefill_kernel(
    const uint16_t* __restrict__ q, const int32_t* __restrict__ cu, int total_q,
    const uint8_t* __restrict__ kpool, const uint8_t* __restrict__ vpool, const float* __restrict__ kscales,
    const float* __restrict__ vscales, const int32_t* __restrict__ bt, const int32_t* __restrict__ seq_lens,
    void* __restrict__ out_, int B, int MP, int NP, int Hq, int Hkv, int G, int TPW, int P, float scale_log2,
    uint32_t q_sign) {
  // bf16 cache: a tile is one 32-token V block.  fp8 cache (e4m3 codes, a
  // scale per (page, kv head)): a tile is one 64-token V block, the same 16 KB
  // at D = 128, computed as two 32-key halves; codes widen to bf16 exactly on
  // their way from LDS to the MFMA, the K scale joins the softmax scale and
  // the V scale multiplies the probabilities that enter the PV products.
  constexpr bool FP8 = KVT == KV_FP8;
  constexpr int BITS = FP8 ? 8 : 16;
  constexpr int E = 128 / BITS;     // elements per 16-byte group
  constexpr int TS = 4 * E;         // tokens per tile (one V block)
  constexpr int NSUB = TS / 16;     // 16-token QK^T sub-tiles per tile
  constexpr int NHALF = NSUB / 2;   // 32-key halves per tile
  constexpr int NCH = FP8 ? 2 : 1;  // bf16x8 operands per 16-byte group
  constexpr int NKK = D / (4 * E);  // K groups per lane and sub-tile
  constexpr int NQ = NKK * NCH;     // query operands per N tile (k steps of QK^T)
  constexpr int NDT = D / 16;       // 16-dim PV tiles
  constexpr int NT = 2;             // 16-row N tiles per wave
  constexpr int NKOP = NSUB * NKK;  // K slices per tile
  constexpr int NOP = NKOP + NDT;   // K and V slices per tile (16 at D = 128)
  constexpr int OPW = NOP / 4;      // slices each wave fetches
  constexpr float TH = 8.f;         // reference lag allowed before a rescale (log2 units)
  constexpr int NBUF = 3;           // K/V tile buffers (prefetch distance NBUF - 1)
  const float NEG_INF = -__builtin_inff();

  __shared__ u32x4_t s_kv[NBUF][NOP][64];      // K/V tiles

  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15, c4 = lane >> 4;
  const int wv = uniform(threadIdx.x >> 6);
  const int g = uniform((int)(blockIdx.x % (unsigned)Hkv));
  const int unit = uniform((int)(blockIdx.x / (unsigned)Hkv));

  // ---- (sequence, token block) of this workgroup (same in every wave) ---------
  // Unit number u (from blockIdx) is the u-th block in this order: sequences
  // by length L_b descending (ties by index), each sequence's ceil(C_b / TPW)
  // blocks from the last to the first.  With n(w) = the blocks of sequences
  // with L_b >= w, a binary search over w finds the length of unit u's
  // sequence, then a scan over the sequences of that length finds it.
  // Lengths are clamped to the table's reach for the ordering only.
  const int cap = (int)min((int64_t)MP * P, (int64_t)1 << 30);
  auto seq_at = [&](int bb, int& C, int& Lc, int& nb) {
    C = 0;
    Lc = 0;
    if (bb < B) {
      const int ra = cu[bb], rb = cu[bb + 1];
      C = (ra >= 0 && rb <= total_q && rb > ra) ? rb - ra : 0;
      Lc = min(max(seq_lens[bb], 0), cap);
    }
    nb = (C + TPW - 1) / TPW;
  };
  // blocks of one sequence counted by n(w)
  auto n_ge = [&](int C, int Lc, int nb, int w) -> int { return (w <= 0 || Lc >= w) ? nb : 0; };
  auto wave_total = [&](int v) -> int { return uniform(__builtin_amdgcn_readlane(wave_incl_scan(v, lane), 63)); };
  // n(w), over all sequences (wave-uniform)
  auto count_ge = [&](int w) -> int {
    int tot = 0;
    for (int b0 = 0; b0 < B; b0 += 64) {
      int C, Lc, nb;
      seq_at(b0 + lane, C, Lc, nb);
      tot += wave_total(n_ge(C, Lc, nb, w));
    }
    return tot;
  };
  int b = -1, qb = 0;
  {
    int n_units = 0, lmax = 0;
    for (int b0 = 0; b0 < B; b0 += 64) {
      int C, Lc, nb;
      seq_at(b0 + lane, C, Lc, nb);
      n_units += wave_total(nb);
      int x = nb > 0 ? Lc : 0;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) x = max(x, __shfl_xor(x, o));
      lmax = max(lmax, uniform(x));
    }
    if (unit < n_units) {
      // largest w with n(w) > unit: the length of the unit's sequence
      int lo = 0, hi = lmax + 1, c_hi = 0;     // count_ge(lo) > unit >= count_ge(hi)
      while (hi - lo > 1) {
        const int mid = lo + (hi - lo) / 2;
        const int c = count_ge(mid);
        if (c > unit) {
          lo = mid;
        } else {
          hi = mid;
          c_hi = c;
        }
      }
      // the unit is number j among the blocks of sequences of length lo, by sequence
      const int j = unit - c_hi;
      int run = 0;
      for (int b0 = 0; b0 < B; b0 += 64) {
        int C, Lc, nb;
        seq_at(b0 + lane, C, Lc, nb);
        const int top = n_ge(C, Lc, nb, lo);
        const int eq = top - n_ge(C, Lc, nb, lo + 1);
        const int incl = run + wave_incl_scan(eq, lane);
        const uint64_t hit = __ballot(b0 + lane < B && incl > j);
        if (hit) {
          const int f = uniform(__builtin_ctzll(hit));
          b = b0 + f;
          const int excl = __builtin_amdgcn_readlane(incl - eq, f);
          qb = __builtin_amdgcn_readlane(nb, f) - 1 - (j - excl);   // last block first
          break;
        }
        run = uniform(__builtin_amdgcn_readlane(incl, 63));
      }
    }
  }
  if (b < 0) return;                           // the whole workgroup: no unit
  b = uniform(b);
  qb = uniform(qb);
  const int r0 = uniform(cu[b]);
  const int C = uniform(cu[b + 1]) - r0;
  const int L = uniform(seq_lens[b]);
  const int ctx = L - C;                       // position of chunk token 0

  // ---- rows and key ranges -------------------------------------------------------
  const int rows = TPW * G;                    // real rows of the workgroup (before C)
  const int tok_base = qb * TPW;
  const int tok_wg_last = min(C - 1, tok_base + (rows - 1) / G);
  const int kv_end_wg = max(ctx + tok_wg_last + 1, 0);           // keys any wave needs
  const int rho_w0 = 16 * NT * wv;
  const bool has_rows = rho_w0 < rows && tok_base + rho_w0 / G < C;
  const int tok_last = min(C - 1, tok_base + min(rho_w0 + 16 * NT - 1, rows - 1) / G);
  const int pos_first = ctx + tok_base + rho_w0 / G;             // smallest row position
  const int kv_end = has_rows ? max(ctx + tok_last + 1, 0) : 0;  // keys this wave needs

  int pos_n[NT];                // position of this lane's row in each N tile (-1: none)
  u32x4_t Q[NT][NQ];            // query operands (B of QK^T)
  auto out_row = [&](int nt) -> int64_t {
    const int rho = rho_w0 + 16 * nt + r16;
    const int tok = tok_base + rho / G, h = rho % G;
    if (rho >= rows || tok >= C) return -1;
    return ((int64_t)(r0 + tok) * Hq + (int64_t)g * G + h) * D;
  };
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int64_t orow = out_row(nt);
    const int tok = tok_base + (rho_w0 + 16 * nt + r16) / G;
    pos_n[nt] = orow >= 0 ? max(ctx + tok, -1) : -1;
    // operand i: dims E (c4 + 4 (i / NCH)) + 8 (i % NCH) .. + 7, the dims of
    // the K operand it meets (a lane's K group, or half of it for fp8)
#pragma unroll
    for (int i = 0; i < NQ; ++i)
      Q[nt][i] = orow >= 0 ? ld16(reinterpret_cast<const uint8_t*>(q + orow + E * (c4 + 4 * (i / NCH)) + 8 * (i % NCH))) ^ q_sign
                           : u32x4_t{0, 0, 0, 0};
  }

  f32x4_t O[NDT][NT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) O[dt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // m: the softmax reference per row (scaled, log2 domain); Ls: row sums of p
  // (every entry of Ls[nt] holds its column's sum).
  float m[NT];
  f32x4_t Ls[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m[nt] = NEG_INF;
    Ls[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const u32x4_t ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  // fp8: scales of the tiles in the buffers (this tile, the next, the one
  // being fetched), loaded by every wave when it fetches a tile
  float ksq[3] = {1.f, 1.f, 1.f}, vsq[3] = {1.f, 1.f, 1.f};

  const const_i32_ptr btrow = (const_i32_ptr)(bt + (size_t)b * MP);
  // Wave wv fetches slices wv, wv + 4, ...: the first OPW / 2 are K slices, the
  // rest V slices.  A slice's lane offset inside a page chunk is linear in the
  // tile's token offset j (K: 16 bytes per token; V: 2 D bytes per token, j a
  // multiple of 32), so it is computed once here and the fetch adds a
  // wave-uniform base.
  static_assert(NKOP % 4 == 0 && NDT % 4 == 0, "K and V slices must split evenly over four waves");
  uint32_t sl_off[OPW];
#pragma unroll
  for (int o = 0; o < OPW; ++o) {
    const int op = wv + 4 * o;
    if (o < OPW / 2) {
      const int sub = op / NKK, kk = op % NKK;
      sl_off[o] = (uint32_t)(BITS / 8) * (uint32_t)k_elem<E>(16 * sub + r16, (c4 + 4 * kk) * E, P);
    } else {
      sl_off[o] = (uint32_t)(BITS / 8) * (uint32_t)v_elem<E>(4 * c4, (op - NKOP) * 16 + r16, D);
    }
  }
  // Next tile to fetch: page index and token offset in it.  Returns whether its
  // page id is bad (page 0 is read instead).
  int f_pgi = 0, f_j = 0;
  // bytes per page (all kv heads; below 2^32, checked at the boundary) and from
  // a page to kv head g's chunk
  const uint32_t page_bytes = uniform((uint32_t)(Hkv * P * D * (BITS / 8)));
  const uint8_t* kg = kpool + (size_t)g * P * D * (BITS / 8);
  const uint8_t* vg = vpool + (size_t)g * P * D * (BITS / 8);
  auto fetch_next = [&](int buf) -> bool {
    const int page = f_pgi < MP ? btrow[f_pgi] : -1;
    const bool badp = (unsigned)page >= (unsigned)NP;
    if constexpr (FP8) {
      ksq[2] = kscales[(size_t)(badp ? 0 : page) * Hkv + g];
      vsq[2] = vscales[(size_t)(badp ? 0 : page) * Hkv + g];
    }
    const uint64_t ch = (uint64_t)(uint32_t)(badp ? 0 : page) * page_bytes;
    const uint8_t* kc = kg + ch + 16 * f_j;
    const uint8_t* vc = vg + ch + (BITS / 8) * D * f_j;
#pragma unroll
    for (int o = 0; o < OPW; ++o) {
      const uint8_t* src = (o < OPW / 2 ? kc : vc) + sl_off[o];
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                       (__attribute__((address_space(3))) void*)&s_kv[buf][wv + 4 * o][0], 16,
                                       0, 0);
    }
    f_j += TS;
    if (f_j == P) {
      f_j = 0;
      ++f_pgi;
    }
    return badp;
  };
  auto slice = [&](int buf, int op) -> u32x4_t {
    return *(lds_u32x4_t*)(&s_kv[buf][op][lane]);
  };

  // 32 keys (half h of the tile) from buffer buf.  masked (wave-uniform): the
  // keys reach past the wave's first row position (causal mask).  One body for
  // every tile: the mask steps are small uniform branches, so the output
  // accumulators never cross a branch of their own.  Keys past a row's
  // position get p = 0; V of slots at or past L (which may hold anything) was
  // zeroed in LDS when the tile arrived.  ksl: the softmax scale times the
  // tile's K scale (log2 domain); vs: the tile's V scale (fp8, else 1).
  u32x2_t vhi[NDT];            // fp8: the second half's bytes of each V group
  auto tile = [&](const int t, const int buf, const bool masked, const int h, const float ksl, const float vs) {
    // ---- S^T = K Q^T: rows = 16 tokens, columns = query rows (unscaled) ------
    f32x4_t acc[2][NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      acc[0][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      acc[1][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const u32x4_t k0 = slice(buf, (2 * h) * NKK + kk), k1 = slice(buf, (2 * h + 1) * NKK + kk);
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const u32x4_t a0 = FP8 ? byte8_to_bf16x8<KV_FP8>(k0[2 * c], k0[2 * c + 1]) : k0;
        const u32x4_t a1 = FP8 ? byte8_to_bf16x8<KV_FP8>(k1[2 * c], k1[2 * c + 1]) : k1;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          acc[0][nt] = mfma_bf16(a0, Q[nt][kk * NCH + c], acc[0][nt]);
          acc[1][nt] = mfma_bf16(a1, Q[nt][kk * NCH + c], acc[1][nt]);
        }
      }
    }
    // ---- online softmax per row (log2 domain, lazy reference) -----------------
    // Unmasked scores are finite, so a column with any unmasked score has a
    // finite reference after its first tile; masked scores (-inf) get p = 0.
    // The reference of a column grows when the column's max passes it by more
    // than TH.  Each lane first tests its own 8 scores; only when some lane
    // passes does the wave form the column maxima across the four lanes of a
    // column and rescale (the common case needs no cross-lane step).
    const int tk = t + 32 * h;                 // first key of these 32
    float s[NT][2][4];
    float lmax[NT];
    bool pass = false;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[nt][0][i] = acc[0][nt][i];
        s[nt][1][i] = acc[1][nt][i];
      }
      if (masked) {
        // key tk + 16 sub + 4 c4 + i lies past the row's position
        const int lim = pos_n[nt] - tk - 4 * c4;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (16 * sub + i > lim) s[nt][sub][i] = NEG_INF;
      }
      float x = NEG_INF;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int i = 0; i < 4; ++i) x = fmaxf(x, s[nt][sub][i]);
      lmax[nt] = x;
      // m = -inf gives +inf (passes) unless every score is masked (NaN: no)
      pass |= __builtin_fmaf(x, ksl, -m[nt]) > TH;
    }
    if (__ballot(pass)) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const float cmax = colmax4(lmax[nt]);
        const bool grow = __builtin_fmaf(cmax, ksl, -m[nt]) > TH;
        const float mref = grow ? cmax * ksl : m[nt];
        const float alpha = grow ? __builtin_amdgcn_exp2f(m[nt] - mref) : 1.f;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) scale_in_place(O[dt][nt], alpha);
        scale_in_place(Ls[nt], alpha);
        m[nt] = mref;
      }
    }
    u32x4_t pb[NT], pv[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float p[2][4];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          p[sub][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[nt][sub][i], ksl, -m[nt]));
      if (masked) {
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (s[nt][sub][i] == NEG_INF) p[sub][i] = 0.f;
      }
      pb[nt] = u32x4_t{pack_bf16_rne(p[0][0], p[0][1]), pack_bf16_rne(p[0][2], p[0][3]),
                       pack_bf16_rne(p[1][0], p[1][1]), pack_bf16_rne(p[1][2], p[1][3])};
      Ls[nt] = mfma_bf16(ones, pb[nt], Ls[nt]);
      // the PV products take p times the tile's V scale (fp8); the row sums
      // above take p itself
      if constexpr (FP8)
        pv[nt] = u32x4_t{pack_bf16_rne(p[0][0] * vs, p[0][1] * vs), pack_bf16_rne(p[0][2] * vs, p[0][3] * vs),
                         pack_bf16_rne(p[1][0] * vs, p[1][1] * vs), pack_bf16_rne(p[1][2] * vs, p[1][3] * vs)};
      else
        pv[nt] = pb[nt];
    }
    // ---- O^T += V^T P^T: rows = 16 dims, columns = query rows -------------------
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      u32x4_t vv;
      if constexpr (FP8) {
        // the first half reads the whole 16-byte group (conflict-free) and
        // keeps the second half's 8 bytes for it
        u32x2_t w;
        if (h == 0) {
          const u32x4_t f = slice(buf, NKOP + dt);
          w = u32x2_t{f.x, f.y};
          vhi[dt] = u32x2_t{f.z, f.w};
        } else {
          w = vhi[dt];
        }
        vv = byte8_to_bf16x8<KV_FP8>(w.x, w.y);
      } else {
        vv = slice(buf, NKOP + dt);
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) O[dt][nt] = mfma_bf16(vv, pv[nt], O[dt][nt]);
    }
  };

  // s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0, expcnt 6:4 left at
  // its maximum, lgkmcnt 11:8 = 0): all LDS reads done and at most n vector
  // memory operations (this wave's later fetches) outstanding
  constexpr int WAIT_V0 = 0x70, WAIT_V1 = 0x70 | OPW, WAIT_V2 = 0x70 | (2 * OPW);
  static_assert(2 * OPW < 16 && NBUF == 3, "waitcnt immediates assume < 16 loads; the scale slots assume 3 buffers");
  bool bad = false;
  const int ntiles = (kv_end_wg + TS - 1) / TS;
  if (ntiles > 0) {
    uint32_t bad_bits = 0;                     // bit i % 32: tile i's page id is bad
#pragma unroll
    for (int i = 0; i < NBUF - 1; ++i) {
      if (i < ntiles && fetch_next(i)) bad_bits |= 1u << i;
      if constexpr (FP8) {       // tile i's scales into slot i
        ksq[i] = ksq[2];
        vsq[i] = vsq[2];
      }
    }
    for (int it = 0; it < ntiles; ++it) {
      const int buf = it % NBUF;
      // this wave's slices of tile `it` have landed (later tiles may be in flight)
      const int later = min(ntiles - 1 - it, NBUF - 2);
      if (later >= 2) __builtin_amdgcn_s_waitcnt(WAIT_V2);
      else if (later == 1) __builtin_amdgcn_s_waitcnt(WAIT_V1);
      else __builtin_amdgcn_s_waitcnt(WAIT_V0);
      if (it * TS + TS > L) {
        // The tile holds slots at or past L, which may hold anything: each wave
        // zeroes the V elements of those slots in the slices it fetched (element
        // e of a lane's group is token 16 (e / 4) + 4 c4 + e % 4), so no 0 * NaN
        // reaches the products, and waits for its writes before the barrier.
        constexpr int PW = 32 / BITS;          // elements per word
        u32x4_t keep;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint32_t msk = 0;
#pragma unroll
          for (int f = 0; f < PW; ++f) {
            const int e = PW * w + f;
            if (it * TS + 16 * (e >> 2) + 4 * c4 + (e & 3) < L) msk |= ((1u << BITS) - 1u) << (BITS * f);
          }
          keep[w] = msk;
        }
#pragma unroll
        for (int o = OPW / 2; o < OPW; ++o) {
          volatile lds_u32x4_t* slot = (volatile lds_u32x4_t*)(&s_kv[buf][wv + 4 * o][lane]);
          *slot = *slot & keep;
        }
        __builtin_amdgcn_s_waitcnt(WAIT_V0);
      }
      asm volatile("" ::: "memory");           // LDS reads of earlier tiles stay above
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");           // and this tile's reads below the barrier
      const int nf = it + NBUF - 1;
      if (nf < ntiles && fetch_next(nf % NBUF)) bad_bits |= 1u << (nf & 31);
      const int t = it * TS;
      if (t < kv_end) {
        bad |= (bad_bits >> (it & 31)) & 1u;
        const float ksl = FP8 ? scale_log2 * ksq[0] : scale_log2;
#pragma unroll
        for (int h = 0; h < NHALF; ++h)
          if (t + 32 * h < kv_end) tile(t, buf, t + 32 * h + 31 > pos_first, h, ksl, vsq[0]);
      }
      bad_bits &= ~(1u << (it & 31));
      if constexpr (FP8) {       // the next tile's scales move up
        ksq[0] = ksq[1];
        ksq[1] = ksq[2];
        vsq[0] = vsq[1];
        vsq[1] = vsq[2];
      }
    }
  }

  // ---- normalise and store ---------------------------------------------------------
  const float qnan = __builtin_nanf("");
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const float lt = Ls[nt][0];
    const int64_t orow = out_row(nt);
    if (orow < 0) continue;
    // rows with no key (position < 0) give zeros; a bad page id gives NaN
    const float inv = bad ? qnan : (pos_n[nt] < 0 ? 0.f : 1.f / lt);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
      store_out4<OUT_BF16>(out_, (size_t)orow + dt * 16 + 4 * c4, O[dt][nt] * inv);
  }
}

hipError_t launch_append_chunk(const AppendChunkArgs& a, hipStream_t s) {
  if (a.batch <= 0 || a.total <= 0) return hipSuccess;
  if (a.kvt == KV_BF16 && (a.head_dim == 64 || a.head_dim == 128)) {
    // 32-token blocks per sequence: about total / batch / 32 + 1 on average
    const int ny = (int)std::min<int64_t>(64, (int64_t)a.total / a.batch / 32 + 2);
    dim3 bgrid(a.batch, ny, a.num_kv_heads), bblock(256);
#define PKV_APPEND_CHUNK_BF16(DD)                                                                   \
    hipLaunchKernelGGL(append_chunk_bf16_kernel<DD>, bgrid, bblock, 0, s,                           \
                       static_cast<const uint16_t*>(a.k_new), static_cast<const uint16_t*>(a.v_new), \
                       a.cu_new, a.total, a.block_tables, a.seq_lens, static_cast<uint16_t*>(a.k_pool), \
                       static_cast<uint16_t*>(a.v_pool), a.max_pages, a.num_pages, a.num_kv_heads,      \
                       a.page_size)
    if (a.head_dim == 128) PKV_APPEND_CHUNK_BF16(128); else PKV_APPEND_CHUNK_BF16(64);
#undef PKV_APPEND_CHUNK_BF16
    return hipGetLastError();
  }
  dim3 grid(a.batch, 64), block(256);
#define PKV_APPEND_CHUNK(K)                                                                          \
  hipLaunchKernelGGL(append_chunk_kernel<K>, grid, block, 0, s, a.k_new, a.v_new, a.cu_new, a.total,   \
                     a.block_tables, a.seq_lens, a.k_pool, a.v_pool, a.max_pages, a.num_pages,        \
                     a.num_kv_heads, a.head_dim, a.page_size)
  if (a.kvt == KV_F32) PKV_APPEND_CHUNK(KV_F32);
  else if (a.kvt == KV_BF16) PKV_APPEND_CHUNK(KV_BF16);
  else if (a.kvt == KV_INT4) PKV_APPEND_CHUNK(KV_INT4);
  else PKV_APPEND_CHUNK(KV_FP8);          // any one-byte format: a byte copy
#undef PKV_APPEND_CHUNK
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) {
  if (a.batch <= 0 || a.total_q <= 0) return hipSuccess;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int TPW = 128 / G;                       // chunk tokens per workgroup (G <= 128)
  // every sequence's blocks: at most total_q / TPW full ones plus one partial each
  const int64_t units = ((int64_t)a.total_q + TPW - 1) / TPW + a.batch;
  const int64_t blocks = units * a.num_kv_heads;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  // a negative scale is applied as a sign flip of q (exact), so the kernel's
  // scale is never negative
  const float scale_log2 = fabsf(a.scale) * 1.4426950408889634f;
  const uint32_t q_sign = std::signbit(a.scale) ? 0x80008000u : 0u;
  dim3 grid((unsigned)blocks), block(256);
#define PKV_PREFILL(K, DD, OB)                                                                       \
  hipLaunchKernelGGL((prefill_kernel<K, DD, OB>), grid, block, 0, s, static_cast<const uint16_t*>(a.q), \
                     a.cu_q, a.total_q, static_cast<const uint8_t*>(a.k_pool),                         \
                     static_cast<const uint8_t*>(a.v_pool), a.k_scales, a.v_scales, a.block_tables,   \
                     a.seq_lens, a.out, a.batch, a.max_pages, a.num_pages, a.num_q_heads,             \
                     a.num_kv_heads, G, TPW, a.page_size, scale_log2, q_sign)
#define PKV_PREFILL_K(K)                                                                             \
  if (a.head_dim == 128) {                                                                           \
    if (a.out_bf16) PKV_PREFILL(K, 128, true); else PKV_PREFILL(K, 128, false);                      \
  } else if (a.head_dim == 64) {                                                                     \
    if (a.out_bf16) PKV_PREFILL(K, 64, true); else PKV_PREFILL(K, 64, false);                        \
  } else {                                                                                           \
    return hipErrorInvalidValue;                                                                     \
  }
  if (a.kvt == KV_FP8) {
    PKV_PREFILL_K(KV_FP8)
  } else if (a.kvt == KV_BF16) {
    PKV_PREFILL_K(KV_BF16)
  } else {
    return hipErrorInvalidValue;
  }
#undef PKV_PREFILL_K
#undef PKV_PREFILL
  return hipGetLastError();
}

}  // namespace pkv
