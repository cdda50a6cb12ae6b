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
//   four waves owns one (sequence, kv head, block of 256/G chunk tokens); each
//   wave holds 64 rows as four 16-column N tiles of the QK^T and PV MFMAs, the
//   query operand in registers for the whole kv range.
// * K and V come straight from the pages into MFMA operand registers, as in
//   decode (the page layout puts each 16-byte group where a lane needs it), one
//   32-token tile ahead; every K or V operand feeds four MFMAs (one per N tile).
//   The workgroups of a kv head g are blockIdx = g (mod Hkv), so with eight kv
//   heads all readers of one head's pages run on one XCD and share its L2.
// * Workgroups holding the later (longer-range) blocks of a sequence are
//   dispatched first.
// * S^T = K Q^T leaves four tokens of one query row per lane, which is the
//   B-operand layout of O^T += V^T P^T: probabilities never cross lanes.  They
//   enter the MFMA as one bf16 value (round to nearest even).
// * Only tiles that reach past a wave's first row position apply the causal
//   mask; V elements of tokens at or past the wave's last position + 1 are
//   zeroed (they may be unwritten slots).

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "pkv_internal.h"
#include "pkv_device.h"

namespace pkv {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 pair (round to nearest even), element a low.
__device__ __forceinline__ uint32_t pack_bf16_rne(float a, float b) {
  const bf16x2_t r = __builtin_convertvector(f32x2_t{a, b}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, r);
}

// ---------------------------------------------------------------------------
// Chunk append.  Block (b, y) copies the chunk tokens of sequence b whose
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
// Prefill attention, bf16 cache.  TPW = 256 / G chunk tokens per workgroup;
// row rho (0..255) of a workgroup is chunk token qb * TPW + rho / G and head
// rho % G of kv group g (rows at or past TPW * G are padding).  Wave wv owns
// rows 64 wv .. 64 wv + 63; N tile nt holds rows 64 wv + 16 nt + (0..15).
// ---------------------------------------------------------------------------
template <int D, bool OUT_BF16>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void prefill_kernel(
    const uint16_t* __restrict__ q, const int32_t* __restrict__ cu, int total_q,
    const uint8_t* __restrict__ kpool, const uint8_t* __restrict__ vpool, const int32_t* __restrict__ bt,
    const int32_t* __restrict__ seq_lens, void* __restrict__ out_, int B, int MP, int NP, int Hq, int Hkv,
    int G, int TPW, int P, float scale_log2) {
  constexpr int E = 8;              // bf16 elements per 16-byte group
  constexpr int TS = 32;            // tokens per tile (one V block)
  constexpr int NKK = D / 32;       // K groups per lane per 16-token sub-tile
  constexpr int NDT = D / 16;       // 16-dim PV tiles
  constexpr int NT = 4;             // 16-row N tiles per wave
  const float NEG_INF = -__builtin_inff();

  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15, c4 = lane >> 4;
  const int wv = uniform(threadIdx.x >> 6);
  const int g = uniform((int)(blockIdx.x % (unsigned)Hkv));
  const int unit = uniform((int)(blockIdx.x / (unsigned)Hkv));

  // ---- (sequence, token block) of this workgroup --------------------------------
  // blocks of sequence b: ceil(C_b / TPW); units are numbered in sequence order,
  // and within a sequence from the last block to the first.
  int b = -1, qb = 0;
  {
    int run = 0;
    for (int b0 = 0; b0 < B; b0 += 64) {
      const int bb = b0 + lane;
      int C = 0;
      if (bb < B) {
        const int r0 = cu[bb], r1 = cu[bb + 1];
        C = (r0 >= 0 && r1 <= total_q && r1 > r0) ? r1 - r0 : 0;
      }
      const int nb = (C + TPW - 1) / TPW;
      const int incl = run + wave_incl_scan(nb, lane);
      const uint64_t hit = __ballot(bb < B && incl > unit);
      if (hit) {
        const int f = uniform(__builtin_ctzll(hit));
        b = b0 + f;
        const int nbf = __builtin_amdgcn_readlane(nb, f);
        const int excl = __builtin_amdgcn_readlane(incl - nb, f);
        qb = nbf - 1 - (unit - excl);
        break;
      }
      run = uniform(__builtin_amdgcn_readlane(incl, 63));
    }
  }
  if (b < 0) return;
  b = uniform(b);
  qb = uniform(qb);
  const int r0 = uniform(cu[b]);
  const int C = uniform(cu[b + 1]) - r0;
  const int L = uniform(seq_lens[b]);
  const int ctx = L - C;                       // position of chunk token 0

  // ---- this wave's rows ----------------------------------------------------------
  const int rows = TPW * G;                    // real rows of the workgroup
  const int tok_base = qb * TPW;
  const int rho_w0 = 64 * wv;
  if (rho_w0 >= rows || tok_base + rho_w0 / G >= C) return;      // no real row in this wave
  const int rho_last = min(rho_w0 + 63, rows - 1);
  const int tok_last = min(C - 1, tok_base + rho_last / G);
  const int pos_first = ctx + tok_base + rho_w0 / G;             // smallest row position
  const int kv_end = max(ctx + tok_last + 1, 0);                 // keys 0 .. kv_end - 1

  u32x4_t Q[NT][NKK];
  int pos_n[NT];                // position of this lane's row in each N tile (-1: none)
  size_t orow[NT];              // output row offset (elements) of this lane's row
  bool store_n[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int rho = rho_w0 + 16 * nt + r16;
    const int tok = tok_base + rho / G, h = rho % G;
    const bool real = rho < rows && tok < C;
    store_n[nt] = real;
    pos_n[nt] = real ? max(ctx + tok, -1) : -1;
    orow[nt] = real ? ((size_t)(r0 + tok) * Hq + (size_t)g * G + h) * D : 0;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      Q[nt][kk] = real ? ld16(reinterpret_cast<const uint8_t*>(q + orow[nt] + 8 * c4 + 32 * kk))
                       : u32x4_t{0, 0, 0, 0};
  }

  f32x4_t O[NDT][NT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) O[dt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m[NT], l[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m[nt] = NEG_INF;
    l[nt] = 0.f;
  }

  const const_i32_ptr btrow = (const_i32_ptr)(bt + (size_t)b * MP);
  auto page_of = [&](int idx) -> int {
    idx = uniform(idx);
    const int v = btrow[idx < MP ? idx : MP - 1];
    return idx < MP ? v : -1;
  };
  u32x4_t kr[2][NKK], vr[NDT];
  auto load_k = [&](int pg, int j) {
    const uint8_t* kc = kpool + 2 * chunk_elem(pg, g, Hkv, P, D);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
        kr[sub][kk] = ld16(kc + 2u * (uint32_t)k_elem<E>(j + 16 * sub + r16, (c4 + 4 * kk) * E, P));
  };
  auto load_v = [&](int pg, int j) {
    const uint8_t* vc = vpool + 2 * chunk_elem(pg, g, Hkv, P, D);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
      vr[dt] = ld16(vc + 2u * (uint32_t)v_elem<E>(j + 4 * c4, dt * 16 + r16, D));
  };

  bool bad = false;
  if (kv_end > 0) {
    int pgi = 0, j0 = 0;
    int page = page_of(0);
    bad = (unsigned)page >= (unsigned)NP;
    load_k(bad ? 0 : page, 0);
    load_v(bad ? 0 : page, 0);

    auto tile = [&](const int t, auto last_tag) {
      constexpr bool LAST = decltype(last_tag)::value;
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

      // ---- S^T = K Q^T: rows = 16 tokens, columns = query rows ----------------
      float s[2][NT][4];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < NKK; ++kk) acc = mfma_bf16(kr[sub][kk], Q[nt][kk], acc);
#pragma unroll
          for (int i = 0; i < 4; ++i) s[sub][nt][i] = acc[i] * scale_log2;
        }
      if constexpr (!LAST) load_k(pg_ld_n, j_n);

      // ---- causal mask (tiles reaching past the wave's first row) -------------
      if (t + TS - 1 > pos_first) {
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int tau = t + 16 * sub + 4 * c4 + i;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
              if (tau > pos_n[nt]) s[sub][nt][i] = NEG_INF;
          }
      }
      if constexpr (LAST) {
        // keys at or past kv_end may be unwritten slots: zero their V elements
        // (element e of a lane's group is token 16 (e / 4) + 4 c4 + e % 4)
        if (t + TS > kv_end) {
          u32x4_t keep;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            uint32_t msk = 0;
#pragma unroll
            for (int f = 0; f < 2; ++f) {
              const int e = 2 * w + f;
              if (t + 16 * (e >> 2) + 4 * c4 + (e & 3) < kv_end) msk |= 0xFFFFu << (16 * f);
            }
            keep[w] = msk;
          }
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) vr[dt] &= keep;
        }
      }

      // ---- online softmax per query row (log2 domain) --------------------------
      u32x4_t pb[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float tmax = NEG_INF;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, s[sub][nt][i]);
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float mnew = fmaxf(m[nt], tmax);
        const float msafe = mnew == NEG_INF ? 0.f : mnew;
        const float alpha = __builtin_amdgcn_exp2f(m[nt] - msafe);
        float p[2][4], lsum = 0.f;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            p[sub][i] = __builtin_amdgcn_exp2f(s[sub][nt][i] - msafe);
            lsum += p[sub][i];
          }
        l[nt] = l[nt] * alpha + lsum;
        if (__ballot(mnew > m[nt])) {
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) O[dt][nt] *= alpha;
        }
        m[nt] = mnew;
        pb[nt] = u32x4_t{pack_bf16_rne(p[0][0], p[0][1]), pack_bf16_rne(p[0][2], p[0][3]),
                         pack_bf16_rne(p[1][0], p[1][1]), pack_bf16_rne(p[1][2], p[1][3])};
      }

      // ---- O^T += V^T P^T: rows = 16 dims, columns = query rows -----------------
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) O[dt][nt] = mfma_bf16(vr[dt], pb[nt], O[dt][nt]);
      if constexpr (!LAST) {
        load_v(pg_ld_n, j_n);
        bad |= bad_n;
        page = page_n;
        pgi = pgi_n;
        j0 = j_n;
      }
    };

    int t = 0;
    for (; t + TS < kv_end; t += TS) tile(t, std::false_type{});
    tile(t, std::true_type{});
  }

  // ---- normalise and store ---------------------------------------------------------
  const float qnan = __builtin_nanf("");
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float lt = l[nt] + __shfl_xor(l[nt], 16);
    lt += __shfl_xor(lt, 32);
    if (!store_n[nt]) continue;
    // rows with no key (position < 0) give zeros; a bad page id gives NaN
    const float inv = bad ? qnan : (pos_n[nt] < 0 ? 0.f : 1.f / lt);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) store_out4<OUT_BF16>(out_, orow[nt] + dt * 16 + 4 * c4, O[dt][nt] * inv);
  }
}

hipError_t launch_append_chunk(const AppendChunkArgs& a, hipStream_t s) {
  if (a.batch <= 0 || a.total <= 0) return hipSuccess;
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
  const int TPW = 256 / G;                       // chunk tokens per workgroup (G <= 256)
  // every sequence's blocks: at most total_q / TPW full ones plus one partial each
  const int64_t units = ((int64_t)a.total_q + TPW - 1) / TPW + a.batch;
  const int64_t blocks = units * a.num_kv_heads;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const float scale_log2 = a.scale * 1.4426950408889634f;
  dim3 grid((unsigned)blocks), block(256);
#define PKV_PREFILL(DD, OB)                                                                          \
  hipLaunchKernelGGL((prefill_kernel<DD, OB>), grid, block, 0, s, static_cast<const uint16_t*>(a.q),  \
                     a.cu_q, a.total_q, static_cast<const uint8_t*>(a.k_pool),                         \
                     static_cast<const uint8_t*>(a.v_pool), a.block_tables, a.seq_lens, a.out,        \
                     a.batch, a.max_pages, a.num_pages, a.num_q_heads, a.num_kv_heads, G, TPW,        \
                     a.page_size, scale_log2)
  if (a.head_dim == 128) {
    if (a.out_bf16) PKV_PREFILL(128, true); else PKV_PREFILL(128, false);
  } else if (a.head_dim == 64) {
    if (a.out_bf16) PKV_PREFILL(64, true); else PKV_PREFILL(64, false);
  } else {
    return hipErrorInvalidValue;
  }
#undef PKV_PREFILL
  return hipGetLastError();
}

}  // namespace pkv
