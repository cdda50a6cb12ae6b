// Internal host interface between the C-ABI entry points (pkv_api.cpp) and the
// HIP kernels (pkv_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

enum KvType { KV_F32 = 0, KV_BF16 = 1, KV_FP8 = 2, KV_INT8 = 3, KV_INT4 = 4 };

inline int elem_bits(int kvt) { return kvt == KV_F32 ? 32 : kvt == KV_BF16 ? 16 : kvt == KV_INT4 ? 4 : 8; }
// Tokens per V block (and per decode step): 4 * E, E = elements per 16-byte group.
inline int v_block_tokens(int kvt) { return 4 * (128 / elem_bits(kvt)); }

// Upper bound on decode wavefronts per compute unit; sizes the partial-result
// workspace together with the device's compute-unit count.  The launch never
// exceeds it: at most 512 / D waves per CU (1024 / D for int4, D = 128 only).
constexpr int kMaxWavesPerCU = 8;

// Size of the library's static device scratch array, the workspace of the
// allocation-free step entry point (one copy per device, held until the
// process ends).  40 MiB covers the partial slots of every accepted group
// size and head dimension on a 256-CU device (34 MB at G = 16, D = 128) plus
// the 32 bytes of per-pair records of up to ~245 000 (sequence, kv head) pairs.
constexpr size_t kStaticScratchBytes = (size_t)40 << 20;

// Workspace layout: partial slots (2 per wave), then B * Hkv 16-byte merge
// descriptors, then B * Hkv 16-byte records of the quantising step.
inline size_t partials_bytes(int cus, int G, int D) {
  size_t b = 2 * (size_t)cus * kMaxWavesPerCU * (size_t)G * ((size_t)D + 2) * sizeof(float);
  return (b + 255) & ~(size_t)255;
}

struct AppendQuantArgs {
  const void* k_new;
  const void* v_new;
  int kvt;                  // KV_FP8, KV_INT8 or KV_INT4: the format written
  bool new_bf16;            // rows are bf16 (else fp32)
  const int32_t* block_tables;
  const int32_t* seq_lens;
  void* k_pool;
  void* v_pool;
  float* k_scales;
  float* v_scales;
  int batch, max_pages, num_pages, num_kv_heads, head_dim, page_size;
};

struct AppendArgs {
  const void* k_new;
  const void* v_new;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  void* k_pool;
  void* v_pool;
  int kvt, batch, max_pages, num_pages, num_kv_heads, head_dim, page_size;
};

struct GatherArgs {
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  void* k_out;
  void* v_out;
  int kvt, batch, max_pages, num_pages, num_kv_heads, head_dim, page_size;
};

struct DecodeArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const void* k_new;       // step entry only (else null): token appended at L_b - 1
  const void* v_new;
  const float* k_scales;   // fp8 only
  const float* v_scales;   // fp8 only
  const int32_t* block_tables;
  const int32_t* seq_lens;
  void* out;
  float* partials;         // workspace: partial-result slots
  int4* descs;             // workspace: per-(b, g) merge descriptors
  int4* qdescs;            // workspace: per-(b, g) old page scales (quantising step)
  int kvt;                 // KvType; q is f32 for KV_F32, bf16 otherwise
  bool out_bf16;
  int batch, max_pages, num_pages, num_q_heads, num_kv_heads, head_dim, page_size;
  int partition_tokens;    // > 0, multiple of v_block_tokens(kvt)
  float scale;
  bool new_quant = false;  // quantising step: k_new / v_new are rows to quantise on write
  bool new_bf16 = false;   // ... bf16 rows (else fp32)
};

// Chunk append: rows cu_new[b] .. cu_new[b+1] of k_new / v_new ([total][Hkv][D])
// into positions L_b - C_b .. L_b - 1 of sequence b.
struct AppendChunkArgs {
  const void* k_new;
  const void* v_new;
  const int32_t* cu_new;
  int total;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  void* k_pool;
  void* v_pool;
  int kvt, batch, max_pages, num_pages, num_kv_heads, head_dim, page_size;
};

// Causal chunked prefill over a bf16 or fp8 cache: q and out are
// [total_q][Hq][D], rows cu_q[b] .. cu_q[b+1] belong to sequence b.
struct PrefillArgs {
  const void* q;            // bf16
  const int32_t* cu_q;
  int total_q;
  const void* k_pool;
  const void* v_pool;
  int kvt;                  // KV_BF16 or KV_FP8
  const float* k_scales;    // fp8 only
  const float* v_scales;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  void* out;
  bool out_bf16;
  int batch, max_pages, num_pages, num_q_heads, num_kv_heads, head_dim, page_size;
  float scale;
};

// Device page allocation: a free-page stack free_pages[0 .. *free_count - 1].
struct PageArgs {
  const int32_t* release;   // release only: nonzero marks a finished sequence
  const int32_t* seq_lens;
  int32_t* block_tables;
  int32_t* free_pages;
  int32_t* free_count;      // one int32 in device memory
  int batch, max_pages, page_size, num_pages, capacity;
};

hipError_t launch_alloc_pages(const PageArgs& a, hipStream_t s);
hipError_t launch_release_pages(const PageArgs& a, hipStream_t s);
hipError_t launch_append(const AppendArgs& a, hipStream_t s);
hipError_t launch_append_chunk(const AppendChunkArgs& a, hipStream_t s);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s);
// Quantising append into a one-byte cache (fp8 or int8) with dynamic page scales.
hipError_t launch_append_quant(const AppendQuantArgs& a, hipStream_t s);
hipError_t launch_gather(const GatherArgs& a, hipStream_t s);
hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* out, hipStream_t s);
// Launches the decode kernel and the log-sum-exp merge kernel.
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);
// Compute units of the current device (cached per device); <= 0 on failure.
int device_cu_count();
// Device address of the current device's static scratch array
// (kStaticScratchBytes), looked up once per device and cached.
hipError_t static_scratch(void** ptr);

}  // namespace pkv
