// C-ABI entry points of libpkv.so (declared in include/pkv.h): argument
// validation, workspace sizing and dispatch to the HIP kernels.  Every check
// runs before any HIP call, so invalid arguments never touch the device.
#include "pkv.h"

#include <hip/hip_runtime_api.h>
#include <stdarg.h>
#include <stdio.h>

#include <initializer_list>
#include <string>

#include "pkv_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(PKV_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// Tensor pointers must be 16-byte aligned (NULLs are reported elsewhere).
int check_align(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs)
    if (p && misaligned(p)) return fail(PKV_E_ALIGN, "tensor pointer %p is not 16-byte aligned", p);
  return PKV_OK;
}

bool valid_dtype(int d) {
  return d == PKV_F32 || d == PKV_BF16 || d == PKV_FP8_E4M3 || d == PKV_INT8 || d == PKV_INT4;
}
// Formats of one byte or less carry per-(page, kv head) scales.
bool scaled_dtype(int d) { return d == PKV_FP8_E4M3 || d == PKV_INT8 || d == PKV_INT4; }

// Shared size checks for every entry point that reads the pools.
int check_pool_shape(int kv_dtype, int max_pages, int batch, int num_pages, int num_kv_heads,
                     int head_dim, int page_size) {
  if (!valid_dtype(kv_dtype)) return fail(PKV_E_DTYPE, "unknown kv dtype %d", kv_dtype);
  if (batch < 0) return fail(PKV_E_SHAPE, "batch %d < 0", batch);
  if (max_pages <= 0 || num_pages <= 0 || num_kv_heads <= 0)
    return fail(PKV_E_SHAPE, "max_pages_per_seq %d, num_pages %d, num_kv_heads %d must be > 0",
                max_pages, num_pages, num_kv_heads);
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_E_SHAPE, "head_dim %d not supported (64 or 128)", head_dim);
  if (kv_dtype == PKV_INT4 && head_dim != 128)
    return fail(PKV_E_SHAPE, "int4 cache: head_dim %d not supported (128)", head_dim);
  const int tb = pkv::v_block_tokens(kv_dtype);
  if (page_size <= 0 || page_size > 1024 || page_size % tb)
    return fail(PKV_E_SHAPE, "page_size %d must be a positive multiple of %d and <= 1024", page_size, tb);
  return PKV_OK;
}

int check_decode(const void* q, int q_dtype, const void* k_pool, const void* v_pool, int kv_dtype,
                 const int32_t* block_tables, int max_pages, const int32_t* seq_lens, int batch,
                 int num_pages, int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                 int partition_tokens, const void* out, int out_dtype, const void* workspace,
                 size_t workspace_bytes, bool static_ws) {
  if (batch > 0 && (!q || !k_pool || !v_pool || !block_tables || !seq_lens || !out))
    return fail(PKV_E_NULL, "a required pointer is NULL");
  if (batch > 0 && !static_ws && !workspace) return fail(PKV_E_NULL, "workspace is NULL");
  int rc = check_pool_shape(kv_dtype, max_pages, batch, num_pages, num_kv_heads, head_dim, page_size);
  if (rc) return rc;
  if (batch > 0 && (rc = check_align({q, k_pool, v_pool, out, static_ws ? nullptr : workspace}))) return rc;
  const int want_q = kv_dtype == PKV_F32 ? PKV_F32 : PKV_BF16;
  if (q_dtype != want_q)
    return fail(PKV_E_DTYPE, "q dtype %d unsupported with kv dtype %d (need %d)", q_dtype, kv_dtype, want_q);
  if (out_dtype != PKV_F32 && !(out_dtype == PKV_BF16 && kv_dtype != PKV_F32))
    return fail(PKV_E_DTYPE, "out dtype %d unsupported with kv dtype %d", out_dtype, kv_dtype);
  if (num_q_heads <= 0 || num_q_heads % num_kv_heads)
    return fail(PKV_E_SHAPE, "num_q_heads %d not a positive multiple of num_kv_heads %d", num_q_heads,
                num_kv_heads);
  const int G = num_q_heads / num_kv_heads;
  if (G > 16) return fail(PKV_E_SHAPE, "group size %d > 16", G);
  const int tb = pkv::v_block_tokens(kv_dtype);
  if (partition_tokens < 0 || partition_tokens % tb)
    return fail(PKV_E_SHAPE, "partition_tokens %d must be 0 or a positive multiple of %d", partition_tokens, tb);
  if (batch > 0) {
    const size_t need = pkv_decode_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim);
    if (need == 0) return fail(PKV_E_HIP, "could not query the current HIP device");
    if (static_ws && need > pkv::kStaticScratchBytes)
      return fail(PKV_E_WORKSPACE, "this shape needs %zu bytes of workspace; the static scratch holds %zu", need,
                  pkv::kStaticScratchBytes);
    if (!static_ws && workspace_bytes < need)
      return fail(PKV_E_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, need);
  }
  return PKV_OK;
}

int run_decode(const void* q, int q_dtype, const void* k_pool, const void* v_pool, int kv_dtype,
               const float* k_scales, const float* v_scales, const int32_t* block_tables,
               int max_pages, const int32_t* seq_lens, int batch, int num_pages, int num_q_heads,
               int num_kv_heads, int head_dim, int page_size, float scale, int partition_tokens,
               void* out, int out_dtype, void* workspace, size_t workspace_bytes, void* stream,
               const void* k_new = nullptr, const void* v_new = nullptr, bool static_ws = false,
               int new_quant_dtype = -1) {
  int rc = check_decode(q, q_dtype, k_pool, v_pool, kv_dtype, block_tables, max_pages, seq_lens, batch,
                        num_pages, num_q_heads, num_kv_heads, head_dim, page_size, partition_tokens,
                        out, out_dtype, workspace, workspace_bytes, static_ws);
  if (rc) return rc;
  if (batch == 0) return PKV_OK;
  if (static_ws) {      // every check has passed: only now look up this device's scratch array
    hipError_t e = pkv::static_scratch(&workspace);
    if (e != hipSuccess) return hip_fail(e, "static scratch lookup");
  }
  pkv::DecodeArgs a;
  a.q = q;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.out = out;
  a.partials = static_cast<float*>(workspace);
  a.descs = reinterpret_cast<int4*>(static_cast<char*>(workspace) +
                                      pkv::partials_bytes(pkv::device_cu_count(), num_q_heads / num_kv_heads,
                                                          head_dim));
  a.qdescs = a.descs + (size_t)batch * num_kv_heads;
  a.kvt = kv_dtype;
  a.out_bf16 = out_dtype == PKV_BF16;
  a.batch = batch;
  a.max_pages = max_pages;
  a.num_pages = num_pages;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.page_size = page_size;
  // Default range granularity: one decode step (the V block), the finest split.
  a.partition_tokens = partition_tokens ? partition_tokens : pkv::v_block_tokens(kv_dtype);
  a.scale = scale;
  a.new_quant = new_quant_dtype >= 0;
  a.new_bf16 = new_quant_dtype == PKV_BF16;
  hipError_t e = pkv::launch_decode(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return PKV_OK;
}

int append_quant(int kv_dtype, const void* k_new, const void* v_new, pkv_dtype new_dtype,
                 const int32_t* block_tables, int max_pages_per_seq, const int32_t* seq_lens, int batch,
                 void* k_pool, void* v_pool, float* k_scales, float* v_scales, int num_pages, int num_kv_heads,
                 int head_dim, int page_size, void* stream) {
  g_last_error.clear();
  if (batch > 0 && (!k_new || !v_new || !block_tables || !seq_lens || !k_pool || !v_pool || !k_scales ||
                    !v_scales))
    return fail(PKV_E_NULL, "a required pointer is NULL");
  int rc = check_pool_shape(kv_dtype, max_pages_per_seq, batch, num_pages, num_kv_heads, head_dim, page_size);
  if (rc) return rc;
  if (new_dtype != PKV_BF16 && new_dtype != PKV_F32)
    return fail(PKV_E_DTYPE, "new-row dtype %d unsupported (bf16 or f32)", new_dtype);
  if (batch == 0) return PKV_OK;
  if ((rc = check_align({k_new, v_new, k_pool, v_pool}))) return rc;
  pkv::AppendQuantArgs a{k_new,  v_new,    kv_dtype, new_dtype == PKV_BF16, block_tables, seq_lens,
                         k_pool, v_pool,   k_scales, v_scales,              batch,        max_pages_per_seq,
                         num_pages, num_kv_heads, head_dim, page_size};
  hipError_t e = pkv::launch_append_quant(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "quantising append launch");
  return PKV_OK;
}

// Append + decode (the step entries): step-specific checks, then run_decode.
int run_step(const void* q, pkv_dtype q_dtype, const void* k_new, const void* v_new, void* k_pool, void* v_pool,
             pkv_dtype kv_dtype, const float* k_scales, const float* v_scales, const int32_t* block_tables,
             int max_pages_per_seq, const int32_t* seq_lens, int batch, int num_pages, int num_q_heads,
             int num_kv_heads, int head_dim, int page_size, float scale, int partition_tokens, void* out,
             pkv_dtype out_dtype, void* workspace, size_t workspace_bytes, void* stream, bool static_ws) {
  if (batch > 0 && (!k_new || !v_new)) return fail(PKV_E_NULL, "k_new / v_new are NULL");
  if (batch > 0) {
    const int rc = check_align({k_new, v_new});
    if (rc) return rc;
  }
  if (scaled_dtype(kv_dtype)) {
    if (batch > 0 && (!k_scales || !v_scales)) return fail(PKV_E_NULL, "fp8 / int8 / int4 scales are NULL");
  } else {
    k_scales = v_scales = nullptr;
  }
  return run_decode(q, q_dtype, k_pool, v_pool, kv_dtype, k_scales, v_scales, block_tables, max_pages_per_seq,
                    seq_lens, batch, num_pages, num_q_heads, num_kv_heads, head_dim, page_size, scale,
                    partition_tokens, out, out_dtype, workspace, workspace_bytes, stream, k_new, v_new, static_ws);
}

// Chunked prefill (bf16 or fp8 cache): checks, then the launch.
int run_prefill(const void* q, pkv_dtype q_dtype, const int32_t* cu_q, int total_q, const void* k_pool,
                const void* v_pool, pkv_dtype kv_dtype, const float* k_scales, const float* v_scales,
                const int32_t* block_tables, int max_pages_per_seq, const int32_t* seq_lens, int batch, int num_pages,
                int num_q_heads, int num_kv_heads, int head_dim, int page_size, float scale, void* out,
                pkv_dtype out_dtype, void* stream) {
  if (total_q < 0) return fail(PKV_E_SHAPE, "total_q %d < 0", total_q);
  if (batch > 0 && (!cu_q || !block_tables || !seq_lens || !k_pool || !v_pool))
    return fail(PKV_E_NULL, "a required pointer is NULL");
  if (batch > 0 && total_q > 0 && (!q || !out)) return fail(PKV_E_NULL, "q / out is NULL");
  int rc = check_pool_shape(kv_dtype, max_pages_per_seq, batch, num_pages, num_kv_heads, head_dim, page_size);
  if (rc) return rc;
  if (q_dtype != PKV_BF16) return fail(PKV_E_DTYPE, "chunked prefill takes bf16 queries (q dtype %d)", q_dtype);
  if (out_dtype != PKV_BF16 && out_dtype != PKV_F32)
    return fail(PKV_E_DTYPE, "out dtype %d not supported (bf16 or fp32)", out_dtype);
  if (num_q_heads <= 0 || num_q_heads % num_kv_heads)
    return fail(PKV_E_SHAPE, "num_q_heads %d is not a positive multiple of num_kv_heads %d", num_q_heads,
                num_kv_heads);
  if (num_q_heads / num_kv_heads > 128)
    return fail(PKV_E_SHAPE, "group size %d > 128", num_q_heads / num_kv_heads);
  const int eb = kv_dtype == PKV_FP8_E4M3 ? 1 : 2;
  if ((uint64_t)num_kv_heads * page_size * head_dim * eb >= (1ull << 32))
    return fail(PKV_E_SHAPE, "a page of all kv heads (%d x %d x %d x %d bytes) must be below 4 GiB", num_kv_heads,
                page_size, head_dim, eb);
  if (batch == 0 || total_q == 0) return PKV_OK;
  if ((rc = check_align({q, k_pool, v_pool, out}))) return rc;
  pkv::PrefillArgs a{q,        cu_q,     total_q,      k_pool,   v_pool,    (int)kv_dtype, k_scales,
                     v_scales, block_tables, seq_lens, out,      out_dtype == PKV_BF16, batch, max_pages_per_seq,
                     num_pages, num_q_heads, num_kv_heads, head_dim, page_size, scale};
  hipError_t e = pkv::launch_prefill(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "prefill launch");
  return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_version(void) { return 100; }

const char* pkv_strerror(int code) {
  switch (code) {
    case PKV_OK: return "success";
    case PKV_E_NULL: return "null pointer argument";
    case PKV_E_SHAPE: return "unsupported or inconsistent sizes";
    case PKV_E_DTYPE: return "unsupported dtype combination";
    case PKV_E_WORKSPACE: return "workspace missing or too small";
    case PKV_E_HIP: return "HIP runtime error";
    case PKV_E_ALIGN: return "tensor pointer not 16-byte aligned";
    default: return "unknown error code";
  }
}

const char* pkv_last_error(void) { return g_last_error.c_str(); }

size_t pkv_decode_workspace_bytes(int batch, int num_q_heads, int num_kv_heads, int head_dim) {
  if (batch < 0 || num_kv_heads <= 0 || num_q_heads <= 0 || num_q_heads % num_kv_heads || head_dim <= 0)
    return 0;
  const int cus = pkv::device_cu_count();
  if (cus <= 0) return 0;
  // two partial slots (first and last range) per resident wave, then the
  // merge descriptors and the quantising step's records (16 bytes each per (b, g))
  return pkv::partials_bytes(cus, num_q_heads / num_kv_heads, head_dim) +
         (size_t)batch * (size_t)num_kv_heads * 32;
}

int pkv_kv_append(const void* k_new, const void* v_new, pkv_dtype kv_dtype, const int32_t* block_tables,
                  int max_pages_per_seq, const int32_t* seq_lens, int batch, void* k_pool, void* v_pool,
                  int num_pages, int num_kv_heads, int head_dim, int page_size, void* stream) {
  g_last_error.clear();
  if (batch > 0 && (!k_new || !v_new || !block_tables || !seq_lens || !k_pool || !v_pool))
    return fail(PKV_E_NULL, "a required pointer is NULL");
  int rc = check_pool_shape(kv_dtype, max_pages_per_seq, batch, num_pages, num_kv_heads, head_dim, page_size);
  if (rc) return rc;
  if (batch == 0) return PKV_OK;
  if ((rc = check_align({k_new, v_new, k_pool, v_pool}))) return rc;
  pkv::AppendArgs a{k_new, v_new, block_tables, seq_lens, k_pool, v_pool, (int)kv_dtype, batch,
                    max_pages_per_seq, num_pages, num_kv_heads, head_dim, page_size};
  hipError_t e = pkv::launch_append(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "append launch");
  return PKV_OK;
}

int pkv_kv_append_chunk(const void* k_new, const void* v_new, pkv_dtype kv_dtype, const int32_t* cu_new,
                        int total_new, const int32_t* block_tables, int max_pages_per_seq, const int32_t* seq_lens,
                        int batch, void* k_pool, void* v_pool, int num_pages, int num_kv_heads, int head_dim,
                        int page_size, void* stream) {
  g_last_error.clear();
  if (total_new < 0) return fail(PKV_E_SHAPE, "total_new %d < 0", total_new);
  if (batch > 0 && (!cu_new || !block_tables || !seq_lens || !k_pool || !v_pool))
    return fail(PKV_E_NULL, "a required pointer is NULL");
  if (batch > 0 && total_new > 0 && (!k_new || !v_new)) return fail(PKV_E_NULL, "k_new / v_new is NULL");
  int rc = check_pool_shape(kv_dtype, max_pages_per_seq, batch, num_pages, num_kv_heads, head_dim, page_size);
  if (rc) return rc;
  if (batch == 0 || total_new == 0) return PKV_OK;
  if ((rc = check_align({k_new, v_new, k_pool, v_pool}))) return rc;
  pkv::AppendChunkArgs a{k_new, v_new, cu_new, total_new, block_tables, seq_lens, k_pool, v_pool,
                         (int)kv_dtype, batch, max_pages_per_seq, num_pages, num_kv_heads, head_dim, page_size};
  hipError_t e = pkv::launch_append_chunk(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "chunk append launch");
  return PKV_OK;
}

int pkv_paged_prefill(const void* q, pkv_dtype q_dtype, const int32_t* cu_q, int total_q, const void* k_pool,
                      const void* v_pool, pkv_dtype kv_dtype, const int32_t* block_tables, int max_pages_per_seq,
                      const int32_t* seq_lens, int batch, int num_pages, int num_q_heads, int num_kv_heads,
                      int head_dim, int page_size, float scale, void* out, pkv_dtype out_dtype, void* stream) {
  g_last_error.clear();
  if (kv_dtype != PKV_BF16)
    return fail(PKV_E_DTYPE, "chunked prefill reads a bf16 cache here (kv dtype %d; fp8: pkv_paged_prefill_fp8)",
                kv_dtype);
  return run_prefill(q, q_dtype, cu_q, total_q, k_pool, v_pool, PKV_BF16, nullptr, nullptr, block_tables,
                     max_pages_per_seq, seq_lens, batch, num_pages, num_q_heads, num_kv_heads, head_dim, page_size,
                     scale, out, out_dtype, stream);
}

int pkv_paged_prefill_fp8(const void* q, pkv_dtype q_dtype, const int32_t* cu_q, int total_q, const void* k_pool,
                          const void* v_pool, const float* k_scales, const float* v_scales,
                          const int32_t* block_tables, int max_pages_per_seq, const int32_t* seq_lens, int batch,
                          int num_pages, int num_q_heads, int num_kv_heads, int head_dim, int page_size, float scale,
                          void* out, pkv_dtype out_dtype, void* stream) {
  g_last_error.clear();
  if (batch > 0 && total_q > 0 && (!k_scales || !v_scales)) return fail(PKV_E_NULL, "fp8 scales are NULL");
  return run_prefill(q, q_dtype, cu_q, total_q, k_pool, v_pool, PKV_FP8_E4M3, k_scales, v_scales, block_tables,
                     max_pages_per_seq, seq_lens, batch, num_pages, num_q_heads, num_kv_heads, head_dim, page_size,
                     scale, out, out_dtype, stream);
}

namespace {
int check_pages(const void* seq_lens, int batch, const void* block_tables, int max_pages, int page_size,
                const void* free_pages, const void* free_count, int capacity) {
  if (batch < 0) return fail(PKV_E_SHAPE, "batch %d < 0", batch);
  if (max_pages <= 0 || page_size <= 0 || capacity <= 0)
    return fail(PKV_E_SHAPE, "max_pages_per_seq %d, page_size %d, capacity %d must be > 0", max_pages, page_size,
                capacity);
  if (!free_pages || !free_count) return fail(PKV_E_NULL, "free_pages / free_count is NULL");
  if (batch > 0 && (!seq_lens || !block_tables)) return fail(PKV_E_NULL, "seq_lens / block_tables is NULL");
  return PKV_OK;
}
}  // namespace

int pkv_alloc_pages(const int32_t* seq_lens, int batch, int32_t* block_tables, int max_pages_per_seq, int page_size,
                    const int32_t* free_pages, int32_t* free_count, int capacity, void* stream) {
  g_last_error.clear();
  int rc = check_pages(seq_lens, batch, block_tables, max_pages_per_seq, page_size, free_pages, free_count, capacity);
  if (rc) return rc;
  if (batch == 0) return PKV_OK;
  pkv::PageArgs a{nullptr, seq_lens, block_tables, const_cast<int32_t*>(free_pages), free_count, batch,
                  max_pages_per_seq, page_size, 0, capacity};
  hipError_t e = pkv::launch_alloc_pages(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "page allocation launch");
  return PKV_OK;
}

int pkv_release_pages(const int32_t* release, const int32_t* seq_lens, int batch, int32_t* block_tables,
                      int max_pages_per_seq, int page_size, int num_pages, int32_t* free_pages, int32_t* free_count,
                      int capacity, void* stream) {
  g_last_error.clear();
  int rc = check_pages(seq_lens, batch, block_tables, max_pages_per_seq, page_size, free_pages, free_count, capacity);
  if (rc) return rc;
  if (num_pages <= 0) return fail(PKV_E_SHAPE, "num_pages %d must be > 0", num_pages);
  if (batch > 0 && !release) return fail(PKV_E_NULL, "release is NULL");
  if (batch == 0) return PKV_OK;
  pkv::PageArgs a{release, seq_lens, block_tables, free_pages, free_count, batch, max_pages_per_seq, page_size,
                  num_pages, capacity};
  hipError_t e = pkv::launch_release_pages(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "page release launch");
  return PKV_OK;
}

int pkv_kv_append_fp8(const void* k_new, const void* v_new, pkv_dtype new_dtype, const int32_t* block_tables,
                      int max_pages_per_seq, const int32_t* seq_lens, int batch, void* k_pool, void* v_pool,
                      float* k_scales, float* v_scales, int num_pages, int num_kv_heads, int head_dim,
                      int page_size, void* stream) {
  return append_quant(PKV_FP8_E4M3, k_new, v_new, new_dtype, block_tables, max_pages_per_seq, seq_lens, batch,
                      k_pool, v_pool, k_scales, v_scales, num_pages, num_kv_heads, head_dim, page_size, stream);
}

int pkv_kv_append_int8(const void* k_new, const void* v_new, pkv_dtype new_dtype, const int32_t* block_tables,
                       int max_pages_per_seq, const int32_t* seq_lens, int batch, void* k_pool, void* v_pool,
                       float* k_scales, float* v_scales, int num_pages, int num_kv_heads, int head_dim,
                       int page_size, void* stream) {
  return append_quant(PKV_INT8, k_new, v_new, new_dtype, block_tables, max_pages_per_seq, seq_lens, batch,
                      k_pool, v_pool, k_scales, v_scales, num_pages, num_kv_heads, head_dim, page_size, stream);
}

int pkv_kv_append_int4(const void* k_new, const void* v_new, pkv_dtype new_dtype, const int32_t* block_tables,
                       int max_pages_per_seq, const int32_t* seq_lens, int batch, void* k_pool, void* v_pool,
                       float* k_scales, float* v_scales, int num_pages, int num_kv_heads, int head_dim,
                       int page_size, void* stream) {
  return append_quant(PKV_INT4, k_new, v_new, new_dtype, block_tables, max_pages_per_seq, seq_lens, batch,
                      k_pool, v_pool, k_scales, v_scales, num_pages, num_kv_heads, head_dim, page_size, stream);
}

int pkv_paged_attn_decode(const void* q, pkv_dtype q_dtype, const void* k_pool, const void* v_pool,
                          pkv_dtype kv_dtype, const int32_t* block_tables, int max_pages_per_seq,
                          const int32_t* seq_lens, int batch, int num_pages, int num_q_heads,
                          int num_kv_heads, int head_dim, int page_size, float scale,
                          int partition_tokens, void* out, pkv_dtype out_dtype, void* workspace,
                          size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (scaled_dtype(kv_dtype))
    return fail(PKV_E_DTYPE, "fp8 / int8 / int4 cache: use the _fp8 / _int8 / _int4 entry (they carry the scales)");
  return run_decode(q, q_dtype, k_pool, v_pool, kv_dtype, nullptr, nullptr, block_tables, max_pages_per_seq,
                    seq_lens, batch, num_pages, num_q_heads, num_kv_heads, head_dim, page_size, scale,
                    partition_tokens, out, out_dtype, workspace, workspace_bytes, stream);
}

int pkv_paged_attn_decode_fp8(const void* q, pkv_dtype q_dtype, const void* k_pool, const void* v_pool,
                              const float* k_scales, const float* v_scales, const int32_t* block_tables,
                              int max_pages_per_seq, const int32_t* seq_lens, int batch, int num_pages,
                              int num_q_heads, int num_kv_heads, int head_dim, int page_size, float scale,
                              int partition_tokens, void* out, pkv_dtype out_dtype, void* workspace,
                              size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (batch > 0 && (!k_scales || !v_scales)) return fail(PKV_E_NULL, "fp8 scales are NULL");
  return run_decode(q, q_dtype, k_pool, v_pool, PKV_FP8_E4M3, k_scales, v_scales, block_tables,
                    max_pages_per_seq, seq_lens, batch, num_pages, num_q_heads, num_kv_heads, head_dim,
                    page_size, scale, partition_tokens, out, out_dtype, workspace, workspace_bytes, stream);
}

int pkv_paged_attn_decode_int4(const void* q, pkv_dtype q_dtype, const void* k_pool, const void* v_pool,
                               const float* k_scales, const float* v_scales, const int32_t* block_tables,
                               int max_pages_per_seq, const int32_t* seq_lens, int batch, int num_pages,
                               int num_q_heads, int num_kv_heads, int head_dim, int page_size, float scale,
                               int partition_tokens, void* out, pkv_dtype out_dtype, void* workspace,
                               size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (batch > 0 && (!k_scales || !v_scales)) return fail(PKV_E_NULL, "int4 scales are NULL");
  return run_decode(q, q_dtype, k_pool, v_pool, PKV_INT4, k_scales, v_scales, block_tables, max_pages_per_seq,
                    seq_lens, batch, num_pages, num_q_heads, num_kv_heads, head_dim, page_size, scale,
                    partition_tokens, out, out_dtype, workspace, workspace_bytes, stream);
}

int pkv_paged_attn_decode_int8(const void* q, pkv_dtype q_dtype, const void* k_pool, const void* v_pool,
                               const float* k_scales, const float* v_scales, const int32_t* block_tables,
                               int max_pages_per_seq, const int32_t* seq_lens, int batch, int num_pages,
                               int num_q_heads, int num_kv_heads, int head_dim, int page_size, float scale,
                               int partition_tokens, void* out, pkv_dtype out_dtype, void* workspace,
                               size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (batch > 0 && (!k_scales || !v_scales)) return fail(PKV_E_NULL, "int8 scales are NULL");
  return run_decode(q, q_dtype, k_pool, v_pool, PKV_INT8, k_scales, v_scales, block_tables, max_pages_per_seq,
                    seq_lens, batch, num_pages, num_q_heads, num_kv_heads, head_dim, page_size, scale,
                    partition_tokens, out, out_dtype, workspace, workspace_bytes, stream);
}

int pkv_decode_step(const void* q, pkv_dtype q_dtype, const void* k_new, const void* v_new, void* k_pool,
                    void* v_pool, pkv_dtype kv_dtype, const float* k_scales, const float* v_scales,
                    const int32_t* block_tables, int max_pages_per_seq, const int32_t* seq_lens, int batch,
                    int num_pages, int num_q_heads, int num_kv_heads, int head_dim, int page_size, float scale,
                    int partition_tokens, void* out, pkv_dtype out_dtype, void* workspace,
                    size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  return run_step(q, q_dtype, k_new, v_new, k_pool, v_pool, kv_dtype, k_scales, v_scales, block_tables,
                  max_pages_per_seq, seq_lens, batch, num_pages, num_q_heads, num_kv_heads, head_dim, page_size,
                  scale, partition_tokens, out, out_dtype, workspace, workspace_bytes, stream, false);
}

int pkv_decode_step_noalloc(const void* q, pkv_dtype q_dtype, const void* k_new, const void* v_new, void* k_pool,
                            void* v_pool, pkv_dtype kv_dtype, const float* k_scales, const float* v_scales,
                            const int32_t* block_tables, int max_pages_per_seq, const int32_t* seq_lens, int batch,
                            int num_pages, int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                            float scale, int partition_tokens, void* out, pkv_dtype out_dtype, void* stream) {
  g_last_error.clear();
  return run_step(q, q_dtype, k_new, v_new, k_pool, v_pool, kv_dtype, k_scales, v_scales, block_tables,
                  max_pages_per_seq, seq_lens, batch, num_pages, num_q_heads, num_kv_heads, head_dim, page_size,
                  scale, partition_tokens, out, out_dtype, nullptr, 0, stream, true);
}

int pkv_decode_step_quant(const void* q, pkv_dtype q_dtype, const void* k_new, const void* v_new,
                          pkv_dtype new_dtype, void* k_pool, void* v_pool, pkv_dtype kv_dtype, float* k_scales,
                          float* v_scales, const int32_t* block_tables, int max_pages_per_seq,
                          const int32_t* seq_lens, int batch, int num_pages, int num_q_heads, int num_kv_heads,
                          int head_dim, int page_size, float scale, int partition_tokens, void* out,
                          pkv_dtype out_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (!scaled_dtype(kv_dtype))
    return fail(PKV_E_DTYPE, "quantising step: kv dtype %d is not fp8, int8 or int4", kv_dtype);
  if (new_dtype != PKV_BF16 && new_dtype != PKV_F32)
    return fail(PKV_E_DTYPE, "new-row dtype %d unsupported (bf16 or f32)", new_dtype);
  if (batch > 0 && (!k_new || !v_new)) return fail(PKV_E_NULL, "k_new / v_new are NULL");
  if (batch > 0 && (!k_scales || !v_scales)) return fail(PKV_E_NULL, "fp8 / int8 / int4 scales are NULL");
  if (batch > 0) {
    const int rc = check_align({k_new, v_new});
    if (rc) return rc;
  }
  return run_decode(q, q_dtype, k_pool, v_pool, kv_dtype, k_scales, v_scales, block_tables, max_pages_per_seq,
                    seq_lens, batch, num_pages, num_q_heads, num_kv_heads, head_dim, page_size, scale,
                    partition_tokens, out, out_dtype, workspace, workspace_bytes, stream, k_new, v_new, false,
                    (int)new_dtype);
}

int pkv_debug_gather(const void* k_pool, const void* v_pool, pkv_dtype kv_dtype, const int32_t* block_tables,
                     int max_pages_per_seq, const int32_t* seq_lens, int batch, int num_pages,
                     int num_kv_heads, int head_dim, int page_size, void* k_out, void* v_out, void* stream) {
  g_last_error.clear();
  if (batch > 0 && (!k_pool || !v_pool || !block_tables || !seq_lens || !k_out || !v_out))
    return fail(PKV_E_NULL, "a required pointer is NULL");
  int rc = check_pool_shape(kv_dtype, max_pages_per_seq, batch, num_pages, num_kv_heads, head_dim, page_size);
  if (rc) return rc;
  if (batch == 0) return PKV_OK;
  if ((rc = check_align({k_pool, v_pool, k_out, v_out}))) return rc;
  pkv::GatherArgs a{k_pool, v_pool, block_tables, seq_lens, k_out, v_out, (int)kv_dtype, batch,
                    max_pages_per_seq, num_pages, num_kv_heads, head_dim, page_size};
  hipError_t e = pkv::launch_gather(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gather launch");
  return PKV_OK;
}

int pkv_debug_read_probe(const void* buf, size_t bytes, uint32_t* out, void* stream) {
  g_last_error.clear();
  if (bytes == 0) return PKV_OK;
  if (!buf || !out) return fail(PKV_E_NULL, "a required pointer is NULL");
  if (bytes % 16) return fail(PKV_E_SHAPE, "bytes %zu not a multiple of 16", bytes);
  int rc = check_align({buf});
  if (rc) return rc;
  hipError_t e = pkv::launch_read_probe(buf, bytes, out, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "read probe launch");
  return PKV_OK;
}

}  // extern "C"
