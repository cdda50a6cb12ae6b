/*
 * pkv.h - paged KV-cache decode attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libpkv.so.  Every pointer argument is DEVICE memory owned by the
 * caller unless stated otherwise; the library allocates and frees nothing.
 * Every tensor pointer (q, out, k_new, v_new, k_pool, v_pool, workspace,
 * k_out, v_out) must be 16-byte aligned, as the kernels move 16-byte groups;
 * a misaligned one is rejected with PKV_E_ALIGN.  int32 / fp32 arrays
 * (block_tables, seq_lens, scales) need only their natural alignment.
 * Calls are asynchronous and ordered on the given HIP stream (`stream` is a
 * hipStream_t passed as void*, NULL = the null stream); they never synchronise
 * and never read device memory from the host.  Pointers must stay valid until
 * the stream work has completed.  Calls on different streams may run
 * concurrently provided they do not write the same memory.
 *
 * Source of the operations.  The first page (TensorRT-LLM concept page,
 * "key mechanisms" section) stores each sequence's K/V cache in fixed-size
 * pages of, e.g., 64 or 128 tokens drawn from a shared pool, maps logical
 * token positions to physical pages through a page table, and allocates new
 * pages as a sequence grows.  Its "compile-time graph optimization" section
 * puts a page-table lookup in front of every cache read and write, and its
 * "runtime execution model" section has each decode iteration's attention
 * read and update those pages, with the host passing the page tables in for
 * every iteration.  The attention computed is single-query softmax attention
 * softmax(scale * q K^T) V per query head over the tokens of its sequence.
 *
 * ---------------------------------------------------------------------------
 * Shapes and notation
 *   B   batch (sequences)          Hq  query heads     Hkv  kv heads
 *   G = Hq / Hkv (query heads per kv head; query head h reads kv head h / G)
 *   D   head dimension (64 or 128)  P   page size in tokens
 *   NP  pages in the pool           MP  block-table width (pages per sequence)
 *   L_b = seq_lens[b]
 *
 * Tensors (row-major, element types given by the dtype arguments)
 *   q            [B][Hq][D]
 *   out          [B][Hq][D]
 *   k_new, v_new [B][Hkv][D]
 *   block_tables int32 [B][MP]; entry j of row b is the physical page holding
 *                tokens [j*P, (j+1)*P) of sequence b.  Entries at or past
 *                ceil(L_b / P) are never read (may be -1).
 *   seq_lens     int32 [B]; number of tokens of sequence b in the cache,
 *                INCLUDING the token appended this step.  0 is allowed.
 *   k_scales, v_scales  fp32 [NP][Hkv], fp8, int8 and int4 caches only:
 *                stored value times scale is the real value, one scale per
 *                (page, kv head).  int8 elements are two's complement bytes
 *                in [-127, 127]; int4 elements are two's complement nibbles in
 *                [-7, 7], two per byte, element 2i in the low nibble of byte i
 *                (in the pools by element index within a chunk, and in k_new /
 *                v_new rows, which are then D / 2 bytes).
 *   k_pool, v_pool      NP * Hkv chunks, one per (page, kv head), each holding
 *                P * D elements; chunk (pg, g) starts at element
 *                (pg * Hkv + g) * P * D.
 *
 * Layout inside one chunk.  Let E = 128 / (element bits) (fp32 4, bf16 8,
 * fp8 and int8 16, int4 32) and TB = 4 * E.  For token slot j in [0, P) and dimension d:
 *   K (j, d) at element ((d / E) * P + j) * E + d % E
 *   V (j, d) at element blk * TB * D + (c * D + d) * E + e, where
 *            blk = j / TB, r = j % TB, c = (r % 16) / 4, e = 4 * (r / 16) + r % 4
 * i.e. each 16-byte group holds E consecutive dimensions of one token for K,
 * and E tokens of one dimension for V, arranged so that a 64-lane wavefront
 * reading one 16-byte group per lane receives matrix-core operand fragments
 * directly.  P must be a multiple of TB (fp32: 16, bf16: 32, fp8 and int8: 64,
 * int4: 128); an int4 cache needs D = 128.
 * ---------------------------------------------------------------------------
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PKV_F32 = 0, PKV_BF16 = 1, PKV_FP8_E4M3 = 2, PKV_INT8 = 3, PKV_INT4 = 4 } pkv_dtype;

/* Return codes.  0 is success; every failure is negative and leaves all device
 * memory untouched (arguments are checked before anything is launched). */
enum {
  PKV_OK = 0,
  PKV_E_NULL = -1,      /* a required pointer is NULL                       */
  PKV_E_SHAPE = -2,     /* unsupported or inconsistent sizes                 */
  PKV_E_DTYPE = -3,     /* unsupported dtype combination                     */
  PKV_E_WORKSPACE = -4, /* workspace NULL or smaller than required           */
  PKV_E_HIP = -5,       /* a HIP runtime call or kernel launch failed        */
  PKV_E_ALIGN = -6      /* a tensor pointer is not 16-byte aligned           */
};

/* kv_append - write this step's new K/V token of every sequence into its page.
 *
 * The "paged store" of the first page ("key mechanisms"), preceded by the
 * page-table lookup of its "compile-time graph optimization" section: for each
 * b with L_b >= 1, token position t = L_b - 1 goes to slot t % P of page
 * block_tables[b][t / P]; k_new[b][g][:] and v_new[b][g][:] are copied there
 * bit for bit for every kv head g.  Sequences with L_b <= 0 are skipped.
 *
 * kv_dtype: element type of k_new/v_new and of the pools (any pkv_dtype; fp8
 *   and int8 bytes are copied as given, already quantised with the page's scale).
 * Writes only the addressed slots of k_pool/v_pool.  Two sequences must not
 * address the same slot in one call (the writes would race).  A page id
 * outside [0, num_pages), or t / P >= max_pages_per_seq, skips that sequence.
 * Errors: PKV_E_NULL, PKV_E_SHAPE (sizes <= 0, D not 64/128, P not a multiple
 * of TB or > 1024), PKV_E_DTYPE, PKV_E_ALIGN, PKV_E_HIP. */
int pkv_kv_append(const void* k_new, const void* v_new, pkv_dtype kv_dtype,
                  const int32_t* block_tables, int max_pages_per_seq,
                  const int32_t* seq_lens, int batch,
                  void* k_pool, void* v_pool, int num_pages,
                  int num_kv_heads, int head_dim, int page_size, void* stream);

/* kv_append_fp8 - append into an fp8 e4m3 cache, quantising on write with
 * dynamic per-(page, kv head) scales.
 *
 * The concept page's "compile-time graph optimization" section computes a
 * dynamic scaling factor where data enters FP8 arithmetic; the yololab page's
 * FP8 section gives FP8 as the way to halve memory bandwidth.  Here new K/V rows
 * enter the fp8 cache: for each b with L_b >= 1, token t = L_b - 1 goes to slot
 * j = t % P of page pg = block_tables[b][t / P], and for each kv head g, for K
 * and V separately, with x = the new row widened to fp32 and a = max |x|:
 *   j == 0 (first token of the page): s = a / 448 (1 if a == 0);
 *   j > 0, s0 = scales[pg][g]: s = s0 if a / s0 <= 464 (the row's largest
 *     element still rounds to +-448, no clipping); otherwise s = a / 448 and
 *     every earlier slot of the page is re-encoded as enc((dec(byte) * s0) / s);
 *   the new row is stored as enc(x / s); scales[pg][g] = s.
 * Each division and product is one fp32 operation rounded to nearest even;
 * enc is e4m3 round-to-nearest-even saturating at +-448; dec is exact.  So
 * the bytes and scales written are fully determined by the inputs.
 *
 * new_dtype: BF16 or F32 (k_new, v_new [B][Hkv][D]; finite values).
 * k_pool/v_pool: fp8 pools; k_scales/v_scales fp32 [NP][Hkv], read and written
 *   (a page's scale must be the one this function last wrote for it, or any
 *   positive scale that encodes the page's bytes, when j > 0).
 * Writes only the addressed page of each sequence (all its earlier slots when
 * its scale grows) and its two scales.  Two sequences must not append into the
 * same page in one call.  Sequences with L_b <= 0, t / P >= max_pages_per_seq or
 * a page id outside [0, num_pages) are skipped.
 * Errors: PKV_E_NULL, PKV_E_SHAPE (as pkv_kv_append with P a multiple of 64),
 * PKV_E_DTYPE (new_dtype), PKV_E_ALIGN, PKV_E_HIP. */
int pkv_kv_append_fp8(const void* k_new, const void* v_new, pkv_dtype new_dtype,
                      const int32_t* block_tables, int max_pages_per_seq,
                      const int32_t* seq_lens, int batch,
                      void* k_pool, void* v_pool, float* k_scales, float* v_scales,
                      int num_pages, int num_kv_heads, int head_dim, int page_size,
                      void* stream);

/* kv_append_int8 - pkv_kv_append_fp8 for a symmetric int8 cache.
 *
 * The solosoft.dev page ("TensorRT-LLM：NVIDIA 的開源最佳化 LLM 推論函式庫")
 * lists INT8 among the supported quantisation formats in its FAQ, and its
 * performance and memory figures give INT8 half the memory of FP16 and a
 * higher throughput; here INT8 is the cache format, with the same dynamic
 * per-(page, kv head)
 * scales as the fp8 append and QMAX = 127: the first token of a page sets
 * s = a / 127 (1 if a == 0); a later row keeps the scale while a / s0 <= 127.5
 * (its largest element rounds to 128 at most, clamped to 127: within half a
 * step), else s = a / 127 and earlier slots are re-encoded; enc(y) = y rounded
 * to the nearest integer (ties to even) and clamped to [-127, 127].
 * Same arguments, contract and errors as pkv_kv_append_fp8. */
int pkv_kv_append_int8(const void* k_new, const void* v_new, pkv_dtype new_dtype,
                       const int32_t* block_tables, int max_pages_per_seq,
                       const int32_t* seq_lens, int batch,
                       void* k_pool, void* v_pool, float* k_scales, float* v_scales,
                       int num_pages, int num_kv_heads, int head_dim, int page_size,
                       void* stream);

/* kv_append_int4 - pkv_kv_append_fp8 for a symmetric int4 cache: QMAX = 7,
 * a later row keeps the page scale while a / s0 <= 7.5, enc(y) = y rounded to
 * the nearest integer (ties to even) and clamped to [-7, 7], stored as a
 * nibble.  The same solosoft.dev FAQ and figures list INT4 beside INT8.
 * Same arguments, contract and errors as pkv_kv_append_fp8 (D = 128). */
int pkv_kv_append_int4(const void* k_new, const void* v_new, pkv_dtype new_dtype,
                       const int32_t* block_tables, int max_pages_per_seq,
                       const int32_t* seq_lens, int batch,
                       void* k_pool, void* v_pool, float* k_scales, float* v_scales,
                       int num_pages, int num_kv_heads, int head_dim, int page_size,
                       void* stream);

/* Bytes of scratch that pkv_paged_attn_decode / pkv_paged_attn_decode_fp8 need
 * for these sizes on the current HIP device (0 if the sizes are invalid).
 * The workspace holds split-KV partial results (per-head running max, sum and
 * unnormalised output of each partial range) followed by one 16-byte merge
 * descriptor per (sequence, kv head).  It needs no initialisation and its
 * contents after a call are unspecified.  Calls that share a workspace must not
 * overlap in time (issue them on one stream); a workspace sized for batch B
 * serves any call with batch <= B and the same head counts and head_dim. */
size_t pkv_decode_workspace_bytes(int batch, int num_q_heads, int num_kv_heads, int head_dim);

/* paged_attn_decode - one decode step of attention over the paged cache.
 *
 * For b in [0,B), h in [0,Hq), g = h / G, tokens t < L_b read through the
 * page table (see the header comment):
 *   out[b][h][:] = sum_t softmax_t(scale * q[b][h] . k_t) v_t     (0 if L_b = 0)
 * Each kv page chunk is read once per kv head and shared by its G query heads.
 * Long sequences are split into ranges processed in parallel and combined by
 * their log-sum-exp; partition_tokens chooses the range granularity: 0 lets
 * the library choose, otherwise a positive multiple of TB (e.g. 512 tokens).
 * Accumulation is fp32; the bf16 products take each probability as a pair of
 * bf16 values (about 16 significant bits); out is rounded to nearest-even
 * when bf16.
 *
 * Supported dtypes (q / kv / out): F32/F32/F32, BF16/BF16/BF16, BF16/BF16/F32.
 * Sizes: D in {64, 128}; 1 <= G <= 16 with Hq % Hkv == 0; P a multiple of TB
 * and <= 1024; batch >= 0 (batch 0 is a no-op).
 * Page ids used must lie in [0, num_pages) and L_b <= MP * P; a row whose
 * sequence breaks this gets NaN outputs (nothing outside the pools is read).
 * workspace: device memory of at least pkv_decode_workspace_bytes(...) bytes.
 * The call launches two kernels on the stream: the split kernel (which also
 * finishes every (sequence, kv head) that one wavefront covered entirely) and
 * a merge kernel for the pairs split over several wavefronts.
 * Writes out and workspace only. */
int pkv_paged_attn_decode(const void* q, pkv_dtype q_dtype,
                          const void* k_pool, const void* v_pool, pkv_dtype kv_dtype,
                          const int32_t* block_tables, int max_pages_per_seq,
                          const int32_t* seq_lens, int batch, int num_pages,
                          int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                          float scale, int partition_tokens,
                          void* out, pkv_dtype out_dtype,
                          void* workspace, size_t workspace_bytes, void* stream);

/* paged_attn_decode_fp8 - as pkv_paged_attn_decode for an fp8 e4m3 cache.
 *
 * The pools hold OCP fp8 e4m3 ("fn") bytes; real value = decoded byte times
 * k_scales / v_scales [page][kv head].  Following the first page ("key
 * mechanisms": FP8 data is widened to 16 bits before the matrix product and
 * accumulated wide), bytes are widened exactly in registers; the K scale is
 * folded into the logits and the V scale into the probabilities, which enter
 * the value product as a pair of bf16 each (a rounded high part and the
 * remainder, 16 significant bits together); accumulation is fp32.  q is
 * BF16; out is BF16 or F32.  Same sizes and errors as above, plus PKV_E_NULL
 * when a scale pointer is NULL. */
int pkv_paged_attn_decode_fp8(const void* q, pkv_dtype q_dtype,
                              const void* k_pool, const void* v_pool,
                              const float* k_scales, const float* v_scales,
                              const int32_t* block_tables, int max_pages_per_seq,
                              const int32_t* seq_lens, int batch, int num_pages,
                              int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                              float scale, int partition_tokens,
                              void* out, pkv_dtype out_dtype,
                              void* workspace, size_t workspace_bytes, void* stream);

/* paged_attn_decode_int8 - as pkv_paged_attn_decode_fp8 for a symmetric int8
 * cache: bytes are two's complement integers, real value = byte * scale.
 * K bytes widen to bf16 exactly (at most 8 significant bits) and the K scale
 * is folded into the logits; V bytes widen to fp16 as 1152 + b exactly, the
 * value products take each probability as one fp16 (11 significant bits,
 * p * 2^7), 1152 * (sum of the probabilities, as the products see them) is
 * taken back out of each output, and the V scale multiplies each tile's fp32
 * result; accumulation is fp32.  q is BF16; out is BF16 or F32.  Same sizes
 * and errors as pkv_paged_attn_decode_fp8. */
int pkv_paged_attn_decode_int8(const void* q, pkv_dtype q_dtype,
                               const void* k_pool, const void* v_pool,
                               const float* k_scales, const float* v_scales,
                               const int32_t* block_tables, int max_pages_per_seq,
                               const int32_t* seq_lens, int batch, int num_pages,
                               int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                               float scale, int partition_tokens,
                               void* out, pkv_dtype out_dtype,
                               void* workspace, size_t workspace_bytes, void* stream);

/* paged_attn_decode_int4 - as pkv_paged_attn_decode_fp8 for a symmetric int4
 * cache (D = 128, P a multiple of 128).  K codes n widen to bf16 as 136 + n
 * and V codes to fp16 as 1032 + n, exactly (integer bit patterns, no
 * conversion); 136 * (sum of q) is taken back out of each logit and 1032 *
 * (sum of the probabilities, as the products see them) out of each output.
 * The value products take each probability as one fp16 (11 significant bits,
 * p * 2^7 so that small weights stay in range) and apply the V scale to each
 * tile's fp32 result.  Same sizes and errors as the fp8 entry. */
int pkv_paged_attn_decode_int4(const void* q, pkv_dtype q_dtype,
                               const void* k_pool, const void* v_pool,
                               const float* k_scales, const float* v_scales,
                               const int32_t* block_tables, int max_pages_per_seq,
                               const int32_t* seq_lens, int batch, int num_pages,
                               int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                               float scale, int partition_tokens,
                               void* out, pkv_dtype out_dtype,
                               void* workspace, size_t workspace_bytes, void* stream);

/* decode_step - one whole decode iteration of the cache for one layer: the
 * append of pkv_kv_append followed by the attention of pkv_paged_attn_decode
 * (or of pkv_paged_attn_decode_fp8 / _int8 / _int4 for those cache types),
 * with no launch of its own for the append.
 *
 * The first page's "runtime execution model" has each iteration's attention
 * both update and read the cache pages.  Here the wavefront of the split
 * kernel that owns the tile holding token L_b - 1 of (b, g) takes
 * k_new[b][g] / v_new[b][g] straight into its registers in place of the
 * slot's old contents, and the merge kernel, which runs after it on the
 * stream, stores them into the page slot.  Results equal pkv_kv_append then decode with the same
 * seq_lens (the pool bytes exactly; out up to the rounding order).
 * k_scales / v_scales: required for FP8_E4M3, INT8 and INT4 (k_new / v_new are
 * then already quantised with that page's scale; int4 rows packed), ignored
 * otherwise.
 * Same sizes, dtypes, workspace and errors as the decode entry points, plus
 * PKV_E_NULL for a NULL k_new / v_new.  A sequence whose slot L_b - 1 lies on
 * a bad page id stores nothing and gets NaN rows. */
int pkv_decode_step(const void* q, pkv_dtype q_dtype, const void* k_new, const void* v_new,
                    void* k_pool, void* v_pool, pkv_dtype kv_dtype,
                    const float* k_scales, const float* v_scales,
                    const int32_t* block_tables, int max_pages_per_seq,
                    const int32_t* seq_lens, int batch, int num_pages,
                    int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                    float scale, int partition_tokens,
                    void* out, pkv_dtype out_dtype,
                    void* workspace, size_t workspace_bytes, void* stream);

/* decode_step_quant - one decode iteration of a quantised cache (fp8-e4m3,
 * int8 or int4) whose new rows arrive in bf16 or fp32: the quantising append
 * of pkv_kv_append_fp8 / _int8 / _int4 followed by the attention of
 * pkv_paged_attn_decode_fp8 / _int8 / _int4, with no launch of its own for
 * the append.
 *
 * The first page's "compile-time graph optimization" section computes a
 * dynamic scaling factor where data enters FP8, and its "runtime execution
 * model" section has each iteration's attention update and read the cache
 * pages.  Here the split kernel's waves that read the page holding slot
 * L_b - 1 of (b, g) derive that page's new scales from the new rows and read
 * the page as the append leaves it (earlier slots re-encoded in registers
 * when a scale rises, the new token encoded); the merge kernel, after them
 * on the stream, stores the codes, the re-encoded slots and the new scales.
 * Results: pools and scales byte-identical to the quantising append of the
 * same rows and seq_lens; out equal to the decode of that cache up to the
 * rounding order.
 * k_new, v_new: [B][Hkv][D] of new_dtype (PKV_BF16 or PKV_F32).
 * k_scales, v_scales: read and written.  Other arguments, sizes, workspace and
 * errors as pkv_decode_step; PKV_E_DTYPE unless kv_dtype is FP8_E4M3, INT8 or
 * INT4 and new_dtype is BF16 or F32. */
int pkv_decode_step_quant(const void* q, pkv_dtype q_dtype, const void* k_new, const void* v_new,
                          pkv_dtype new_dtype, void* k_pool, void* v_pool, pkv_dtype kv_dtype,
                          float* k_scales, float* v_scales,
                          const int32_t* block_tables, int max_pages_per_seq,
                          const int32_t* seq_lens, int batch, int num_pages,
                          int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                          float scale, int partition_tokens,
                          void* out, pkv_dtype out_dtype,
                          void* workspace, size_t workspace_bytes, void* stream);

/* decode_step_noalloc - pkv_decode_step without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  It runs the same
 * kernels as pkv_decode_step (same results, bit for bit) and makes no
 * allocation of any kind: the workspace is a static device array inside the
 * library, 40 MiB (41943040 bytes), one copy per device, created with the
 * library's code on that device and held until the process ends.  Its address
 * is looked up once per device, on the first call made with that device
 * current.  Shapes whose pkv_decode_workspace_bytes exceed 40 MiB are rejected
 * with PKV_E_WORKSPACE (on a 256-CU device every G <= 16 and D <= 128 fits
 * for up to ~245 000 (sequence, kv head) pairs).  Nothing in the array needs
 * to start at zero; each call overwrites what it reads.  Every call on one
 * device shares that device's array: calls that may overlap on one device
 * (different streams, or different host threads without ordering) race and
 * give wrong results; serialise them.  Arguments, dtypes and errors are those
 * of pkv_decode_step minus workspace / workspace_bytes. */
int pkv_decode_step_noalloc(const void* q, pkv_dtype q_dtype, const void* k_new, const void* v_new,
                            void* k_pool, void* v_pool, pkv_dtype kv_dtype,
                            const float* k_scales, const float* v_scales,
                            const int32_t* block_tables, int max_pages_per_seq,
                            const int32_t* seq_lens, int batch, int num_pages,
                            int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                            float scale, int partition_tokens,
                            void* out, pkv_dtype out_dtype, void* stream);

/* kv_append_chunk - write a chunk of new K/V tokens per sequence into its pages.
 *
 * The paged store of the first page ("key mechanisms", after the page-table
 * lookup of "compile-time graph optimization") for the context tokens that its
 * "key performance parameters" section processes many at a time.  Sequence b
 * owns rows cu_new[b] .. cu_new[b+1] - 1 of k_new / v_new ([total_new][Hkv][D]
 * elements of kv_dtype, int4 rows packed two per byte): C_b = cu_new[b+1] -
 * cu_new[b] tokens that take positions L_b - C_b .. L_b - 1 (seq_lens counts
 * them), each copied bit for bit to slot t % P of page block_tables[b][t / P].
 *
 * cu_new: int32 [batch + 1] device array, non-decreasing, cu_new[batch] <=
 *   total_new.  kv_dtype: any pkv_dtype (fp8 / int8 / int4 bytes copied as
 *   given).  Writes only the addressed slots.  Sequences must not share slots.
 * A sequence with C_b <= 0 is untouched; one whose chunk does not fit (C_b >
 * L_b, L_b > max_pages_per_seq * P, or rows outside [0, total_new)) is skipped,
 * and so is a token whose page id lies outside [0, num_pages).
 * Errors: PKV_E_NULL, PKV_E_SHAPE (as pkv_kv_append, and total_new < 0),
 * PKV_E_DTYPE, PKV_E_ALIGN, PKV_E_HIP. */
int pkv_kv_append_chunk(const void* k_new, const void* v_new, pkv_dtype kv_dtype,
                        const int32_t* cu_new, int total_new,
                        const int32_t* block_tables, int max_pages_per_seq,
                        const int32_t* seq_lens, int batch,
                        void* k_pool, void* v_pool, int num_pages,
                        int num_kv_heads, int head_dim, int page_size, void* stream);

/* paged_prefill - causal attention of a chunk of query tokens per sequence
 * over the paged cache (chunked prefill).
 *
 * The first page's "key performance parameters" section has paged attention
 * process the context in parallel over many tokens; its "runtime execution
 * model" has the same pages read and updated by the decode iterations.  With
 * G = num_q_heads / num_kv_heads and C_b = cu_q[b+1] - cu_q[b], row
 * r = cu_q[b] + i of q is chunk token i of sequence b at position
 * p = L_b - C_b + i (its K/V already in the pages, e.g. by
 * pkv_kv_append_chunk); for each query head h (kv head h / G):
 *   out[r][h][:] = sum_{t <= p} softmax_t(scale * q[r][h] . k_t) v_t.
 * A row with p < 0 (C_b > L_b) gets zeros.
 *
 * q: bf16 [total_q][num_q_heads][head_dim]; out: bf16 or fp32, same shape;
 * cu_q: int32 [batch + 1] device array, non-decreasing, cu_q[batch] <= total_q
 * (rows of a sequence with a decreasing or out-of-range pair are not written);
 * kv_dtype must be BF16 (fp8: pkv_paged_prefill_fp8).  Pool layout and sizes as for decode.  Writes only the
 * rows of out that belong to a sequence.  No workspace.  A key position whose
 * page id lies outside [0, num_pages) (or past the table row) makes every row
 * of that (sequence, kv head) block NaN.
 * Errors: PKV_E_NULL, PKV_E_SHAPE (as decode, total_q < 0, G > 128, a page of
 * all kv heads of 4 GiB or more),
 * PKV_E_DTYPE (kv not bf16, q not bf16, out not bf16 / fp32), PKV_E_ALIGN,
 * PKV_E_HIP. */
int pkv_paged_prefill(const void* q, pkv_dtype q_dtype, const int32_t* cu_q, int total_q,
                      const void* k_pool, const void* v_pool, pkv_dtype kv_dtype,
                      const int32_t* block_tables, int max_pages_per_seq,
                      const int32_t* seq_lens, int batch, int num_pages,
                      int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                      float scale, void* out, pkv_dtype out_dtype, void* stream);

/* paged_prefill_fp8 - pkv_paged_prefill over an fp8-e4m3 cache with
 * per-(page, kv head) scales (a stored value is its code times the scale).
 *
 * The first page's "key mechanisms" section widens FP8 data back to 16 bits
 * before the matrix product accumulates, and the yololab page ("NVIDIA
 * TensorRT-LLM deep dive", FP8 section) gives FP8 as the way to halve the
 * memory a cache needs.  Here every e4m3 code widens to bf16 exactly on its
 * way into the products; the K scale joins the softmax scale of its tile and
 * the V scale multiplies the probabilities that enter the value products (the
 * row sums take the probabilities unscaled).
 * k_scales, v_scales: fp32 [num_pages][num_kv_heads].  page_size a multiple of
 * 64 (the fp8 V block).  Other arguments, results and errors as
 * pkv_paged_prefill, with PKV_E_NULL for NULL scales. */
int pkv_paged_prefill_fp8(const void* q, pkv_dtype q_dtype, const int32_t* cu_q, int total_q,
                          const void* k_pool, const void* v_pool,
                          const float* k_scales, const float* v_scales,
                          const int32_t* block_tables, int max_pages_per_seq,
                          const int32_t* seq_lens, int batch, int num_pages,
                          int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                          float scale, void* out, pkv_dtype out_dtype, void* stream);

/* alloc_pages - give every sequence the page its newest token opens, from a
 * free-page stack in device memory (no host round trip per step).
 *
 * The first page's "key mechanisms" section takes pages from a shared pool as a
 * sequence grows.  free_pages[0 .. *free_count - 1] is the stack (top at
 * *free_count - 1); capacity is free_pages' length.  In sequence order, each b
 * with L_b >= 1, (L_b - 1) % P == 0, (L_b - 1) / P < max_pages_per_seq and a
 * negative entry block_tables[b][(L_b - 1) / P] takes the top page into that
 * entry (so a sequence that did not grow this step takes nothing); when the
 * stack runs out the remaining entries stay negative.  *free_count is updated.
 * Call it with the step's seq_lens before the append (pkv_kv_append or
 * pkv_decode_step), which then writes into the new page.
 * seq_lens, block_tables, free_pages, free_count: device int32 arrays
 * ([batch], [batch][max_pages_per_seq], [capacity], [1]).  A *free_count
 * outside [0, capacity] is clamped.  Calls on one stack must not overlap.
 * Errors: PKV_E_NULL, PKV_E_SHAPE (batch < 0; max_pages_per_seq, page_size or
 * capacity <= 0), PKV_E_HIP. */
int pkv_alloc_pages(const int32_t* seq_lens, int batch, int32_t* block_tables,
                    int max_pages_per_seq, int page_size,
                    const int32_t* free_pages, int32_t* free_count, int capacity, void* stream);

/* release_pages - return the pages of finished sequences to the stack.
 *
 * The first page's "runtime execution model" has finished requests release
 * their KV pages for reuse.  In sequence order, each b with release[b] != 0
 * pushes the ids in [0, num_pages) among the first ceil(L_b / P) entries of its
 * row (at most max_pages_per_seq) onto the stack and sets those entries to -1;
 * pushes past capacity are dropped.  *free_count is updated.
 * release: device int32 [batch]; other arguments as for pkv_alloc_pages.
 * Errors: as pkv_alloc_pages, plus PKV_E_NULL for release and PKV_E_SHAPE
 * for num_pages <= 0. */
int pkv_release_pages(const int32_t* release, const int32_t* seq_lens, int batch,
                      int32_t* block_tables, int max_pages_per_seq, int page_size, int num_pages,
                      int32_t* free_pages, int32_t* free_count, int capacity, void* stream);

/* debug_read_probe - read every byte of buf once with 16-byte nontemporal loads
 * (the access of the decode's K/V stream) and nothing else: a measurement
 * aid.  The first page ties decode throughput to memory bandwidth ("key
 * performance parameters"); timing this call on a buffer much larger than
 * the caches gives the streaming-read rate the decode is compared with.
 * buf: device memory, 16-byte aligned, bytes a multiple of 16.  out: one
 * device uint32, written only in the unlikely case that the folded words
 * equal a fixed constant (so the loads cannot be dropped).
 * Errors: PKV_E_NULL, PKV_E_SHAPE (bytes % 16), PKV_E_ALIGN, PKV_E_HIP. */
int pkv_debug_read_probe(const void* buf, size_t bytes, uint32_t* out, void* stream);

/* debug_gather - copy each sequence's cached tokens out of the pages into
 * contiguous rows, through the same page-table lookup and chunk addressing
 * the decode kernels use (for bit-exact tests of that address path).
 * k_out, v_out: [B][Hkv][max_pages_per_seq * P][D] elements of kv_dtype; row
 * t < L_b of (b, g) receives token t; rows at or past L_b are not written.
 * Sequences with a bad page id or L_b > MP * P are skipped entirely. */
int pkv_debug_gather(const void* k_pool, const void* v_pool, pkv_dtype kv_dtype,
                     const int32_t* block_tables, int max_pages_per_seq,
                     const int32_t* seq_lens, int batch, int num_pages,
                     int num_kv_heads, int head_dim, int page_size,
                     void* k_out, void* v_out, void* stream);

/* Static text for a return code. */
const char* pkv_strerror(int code);

/* Detail of the last failure on the calling thread ("" if none).  The string
 * is thread-local and valid until the thread's next pkv call. */
const char* pkv_last_error(void);

/* Library version as major * 10000 + minor * 100 + patch. */
int pkv_version(void);

#ifdef __cplusplus
}
#endif
#endif /* PKV_H */
