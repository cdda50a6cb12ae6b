// Device-side page allocation for the paged KV cache (gfx950).
//
// The first page (TensorRT-LLM concept page) takes pages from a shared pool as
// a sequence grows ("key mechanisms") and returns the pages of finished
// requests for reuse ("runtime execution model").  Here the free pages are a
// stack in device memory (free_pages[0 .. count - 1], top at count - 1), so a
// decode step can take the page its new tokens open without a host round trip.
//
// alloc: in sequence order, every sequence whose last token L_b - 1 opens a
// page (L_b >= 1, (L_b - 1) % P == 0, page index < MP) and whose table entry
// for it is empty (negative) takes the top page; when the stack runs out the
// remaining entries stay as they are.  release: in sequence order, every
// marked sequence pushes the valid ids (in [0, NP)) among the first
// ceil(L_b / P) entries of its row and sets those entries to -1; pushes past
// the stack's capacity are dropped.
//
// One wave does each of them, so the result does not depend on timing.
// alloc takes 64 sequences at a time, and a prefix scan over the requests
// gives each its rank.  release walks the marked sequences in order; for
// each, the wave reads 64 table entries at a time, and a prefix scan over the
// valid ones gives each its stack slot.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_internal.h"
#include "pkv_device.h"

namespace pkv {

__global__ __launch_bounds__(64) void alloc_pages_kernel(const int32_t* __restrict__ seq_lens, int B,
                                                         int32_t* __restrict__ bt, int MP, int P,
                                                         const int32_t* __restrict__ free_pages,
                                                         int32_t* __restrict__ free_count, int capacity) {
  const int lane = threadIdx.x;
  // a count outside [0, capacity] is clamped, so no read leaves the stack
  const int count = uniform(min(max(free_count[0], 0), capacity));
  int taken = 0;
  for (int b0 = 0; b0 < B; b0 += 64) {
    const int b = b0 + lane;
    int want = 0, idx = 0;
    if (b < B) {
      const int L = seq_lens[b];
      if (L >= 1 && (L - 1) % P == 0) {
        idx = (L - 1) / P;
        if (idx < MP && bt[(size_t)b * MP + idx] < 0) want = 1;
      }
    }
    const int incl = wave_incl_scan(want, lane);
    const int k = taken + incl - want;               // requests before this one
    if (want && k < count) bt[(size_t)b * MP + idx] = free_pages[count - 1 - k];
    taken = uniform(taken + __builtin_amdgcn_readlane(incl, 63));
  }
  if (lane == 0) free_count[0] = max(count - taken, 0);
}

__global__ __launch_bounds__(64) void release_pages_kernel(const int32_t* __restrict__ release,
                                                           const int32_t* __restrict__ seq_lens, int B,
                                                           int32_t* __restrict__ bt, int MP, int P, int NP,
                                                           int32_t* __restrict__ free_pages,
                                                           int32_t* __restrict__ free_count, int capacity) {
  const int lane = threadIdx.x;
  const int count = uniform(min(max(free_count[0], 0), capacity));
  int pushed = 0;
  for (int b0 = 0; b0 < B; b0 += 64) {
    const int b = b0 + lane;
    const bool mark = b < B && release[b] != 0;
    const int L = mark ? seq_lens[b] : 0;
    uint64_t todo = __ballot(mark);
    // marked sequences in order; the whole wave walks one sequence's table
    // entries 64 at a time, and a prefix scan over the valid ones gives each
    // its stack slot, so pages are pushed in sequence order, then entry order
    while (todo) {
      const int f = uniform(__builtin_ctzll(todo));
      todo &= todo - 1;
      const int be = b0 + f;
      const int Lb = uniform(__builtin_amdgcn_readlane(L, f));
      const int n = Lb > 0 ? min((Lb - 1) / P + 1, MP) : 0;
      int32_t* row = bt + (size_t)be * MP;
      for (int i0 = 0; i0 < n; i0 += 64) {
        const int i = i0 + lane;
        const int pg = i < n ? row[i] : -1;
        const int valid = (unsigned)pg < (unsigned)NP;
        const int incl = wave_incl_scan(valid, lane);
        const int pos = count + pushed + incl - valid;
        if (valid && pos < capacity) free_pages[pos] = pg;
        if (i < n) row[i] = -1;
        pushed = uniform(pushed + __builtin_amdgcn_readlane(incl, 63));
      }
    }
  }
  if (lane == 0) free_count[0] = min(count + pushed, capacity);
}

hipError_t launch_alloc_pages(const PageArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(alloc_pages_kernel, dim3(1), dim3(64), 0, s, a.seq_lens, a.batch, a.block_tables, a.max_pages,
                     a.page_size, a.free_pages, a.free_count, a.capacity);
  return hipGetLastError();
}

hipError_t launch_release_pages(const PageArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(release_pages_kernel, dim3(1), dim3(64), 0, s, a.release, a.seq_lens, a.batch,
                     a.block_tables, a.max_pages, a.page_size, a.num_pages, a.free_pages, a.free_count,
                     a.capacity);
  return hipGetLastError();
}

}  // namespace pkv
