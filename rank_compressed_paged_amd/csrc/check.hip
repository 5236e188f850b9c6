// Index checks, a debugging aid beside the attention path: the decode,
// prefill and append kernels skip out-of-range block ids and slots instead of
// failing, so this kernel scans the same index arrays and reports what lies
// outside the ranges those kernels assume (the paged cache of 16-token
// blocks reached through a block table, Proxima README "KV-cache capacity").
#include "common.h"
#include "kernels.h"

namespace starkv {

constexpr int kCheckThreads = 1024;

// One work group: every thread scans a strided share of the lengths, the
// block-table entries in use and the slots, keeping a bit mask and the
// smallest offending index of each kind; LDS atomics combine them, so the
// report does not depend on the order in which threads run.
__global__ __launch_bounds__(kCheckThreads) void check_indices_kernel(
    const int32_t* __restrict__ block_tables, int max_blocks, const int32_t* __restrict__ seq_lens,
    int batch, int max_seq_len, int num_blocks, const int64_t* __restrict__ slots, int n_slots,
    int64_t slot_limit, uint32_t* __restrict__ report) {
  __shared__ uint32_t s_rep[4];
  const int tid = threadIdx.x;
  if (tid == 0) {
    s_rep[0] = 0u;
    s_rep[1] = s_rep[2] = s_rep[3] = 0xFFFFFFFFu;
  }
  __syncthreads();
  uint32_t flags = 0u, bad_blk = 0xFFFFFFFFu, bad_len = 0xFFFFFFFFu, bad_slot = 0xFFFFFFFFu;
  for (int b = tid; b < batch; b += kCheckThreads) {
    const int L = seq_lens[b];
    if (L < 0 || L > max_seq_len) {
      flags |= 2u;
      bad_len = min(bad_len, (uint32_t)b);
    }
  }
  const int64_t entries = (int64_t)batch * max_blocks;
  for (int64_t i = tid; i < entries; i += kCheckThreads) {
    const int b = (int)(i / max_blocks), j = (int)(i % max_blocks);
    const int L = min(max(seq_lens[b], 0), max_seq_len);
    if (j < (L + 15) / 16 && (uint32_t)block_tables[i] >= (uint32_t)num_blocks) {
      flags |= 1u;
      bad_blk = min(bad_blk, (uint32_t)b);
    }
  }
  for (int n = tid; n < n_slots; n += kCheckThreads) {
    if (slots[n] >= slot_limit) {
      flags |= 4u;
      bad_slot = min(bad_slot, (uint32_t)n);
    }
  }
  if (flags) {
    atomicOr(&s_rep[0], flags);
    atomicMin(&s_rep[1], bad_blk);
    atomicMin(&s_rep[2], bad_len);
    atomicMin(&s_rep[3], bad_slot);
  }
  __syncthreads();
  if (tid < 4) report[tid] = s_rep[tid];
}

hipError_t launch_check_indices(const int32_t* block_tables, int max_blocks,
                                const int32_t* seq_lens, int batch, int max_seq_len,
                                int num_blocks, const int64_t* slots, int n_slots,
                                uint32_t* report, hipStream_t st) {
  hipLaunchKernelGGL(check_indices_kernel, dim3(1), dim3(kCheckThreads), 0, st, block_tables,
                     max_blocks, seq_lens, batch, max_seq_len, num_blocks, slots, n_slots,
                     (int64_t)num_blocks * 16, report);
  return hipGetLastError();
}

}  // namespace starkv
