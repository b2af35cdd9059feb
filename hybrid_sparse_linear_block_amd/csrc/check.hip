// Checks of what the decode kernels take on trust: sequence lengths and
// the block-table entries they turn into page indices (the paged cache of
// "SPLA: Block Sparse Plus Linear Attention for Long Context Modeling",
// section "Page Attention and Selection").  The same rule runs on the GPU
// (k_check_tables, for device-resident tables) and on the host
// (check_tables_host, for host copies and CPU-only tests).
#include <limits.h>

#include <algorithm>

#include "common.h"
#include "internal.h"

namespace hsla {

namespace {

constexpr int kCheckThreads = 256;

// Item key of the first violation: row b's length is item b (M + 1), its
// entry j is item b (M + 1) + j + 1 (M = entries per row).
__global__ __launch_bounds__(kCheckThreads) void k_check_tables(CheckTablesArgs a) {
  const int b = blockIdx.x;
  const int T = a.seq_lens[b];
  const long rowkey = static_cast<long>(b) * (a.max_blocks + 1);
  int bad = 0;
  long first = LONG_MAX;
  const bool len_ok = T >= a.min_len && static_cast<long>(T) + a.extra <= a.max_seq_len;
  if (!len_ok) {
    if (threadIdx.x == 0) {
      bad = 1;
      first = rowkey;
    }
  } else {
    const long used = (static_cast<long>(T) + a.extra + a.B - 1) / a.B;   // <= max_blocks (checked on the host)
    const int32_t* row = a.block_table + static_cast<size_t>(b) * a.max_blocks;
    for (long j = threadIdx.x; j < used; j += blockDim.x) {
      const int32_t p = row[j];
      if (p < 0 || p >= a.num_pages) {
        ++bad;
        first = min(first, rowkey + j + 1);
      }
    }
  }
  if (bad) {
    atomicAdd(a.result, bad);
    atomicMin(a.result + 1, static_cast<int32_t>(min(first, static_cast<long>(INT_MAX - 1))));
  }
}

// Result slots to (0, INT_MAX) with a kernel (no memset node in a captured graph).
__global__ void k_check_init(int32_t* result) {
  if (threadIdx.x == 0) {
    result[0] = 0;
    result[1] = INT_MAX;
  }
}

}  // namespace

hipError_t launch_check_tables(const CheckTablesArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(k_check_init, dim3(1), dim3(kWave), 0, stream, a.result);
  hipError_t e = launch_status("k_check_init");
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_check_tables, dim3(a.batch), dim3(kCheckThreads), 0, stream, a);
  return launch_status("k_check_tables");
}

void check_tables_host(const CheckTablesArgs& a) {
  int bad = 0;
  long first = LONG_MAX;
  for (int b = 0; b < a.batch; ++b) {
    const int T = a.seq_lens[b];
    const long rowkey = static_cast<long>(b) * (a.max_blocks + 1);
    if (T < a.min_len || static_cast<long>(T) + a.extra > a.max_seq_len) {
      ++bad;
      first = std::min(first, rowkey);
      continue;
    }
    const long used = (static_cast<long>(T) + a.extra + a.B - 1) / a.B;
    const int32_t* row = a.block_table + static_cast<size_t>(b) * a.max_blocks;
    for (long j = 0; j < used; ++j) {
      if (row[j] < 0 || row[j] >= a.num_pages) {
        ++bad;
        first = std::min(first, rowkey + j + 1);
      }
    }
  }
  a.result[0] = bad;
  a.result[1] = static_cast<int32_t>(std::min(first, static_cast<long>(INT_MAX)));
}

}  // namespace hsla
