// Device-side check of a step's metadata: block tables, context lengths and,
// for a chunked-prefill step, the query offsets.
//
// The attention and append kernels trust these device arrays, as the pages'
// gather trusts its block table (scalablesystem.dev, "PagedAttention Block
// Table Lookup"); they only keep a bad entry from reaching memory outside the
// pool (an id outside the pool reads as zero, a length past max_context_len
// is clamped).  A wrong id is still a wrong answer, and one row reading
// another request's blocks is on the faangrind failure list.  Checking the
// contents on the host would need a device-to-host copy and a
// synchronisation, so this call counts the violations on the device and
// leaves a small report there for the caller to read when it likes.
//
// One workgroup of 16 waves scans the rows (wave w takes rows w, w + 16, ...)
// with each lane reading one table entry per pass, counts in LDS, and writes
// the whole report at the end: no global atomics and nothing the caller must
// clear first, so the call is the same every time it is replayed.

#include <climits>

#include "device_common.h"

namespace pkv {
namespace {

constexpr int kCheckWaves = 16;

struct CheckArgs {
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* query_start;  // may be null
  int32_t* report;
  int bt_stride, num_rows, max_context_len, num_blocks, total_q;
};

__global__ __launch_bounds__(64 * kCheckWaves) void check_tables_kernel(CheckArgs a) {
  __shared__ int s_bad_len, s_bad_id, s_bad_q, s_first;
  if (threadIdx.x == 0) {
    s_bad_len = 0;
    s_bad_id = 0;
    s_bad_q = 0;
    s_first = INT_MAX;
  }
  __syncthreads();
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  for (int r = wave; r < a.num_rows; r += kCheckWaves) {
    const int L = a.context_lens[r];
    const bool len_bad = L < 1 || L > a.max_context_len;
    // the table entries a kernel would read for this row: those of its first
    // min(L, max_context_len) tokens
    const int Lc = L < 0 ? 0 : (L > a.max_context_len ? a.max_context_len : L);
    const int nb = (Lc + kBlockSize - 1) / kBlockSize;
    const int32_t* row = a.block_tables + (size_t)r * a.bt_stride;
    int ids_bad = 0;
    for (int j0 = 0; j0 < nb; j0 += 64) {
      const int j = j0 + lane;
      const bool bad = j < nb && (unsigned)row[j] >= (unsigned)a.num_blocks;
      ids_bad += __popcll(__ballot(bad));
    }
    bool q_bad = false;
    if (a.query_start) {
      const int q0 = a.query_start[r], q1 = a.query_start[r + 1];
      const int n = q1 - q0;
      q_bad = q0 < 0 || q1 > a.total_q || n < 1 || n > L;
    }
    if (lane == 0 && (len_bad || ids_bad || q_bad)) {
      if (len_bad) atomicAdd(&s_bad_len, 1);
      if (ids_bad) atomicAdd(&s_bad_id, ids_bad);
      if (q_bad) atomicAdd(&s_bad_q, 1);
      atomicMin(&s_first, r);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    a.report[0] = s_bad_len;
    a.report[1] = s_bad_id;
    a.report[2] = s_bad_q;
    a.report[3] = s_first == INT_MAX ? -1 : s_first;
  }
}

}  // namespace
}  // namespace pkv

extern "C" int pkv_check_tables(const pkv_cache* cache, const int32_t* block_tables, int32_t bt_stride,
                                const int32_t* context_lens, int32_t num_rows, int32_t max_context_len,
                                const int32_t* query_start, int32_t total_q, int32_t* report, void* stream) {
  using namespace pkv;
  if (int rc = check_cache(cache)) return rc;
  if (num_rows < 1) return fail(PKV_ERR_INVALID_ARG, "num_rows must be >= 1");
  if (!block_tables || !context_lens || !report) return fail(PKV_ERR_INVALID_ARG, "null device pointer");
  if (bt_stride < 1) return fail(PKV_ERR_INVALID_ARG, "bt_stride must be >= 1");
  if (max_context_len < 1 || (int64_t)max_context_len > (int64_t)bt_stride * kBlockSize)
    return fail(PKV_ERR_INVALID_ARG, "max_context_len must be in [1, bt_stride * 16]");
  if (query_start && total_q < 1) return fail(PKV_ERR_INVALID_ARG, "total_q must be >= 1 with query_start");
  CheckArgs a;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start = query_start;
  a.report = report;
  a.bt_stride = bt_stride;
  a.num_rows = num_rows;
  a.max_context_len = max_context_len;
  a.num_blocks = cache->num_blocks;
  a.total_q = total_q;
  check_tables_kernel<<<dim3(1), dim3(64 * kCheckWaves), 0, static_cast<hipStream_t>(stream)>>>(a);
  return check_launch("table check kernel");
}
