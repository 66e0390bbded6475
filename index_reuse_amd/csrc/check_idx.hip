// Device-side check of an index tensor against the index format and the
// row domain, for callers that want to catch a corrupted or misaligned index
// set before it is gathered ("CSA, HCA and CSA2", section 5.1, fault
// injection: a Reuse layer's indices shifted by a token must be caught by
// assertions, not by the output looking wrong).
//
// Row r passes when 0 <= count[r] <= k, idx[r][0 .. count) is strictly
// ascending and every entry lies among the row's candidates (token mode:
// [0, win_lo); candidate mode: at or above 0 and below n_avail, outside the
// window), and idx[r][count .. k) are all -1.  The kernels only read idx,
// count and the row geometry, so any contents are safe to check.
#include "kernels.hpp"

namespace sa {

namespace {

__global__ void check_init_kernel(uint32_t* err) {
  if (threadIdx.x == 0) err[0] = 0xFFFFFFFFu;
}

// One workgroup per row; the smallest (row, code) pair found wins.
__global__ __launch_bounds__(256) void check_idx_kernel(CheckArgs a) {
  const int r = blockIdx.x;
  const RowInfo ri = row_info(a.rows, r);
  const int32_t* idx = a.idx + (int64_t)r * a.idx_stride;
  const int cnt = a.count[r];
  const int hi = a.candidate_mode ? ri.n_avail : ri.win_lo;
  uint32_t code = 0;
  if (cnt < 0 || cnt > a.k) {
    code = kCheckCount;
  } else {
    for (int j = threadIdx.x; j < a.k; j += 256) {
      const int v = idx[j];
      uint32_t c = 0;
      if (j < cnt) {
        const bool in_window = a.candidate_mode && v >= ri.win_lo;
        if (v < 0 || v >= hi || in_window) c = kCheckDomain;
        else if (j > 0 && idx[j - 1] >= v) c = kCheckOrder;
      } else if (v != -1) {
        c = kCheckPadding;
      }
      if (c && (code == 0 || c < code)) code = c;
    }
  }
  if (code) atomicMin(a.err, ((uint32_t)r << 3) | code);
}

}  // namespace

hipError_t launch_check_indices(const CheckArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(check_init_kernel, dim3(1), dim3(64), 0, s, a.err);
  if (a.rows.n_rows > 0)
    hipLaunchKernelGGL(check_idx_kernel, dim3(a.rows.n_rows), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace sa
