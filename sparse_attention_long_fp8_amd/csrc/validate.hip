// On-request checks of the device-side preconditions that the path's entry
// points document but do not test while they run (the batch arrays, the key
// rows and page ids they address, the selected positions, NaN scores).  The
// checks only read and compare: every address they form is bounded by sizes
// the host has validated, so a violating input yields a report, never an
// access outside its arrays.  The first violation found wins the report.
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {

namespace {

__device__ void report_violation(int32_t *report, int code, int a, int b, int v) {
  if (atomicCAS(&report[0], 0, code) == 0) {
    report[1] = a;
    report[2] = b;
    report[3] = v;
  }
}

__global__ void validate_init_kernel(int32_t *report) {
  if (threadIdx.x < 4) report[threadIdx.x] = 0;
}

// One workgroup per sequence: thread 0 checks the batch arrays and the
// sequence's row range; all threads check its page ids.
__global__ __launch_bounds__(256) void validate_seq_kernel(ValidateArgs a, int32_t *report) {
  const int b = blockIdx.x;
  const int q0 = a.q_seq_start[b], q1 = a.q_seq_start[b + 1];
  const int kl = a.k_len[b];
  const int nq = q1 - q0;
  const bool batch_ok = (b > 0 || q0 == 0) && nq >= 0 && nq <= a.max_q_per_seq &&
                        (b < a.num_seqs - 1 || q1 == a.num_queries) && kl >= nq && kl <= a.max_k_len;
  if (threadIdx.x == 0) {
    if (!batch_ok) {
      report_violation(report, kCheckBatch, b, nq, kl);
    } else if (a.has_layout && !a.paged) {
      const int64_t ks = a.k_seq_start[b];
      if (ks < 0 || ks + kl > a.num_rows) report_violation(report, kCheckRows, b, kl, (int)ks);
    }
  }
  if (a.has_layout && a.paged && batch_ok) {
    // kl <= max_k_len, whose pages fit the table's stride (host-checked)
    const int pages = (kl + kPageSize - 1) >> kPageShift;
    for (int p = threadIdx.x; p < pages; p += blockDim.x) {
      const int id = a.page_table[(int64_t)b * a.page_table_stride + p];
      if (id < 0 || id >= a.num_rows) report_violation(report, kCheckPage, b, p, id);
    }
  }
}

// One workgroup per query row: its selected positions are -1 or below n_t,
// and its scores below n_t are not NaN.  n_t comes from the batch arrays;
// reads stay inside the row (s < ld, j < k) whatever it is.
__global__ __launch_bounds__(256) void validate_row_kernel(ValidateArgs a, int32_t *report) {
  const int t = blockIdx.x;
  const BatchDev bt{a.num_seqs, a.q_seq_start, a.k_len};
  const int b = seq_of_row(bt, t);
  const int n = candidates_of_row(bt, b, t);
  if (a.indices) {
    const int32_t *row = a.indices + (int64_t)t * a.k;
    for (int j = threadIdx.x; j < a.k; j += blockDim.x) {
      const int s = row[j];
      if (s != -1 && (s < 0 || s >= n)) report_violation(report, kCheckIndex, t, j, s);
    }
  }
  if (a.scores) {
    const float *row = a.scores + (int64_t)t * a.ld;
    const int64_t m = n < 0 ? 0 : (n < a.ld ? n : a.ld);
    for (int64_t s = threadIdx.x; s < m; s += blockDim.x)
      if ((__float_as_uint(row[s]) & 0x7FFFFFFFu) > 0x7F800000u) report_violation(report, kCheckNanScore, t, (int)s, 0);
  }
}

}  // namespace

hipError_t launch_validate(const ValidateArgs &a, int32_t *report, hipStream_t stream) {
  hipLaunchKernelGGL(validate_init_kernel, dim3(1), dim3(64), 0, stream, report);
  if (!a.q_seq_start || !a.k_len) return hipGetLastError();
  hipLaunchKernelGGL(validate_seq_kernel, dim3(a.num_seqs), dim3(256), 0, stream, a, report);
  if (a.num_queries > 0 && (a.indices || a.scores))
    hipLaunchKernelGGL(validate_row_kernel, dim3(a.num_queries), dim3(256), 0, stream, a, report);
  return hipGetLastError();
}

}  // namespace dsa
