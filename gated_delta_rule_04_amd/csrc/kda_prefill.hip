// KDA chunked prefill: host-side dispatch and the small helper kernels.
//
// The prefill kernel itself (chunk_fwd_pipe_kernel, bf16 and fp32 inputs) is
// in kda_prefill_pipe.hip.  Here: the packed-document ordering kernel, the
// fill kernel (no hipMemsetAsync, so calls can be captured in graphs), the
// value-slice choice and the dispatch.

#include "kda_prefill_common.h"
#include "kda_launch.h"

namespace kda {

// ---------------------------------------------------------------------------
// Varlen prep: documents ordered by decreasing length (ties by index), so the
// longest chains start first.  One thread per document; O(N) scan each.
// ---------------------------------------------------------------------------
__global__ void varlen_order_kernel(const int* __restrict__ cu, int N, int T, int* __restrict__ order) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= N) return;
  auto length = [&](int n) {
    int a = min(max(cu[n], 0), T);
    int b = min(max(cu[n + 1], a), T);
    return b - a;
  };
  const int li = length(i);
  int r = 0;
  for (int j = 0; j < N; ++j) {
    const int lj = length(j);
    r += (lj > li) || (lj == li && j < i);
  }
  order[r] = i;
}

// Fill helpers (no hipMemsetAsync: safe to capture in graphs).
__global__ void fill_zero_kernel(float* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0.f;
}

// Value-slice width for a shape: fill the CUs with one workgroup wave where
// possible; narrower slices cost a repeated intra-chunk transform.
int prefill_slice_width(bool bf16_io, int Dk, int Dv, long long units, int num_cus) {
  if (!bf16_io) return units * (Dv / 16) <= num_cus ? 16 : 32;
  // widest slice that still gives every CU a workgroup (64 at most with 128
  // key channels: wider state slices do not fit the register budget)
  for (int vs = (Dk == 128 ? 64 : Dv); vs > 32; vs /= 2)
    if (units * (Dv / vs) >= num_cus / 2) return vs;
  return 32;
}

bool prefill_supported(bool bf16_io, int Dk, int Dv) {
  (void)bf16_io;
  return (Dk == 64 || Dk == 128) && (Dv == 64 || Dv == 128);
}

hipError_t launch_prefill(bool bf16_io, int Dk, int Dv, int g_group, int VS, const PrefillArgs& a,
                          hipStream_t stream) {
  return launch_prefill_pipe(bf16_io, Dk, Dv, g_group, VS, a, stream);  // kda_prefill_pipe.hip
}

hipError_t launch_varlen_order(const int* cu, int N, int T, int* order, hipStream_t stream) {
  if (N <= 0) return hipSuccess;
  hipLaunchKernelGGL(varlen_order_kernel, dim3((N + 255) / 256), dim3(256), 0, stream, cu, N, T, order);
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, size_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

}  // namespace kda

