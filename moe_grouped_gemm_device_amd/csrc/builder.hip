// Standalone argument builder (K1): runs the same device group table that
// every grouped-GEMM kernel builds in its prologue, and writes it out.
//
// Output (grouped_gemm PR "Support GPU-resident batch sizes", review thread:
// the batch sizes are scanned on the device by a single block; kDynamicK
// problems are sorted by k, descending.  FBGEMM PR "F8I4 Grouped Gemm
// Optimization for Sparse M": only non-empty groups become problems):
//   offs[E+1]; count; entries {g, first row, rows, 0}:
//     fixed-M  : one per bm-row slice of every non-empty group, g ascending;
//     dynamic-K: every group, by size descending then g ascending.
#include "kernels.h"
#include "worklist.h"

namespace mg {

__global__ void __launch_bounds__(kTableThreads) build_worklist_kernel(BuildArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  GroupTable t = carve_table(lds, a.E);
  build_group_table(a.sizes, a.E, a.total_M, a.bm, a.kind == 1, t);
  const int tid = threadIdx.x;
  for (int g = tid; g <= a.E; g += kTableThreads) a.offs[g] = t.off[g];
  int4* out = reinterpret_cast<int4*>(a.entries);
  if (a.kind == 0) {
    const int32_t n = t.tstart[a.E];
    if (tid == 0) *a.count = n;
    for (int32_t i = tid; i < n; i += kTableThreads) out[i] = fixed_m_entry(t, a.E, a.bm, i);
  } else {
    if (tid == 0) *a.count = a.E;
    for (int i = tid; i < a.E; i += kTableThreads) {
      const int g = t.order[i];
      out[i] = make_int4(g, t.off[g], t.eff[g], 0);
    }
  }
}

hipError_t launch_build_worklist(const BuildArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(build_worklist_kernel, dim3(1), dim3(kTableThreads), (size_t)table_lds_bytes(a.E), stream, a);
  return hipGetLastError();
}

}  // namespace mg
