// Expert placement and online load statistics.
//
// Large-scale expert parallelism replicates hot experts and places the
// copies on physical expert slots; the routing step then sends each pick to
// one physical copy of its logical expert, and a statistics component on the
// GPU counts how many picks every logical expert received, as input for the
// placement computed elsewhere (TensorRT-LLM large-EP page, high-level
// design: the GPU-side routing component reads the placement information,
// the online statistics collector feeds the replication and placement
// computation).
//
// Placement information (caller-owned, on the device), in CSR form:
//   rep_offsets[E_log + 1]  logical expert e owns entries
//                           [rep_offsets[e], rep_offsets[e + 1]) of rep_phys
//   rep_phys[...]           the physical slot of each copy, in [0, E_phys)
// The copy serving pick j of token t is entry t mod n_e of its expert
// (n_e = number of copies): successive tokens of an expert take its copies
// in turn, a stateless and deterministic spread.

#include "moe_internal.h"

namespace moe {

__global__ void __launch_bounds__(256)
    place_kernel(const int32_t* __restrict__ idx, int T, int k, int E_log, int E_phys,
                 const int32_t* __restrict__ rep_offsets, const int32_t* __restrict__ rep_phys,
                 int32_t* __restrict__ phys) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)T * k) return;
  const int t = (int)(i / k);
  const int e = idx[i];
  int out = -1;  // dropped picks stay dropped
  if (e >= 0 && e < E_log) {
    const int b = rep_offsets[e], n = rep_offsets[e + 1] - b;
    if (n > 0) {
      const int p = rep_phys[b + t % n];
      // a malformed entry drops the pick instead of indexing out of range
      out = (p >= 0 && p < E_phys) ? p : -1;
    }
  }
  phys[i] = out;
}

// Per 256-token tile an LDS histogram over the logical experts, then one
// 64-bit atomic add per expert with a nonzero count: integer sums, so the
// totals do not depend on the order of the atomics.
__global__ void __launch_bounds__(256)
    load_stats_kernel(const int32_t* __restrict__ idx, int T, int k, int E,
                      unsigned long long* __restrict__ stats) {
  extern __shared__ int hist[];
  for (int e = threadIdx.x; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  const int t = (int)blockIdx.x * 256 + (int)threadIdx.x;
  if (t < T)
    for (int j = 0; j < k; ++j) {
      const int e = idx[(long long)t * k + j];
      if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
    }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256)
    if (hist[e]) atomicAdd(&stats[e], (unsigned long long)hist[e]);
}

int place_impl(const int32_t* idx, int T, int k, int E_log, int E_phys,
               const int32_t* rep_offsets, const int32_t* rep_phys, int32_t* phys,
               hipStream_t s) {
  const long long n = (long long)T * k;
  if (n == 0) return MOE_OK;
  hipLaunchKernelGGL(place_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, idx,
                     T, k, E_log, E_phys, rep_offsets, rep_phys, phys);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int load_stats_impl(const int32_t* idx, int T, int k, int E, unsigned long long* stats,
                    hipStream_t s) {
  if (T == 0) return MOE_OK;
  hipLaunchKernelGGL(load_stats_kernel, dim3((T + 255) / 256), dim3(256), E * sizeof(int), s,
                     idx, T, k, E, stats);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
