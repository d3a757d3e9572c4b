// Dispatch: per-expert counts, offsets, the token <-> layout-row map and the
// permute-gather of token activations into expert-contiguous rows.
//
// Each token is written once for every expert it picked (DySHARP page,
// section 1: dispatch sends the same token to k experts); rows bound for one
// expert form one dense, contiguous segment, allocated incrementally in
// arrival (= token) order, and the algebraic -> layout index table is kept
// for combine's reverse lookup (DySHARP page, section 3.1 item 3; ThunderEP
// page, sections 3.4 and 5.2 on gathering one expert's tokens into one
// buffer).  Counts stay on the device (TensorRT-LLM large-EP page, EP
// communication kernels).
//
// Kernels (tile = 256 tokens = 4 waves):
//   hist    per-tile expert histogram (LDS integer atomics: exact counts)
//   scan    per-expert prefix over tiles -> tile bases, counts, offsets
//   slots   rank of each pick among earlier picks of the same expert:
//           earlier waves via per-wave LDS histograms, earlier lanes of the
//           same wave via ballots over the expert-id bits; no atomics decide
//           any order, so the layout is deterministic and token-stable
//   gather  one wave per token: each 16-byte chunk of x[t] is loaded once and
//           stored to every local row of that token

#include "moe_internal.h"

namespace moe {

constexpr int TILE = 256;

__global__ void __launch_bounds__(TILE)
    hist_kernel(const int32_t* __restrict__ idx, int T, int E, int k, int n_tiles,
                int32_t* __restrict__ tile_counts /* [E][n_tiles] */) {
  extern __shared__ int hist[];
  const int tile = (int)blockIdx.x;
  for (int e = threadIdx.x; e < E; e += TILE) hist[e] = 0;
  __syncthreads();
  const int t = tile * TILE + (int)threadIdx.x;
  if (t < T) {
    const int32_t* p = idx + (long long)t * k;
    for (int j = 0; j < k; ++j) atomicAdd(&hist[p[j]], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += TILE)
    tile_counts[(long long)e * n_tiles + tile] = hist[e];
}

// One block: thread e turns its expert's tile counts into exclusive bases;
// then a block scan over experts gives the offsets.
__global__ void __launch_bounds__(1024)
    scan_kernel(const int32_t* __restrict__ tile_counts, int E, int n_tiles,
                int32_t* __restrict__ tile_base, int32_t* __restrict__ counts,
                int32_t* __restrict__ offsets) {
  __shared__ int s[1024];
  const int e = (int)threadIdx.x;
  int total = 0;
  if (e < E) {
    const int32_t* src = tile_counts + (long long)e * n_tiles;
    int32_t* dst = tile_base + (long long)e * n_tiles;
    int tb = 0;
    for (; tb + 8 <= n_tiles; tb += 8) {
      int v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = src[tb + q];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        dst[tb + q] = total;
        total += v[q];
      }
    }
    for (; tb < n_tiles; ++tb) {
      const int v = src[tb];
      dst[tb] = total;
      total += v;
    }
    counts[e] = total;
  }
  // inclusive scan of totals over experts (Hillis-Steele)
  s[e] = total;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int add = e >= o ? s[e - o] : 0;
    __syncthreads();
    s[e] += add;
    __syncthreads();
  }
  if (e < E) offsets[e] = s[e] - total;
  if (e == 0) offsets[E] = s[1023];
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = lane_id();
  return l ? (~0ull >> (64 - l)) : 0ull;
}

__global__ void __launch_bounds__(TILE)
    slots_kernel(const int32_t* __restrict__ idx, int T, int E, int k, int n_tiles,
                 int nbits, const int32_t* __restrict__ tile_base,
                 const int32_t* __restrict__ offsets, int32_t* __restrict__ slot_of,
                 int32_t* __restrict__ row_token) {
  extern __shared__ int wcnt[];  // [4][E] per-wave counts, then exclusive
  const int tile = (int)blockIdx.x;
  const int wave = (int)threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 4 * E; i += TILE) wcnt[i] = 0;
  __syncthreads();
  const int t = tile * TILE + (int)threadIdx.x;
  const bool valid = t < T;
  const int32_t* p = idx + (long long)(valid ? t : 0) * k;
  if (valid)
    for (int j = 0; j < k; ++j) atomicAdd(&wcnt[wave * E + p[j]], 1);
  __syncthreads();
  // exclusive prefix over the 4 waves, per expert
  for (int e = threadIdx.x; e < E; e += TILE) {
    int run = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int c = wcnt[w * E + e];
      wcnt[w * E + e] = run;
      run += c;
    }
  }
  __syncthreads();
  const uint64_t lt = lanemask_lt();
  for (int j = 0; j < k; ++j) {
    const int e = valid ? p[j] : -1;
    uint64_t same = 0;  // lanes of this wave whose picks include e
    for (int jj = 0; jj < k; ++jj) {
      const int o = valid ? p[jj] : -1;
      uint64_t eq = __ballot(valid);
      for (int b = 0; b < nbits; ++b) {
        const uint64_t ob = __ballot(valid && ((o >> b) & 1));
        eq &= ((e >> b) & 1) ? ob : ~ob;
      }
      same |= eq;
    }
    if (valid) {
      const int rank = __popcll(same & lt);
      const int r = offsets[e] + tile_base[(long long)e * n_tiles + tile] +
                    wcnt[wave * E + e] + rank;
      slot_of[(long long)t * k + j] = r;
      row_token[r] = t;
    }
  }
}

// One wave per token; rows of local experts only.  KMAX >= k bounds the
// unrolled pick loop so the (wave-uniform) row numbers stay in registers.
template <int KMAX>
__global__ void __launch_bounds__(256)
    gather_kernel(const uint4* __restrict__ x, const int32_t* __restrict__ idx,
                  const int32_t* __restrict__ slot_of, int T, int k, int e_begin,
                  int e_end, int nch /* 16-byte chunks per row */,
                  uint4* __restrict__ x_perm) {
  const int t = __builtin_amdgcn_readfirstlane(
      (int)(blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)));
  if (t >= T) return;
  const int lane = lane_id();
  long long rows[KMAX];
  bool loc[KMAX];
  bool any = false;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    loc[j] = false;
    rows[j] = 0;
    if (j < k) {
      const int e = idx[(long long)t * k + j];
      loc[j] = e >= e_begin && e < e_end;
      rows[j] = (long long)slot_of[(long long)t * k + j] * nch;
      any |= loc[j];
    }
  }
  if (!any) return;
  const uint4* src = x + (long long)t * nch;
  constexpr int U = 4;
  int c = lane;
  for (; c + (U - 1) * 64 < nch; c += U * 64) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = src[c + u * 64];
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (loc[j])
#pragma unroll
        for (int u = 0; u < U; ++u) x_perm[rows[j] + c + u * 64] = v[u];
  }
  for (; c < nch; c += 64) {
    const uint4 v = src[c];
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (loc[j]) x_perm[rows[j] + c] = v;
  }
}

int dispatch_impl(const void* x, int act_dtype, const int32_t* idx, int T, int H,
                  int E, int k, int e_begin, int e_end, int32_t* counts,
                  int32_t* offsets, int32_t* slot_of, int32_t* row_token,
                  void* x_perm, void* ws, hipStream_t s) {
  const int n_tiles = (T + TILE - 1) / TILE;
  int32_t* tile_counts = (int32_t*)ws;
  int32_t* tile_base = tile_counts + (size_t)E * (n_tiles > 0 ? n_tiles : 1);
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  if (n_tiles > 0) {
    hipLaunchKernelGGL(hist_kernel, dim3(n_tiles), dim3(TILE), E * sizeof(int), s, idx,
                       T, E, k, n_tiles, tile_counts);
  }
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, tile_counts, E, n_tiles,
                     tile_base, counts, offsets);
  if (n_tiles > 0) {
    hipLaunchKernelGGL(slots_kernel, dim3(n_tiles), dim3(TILE), 4 * E * sizeof(int), s,
                       idx, T, E, k, n_tiles, nbits, tile_base, offsets, slot_of,
                       row_token);
    const int elem = act_dtype == MOE_DTYPE_F32 ? 4 : 2;
    const int nch = H * elem / 16;
    if (e_end > e_begin) {
      const dim3 grid((T + 3) / 4), block(256);
#define MOE_GATHER(KM)                                                         \
  hipLaunchKernelGGL((gather_kernel<KM>), grid, block, 0, s, (const uint4*)x, idx, \
                     slot_of, T, k, e_begin, e_end, nch, (uint4*)x_perm)
      if (k <= 1) MOE_GATHER(1);
      else if (k <= 2) MOE_GATHER(2);
      else if (k <= 4) MOE_GATHER(4);
      else if (k <= 8) MOE_GATHER(8);
      else if (k <= 16) MOE_GATHER(16);
      else MOE_GATHER(32);
#undef MOE_GATHER
    }
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

size_t dispatch_ws_bytes(int T, int E) {
  const size_t n_tiles = (size_t)((T + TILE - 1) / TILE);
  return 2 * (size_t)E * (n_tiles > 0 ? n_tiles : 1) * sizeof(int32_t);
}

}  // namespace moe
