// Combine: the gate-weighted un-permute reduction.
//
// The k expert results of a token come back to it and are reduced into one
// (DySHARP page, section 1), as the weighted sum of the expert outputs
// (ThunderEP page, section 2.1).  The layout map built at dispatch is used in
// reverse: row slot_of[t][j] of y_perm holds the j-th expert's output for t
// (DySHARP page, section 3.1 item 3).
//
// One wave per token and column slice (a small batch is cut into slices of
// the row so that enough waves are in flight): the token's k row numbers and
// weights are wave-uniform (scalar loads); each lane owns 16-byte chunks of
// the slice, accumulates the k products in float32 in pick order and rounds
// once.  The k loads of a chunk are independent, so each lane keeps k x 16
// bytes in flight; they are non-temporal loads, since every expert-output
// row is read exactly once.  Picks with slot -1 (dropped by the gate threshold) add
// nothing; a token with no kept pick gets a zero row.

#include "moe_internal.h"

namespace moe {

template <int DT, int KMAX>
__global__ void __launch_bounds__(256)
    combine_kernel(const uint4* __restrict__ y_perm, const int32_t* __restrict__ slot_of,
                   const float* __restrict__ topk_w, int T, int k, int nch, int cps,
                   uint4* __restrict__ out) {
  constexpr int EPC = DT == MOE_DTYPE_F32 ? 4 : 8;  // elements per chunk
  const int t = __builtin_amdgcn_readfirstlane(
      (int)(blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)));
  if (t >= T) return;
  const int lane = lane_id();
  long long rows[KMAX];
  float w[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    rows[j] = 0;
    w[j] = 0.0f;
    if (j < k) {
      rows[j] = (long long)slot_of[(long long)t * k + j] * nch;
      w[j] = topk_w[(long long)t * k + j];
    }
  }
  // slot -1: a pick dropped by the gate threshold, nothing to add
  bool has[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) has[j] = j < k && rows[j] >= 0;
  uint4* dst = out + (long long)t * nch;
  const int c0 = (int)blockIdx.y * cps;
  const int c1 = min(nch, c0 + cps);
  for (int c = c0 + lane; c < c1; c += 64) {
    uint4 q[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (has[j])  // each row is read once: stream it past the caches
        q[j] = __builtin_bit_cast(
            uint4, __builtin_nontemporal_load((const u32x4*)&y_perm[rows[j] + c]));
    float acc[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] = 0.0f;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (has[j]) {
        float v[EPC];
        if (DT == MOE_DTYPE_F32) {
          v[0] = __uint_as_float(q[j].x);
          v[1] = __uint_as_float(q[j].y);
          v[2] = __uint_as_float(q[j].z);
          v[3] = __uint_as_float(q[j].w);
        } else {
          unpack8<DT>(q[j], v);
        }
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[e] = fmaf(w[j], v[e], acc[e]);
      }
    }
    if (DT == MOE_DTYPE_F32)
      dst[c] = make_uint4(__float_as_uint(acc[0]), __float_as_uint(acc[1]),
                          __float_as_uint(acc[2]), __float_as_uint(acc[3]));
    else
      dst[c] = pack8<DT>(acc);
  }
}

namespace {
template <int DT>
int launch_combine_dt(const void* y_perm, const int32_t* slot_of, const float* w,
                      int T, int k, int nch, void* out, hipStream_t s) {
  int slices, cps;
  row_slices(T, nch, slices, cps);
  const dim3 grid((T + 3) / 4, slices), block(256);
#define MOE_COMBINE(KM)                                                        \
  hipLaunchKernelGGL((combine_kernel<DT, KM>), grid, block, 0, s,             \
                     (const uint4*)y_perm, slot_of, w, T, k, nch, cps, (uint4*)out)
  if (k <= 1) MOE_COMBINE(1);
  else if (k <= 2) MOE_COMBINE(2);
  else if (k <= 4) MOE_COMBINE(4);
  else if (k <= 8) MOE_COMBINE(8);
  else if (k <= 16) MOE_COMBINE(16);
  else MOE_COMBINE(32);
#undef MOE_COMBINE
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
}  // namespace

int combine_impl(const void* y_perm, const int32_t* slot_of, const float* w,
                 int act_dtype, int T, int H, int k, void* out, hipStream_t s) {
  if (T == 0) return MOE_OK;
  const int elem = act_dtype == MOE_DTYPE_F32 ? 4 : 2;
  const int nch = H * elem / 16;
  switch (act_dtype) {
    case MOE_DTYPE_F32: return launch_combine_dt<MOE_DTYPE_F32>(y_perm, slot_of, w, T, k, nch, out, s);
    case MOE_DTYPE_F16: return launch_combine_dt<MOE_DTYPE_F16>(y_perm, slot_of, w, T, k, nch, out, s);
    case MOE_DTYPE_BF16: return launch_combine_dt<MOE_DTYPE_BF16>(y_perm, slot_of, w, T, k, nch, out, s);
  }
  return MOE_ERR_UNSUPPORTED;
}

}  // namespace moe
