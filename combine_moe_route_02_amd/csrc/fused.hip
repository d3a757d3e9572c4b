// Fused dispatch -> GEMM-1 -> GEMM-2 -> combine, pipelined at token tiles.
//
// The DySHARP page (section 3.2) fuses the chain Dispatch -> GEMM-1 -> GEMM-2
// -> Combine at token granularity: a GEMM row tile starts as soon as the
// tokens it needs are present, and a token's combine fires once its expert
// outputs are ready, with the synchronisation tile aligned to the GEMM tile.
// On one GPU the dispatch is fused into GEMM-1's A load (rows of x are read
// through the layout map, so no permuted copy is written), and the overlap
// is between stages inside one persistent kernel:
//
//   * Eight work queues (workgroup i serves queue i % 8, i.e. one XCD).
//     Each queue holds, in order, its contiguous slice of the GEMM-1 tiles,
//     then of the GEMM-2 tiles, then of the combine token blocks, and hands
//     them out through an atomic counter.
//   * GEMM-1 tile (m, n) signals m's counter after its h stores; a GEMM-2
//     tile of m-tile m waits until all GEMM-1 n-tiles of m are done.
//   * GEMM-2 tile (m, n) signals m's second counter; the combine of a token
//     waits until every m-tile holding one of its local rows is complete.
//     Rows of experts on other GPUs are already present in y_perm.
//   * An item only waits on items of an earlier phase, which running
//     workgroups have taken and finish without waiting on later ones, and
//     the grid never exceeds co-resident capacity, so the queue drains.  A
//     bounded spin backs this up: past the limit the workgroup raises an
//     error flag in the workspace and stops.
//
// Results equal the unfused path: the same tiles, the same accumulation
// order and the same combine order.

#include "gemm_tile.h"

namespace moe {

namespace {

constexpr int kQueues = 8;
constexpr int kHeaderInts = 16;          // queue counters, error flag, padding
// The error flag (header int kQueues) is cleared with the header before every
// launch and raised by a timed-out wait, so after the call it is the call's
// status word at the byte offset the header documents.
static_assert(kQueues * 4 == MOE_FUSED_STATUS_BYTE, "status word offset");
constexpr int kTokensPerItem = 64;       // combine block (16 tokens per wave)
constexpr int kSpinLimit = 1 << 20;      // ~seconds of sleeping spins

struct FusedArgs {
  GemmArgs g1;            // A = x gathered by row_token, B = w13, C = h
  GemmArgs g2;            // A = h, B = w2, C = y_perm
  const int32_t* row_token;
  const int32_t* slot_of;
  const float* topk_w;
  const uint4* y_perm;
  uint4* out;
  int T, k, nch;          // nch: 16-byte chunks per row of H
  int* ws;                // header + cnt1[max_mt] + cnt2[max_mt]
  int max_mt;
};

// Polls use relaxed agent-scope loads (coherent across XCDs, no cache
// maintenance).  A producer makes its rows visible with an agent-scope
// release (a writeback of its XCD's L2) before counting its tile as done.
// The waiting side needs no agent-scope acquire, which on this GPU
// invalidates the whole L2 of the XCD (and with it the weight lines the
// XCD's other workgroups are streaming): the rows a wait guards (h of an
// m-tile, y_perm rows of local experts) are written once per launch, every
// cache starts the launch without them, and no workgroup reads them before
// their producer has written them back and signalled, so no cache can hold
// a stale copy.  A workgroup-scope acquire orders the later loads after the
// poll that saw the count.
__device__ __forceinline__ int load_relaxed(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Block-wide wait until *p >= target (thread 0 spins).  Returns false (for
// the whole block) if the spin limit was hit.
__device__ bool block_wait(const int* p, int target, int* err, int* s_flag) {
  if (threadIdx.x == 0) {
    int ok = 1, spins = 0;
    while (load_relaxed(p) < target) {
      __builtin_amdgcn_s_sleep(8);
      if (++spins > kSpinLimit) {
        __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ok = 0;
        break;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    *s_flag = ok;
  }
  __syncthreads();
  return *s_flag != 0;
}

// Every thread's stores of the tile have completed (vmcnt 0) before the
// barrier; one thread then makes them visible at agent scope and counts the
// tile as done.
__device__ void block_signal(int* p) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __hip_atomic_fetch_add(p, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

__device__ __forceinline__ void slice(int total, int q, int& lo, int& len) {
  const long long a = (long long)total * q / kQueues;
  const long long b = (long long)total * (q + 1) / kQueues;
  lo = (int)a;
  len = (int)(b - a);
}

// One token's output row by one wave: out = sum over picks j < k of
// w_j * y_perm[row_j], in pick order, in float32, rounded once (as
// moe_combine); a dropped pick (row -1) adds nothing.  KM >= k picks are
// loaded for U 16-byte chunks per lane at a time with no condition on any
// load (picks past k and dropped picks load row 0, a lane past the row end
// loads its last chunk; neither is used), so all KM x U loads are in flight
// together: with one wave per SIMD in this kernel, that is what keeps HBM
// busy (one chunk per pick at a time ran the fused combine at under half
// the standalone combine's rate).  Each row is read once: non-temporal loads.
template <int DT, int KM>
__device__ __forceinline__ void combine_row(const uint4* __restrict__ y_perm,
                                            const long long (&rj)[8], const float (&wj)[8],
                                            int k, int nch, uint4* __restrict__ dst,
                                            int lane) {
  constexpr int U = 32 / KM;
  for (int cb = 0; cb < nch; cb += 64 * U) {
    uint4 qv[U][KM];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = min(cb + 64 * u + lane, nch - 1);
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        const long long r = j < k && rj[j] >= 0 ? rj[j] : 0;
        qv[u][j] = __builtin_bit_cast(
            uint4, __builtin_nontemporal_load((const u32x4*)&y_perm[r + c]));
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        if (j < k && rj[j] >= 0) {
          float v[8];
          unpack8<DT>(qv[u][j], v);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] = fmaf(wj[j], v[e], acc[e]);
        }
      }
      const int c = cb + 64 * u + lane;
      if (c < nch) dst[c] = pack8<DT>(acc);
    }
  }
}

template <int DT, int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(WM * WN * 64) fused_layer_kernel(FusedArgs f) {
  typedef DmaTile<DT, EPI_SWIGLU, BM, BN, WM, WN> T1;
  typedef DmaTile<DT, EPI_STORE, BM, BN, WM, WN> T2;
  constexpr int NT = WM * WN * 64;
  constexpr int NWAVE = NT / 64;
  static_assert(T1::SMEM == T2::SMEM, "same stage layout");
  __shared__ __attribute__((aligned(1024))) char smem[T1::SMEM];
  __shared__ int s_pre[1024];
  __shared__ int s_scan[NT];
  __shared__ int s_item, s_flag;

  int* hdr = f.ws;
  int* err = hdr + kQueues;
  int* cnt1 = hdr + kHeaderInts;
  int* cnt2 = cnt1 + f.max_mt;

  const int total_m = build_mtile_table<NT, BM>(f.g1, s_pre, s_scan);
  const int nt1 = f.g1.n_tiles, nt2 = f.g2.n_tiles;
  const int q = (int)blockIdx.x % kQueues;
  int lo1, len1, lo2, len2, lo3, len3;
  slice(total_m * nt1, q, lo1, len1);
  slice(total_m * nt2, q, lo2, len2);
  slice((f.T + kTokensPerItem - 1) / kTokensPerItem, q, lo3, len3);
  const int lane = (int)threadIdx.x & 63;
  const int wave = (int)threadIdx.x >> 6;
  const int e0 = f.g1.e_begin, ng = f.g1.n_groups;
  // When this queue's GEMM-2 slice starts inside a band that began in the
  // previous queue's slice, the band's m-tiles got part of their GEMM-1
  // tiles at the end of the previous queue's GEMM-1 work, so they are the
  // last to be ready; the rest of the slice's bands finished GEMM-1 in this
  // queue, in order.  Their items go first and the straddling band's last.
  int rot2 = 0;
  if (len2 > 0) {
    int b0, b1;
    band_bounds(f.g2, s_pre, lo2, nt2, f.g2.gm, b0, b1);
    if (b0 < lo2 && b1 - lo2 < len2) rot2 = b1 - lo2;
  }

  for (;;) {
    if (threadIdx.x == 0) s_item = __hip_atomic_fetch_add(hdr + q, 1, __ATOMIC_RELAXED,
                                                          __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    int it = s_item;
    __syncthreads();
    if (it < len1) {
      int mt, nt;
      const TileInfo ti = band_tile<BM>(f.g1, s_pre, lo1 + it, nt1, f.g1.gm, mt, nt);
      T1::run(f.g1, ti, nt, smem, f.row_token);
      block_signal(cnt1 + mt);
      continue;
    }
    it -= len1;
    if (it < len2) {
      int mt, nt;
      const int it2 = it + rot2 < len2 ? it + rot2 : it + rot2 - len2;
      const TileInfo ti = band_tile<BM>(f.g2, s_pre, lo2 + it2, nt2, f.g2.gm, mt, nt);
      if (!block_wait(cnt1 + mt, nt1, err, &s_flag)) return;
      T2::run(f.g2, ti, nt, smem, nullptr);
      block_signal(cnt2 + mt);
      continue;
    }
    it -= len2;
    if (it >= len3) return;

    // Combine block: one wave per token, kTokensPerItem / 4 tokens per wave.
    const int r_lo = f.g1.offsets[e0];
    const int r_hi = f.g1.offsets[e0 + ng];
    const int tb = (lo3 + it) * kTokensPerItem;
    for (int ti_ = wave; ti_ < kTokensPerItem; ti_ += NWAVE) {
      const int t = __builtin_amdgcn_readfirstlane(tb + ti_);
      if (t >= f.T) break;
      // lane j < k: the row of pick j and the m-tile that produces it
      int row = 0, mt = -1;
      if (lane < f.k) {
        row = f.slot_of[(long long)t * f.k + lane];
        if (row >= r_lo && row < r_hi) {
          int a = 0, b = ng - 1;  // expert g with offsets[e0+g] <= row < offsets[e0+g+1]
          while (a < b) {
            const int mid = (a + b + 1) >> 1;
            if (f.g1.offsets[e0 + mid] <= row) a = mid; else b = mid - 1;
          }
          mt = (a > 0 ? s_pre[a - 1] : 0) + (row - f.g1.offsets[e0 + a]) / BM;
        }
      }
      int spins = 0;
      bool timed_out = false;
      for (;;) {
        const bool ready = mt < 0 || load_relaxed(cnt2 + mt) >= nt2;
        if (__ballot(!ready) == 0) break;
        __builtin_amdgcn_s_sleep(8);
        if (++spins > kSpinLimit) {
          __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          timed_out = true;
          break;
        }
      }
      if (timed_out) break;
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      const float w = lane < f.k ? f.topk_w[(long long)t * f.k + lane] : 0.0f;
      uint4* dst = f.out + (long long)t * f.nch;
      if (f.k <= 8) {
        // rows and weights in scalar registers (lane j holds pick j), so
        // every test on them is a uniform branch
        long long rj[8];
        float wj[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          rj[j] = (long long)__builtin_amdgcn_readlane(row, j < f.k ? j : 0) * f.nch;
          wj[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j));
        }
        if (f.k <= 1) combine_row<DT, 1>(f.y_perm, rj, wj, f.k, f.nch, dst, lane);
        else if (f.k <= 2) combine_row<DT, 2>(f.y_perm, rj, wj, f.k, f.nch, dst, lane);
        else if (f.k <= 4) combine_row<DT, 4>(f.y_perm, rj, wj, f.k, f.nch, dst, lane);
        else combine_row<DT, 8>(f.y_perm, rj, wj, f.k, f.nch, dst, lane);
        continue;
      }
      for (int c = lane; c < f.nch; c += 64) {
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
        for (int j = 0; j < f.k; ++j) {
          const int rjj = __shfl(row, j, 64);
          const float wjj = __shfl(w, j, 64);
          if (rjj < 0) continue;  // dropped pick
          float v[8];
          unpack8<DT>(f.y_perm[(long long)rjj * f.nch + c], v);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] = fmaf(wjj, v[e], acc[e]);
        }
        dst[c] = pack8<DT>(acc);
      }
    }
    __syncthreads();
    if (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) return;
  }
}

__global__ void zero_ints(int* p, int n) {
  for (int i = (int)(blockIdx.x * blockDim.x + threadIdx.x); i < n;
       i += (int)(gridDim.x * blockDim.x))
    p[i] = 0;
}

int max_mtiles(int T, int k, int E) {
  const long long rows = (long long)T * k;
  return (int)((rows + 127) / 128 + E + 8);
}

template <int DT, int BM, int BN, int WM, int WN>
int launch_fused(FusedArgs f, int max_rows, hipStream_t s) {
  auto kern = fused_layer_kernel<DT, BM, BN, WM, WN>;
  static int occ = 0;
  if (occ == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, WM * WN * 64, 0) !=
            hipSuccess ||
        n <= 0)
      n = 1;
    occ = n;
  }
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return MOE_ERR_HIP;
  f.g1.n_tiles = f.g1.Nb / BN;
  f.g2.n_tiles = f.g2.Nb / BN;
  f.g1.gm = f.g2.gm = 8;
  // grid within co-resident capacity (forward progress), a multiple of 8
  int grid = (cus * occ) / kQueues * kQueues;
  if (grid < kQueues) return MOE_ERR_UNSUPPORTED;
  const int nz = kHeaderInts + 2 * f.max_mt;
  hipLaunchKernelGGL(zero_ints, dim3((nz + 255) / 256), dim3(256), 0, s, f.ws, nz);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(WM * WN * 64), 0, s, f);
  (void)max_rows;
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace

size_t fused_ws_bytes(int T, int H, int E, int k, int I) {
  (void)H;
  (void)I;
  return (size_t)(kHeaderInts + 2 * max_mtiles(T, k, E)) * sizeof(int);
}

int fused_impl(const void* x, const int32_t* offsets, const int32_t* slot_of,
               const int32_t* row_token, const float* topk_w, int act_dtype, int T, int H,
               int E, int k, int I, int e_begin, int e_end, int act, const void* w13,
               const void* w2, void* h_ws, void* y_perm, void* out, void* ws, size_t ws_bytes,
               hipStream_t s) {
  (void)act;
  (void)ws_bytes;
  const int n_groups = e_end - e_begin;
  if (n_groups > 1024) return MOE_ERR_UNSUPPORTED;
  const int max_rows = T * (k < n_groups ? k : n_groups);
  FusedArgs f{};
  GemmArgs& a = f.g1;
  a.A = x;
  a.lda = H;
  a.B = w13;
  a.strideB = 2ll * I * H;
  a.ldb = H;
  a.C = h_ws;
  a.ldc = I;
  a.offsets = offsets;
  a.e_begin = e_begin;
  a.n_groups = n_groups;
  a.c_local = 1;
  a.c_rows = max_rows;
  a.Nb = 2 * I;
  a.I = I;
  a.K = H;
  GemmArgs& b = f.g2;
  b.A = h_ws;
  b.lda = I;
  b.B = w2;
  b.strideB = (long long)H * I;
  b.ldb = I;
  b.C = y_perm;
  b.ldc = H;
  b.offsets = offsets;
  b.e_begin = e_begin;
  b.n_groups = n_groups;
  b.a_local = 1;
  b.a_rows = max_rows;
  b.Nb = H;
  b.K = I;
  f.row_token = row_token;
  f.slot_of = slot_of;
  f.topk_w = topk_w;
  f.y_perm = (const uint4*)y_perm;
  f.out = (uint4*)out;
  f.T = T;
  f.k = k;
  f.nch = H * 2 / 16;
  f.ws = (int*)ws;
  f.max_mt = max_mtiles(T, k, E);
  if ((2 * I) % 256 || H % 256) return MOE_ERR_UNSUPPORTED;
  // the GEMM tiles address x rows and one expert's weights with 32-bit offsets
  if ((long long)T * H * 2 >= (1ll << 32) || 2ll * I * H * 2 >= (1ll << 32))
    return MOE_ERR_UNSUPPORTED;
  const double avg = (double)max_rows / (n_groups > 0 ? n_groups : 1);
  const bool big = avg >= 384.0;
  if (act_dtype == MOE_DTYPE_BF16) {
    return big ? launch_fused<MOE_DTYPE_BF16, 256, 256, 2, 2>(f, max_rows, s)
               : launch_fused<MOE_DTYPE_BF16, 128, 256, 2, 2>(f, max_rows, s);
  }
  return big ? launch_fused<MOE_DTYPE_F16, 256, 256, 2, 2>(f, max_rows, s)
             : launch_fused<MOE_DTYPE_F16, 128, 256, 2, 2>(f, max_rows, s);
}

}  // namespace moe
