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
//   layout_one_tile  hist + scan + slots in one block for T <= 256
//   layout_few_experts  hist + scan + slots in one launch for E <= 32: every
//           block counts all picks, then ranks its own tile's
//   slots_from_table  after hist: totals, offsets, tile bases and slots in
//           one kernel for up to kTableMaxTiles tiles (every block reads
//           the whole tile-count table)
//   hist    per-tile expert histogram (LDS integer atomics: exact counts)
//   scan    per-expert prefix over tiles -> tile bases, counts, offsets
//   slots   rank of each pick among earlier picks of the same expert:
//           per wave and expert a 64-bit mask of the lanes that picked it
//           (LDS atomic OR); earlier waves add their popcounts, earlier lanes
//           of the same wave the popcount of the lanes below; no atomic
//           decides any order, so the layout is deterministic and
//           token-stable
//   gather  one wave per token (and column slice, for small batches): each
//           16-byte chunk of x[t] is loaded once and stored to every local
//           row of that token
// A pick of -1 (dropped by the gate threshold) is not counted, gets slot -1
// and no row; offsets[E] is then the number of kept picks.

#include "moe_internal.h"

namespace moe {

constexpr int TILE = 256;
// Batches of at most this many picks and at most 32 experts take the
// one-launch layout (each block counts every pick).
constexpr long long kFewExpertsMaxPicks = 32768;

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
    for (int j = 0; j < k; ++j) {
      const int e = p[j];
      if (e >= 0) atomicAdd(&hist[e], 1);  // -1: dropped by the gate threshold
    }
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

// Lanes of this wave that picked expert e, as a 64-bit mask per wave and
// expert in LDS (set with atomic OR, so the result does not depend on the
// order of the atomics): the per-wave count of e is its popcount and the
// rank of a pick among the wave's earlier picks of e is the popcount of the
// lanes below it.  The k picks of a token are distinct experts.
template <int KMAX>
__global__ void __launch_bounds__(TILE)
    slots_kernel(const int32_t* __restrict__ idx, int T, int E, int k, int n_tiles,
                 const int32_t* __restrict__ tile_base, const int32_t* __restrict__ offsets,
                 int32_t* __restrict__ slot_of, int32_t* __restrict__ row_token) {
  extern __shared__ uint64_t lanes_of[];  // [4][E] lane masks
  int* wbase = (int*)(lanes_of + 4 * E);  // [4][E] exclusive prefix over waves
  const int tile = (int)blockIdx.x;
  const int wave = (int)threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 4 * E; i += TILE) lanes_of[i] = 0;
  __syncthreads();
  const int t = tile * TILE + (int)threadIdx.x;
  const bool valid = t < T;
  int pk[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) pk[j] = (valid && j < k) ? idx[(long long)t * k + j] : 0;
  const uint64_t bit = 1ull << lane_id();
  if (valid)
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (j < k && pk[j] >= 0) atomicOr((unsigned long long*)&lanes_of[wave * E + pk[j]], bit);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += TILE) {
    int run = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      wbase[w * E + e] = run;
      run += __popcll(lanes_of[w * E + e]);
    }
  }
  __syncthreads();
  if (!valid) return;
  const uint64_t lt = bit - 1;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j >= k) break;
    const int e = pk[j];
    if (e < 0) {  // dropped pick: no row
      slot_of[(long long)t * k + j] = -1;
      continue;
    }
    const int r = offsets[e] + tile_base[(long long)e * n_tiles + tile] + wbase[wave * E + e] +
                  __popcll(lanes_of[wave * E + e] & lt);
    slot_of[(long long)t * k + j] = r;
    row_token[r] = t;
  }
}

// Whole layout of a batch of at most one tile (T <= 256, a decode batch) in
// one block: lane masks per wave and expert as in slots_kernel, counts and
// offsets from a block scan over experts, tile base 0.
template <int KMAX>
__global__ void __launch_bounds__(TILE)
    layout_one_tile_kernel(const int32_t* __restrict__ idx, int T, int E, int k,
                           int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                           int32_t* __restrict__ slot_of, int32_t* __restrict__ row_token) {
  extern __shared__ uint64_t lanes_of[];  // [4][E] lane masks
  int* wbase = (int*)(lanes_of + 4 * E);  // [4][E] exclusive prefix over waves
  int* s_off = wbase + 4 * E;             // [E] offsets
  __shared__ int s_part[TILE];
  const int wave = (int)threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 4 * E; i += TILE) lanes_of[i] = 0;
  __syncthreads();
  const int t = (int)threadIdx.x;
  const bool valid = t < T;
  int pk[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) pk[j] = (valid && j < k) ? idx[(long long)t * k + j] : 0;
  const uint64_t bit = 1ull << lane_id();
  if (valid)
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (j < k && pk[j] >= 0) atomicOr((unsigned long long*)&lanes_of[wave * E + pk[j]], bit);
  __syncthreads();
  // thread i owns experts [i * per, (i + 1) * per): prefix over the 4 waves
  // and the expert's count
  const int per = (E + TILE - 1) / TILE;
  int run_total = 0;
  for (int q = 0; q < per; ++q) {
    const int e = (int)threadIdx.x * per + q;
    if (e < E) {
      int run = 0;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        wbase[w * E + e] = run;
        run += __popcll(lanes_of[w * E + e]);
      }
      counts[e] = run;
      s_off[e] = run;  // count for now
      run_total += run;
    }
  }
  // block scan of the per-thread totals -> exclusive base of each thread
  s_part[threadIdx.x] = run_total;
  __syncthreads();
  for (int o = 1; o < TILE; o <<= 1) {
    const int add = (int)threadIdx.x >= o ? s_part[threadIdx.x - o] : 0;
    __syncthreads();
    s_part[threadIdx.x] += add;
    __syncthreads();
  }
  int base = s_part[threadIdx.x] - run_total;
  for (int q = 0; q < per; ++q) {
    const int e = (int)threadIdx.x * per + q;
    if (e < E) {
      const int c = s_off[e];
      s_off[e] = base;
      offsets[e] = base;
      base += c;
    }
  }
  if (threadIdx.x == TILE - 1) offsets[E] = s_part[TILE - 1];
  __syncthreads();
  if (!valid) return;
  const uint64_t lt = bit - 1;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j >= k) break;
    const int e = pk[j];
    if (e < 0) {  // dropped pick: no row
      slot_of[(long long)t * k + j] = -1;
      continue;
    }
    const int r = s_off[e] + wbase[wave * E + e] + __popcll(lanes_of[wave * E + e] & lt);
    slot_of[(long long)t * k + j] = r;
    row_token[r] = t;
  }
}

// Whole layout of a multi-tile batch with few experts (E <= EMAX) in one
// launch, one block per 256-token tile: every block counts all picks itself
// (16-byte coalesced reads of topk_idx, one counter per expert in each
// thread, so no atomics pile onto a few hot counters), which gives the
// totals (counts, offsets) and the picks of each expert before its own tile
// (its tile base); then its tile's slots exactly as in slots_kernel.  One
// launch instead of histogram, scan and slots; the same layout.
__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, MOE_WAVE);
  return v;
}

// Picks per expert of the whole batch (all) and of the picks before n_bef
// (bef), in one pass over topk_idx with up to 16 16-byte loads in flight per
// thread.  Counters are packed eight to a 64-bit register, 8 bits each: a
// thread sees at most kFewExpertsMaxPicks / TILE = 128 picks.  n_bef is a
// multiple of 4.
template <int EMAX>
__device__ __forceinline__ void add_pick(int e, bool before, uint64_t* all, uint64_t* bef) {
  // e outside [0, EMAX) (a dropped pick, -1) adds nothing
  const uint64_t inc = (e >= 0 && e < EMAX) ? 1ull << (8 * (e & 7)) : 0ull;
#pragma unroll
  for (int g = 0; g < EMAX / 8; ++g) {
    const uint64_t x = (e >> 3) == g ? inc : 0ull;
    all[g] += x;
    bef[g] += before ? x : 0ull;
  }
}

template <int EMAX>
__device__ __forceinline__ void count_picks(const int32_t* __restrict__ idx, int n_all,
                                            int n_bef, uint64_t* all, uint64_t* bef) {
  constexpr int U = 16;
  const int v_end = n_all >> 2, v_bef = n_bef >> 2;
  for (int v0 = (int)threadIdx.x; v0 < v_end; v0 += U * TILE) {
    int4 q[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (v0 + u * TILE < v_end) q[u] = ((const int4*)idx)[v0 + u * TILE];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (v0 + u * TILE >= v_end) break;
      const bool before = v0 + u * TILE < v_bef;
      add_pick<EMAX>(q[u].x, before, all, bef);
      add_pick<EMAX>(q[u].y, before, all, bef);
      add_pick<EMAX>(q[u].z, before, all, bef);
      add_pick<EMAX>(q[u].w, before, all, bef);
    }
  }
  // the last n_all % 4 picks (all past n_bef)
  for (int n = (v_end << 2) + (int)threadIdx.x; n < n_all; n += TILE)
    add_pick<EMAX>(idx[n], false, all, bef);
}

template <int KMAX, int EMAX>
__global__ void __launch_bounds__(TILE)
    layout_few_experts_kernel(const int32_t* __restrict__ idx, int T, int E, int k,
                              int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                              int32_t* __restrict__ slot_of, int32_t* __restrict__ row_token) {
  __shared__ uint64_t lanes_of[4][EMAX];
  __shared__ int s_cnt[2][4][EMAX];  // [before this tile, all][wave][expert]
  __shared__ int wbase[4][EMAX];
  __shared__ int s_base[EMAX];       // offsets[e] + picks of e before this tile
  const int tile = (int)blockIdx.x;
  const int wave = (int)threadIdx.x >> 6;
  const int lane = lane_id();
  for (int i = threadIdx.x; i < 4 * EMAX; i += TILE) (&lanes_of[0][0])[i] = 0;
  // 1. this tile's picks (loads issued first, they overlap the count)
  const int t = tile * TILE + (int)threadIdx.x;
  const bool valid = t < T;
  int pk[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) pk[j] = (valid && j < k) ? idx[(long long)t * k + j] : -1;
  // 2. picks per expert over the batch and before this tile
  const int n_all = T * k, n_bef = tile * TILE * k;
  uint64_t all[EMAX / 8], bef[EMAX / 8];
#pragma unroll
  for (int g = 0; g < EMAX / 8; ++g) all[g] = bef[g] = 0;
  count_picks<EMAX>(idx, n_all, n_bef, all, bef);
#pragma unroll
  for (int e = 0; e < EMAX; ++e) {
    const int a = wave_sum_int((int)((all[e >> 3] >> (8 * (e & 7))) & 0xff));
    const int b = wave_sum_int((int)((bef[e >> 3] >> (8 * (e & 7))) & 0xff));
    if (lane == 0) {
      s_cnt[0][wave][e] = b;
      s_cnt[1][wave][e] = a;
    }
  }
  const uint64_t bit = 1ull << lane;
  __syncthreads();  // lanes_of cleared, s_cnt written
  // lane masks of this tile's picks per wave and expert
#pragma unroll
  for (int j = 0; j < KMAX; ++j)
    if (pk[j] >= 0) atomicOr((unsigned long long*)&lanes_of[wave][pk[j]], bit);
  // 3. offsets (exclusive scan over experts of the totals) and tile bases
  if (wave == 0) {
    const int e = lane;
    int tot = 0, before = 0;
    if (e < E) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        before += s_cnt[0][w][e];
        tot += s_cnt[1][w][e];
      }
    }
    int inc = tot;  // inclusive scan over the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(inc, o, MOE_WAVE);
      if (lane >= o) inc += u;
    }
    if (e < E) {
      s_base[e] = inc - tot + before;
      if (tile == 0) {
        counts[e] = tot;
        offsets[e] = inc - tot;
        if (e == E - 1) offsets[E] = inc;
      }
    }
  }
  __syncthreads();  // lane masks and bases complete
  for (int e = threadIdx.x; e < E; e += TILE) {
    int run = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      wbase[w][e] = run;
      run += __popcll(lanes_of[w][e]);
    }
  }
  __syncthreads();
  if (!valid) return;
  const uint64_t lt = bit - 1;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j >= k) break;
    const int e = pk[j];
    if (e < 0) {  // dropped pick: no row
      slot_of[(long long)t * k + j] = -1;
      continue;
    }
    const int r = s_base[e] + wbase[wave][e] + __popcll(lanes_of[wave][e] & lt);
    slot_of[(long long)t * k + j] = r;
    row_token[r] = t;
  }
}

// Layout of a multi-tile batch with many experts after hist_kernel: one
// block per 256-token tile reads the whole tile-count table (each thread the
// row of its experts, 16 bytes at a time), which gives every expert's total
// (counts, offsets by a block scan over experts) and its picks before this
// tile (the tile base); then its tile's slots exactly as in slots_kernel.
// Two launches instead of histogram, scan and slots.  Every block reads the
// whole table, so the host uses it up to kTableMaxTiles tiles.
constexpr int kTableMaxTiles = 256;

template <int KMAX>
__global__ void __launch_bounds__(TILE)
    slots_from_table_kernel(const int32_t* __restrict__ idx, int T, int E, int k,
                            int n_tiles, const int32_t* __restrict__ tile_counts,
                            int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                            int32_t* __restrict__ slot_of, int32_t* __restrict__ row_token) {
  extern __shared__ uint64_t dyn[];
  uint64_t* lanes_of = dyn;                  // [4][E] lane masks of this tile
  int* wbase = (int*)(lanes_of + 4 * E);     // [4][E] exclusive prefix over waves
  int* s_base = wbase + 4 * E;               // [E] offsets[e] + picks before the tile
  __shared__ int s_part[TILE];
  const int tile = (int)blockIdx.x;
  const int tid = (int)threadIdx.x;
  const int wave = tid >> 6;
  for (int i = tid; i < 4 * E; i += TILE) lanes_of[i] = 0;
  const int t = tile * TILE + tid;
  const bool valid = t < T;
  int pk[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) pk[j] = (valid && j < k) ? idx[(long long)t * k + j] : -1;
  // thread i owns the contiguous experts [i * per, (i + 1) * per): their
  // totals and their picks before this tile, from the table rows
  const int per = (E + TILE - 1) / TILE;
  int run_total = 0;
  for (int q = 0; q < per; ++q) {
    const int e = tid * per + q;
    if (e >= E) break;
    const int32_t* row = tile_counts + (long long)e * n_tiles;
    int bef = 0, tot = 0;
    int b = 0;
    if ((n_tiles & 3) == 0) {  // rows start 16-byte aligned: 4 tiles per load
      for (; b < n_tiles; b += 4) {
        const int4 v = *(const int4*)(row + b);
        tot += v.x + v.y + v.z + v.w;
        bef += (b < tile ? v.x : 0) + (b + 1 < tile ? v.y : 0) + (b + 2 < tile ? v.z : 0) +
               (b + 3 < tile ? v.w : 0);
      }
    }
    for (; b < n_tiles; ++b) {
      const int v = row[b];
      tot += v;
      bef += b < tile ? v : 0;
    }
    s_base[e] = bef;   // picks before the tile for now
    wbase[e] = tot;    // total for now (wbase is rebuilt below)
    run_total += tot;
  }
  s_part[tid] = run_total;
  __syncthreads();
  for (int o = 1; o < TILE; o <<= 1) {
    const int add = tid >= o ? s_part[tid - o] : 0;
    __syncthreads();
    s_part[tid] += add;
    __syncthreads();
  }
  int base = s_part[tid] - run_total;
  for (int q = 0; q < per; ++q) {
    const int e = tid * per + q;
    if (e >= E) break;
    const int c = wbase[e];
    s_base[e] += base;
    if (tile == 0) {
      counts[e] = c;
      offsets[e] = base;
    }
    base += c;
  }
  if (tile == 0 && tid == TILE - 1) offsets[E] = s_part[TILE - 1];
  __syncthreads();  // the totals in wbase are read; lane masks cleared
  const uint64_t bit = 1ull << lane_id();
  if (valid)
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (pk[j] >= 0) atomicOr((unsigned long long*)&lanes_of[wave * E + pk[j]], bit);
  __syncthreads();
  for (int e = tid; e < E; e += TILE) {
    int run = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      wbase[w * E + e] = run;
      run += __popcll(lanes_of[w * E + e]);
    }
  }
  __syncthreads();
  if (!valid) return;
  const uint64_t lt = bit - 1;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j >= k) break;
    const int e = pk[j];
    if (e < 0) {  // dropped pick: no row
      slot_of[(long long)t * k + j] = -1;
      continue;
    }
    const int r = s_base[e] + wbase[wave * E + e] + __popcll(lanes_of[wave * E + e] & lt);
    slot_of[(long long)t * k + j] = r;
    row_token[r] = t;
  }
}

// One wave per token; rows of local experts only.  KMAX >= k bounds the
// unrolled pick loop so the (wave-uniform) row numbers stay in registers.
template <int KMAX>
__global__ void __launch_bounds__(256)
    gather_kernel(const uint4* __restrict__ x, const int32_t* __restrict__ idx,
                  const int32_t* __restrict__ slot_of, int T, int k, int e_begin,
                  int e_end, int nch /* 16-byte chunks per row */,
                  int cps /* chunks per column slice */, uint4* __restrict__ x_perm) {
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
  const int c0 = (int)blockIdx.y * cps;
  const int c1 = min(nch, c0 + cps);
  constexpr int U = 4;
  int c = c0 + lane;
  for (; c + (U - 1) * 64 < c1; c += U * 64) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = src[c + u * 64];
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (loc[j])
#pragma unroll
        for (int u = 0; u < U; ++u) x_perm[rows[j] + c + u * 64] = v[u];
  }
  for (; c < c1; c += 64) {
    const uint4 v = src[c];
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (loc[j]) x_perm[rows[j] + c] = v;
  }
}

// fp8 transport of the dispatched rows (ThunderEP page, section 3.3: send
// the activations in 8 bits).  One 256-thread block per token with a local
// pick: the block reads the bf16 row once for its amax, picks the power-of-
// two scale 2^e (the smallest with amax <= 448 * 2^e, so the scaling is
// exact and nothing saturates), then reads the row again (an L2 hit) and
// writes E4M3 codes of x * 2^-e, 8 bytes per 16-byte chunk, to every local
// row of the token, plus 2^e as that row's scale.
template <int KMAX>
__global__ void __launch_bounds__(256)
    gather_fp8_kernel(const uint4* __restrict__ x, const int32_t* __restrict__ idx,
                      const int32_t* __restrict__ slot_of, int T, int k, int e_begin,
                      int e_end, int nch /* 16-byte bf16 chunks per row */,
                      uint2* __restrict__ xq, float* __restrict__ xscale) {
  __shared__ float s_max[4];
  const int t = (int)blockIdx.x;
  const int tid = (int)threadIdx.x;
  long long rows[KMAX];
  int slots[KMAX];
  bool loc[KMAX];
  bool any = false;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    loc[j] = false;
    rows[j] = 0;
    slots[j] = 0;
    if (j < k) {
      const int e = idx[(long long)t * k + j];
      loc[j] = e >= e_begin && e < e_end;
      slots[j] = slot_of[(long long)t * k + j];
      rows[j] = (long long)slots[j] * nch;
      any |= loc[j];
    }
  }
  if (!any) return;  // block-uniform
  const uint4* src = x + (long long)t * nch;
  float m = 0.0f;
  for (int c = tid; c < nch; c += 256) {
    float f[8];
    unpack8<MOE_DTYPE_BF16>(src[c], f);
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
  }
  m = wave_max(m);
  if (lane_id() == 0) s_max[tid >> 6] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
  const int e = e4m3_row_exponent(amax);
  for (int c = tid; c < nch; c += 256) {
    float f[8];
    unpack8<MOE_DTYPE_BF16>(src[c], f);
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i >> 2] |= f32_to_e4m3(ldexpf(f[i], -e)) << (8 * (i & 3));
    const uint2 q = make_uint2(w[0], w[1]);
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (loc[j]) xq[rows[j] + c] = q;
  }
  if (tid == 0) {
    const float sc = ldexpf(1.0f, e);
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (loc[j]) xscale[slots[j]] = sc;
  }
}

int dispatch_impl(const void* x, int act_dtype, const int32_t* idx, int T, int H,
                  int E, int k, int e_begin, int e_end, int32_t* counts,
                  int32_t* offsets, int32_t* slot_of, int32_t* row_token,
                  void* x_perm, float* x_scale, void* ws, hipStream_t s) {
  const int n_tiles = (T + TILE - 1) / TILE;
  int32_t* tile_counts = (int32_t*)ws;
  int32_t* tile_base = tile_counts + (size_t)E * (n_tiles > 0 ? n_tiles : 1);
#define MOE_BY_K(MACRO)                                                         \
  do {                                                                          \
    if (k <= 1) MACRO(1);                                                       \
    else if (k <= 2) MACRO(2);                                                  \
    else if (k <= 4) MACRO(4);                                                  \
    else if (k <= 8) MACRO(8);                                                  \
    else if (k <= 16) MACRO(16);                                                \
    else MACRO(32);                                                             \
  } while (0)
  if (n_tiles == 1) {
#define MOE_LAYOUT1(KM)                                                              \
  hipLaunchKernelGGL((layout_one_tile_kernel<KM>), dim3(1), dim3(TILE), 13 * E * sizeof(int), \
                     s, idx, T, E, k, counts, offsets, slot_of, row_token)
    MOE_BY_K(MOE_LAYOUT1);
#undef MOE_LAYOUT1
  } else if (n_tiles > 1 && E <= 32 && (long long)T * k <= kFewExpertsMaxPicks) {
#define MOE_LAYOUTF(KM)                                                                   \
  do {                                                                                    \
    if (E <= 8)                                                                           \
      hipLaunchKernelGGL((layout_few_experts_kernel<KM, 8>), dim3(n_tiles), dim3(TILE), 0, \
                         s, idx, T, E, k, counts, offsets, slot_of, row_token);           \
    else if (E <= 16)                                                                     \
      hipLaunchKernelGGL((layout_few_experts_kernel<KM, 16>), dim3(n_tiles), dim3(TILE), 0, \
                         s, idx, T, E, k, counts, offsets, slot_of, row_token);           \
    else                                                                                  \
      hipLaunchKernelGGL((layout_few_experts_kernel<KM, 32>), dim3(n_tiles), dim3(TILE), 0, \
                         s, idx, T, E, k, counts, offsets, slot_of, row_token);           \
  } while (0)
    MOE_BY_K(MOE_LAYOUTF);
#undef MOE_LAYOUTF
  } else if (n_tiles > 1 && n_tiles <= kTableMaxTiles) {
    hipLaunchKernelGGL(hist_kernel, dim3(n_tiles), dim3(TILE), E * sizeof(int), s, idx, T, E,
                       k, n_tiles, tile_counts);
    // lane masks, wave bases and tile bases (dynamic LDS)
    const size_t lds = (size_t)E * (4 * sizeof(uint64_t) + 5 * sizeof(int));
#define MOE_SLOTST(KM)                                                                  \
  hipLaunchKernelGGL((slots_from_table_kernel<KM>), dim3(n_tiles), dim3(TILE), lds, s, idx, \
                     T, E, k, n_tiles, tile_counts, counts, offsets, slot_of, row_token)
    MOE_BY_K(MOE_SLOTST);
#undef MOE_SLOTST
  } else {
    if (n_tiles > 0) {
      hipLaunchKernelGGL(hist_kernel, dim3(n_tiles), dim3(TILE), E * sizeof(int), s, idx,
                         T, E, k, n_tiles, tile_counts);
    }
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, tile_counts, E, n_tiles,
                       tile_base, counts, offsets);
    if (n_tiles > 0) {
#define MOE_SLOTS(KM)                                                                \
  hipLaunchKernelGGL((slots_kernel<KM>), dim3(n_tiles), dim3(TILE), 12 * E * sizeof(int), s, \
                     idx, T, E, k, n_tiles, tile_base, offsets, slot_of, row_token)
      MOE_BY_K(MOE_SLOTS);
#undef MOE_SLOTS
    }
  }
  if (n_tiles > 0 && e_end > e_begin && x_scale) {
    // fp8 transport: x_perm holds E4M3 codes, x_scale one scale per row
    const int nch = H * 2 / 16;
#define MOE_GATHER8(KM)                                                        \
  hipLaunchKernelGGL((gather_fp8_kernel<KM>), dim3(T), dim3(256), 0, s,         \
                     (const uint4*)x, idx, slot_of, T, k, e_begin, e_end, nch,  \
                     (uint2*)x_perm, x_scale)
    MOE_BY_K(MOE_GATHER8);
#undef MOE_GATHER8
  } else if (n_tiles > 0 && e_end > e_begin) {
    const int elem = act_dtype == MOE_DTYPE_F32 ? 4 : 2;
    const int nch = H * elem / 16;
    int slices, cps;
    row_slices(T, nch, slices, cps);
    const dim3 grid((T + 3) / 4, slices), block(256);
#define MOE_GATHER(KM)                                                         \
  hipLaunchKernelGGL((gather_kernel<KM>), grid, block, 0, s, (const uint4*)x, idx, \
                     slot_of, T, k, e_begin, e_end, nch, cps, (uint4*)x_perm)
    MOE_BY_K(MOE_GATHER);
#undef MOE_GATHER
  }
#undef MOE_BY_K
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

size_t dispatch_ws_bytes(int T, int E) {
  const size_t n_tiles = (size_t)((T + TILE - 1) / TILE);
  return 2 * (size_t)E * (n_tiles > 0 ? n_tiles : 1) * sizeof(int32_t);
}

}  // namespace moe
