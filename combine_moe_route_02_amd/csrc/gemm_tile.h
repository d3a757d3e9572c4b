// Building blocks of the grouped GEMMs, shared by the standalone kernels and
// the fused dispatch -> GEMM-1 -> GEMM-2 -> combine kernel.
#pragma once

#include "moe_internal.h"

namespace moe {

template <int NT>
__device__ __forceinline__ int block_incl_scan(int v, int* s) {
  s[threadIdx.x] = v;
  __syncthreads();
#pragma unroll
  for (int o = 1; o < NT; o <<= 1) {
    int t = (threadIdx.x >= (unsigned)o) ? s[threadIdx.x - o] : 0;
    __syncthreads();
    s[threadIdx.x] += t;
    __syncthreads();
  }
  return s[threadIdx.x];
}

struct TileInfo {
  int g, r0, r1, base;
};

// Per-workgroup table of m-tiles: s_pre[g] = number of m-tiles of groups
// 0..g (inclusive prefix), built once from the device-side offsets.  Returns
// the total number of m-tiles.  All threads must call it.
template <int NT, int BM>
__device__ __forceinline__ int build_mtile_table(const GemmArgs& p, int* s_pre, int* s_tmp) {
  if (p.offsets == nullptr) {
    if (threadIdx.x == 0) s_pre[0] = (p.dense_M + BM - 1) / BM;
    __syncthreads();
    return s_pre[0];
  }
  int carry = 0;
  for (int b = 0; b < p.n_groups; b += NT) {
    const int g = b + (int)threadIdx.x;
    int tiles = 0;
    if (g < p.n_groups) {
      const int o0 = p.offsets[p.e_begin + g];
      const int o1 = p.offsets[p.e_begin + g + 1];
      tiles = (o1 - o0 + BM - 1) / BM;
    }
    const int incl = block_incl_scan<NT>(tiles, s_tmp) + carry;
    if (g < p.n_groups) s_pre[g] = incl;
    carry += s_tmp[NT - 1];
    __syncthreads();
  }
  return carry;
}

// Tile t of the expert-band order -> its m-tile, n-tile and rows.  The tiles
// of one group (its m-tiles x all n-tiles) are consecutive, so every weight
// tile of a group is used by all of that group's m-tiles close together in
// time: one HBM read, L2 hits after.  A group with more than gm m-tiles is cut
// into bands of gm m-tiles; inside a band the m-tile index runs fastest.
template <int BM>
__device__ __forceinline__ TileInfo band_tile(const GemmArgs& p, const int* s_pre, int t,
                                              int n_tiles, int gm, int& mt, int& nt) {
  int g = 0;
  if (p.offsets != nullptr) {
    int lo = 0, hi = p.n_groups - 1;  // first g whose tiles end after t
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (s_pre[mid] * n_tiles > t) hi = mid; else lo = mid + 1;
    }
    g = lo;
  }
  const int m_before = g > 0 ? s_pre[g - 1] : 0;
  const int mt_g = s_pre[g] - m_before;
  const int w = t - m_before * n_tiles;
  const int full = mt_g / gm;
  const int per_band = gm * n_tiles;
  const int band = w / per_band;
  int mloc;
  if (band < full) {
    const int r = w - band * per_band;
    nt = r / gm;
    mloc = band * gm + r % gm;
  } else {
    const int gl = mt_g - full * gm;
    const int r = w - full * per_band;
    nt = r / gl;
    mloc = full * gm + r % gl;
  }
  mt = m_before + mloc;
  TileInfo ti;
  if (p.offsets == nullptr) {
    ti.g = 0;
    ti.r0 = mt * BM;
    ti.r1 = p.dense_M;
    ti.base = 0;
  } else {
    ti.g = g;
    ti.base = p.offsets[p.e_begin];
    ti.r0 = p.offsets[p.e_begin + g] + mloc * BM;
    ti.r1 = p.offsets[p.e_begin + g + 1];
  }
  return ti;
}

// The share of tiles [lo, hi) of this workgroup's XCD and its stride.  The
// hardware places workgroup i on XCD i % 8, so the persistent grid (a
// multiple of 8) gives every XCD gridDim/8 workgroups and a contiguous,
// equal slice of the tile order.
__device__ __forceinline__ void xcd_share(int total, int& first, int& end, int& stride) {
  const int xcd = (int)blockIdx.x & 7;
  const int per = (int)gridDim.x >> 3;
  const long long lo = (long long)total * xcd / 8;
  const long long hi = (long long)total * (xcd + 1) / 8;
  first = (int)lo + ((int)blockIdx.x >> 3);
  end = (int)hi;
  stride = per;
}

template <int DT>
struct MfmaOp;
template <>
struct MfmaOp<MOE_DTYPE_BF16> {
  typedef bf16x8 V;
  static __device__ __forceinline__ f32x16 run(V a, V b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct MfmaOp<MOE_DTYPE_F16> {
  typedef f16x8 V;
  static __device__ __forceinline__ f32x16 run(V a, V b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + __expf(-g)) * u;
}

__device__ __forceinline__ float gelu_erf(float a) {
  return 0.5f * a * (1.0f + erff(a * 0.70710678118654752f));
}

// ---------------------------------------------------------------------------
// 16-bit weights: direct-to-LDS staging (global_load_lds_dwordx4), BK = 32,
// four LDS stages, loads issued three k-steps ahead.
//
// Stage layout: rows of 64 bytes (32 values); 16-byte chunk kc of row r sits
// at chunk kc ^ dma_swz(r), so the 32 rows an MFMA operand read touches
// (same logical chunk) spread over all bank groups.  One wave instruction
// fills one 1 KB block (16 rows): lane p writes row p/4, physical chunk p%4,
// and fetches the logical chunk that belongs there.  The hardware performs
// these LDS writes; the wave only tracks them with vmcnt, so each k-step
// waits for its own stage's loads (vmcnt = loads issued after it) and then a
// barrier makes every wave's loads visible.
// ---------------------------------------------------------------------------

// LDS chunk swizzle of a 64-byte row: conflict-free for the 32 rows of an
// MFMA operand read whether the LDS serves 8 lanes x 16 B (32 banks) or
// 16 lanes x 16 B (64 banks) per cycle.
__device__ __forceinline__ int dma_swz(int row) { return ((row >> 2) & 3) ^ (row & 2); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Workgroup barrier for LDS hand-off that does not drain outstanding loads.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt((0x3F & 0xF) | (0x7 << 4) | (0x0 << 8) | ((0x3F >> 4) << 14));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One wave-wide 16-byte-per-lane copy global -> LDS (global_load_lds_dwordx4):
// lane l's 16 bytes land at LDS byte address lds_base + 16 * l.  Issued
// from asm so that the compiler does not add its own conservative vmcnt(0)
// before every later LDS read; the instruction writes no VGPR, and the
// kernel's counted vmcnt waits order it before the reads of its stage.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(lds_base)
               : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// One BM x BN output tile of a grouped GEMM with 16-bit weights (see the
// stage layout above).  A rows come from p.A at row r - a_sub, or, with
// a_gather, at row a_gather[r] (the fused kernel reads token rows of x
// through the layout map instead of a gathered copy).  smem must hold
// SMEM bytes; all threads of the block call it.
template <int DT, int EPI, int BM, int BN, int WM, int WN>
struct DmaTile {
  static constexpr int NW = WM * WN;
  static constexpr int NT = NW * 64;
  static constexpr int BK = 32, NS = 4;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int TM = WTM / 32, TN = WTN / 32;
  static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int A_BLK = BM / 16, B_BLK = BN / 16;
  static constexpr int BPW = (A_BLK + B_BLK) / NW;  // DMA blocks per wave
  static constexpr int SMEM = NS * STAGE;
  static_assert((A_BLK + B_BLK) % NW == 0, "blocks per wave");
  static_assert(TM >= 1 && TN >= 1, "tile");
  static_assert(EPI != EPI_SWIGLU || (TN % 2) == 0, "swiglu pairs");

  __device__ static __forceinline__ void run(const GemmArgs& p, const TileInfo& ti, int nt,
                                             char* smem, const int32_t* a_gather) {
    typedef typename MfmaOp<DT>::V V;
    const int tid = (int)threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int lrow = lane & 31;
    const int khalf = lane >> 5;
    const int prow = lane >> 2, pchunk = lane & 3;  // DMA lane -> (row, chunk)
    // MFMA operand read: logical chunk 2s + khalf of a row whose swizzle is
    // that of lrow (tile rows start at multiples of 32).
    const int sw0 = ((0 + khalf) ^ dma_swz(lrow)) << 4;
    const int sw1 = ((2 + khalf) ^ dma_swz(lrow)) << 4;

    const int a_sub = p.a_local ? ti.base : 0;
    const int c_sub = p.c_local ? ti.base : 0;
    const int n0 = nt * BN;
    const int n0h = nt * (BN / 2);

    // Source of each of this wave's DMA blocks (fixed for the tile; the
    // k-step adds BK * 2 bytes).
    const char* src[BPW];
    int ldsoff[BPW];
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
      const int q = wave + NW * j;
      if (q < A_BLK) {
        const int row = 16 * q + prow;
        const int kc = pchunk ^ dma_swz(row);
        int grow = ti.r0 + row;
        grow = grow < ti.r1 ? grow : ti.r1 - 1;
        int arow;
        if (a_gather) {
          arow = a_gather[grow];  // dispatch fused into the A load
        } else {
          arow = grow - a_sub;
          if (p.a_local && arow >= p.a_rows) arow = p.a_rows - 1;
        }
        src[j] = (const char*)p.A + ((long long)arow * p.lda) * 2 + kc * 16;
        ldsoff[j] = q * 1024;
      } else {
        const int row = 16 * (q - A_BLK) + prow;
        const int kc = pchunk ^ dma_swz(row);
        int n;
        if (EPI == EPI_SWIGLU) {
          const int gi = row >> 5;
          n = ((gi & 1) ? p.I : 0) + n0h + (gi >> 1) * 32 + (row & 31);
        } else {
          n = n0 + row;
        }
        src[j] = (const char*)p.B + ((long long)ti.g * p.strideB + (long long)n * p.ldb) * 2 +
                 kc * 16;
        ldsoff[j] = A_BYTES + (q - A_BLK) * 1024;
      }
    }

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    const int nk = p.K / BK;
    const uint32_t lds0 = lds_addr(smem);

// Fragments of one k16 substep (sw = sw0 or sw1) of a stage into FA/FB.
#define MOE_READ_HALF(stage, sw, FA, FB)                                           \
do {                                                                             \
    const char* As_ = smem + (stage) * STAGE;                                      \
    const char* Bs_ = As_ + A_BYTES;                                               \
    _Pragma("unroll") for (int i = 0; i < TM; ++i)                                 \
      FA[i] = *(const V*)(As_ + (wm * WTM + i * 32 + lrow) * 64 + (sw));           \
    _Pragma("unroll") for (int j = 0; j < TN; ++j)                                 \
      FB[j] = *(const V*)(Bs_ + (wn * WTN + j * 32 + lrow) * 64 + (sw));           \
} while (0)
#define MOE_MFMAS(FA, FB)                                                          \
do {                                                                             \
    _Pragma("unroll") for (int i = 0; i < TM; ++i)                                 \
    _Pragma("unroll") for (int j = 0; j < TN; ++j)                                 \
      acc[i][j] = MfmaOp<DT>::run(FA[i], FB[j], acc[i][j]);                        \
} while (0)
// A stage becomes readable: wait until at most `n_after` (0..3) later
// stages of this wave's copies are still in flight, finish this wave's LDS
// reads, then a barrier covers the other waves' copies and reads.
#define MOE_STAGE_READY(n_after)                                                   \
do {                                                                             \
    const int na_ = (n_after);                                                     \
    if (na_ >= 3) wait_vmcnt<3 * BPW>();                                           \
    else if (na_ == 2) wait_vmcnt<2 * BPW>();                                      \
    else if (na_ == 1) wait_vmcnt<BPW>();                                          \
    else wait_vmcnt<0>();                                                          \
    __builtin_amdgcn_s_waitcnt((0x3F & 0xF) | (0x7 << 4) | ((0x3F >> 4) << 14)); \
    __builtin_amdgcn_s_barrier();                                                  \
    asm volatile("" ::: "memory");                                                 \
} while (0)
#define MOE_ISSUE(st)                                                              \
do {                                                                             \
    const uint32_t dst_ = lds0 + ((st) % NS) * STAGE;                              \
    _Pragma("unroll") for (int j = 0; j < BPW; ++j)                                \
      dma16(src[j] + (st) * BK * 2, dst_ + ldsoff[j]);                             \
} while (0)

    static_assert(NS == 4, "wait counts assume four stages");
    static_assert(3 * BPW < 64, "vmcnt range");
    V xa[TM], xb[TN], ya[TM], yb[TN];
    // Every wave is done with the previous tile's stages: fill all four.
    lds_barrier();
#pragma unroll
    for (int st = 0; st < NS; ++st)
      if (st < nk) MOE_ISSUE(st);
    MOE_STAGE_READY(nk - 1 < 3 ? nk - 1 : 3);  // stage 0; stages 1..3 may be in flight
    MOE_READ_HALF(0, sw0, xa, xb);

    // Loop invariant at the top of iteration kt: stage kt is visible, its
    // first k16 half is in (xa, xb) (reads possibly in flight), stages up to
    // kt+3 have been issued.  The second half is read during the first
    // half's MFMAs.  Then stage kt+1 is made visible (stages kt+2, kt+3 may
    // stay in flight), stage kt's buffer, now fully read by every wave, is
    // refilled with stage kt+4, and stage kt+1's first half is read during
    // the second half's MFMAs.  The steady-state body is straight-line so
    // the compiler's own LDS wait counts stay exact; the last iterations
    // (no refill, full drain) are peeled.
    int kt = 0;
    // sched_barrier(0) keeps each phase's LDS reads ahead of the MFMAs that
    // overlap them (the scheduler would otherwise sink each read to its use).
#define MOE_PHASE() __builtin_amdgcn_sched_barrier(0)
    for (; kt < nk - NS; ++kt) {
      MOE_READ_HALF(kt % NS, sw1, ya, yb);
      MOE_PHASE();
      MOE_MFMAS(xa, xb);
      MOE_PHASE();
      MOE_STAGE_READY(2);
      MOE_READ_HALF((kt + 1) % NS, sw0, xa, xb);
      MOE_PHASE();
      {
        // Refill stage kt's buffer with stage kt+NS, one copy every few
        // MFMAs so the issue slots overlap the matrix pipe.
        const uint32_t dst_ = lds0 + ((kt + NS) % NS) * STAGE;
        const int kofs_ = (kt + NS) * BK * 2;
        constexpr int MF = TM * TN;
        constexpr int EVERY = MF / BPW > 0 ? MF / BPW : 1;
#pragma unroll
        for (int q = 0; q < MF; ++q) {
          acc[q / TN][q % TN] = MfmaOp<DT>::run(ya[q / TN], yb[q % TN], acc[q / TN][q % TN]);
          if ((q % EVERY) == EVERY - 1 && q / EVERY < BPW) {
            dma16(src[q / EVERY] + kofs_, dst_ + ldsoff[q / EVERY]);
            MOE_PHASE();
          }
        }
#pragma unroll
        for (int j = MF / EVERY; j < BPW; ++j) dma16(src[j] + kofs_, dst_ + ldsoff[j]);
      }
      MOE_PHASE();
    }
    for (; kt < nk - 1; ++kt) {
      MOE_READ_HALF(kt % NS, sw1, ya, yb);
      MOE_PHASE();
      MOE_MFMAS(xa, xb);
      MOE_PHASE();
      MOE_STAGE_READY(0);
      MOE_READ_HALF((kt + 1) % NS, sw0, xa, xb);
      MOE_PHASE();
      MOE_MFMAS(ya, yb);
      MOE_PHASE();
    }
    MOE_READ_HALF(kt % NS, sw1, ya, yb);
    MOE_PHASE();
    MOE_MFMAS(xa, xb);
    MOE_MFMAS(ya, yb);
#undef MOE_PHASE
#undef MOE_READ_HALF
#undef MOE_MFMAS
#undef MOE_STAGE_READY
#undef MOE_ISSUE

    // Epilogue (32x32 f32 layout: lane l -> column l % 32, rows
    // 8*(v/4) + 4*(l/32) + v%4).
    const int rsub = khalf * 4;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int grow = ti.r0 + wm * WTM + i * 32 + (v >> 2) * 8 + rsub + (v & 3);
        if (grow >= ti.r1) continue;
        const long long crow = grow - c_sub;
        if (p.c_local && crow >= p.c_rows) continue;
        if (EPI == EPI_SWIGLU) {
          uint16_t* C = (uint16_t*)p.C;
#pragma unroll
          for (int jp = 0; jp < TN / 2; ++jp) {
            const float h = silu_mul(acc[i][2 * jp][v], acc[i][2 * jp + 1][v]);
            const int col = n0h + (wn * (TN / 2) + jp) * 32 + lrow;
            C[crow * p.ldc + col] = Act<DT>::store(h);
          }
        } else if (EPI == EPI_F32) {
          float* C = (float*)p.C;
#pragma unroll
          for (int j = 0; j < TN; ++j)
            C[crow * p.ldc + n0 + wn * WTN + j * 32 + lrow] = acc[i][j][v];
        } else {
          uint16_t* C = (uint16_t*)p.C;
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            float y = acc[i][j][v];
            if (EPI == EPI_GELU) y = gelu_erf(y);
            C[crow * p.ldc + n0 + wn * WTN + j * 32 + lrow] = Act<DT>::store(y);
          }
        }
      }
    }
  }
};

}  // namespace moe
