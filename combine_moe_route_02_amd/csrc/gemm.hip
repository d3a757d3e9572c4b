// Grouped expert GEMMs on MFMA (gfx950) and a plain fp32 path.
//
// The expert FFN of each local expert is a dense contraction over that
// expert's contiguous row segment (GPT-4 MoE page, section 3.1 table: each
// expert is Linear -> activation -> Linear; the segments are the dense
// per-expert layout built at dispatch, DySHARP page, section 3.1 item 3).
// Segment sizes are read on the device from `offsets`, so the grid is sized
// from host-known upper bounds only and surplus workgroups exit at once.
//
// Tile order.  The 1-D grid is remapped so that consecutive logical tiles
// land on the same XCD (hardware dispatches workgroup i to XCD i % 8), and
// logical tiles walk bands of `gm` m-tiles for one n-tile before moving to
// the next n-tile: the gm m-tiles of a band share each weight tile in that
// XCD's L2, and a band's activation rows are reused across its n-tiles.
//
// Main loop.  BK = 64; global -> registers -> LDS with a two-buffer ring and
// one barrier per k-step; 16-byte chunks are stored XOR-swizzled
// (chunk ^ (row & 7)) so that the ds_read_b128 of an MFMA operand (32 rows,
// same k-chunk) touches every bank group once.  Each wave owns a
// (BM/WM) x (BN/WN) accumulator block of 32x32 MFMA tiles
// (v_mfma_f32_32x32x16_{bf16,f16}: 8 values of K per lane per operand).
//
// Epilogues: plain store in the activation dtype, SwiGLU (the B tile
// interleaves 32-row groups of gate and up rows so a wave holds both halves
// of the same h columns), exact-erf GELU, or float32 (router logits).
// fp8 E4M3 weights are decoded and scaled by their 128x128 tile scale while
// being staged to LDS as bf16.

#include <math.h>

#include "moe_internal.h"

namespace moe {

enum { W_SAME = 0, W_FP8 = 1 };

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
__device__ int build_mtile_table(const GemmArgs& p, int* s_pre, int* s_tmp) {
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

// m-tile index -> group and row range (binary search in the prefix table).
template <int BM>
__device__ __forceinline__ TileInfo tile_rows(const GemmArgs& p, const int* s_pre, int mt) {
  TileInfo ti;
  if (p.offsets == nullptr) {
    ti.g = 0;
    ti.r0 = mt * BM;
    ti.r1 = p.dense_M;
    ti.base = 0;
    return ti;
  }
  int lo = 0, hi = p.n_groups - 1;   // first g with s_pre[g] > mt
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (s_pre[mid] > mt) hi = mid; else lo = mid + 1;
  }
  const int before = lo > 0 ? s_pre[lo - 1] : 0;
  ti.g = lo;
  ti.base = p.offsets[p.e_begin];
  ti.r0 = p.offsets[p.e_begin + lo] + (mt - before) * BM;
  ti.r1 = p.offsets[p.e_begin + lo + 1];
  return ti;
}

// Tile t of the band order -> (m-tile, n-tile).  Bands hold gm m-tiles (the
// last band may hold fewer); inside a band the m-tile index runs fastest.
__device__ __forceinline__ void band_coords(int t, int total_m, int n_tiles, int gm,
                                            int& mt, int& nt) {
  const int full = total_m / gm;
  const int per_band = gm * n_tiles;
  const int band = t / per_band;
  if (band < full) {
    const int w = t - band * per_band;
    nt = w / gm;
    mt = band * gm + w % gm;
  } else {
    const int gl = total_m - full * gm;
    const int w = t - full * per_band;
    nt = w / gl;
    mt = full * gm + w % gl;
  }
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

// 16 fp8 codes * scale -> 16 bf16 (two 16-byte chunks).
__device__ __forceinline__ void fp8x16_to_bf16(const u32x4& q, float s, u32x4& lo,
                                               u32x4& hi) {
  const uint32_t w[4] = {q[0], q[1], q[2], q[3]};
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t v = w[i];
    const uint16_t b0 = f32_to_bf16(e4m3_to_f32(v & 0xffu) * s);
    const uint16_t b1 = f32_to_bf16(e4m3_to_f32((v >> 8) & 0xffu) * s);
    const uint16_t b2 = f32_to_bf16(e4m3_to_f32((v >> 16) & 0xffu) * s);
    const uint16_t b3 = f32_to_bf16(e4m3_to_f32(v >> 24) * s);
    o[2 * i] = (uint32_t)b0 | ((uint32_t)b1 << 16);
    o[2 * i + 1] = (uint32_t)b2 | ((uint32_t)b3 << 16);
  }
  lo = u32x4{o[0], o[1], o[2], o[3]};
  hi = u32x4{o[4], o[5], o[6], o[7]};
}

template <int DT, int WK, int EPI, int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(WM * WN * 64)
    grouped_gemm_mfma(GemmArgs p) {
  constexpr int NT = WM * WN * 64;
  constexpr int BK = 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int ACH = BM * 8 / NT;                             // 16-B chunks
  constexpr int BCH = (WK == W_FP8) ? BN * 4 / NT : BN * 8 / NT;
  static_assert(TM >= 1 && TN >= 1 && ACH >= 1 && BCH >= 1, "tile");
  static_assert(EPI != EPI_SWIGLU || (TN % 2) == 0, "swiglu pairs");
  typedef typename MfmaOp<DT>::V V;

  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][BN * BK];
  __shared__ int s_pre[1024];
  __shared__ int s_scan[NT];

  const int total_m = build_mtile_table<NT, BM>(p, s_pre, s_scan);
  int t_first, t_end, t_stride;
  xcd_share(total_m * p.n_tiles, t_first, t_end, t_stride);
  for (int t = t_first; t < t_end; t += t_stride) {
  int mt, nt;
  band_coords(t, total_m, p.n_tiles, p.gm, mt, nt);
  const TileInfo ti = tile_rows<BM>(p, s_pre, mt);

  const int tid = (int)threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int a_sub = p.a_local ? ti.base : 0;
  const int c_sub = p.c_local ? ti.base : 0;
  const int n0 = nt * BN;
  const int n0h = nt * (BN / 2);

  // Chunk addresses: 64-bit for activation rows, 32-bit byte offsets from the
  // expert's (uniform) base for weights; the host keeps one expert's weight
  // matrix below 4 GiB.
  const char* Abase = (const char*)p.A;
  const char* Bbase = (const char*)p.B + (long long)ti.g * p.strideB * (WK == W_FP8 ? 1 : 2);
  const char* a_ptr[ACH];
  int a_lds[ACH];
#pragma unroll
  for (int i = 0; i < ACH; ++i) {
    const int c = tid + i * NT;
    const int row = c >> 3, kc = c & 7;
    int grow = ti.r0 + row;
    grow = grow < ti.r1 ? grow : ti.r1 - 1;
    int arow = grow - a_sub;
    if (p.a_local && arow >= p.a_rows) arow = p.a_rows - 1;
    a_ptr[i] = Abase + ((long long)arow * p.lda + kc * 8) * 2;
    a_lds[i] = row * BK + ((kc ^ (row & 7)) << 3);
  }
  uint32_t b_off[BCH];
  int b_lds[BCH], b_lds2[BCH];
  uint32_t s_off[BCH];
#pragma unroll
  for (int i = 0; i < BCH; ++i) {
    const int c = tid + i * NT;
    const int row = (WK == W_FP8) ? (c >> 2) : (c >> 3);
    const int kc = (WK == W_FP8) ? ((c & 3) * 2) : (c & 7);
    int n;
    if (EPI == EPI_SWIGLU) {
      const int gi = row >> 5;
      n = ((gi & 1) ? p.I : 0) + n0h + (gi >> 1) * 32 + (row & 31);
    } else {
      n = n0 + row;
    }
    if (WK == W_FP8) {
      b_off[i] = (uint32_t)n * (uint32_t)p.ldb + kc * 8;
      s_off[i] = (uint32_t)(n >> 7) * (uint32_t)(p.K >> 7);
      b_lds2[i] = row * BK + (((kc + 1) ^ (row & 7)) << 3);
    } else {
      b_off[i] = ((uint32_t)n * (uint32_t)p.ldb + kc * 8) * 2u;
      s_off[i] = 0;
      b_lds2[i] = 0;
    }
    b_lds[i] = row * BK + ((kc ^ (row & 7)) << 3);
  }
  const float* Sbase = (WK == W_FP8) ? p.Bscale + (long long)ti.g * p.strideS : nullptr;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int nk = p.K / BK;

  // Prologue: k-step 0 straight to buffer 0.
  {
  u32x4 ra[ACH], rb[BCH];
  float rs[BCH];
#pragma unroll
  for (int i = 0; i < ACH; ++i) ra[i] = *(const u32x4*)(a_ptr[i]);
#pragma unroll
  for (int i = 0; i < BCH; ++i) {
    rb[i] = *(const u32x4*)(Bbase + b_off[i]);
    if (WK == W_FP8) rs[i] = Sbase[s_off[i]];
  }
#pragma unroll
  for (int i = 0; i < ACH; ++i) *(u32x4*)(&sA[0][a_lds[i]]) = ra[i];
#pragma unroll
  for (int i = 0; i < BCH; ++i) {
    if (WK == W_FP8) {
      u32x4 lo, hi;
      fp8x16_to_bf16(rb[i], rs[i], lo, hi);
      *(u32x4*)(&sB[0][b_lds[i]]) = lo;
      *(u32x4*)(&sB[0][b_lds2[i]]) = hi;
    } else {
      *(u32x4*)(&sB[0][b_lds[i]]) = rb[i];
    }
  }
  }
  __syncthreads();

  const int lrow = lane & 31;
  const int khalf = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    u32x4 ra[ACH], rb[BCH];
    float rs[BCH];
    if (more) {
      const uint32_t ka = (uint32_t)(kt + 1) * BK * 2u;
      const uint32_t kb = (uint32_t)(kt + 1) * BK * (WK == W_FP8 ? 1u : 2u);
#pragma unroll
      for (int i = 0; i < ACH; ++i) ra[i] = *(const u32x4*)(a_ptr[i] + ka);
#pragma unroll
      for (int i = 0; i < BCH; ++i) {
        rb[i] = *(const u32x4*)(Bbase + b_off[i] + kb);
        if (WK == W_FP8) rs[i] = Sbase[s_off[i] + (((kt + 1) * BK) >> 7)];
      }
    }
    const uint16_t* As = sA[cur];
    const uint16_t* Bs = sB[cur];
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      const int sw = ((2 * s + khalf) ^ (lane & 7)) << 3;
      V af[TM], bfv[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *(const V*)(As + (wm * WTM + i * 32 + lrow) * BK + sw);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfv[j] = *(const V*)(Bs + (wn * WTN + j * 32 + lrow) * BK + sw);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = MfmaOp<DT>::run(af[i], bfv[j], acc[i][j]);
    }
    if (more) {
      uint16_t* An = sA[cur ^ 1];
      uint16_t* Bn = sB[cur ^ 1];
#pragma unroll
      for (int i = 0; i < ACH; ++i) *(u32x4*)(An + a_lds[i]) = ra[i];
#pragma unroll
      for (int i = 0; i < BCH; ++i) {
        if (WK == W_FP8) {
          u32x4 lo, hi;
          fp8x16_to_bf16(rb[i], rs[i], lo, hi);
          *(u32x4*)(Bn + b_lds[i]) = lo;
          *(u32x4*)(Bn + b_lds2[i]) = hi;
        } else {
          *(u32x4*)(Bn + b_lds[i]) = rb[i];
        }
      }
    }
    __syncthreads();
  }

  // Epilogue.  32x32 f32 output: lane l holds column l % 32 and rows
  // 8*(v/4) + 4*(l/32) + v%4 for v = 0..15.
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
  }  // tile loop
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

template <int DT, int EPI, int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(WM * WN * 64)
    grouped_gemm_dma(GemmArgs p) {
  constexpr int NW = WM * WN;
  constexpr int NT = NW * 64;
  constexpr int BK = 32, NS = 4;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int A_BLK = BM / 16, B_BLK = BN / 16;
  constexpr int BPW = (A_BLK + B_BLK) / NW;            // DMA blocks per wave
  static_assert((A_BLK + B_BLK) % NW == 0, "blocks per wave");
  static_assert(BPW * 2 < 64, "vmcnt range");
  static_assert(TM >= 1 && TN >= 1, "tile");
  static_assert(EPI != EPI_SWIGLU || (TN % 2) == 0, "swiglu pairs");
  typedef typename MfmaOp<DT>::V V;

  __shared__ __attribute__((aligned(1024))) char smem[NS * STAGE];
  __shared__ int s_pre[1024];
  __shared__ int s_scan[NT];

  const int total_m = build_mtile_table<NT, BM>(p, s_pre, s_scan);
  int t_first, t_end, t_stride;
  xcd_share(total_m * p.n_tiles, t_first, t_end, t_stride);

  const int tid = (int)threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int lrow = lane & 31;
  const int khalf = lane >> 5;
  const int prow = lane >> 2, pchunk = lane & 3;  // DMA lane -> (row, chunk)
  // MFMA operand read: logical chunk 2s + khalf of a row whose (r>>1)&3 is
  // that of lrow (tile rows start at multiples of 32).
  const int sw0 = ((0 + khalf) ^ dma_swz(lrow)) << 4;
  const int sw1 = ((2 + khalf) ^ dma_swz(lrow)) << 4;

  for (int t = t_first; t < t_end; t += t_stride) {
    int mt, nt;
    band_coords(t, total_m, p.n_tiles, p.gm, mt, nt);
    const TileInfo ti = tile_rows<BM>(p, s_pre, mt);
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
        int arow = grow - a_sub;
        if (p.a_local && arow >= p.a_rows) arow = p.a_rows - 1;
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
  }  // tile loop
}

// Plain fp32 grouped GEMM (64x64 tiles, 4x4 outputs per thread).
template <int EPI>
__global__ void __launch_bounds__(256) grouped_gemm_f32(GemmArgs p) {
  constexpr int BM = 64, BN = 64, BK = 16, NT = 256;
  __shared__ float sA[BM][BK + 1];
  __shared__ float sB[BN][BK + 1];
  __shared__ int s_pre[1024];
  __shared__ int s_scan[NT];

  const int total_m = build_mtile_table<NT, BM>(p, s_pre, s_scan);
  int t_first, t_end, t_stride;
  xcd_share(total_m * p.n_tiles, t_first, t_end, t_stride);
  for (int t = t_first; t < t_end; t += t_stride) {
  int mt, nt;
  band_coords(t, total_m, p.n_tiles, p.gm, mt, nt);
  const TileInfo ti = tile_rows<BM>(p, s_pre, mt);

  const int tid = (int)threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const long long a_sub = p.a_local ? ti.base : 0;
  const long long c_sub = p.c_local ? ti.base : 0;
  const float* A = (const float*)p.A;
  const float* B = (const float*)p.B + (long long)ti.g * p.strideB;
  const int n0 = nt * BN, n0h = nt * (BN / 2);

  float acc[4][4] = {};
  for (int k0 = 0; k0 < p.K; k0 += BK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + i * NT;          // 1024 elements per tile
      const int row = c >> 4, kk = c & 15;
      int grow = ti.r0 + row;
      grow = grow < ti.r1 ? grow : ti.r1 - 1;
      long long arow = grow - a_sub;
      if (p.a_local && arow >= p.a_rows) arow = p.a_rows - 1;
      sA[row][kk] = A[arow * p.lda + k0 + kk];
      int n;
      if (EPI == EPI_SWIGLU)
        n = (row < 32) ? n0h + row : p.I + n0h + row - 32;
      else
        n = n0 + row;
      sB[row][kk] = B[(long long)n * p.ldb + k0 + kk];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sA[ty + 16 * i][kk];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = sB[tx + 16 * j][kk];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  float* C = (float*)p.C;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int grow = ti.r0 + ty + 16 * i;
    if (grow >= ti.r1) continue;
    const long long crow = grow - c_sub;
    if (p.c_local && crow >= p.c_rows) continue;
    if (EPI == EPI_SWIGLU) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
        C[crow * p.ldc + n0h + tx + 16 * j] = silu_mul(acc[i][j], acc[i][j + 2]);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float y = acc[i][j];
        if (EPI == EPI_GELU) y = gelu_erf(y);
        C[crow * p.ldc + n0 + tx + 16 * j] = y;
      }
    }
  }
  __syncthreads();
  }  // tile loop
}

// ---------------------------------------------------------------------------
// Host launcher
// ---------------------------------------------------------------------------

namespace {

int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

// Persistent grid: no more workgroups than can be resident at once (so the
// XCD placement i % 8 holds for all of them) and no more than the tile count
// can use; always a multiple of 8.
template <typename Kern>
dim3 persistent_grid(Kern kernel, int threads, GemmArgs& a, int max_rows, int BM, int BN,
                     int gm) {
  static int occ = 0;  // one cache per kernel instantiation
  if (occ == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess ||
        n <= 0)
      n = 1;
    occ = n;
  }
  long long mtiles = a.offsets ? (long long)(max_rows + BM - 1) / BM + a.n_groups
                               : (long long)(a.dense_M + BM - 1) / BM;
  a.n_tiles = a.Nb / BN;
  a.gm = gm < 1 ? 1 : gm;
  a.mt_slots = (int)mtiles;
  long long g = mtiles * a.n_tiles;
  const long long cap = (long long)device_cus() * occ;
  if (g > cap) g = cap;
  g = (g + 7) / 8 * 8;
  return dim3((unsigned)g);
}

template <int DT, int WK, int EPI, int BM, int BN, int WM, int WN>
int run_mfma(GemmArgs a, int max_rows, int gm, hipStream_t s) {
  if (a.Nb % BN || a.K % 64) return MOE_ERR_UNSUPPORTED;
  if (WK == W_FP8 && (a.K % 128 || a.Nb % 128)) return MOE_ERR_UNSUPPORTED;
  if ((long long)a.Nb * a.ldb * (WK == W_FP8 ? 1 : 2) >= (1ll << 32))
    return MOE_ERR_UNSUPPORTED;
  if (a.offsets && a.n_groups > 1024) return MOE_ERR_UNSUPPORTED;
  auto kern = grouped_gemm_mfma<DT, WK, EPI, BM, BN, WM, WN>;
  const dim3 grid = persistent_grid(kern, WM * WN * 64, a, max_rows, BM, BN, gm);
  hipLaunchKernelGGL(kern, grid, dim3(WM * WN * 64), 0, s, a);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

template <int DT, int EPI, int BM, int BN, int WM, int WN>
int run_dma(GemmArgs a, int max_rows, int gm, hipStream_t s) {
  if (a.Nb % BN || a.K % 32) return MOE_ERR_UNSUPPORTED;
  if (a.offsets && a.n_groups > 1024) return MOE_ERR_UNSUPPORTED;
  auto kern = grouped_gemm_dma<DT, EPI, BM, BN, WM, WN>;
  const dim3 grid = persistent_grid(kern, WM * WN * 64, a, max_rows, BM, BN, gm);
  hipLaunchKernelGGL(kern, grid, dim3(WM * WN * 64), 0, s, a);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// Relative MFMA efficiency of each tile shape (larger wave tiles need fewer
// LDS reads per MFMA) used to pick a shape; rounds of 256 workgroups model the
// tail of the last wave of tiles.
struct TileShape {
  int BM, BN;
  float eff;
};

template <int DT, int WK, int EPI>
int pick_tile(GemmArgs a, int max_rows, hipStream_t s) {
  if (EPI == EPI_F32) {
    if (WK == W_SAME) return run_dma<DT, EPI, 64, 128, 2, 2>(a, max_rows, 4, s);
    return run_mfma<DT, WK, EPI, 64, 128, 2, 2>(a, max_rows, 4, s);
  }
  const int groups = a.offsets ? a.n_groups : 1;
  const int rows = a.offsets ? max_rows : a.dense_M;
  const double avg = (double)rows / (groups > 0 ? groups : 1);
  if (avg <= 48.0) return run_mfma<DT, WK, EPI, 32, 256, 1, 4>(a, max_rows, 1, s);
  const TileShape shapes[2] = {{256, 256, 1.0f}, {128, 256, 0.8f}};
  int best = 0;
  double best_t = 1e300;
  for (int c = 0; c < 2; ++c) {
    const TileShape& t = shapes[c];
    if (a.Nb % t.BN) continue;
    // expected m-tiles: a segment's ragged tail costs half a tile on average
    const double mtiles = groups * (avg / t.BM + (a.offsets ? 0.5 : 1.0));
    const double tiles = mtiles * (a.Nb / t.BN);
    const double rounds = ceil(tiles / 256.0);
    const double tm = rounds * (double)t.BM * t.BN / t.eff;
    if (tm < best_t) {
      best_t = tm;
      best = c;
    }
  }
  if (WK == W_SAME) {
    if (best == 0) return run_dma<DT, EPI, 256, 256, 2, 2>(a, max_rows, 4, s);
    return run_dma<DT, EPI, 128, 256, 2, 2>(a, max_rows, 4, s);
  }
  if (best == 0) return run_mfma<DT, WK, EPI, 256, 256, 2, 2>(a, max_rows, 4, s);
  return run_mfma<DT, WK, EPI, 128, 256, 2, 2>(a, max_rows, 4, s);
}

template <int EPI>
int run_f32(GemmArgs a, int max_rows, hipStream_t s) {
  if (a.Nb % 64 || a.K % 16) return MOE_ERR_UNSUPPORTED;
  if (a.offsets && a.n_groups > 1024) return MOE_ERR_UNSUPPORTED;
  auto kern = grouped_gemm_f32<EPI>;
  const dim3 grid = persistent_grid(kern, 256, a, max_rows, 64, 64, 4);
  hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

template <int DT, int WK>
int by_epi(int epi, GemmArgs a, int max_rows, hipStream_t s) {
  switch (epi) {
    case EPI_STORE: return pick_tile<DT, WK, EPI_STORE>(a, max_rows, s);
    case EPI_SWIGLU: return pick_tile<DT, WK, EPI_SWIGLU>(a, max_rows, s);
    case EPI_GELU: return pick_tile<DT, WK, EPI_GELU>(a, max_rows, s);
    case EPI_F32: return pick_tile<DT, WK, EPI_F32>(a, max_rows, s);
  }
  return MOE_ERR_ARG;
}

}  // namespace

int launch_grouped_gemm(int act_dtype, int w_dtype, int epi, GemmArgs a,
                        int max_rows, hipStream_t stream) {
  if (act_dtype == MOE_DTYPE_F32) {
    if (w_dtype != MOE_DTYPE_F32) return MOE_ERR_UNSUPPORTED;
    switch (epi) {
      case EPI_STORE: return run_f32<EPI_STORE>(a, max_rows, stream);
      case EPI_F32: return run_f32<EPI_STORE>(a, max_rows, stream);
      case EPI_SWIGLU: return run_f32<EPI_SWIGLU>(a, max_rows, stream);
      case EPI_GELU: return run_f32<EPI_GELU>(a, max_rows, stream);
    }
    return MOE_ERR_ARG;
  }
  if (act_dtype == MOE_DTYPE_BF16) {
    if (w_dtype == MOE_DTYPE_BF16) return by_epi<MOE_DTYPE_BF16, W_SAME>(epi, a, max_rows, stream);
    if (w_dtype == MOE_DTYPE_FP8_E4M3 && epi != EPI_F32)
      return by_epi<MOE_DTYPE_BF16, W_FP8>(epi, a, max_rows, stream);
    return MOE_ERR_UNSUPPORTED;
  }
  if (act_dtype == MOE_DTYPE_F16) {
    if (w_dtype == MOE_DTYPE_F16) return by_epi<MOE_DTYPE_F16, W_SAME>(epi, a, max_rows, stream);
    return MOE_ERR_UNSUPPORTED;
  }
  return MOE_ERR_UNSUPPORTED;
}

}  // namespace moe
