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

// Tiles [b0, b1) of the expert-band order form the band that holds tile t
// (the same bands as band_tile).
__device__ __forceinline__ void band_bounds(const GemmArgs& p, const int* s_pre, int t,
                                            int n_tiles, int gm, int& b0, int& b1) {
  int g = 0;
  if (p.offsets != nullptr) {
    int lo = 0, hi = p.n_groups - 1;
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
  b0 = m_before * n_tiles + (band < full ? band : full) * per_band;
  b1 = band < full ? b0 + per_band : (m_before + mt_g) * n_tiles;
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

// MFMA instruction of a tile: 32x32x16 (MI = 32, 16 results per lane) or
// 16x16x32 (MI = 16, 4 results per lane); both take 8 16-bit values of K
// per lane and operand.  On gfx950 the two give bit-identical sums over the
// same K order (checked on full expert-FFN GEMMs); the 16x16x32 form is the
// faster one in the tiles below: a k-step is 2 substeps of 64 short MFMAs
// instead of 4 of 16 long ones, which leaves finer slots between them for
// the LDS reads and copies.
template <int DT, int MI>
struct MfmaT;
template <int DT>
struct MfmaT<DT, 32> {
  typedef typename MfmaOp<DT>::V V;
  typedef f32x16 Acc;
  static constexpr int NV = 16;
  static __device__ __forceinline__ Acc run(V a, V b, Acc c) { return MfmaOp<DT>::run(a, b, c); }
};
template <>
struct MfmaT<MOE_DTYPE_BF16, 16> {
  typedef bf16x8 V;
  typedef f32x4 Acc;
  static constexpr int NV = 4;
  static __device__ __forceinline__ Acc run(V a, V b, Acc c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct MfmaT<MOE_DTYPE_F16, 16> {
  typedef f16x8 V;
  typedef f32x4 Acc;
  static constexpr int NV = 4;
  static __device__ __forceinline__ Acc run(V a, V b, Acc c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

// One accumulator value read into a vector register at this point of the
// program (a plain use lets the compiler copy every accumulator out at once).
__device__ __forceinline__ float acc_read(float a) {
  float v;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
  return v;
}

// silu(g) * u with the hardware exp2 and reciprocal (each within about one
// ulp of float32; the result is rounded to 16 bits afterwards).
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

__device__ __forceinline__ float gelu_erf(float a) {
  return 0.5f * a * (1.0f + erff(a * 0.70710678118654752f));
}

// GELU for 16-bit outputs, with erf from Abramowitz & Stegun formula 7.1.26
// (|error| <= 1.5e-7, far below 16-bit rounding): inline and short, where
// the library erf can end up as a call that forces every live accumulator
// register out to memory.
__device__ __forceinline__ float gelu_erf16(float a) {
  const float x = a * 0.70710678118654752f;
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * ax);
  const float poly =
      t * (0.254829592f +
           t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
  const float e = 1.0f - poly * __expf(-ax * ax);
  return 0.5f * a * (1.0f + (x < 0.0f ? -e : e));
}

// ---------------------------------------------------------------------------
// 16-bit weights: direct-to-LDS staging (global_load_lds_dwordx4), BK = 64,
// two LDS stages; the next stage loads during the whole current k-step.
//
// Stage layout: rows of 128 bytes (64 values, one full cache line of a
// K-contiguous row); 16-byte chunk kc of row r sits at chunk kc ^ dma_swz(r),
// so the 16 or 32 rows an MFMA operand read touches (same logical chunk)
// spread over all bank groups.  One wave instruction fills one 1 KB block
// (8 rows): lane p writes row p/8, physical chunk p%8, and fetches the
// logical chunk that belongs there.  Whole 128-byte lines per row matter: the same bytes
// fetched as 64-byte halves of twice as many lines take twice as many L2
// requests, and the request rate, not the byte rate, bounds a CU's copies
// when every k-step touches hundreds of rows.  The hardware performs the LDS
// writes; the wave only tracks them with vmcnt, so a k-step waits for its
// stage's loads and then a barrier makes every wave's loads visible.
// ---------------------------------------------------------------------------

// LDS chunk swizzle of a 128-byte row: conflict-free for the 32 rows x 2
// chunks of a 32x32x16 operand read and the 16 rows x 4 chunks of a
// 16x16x32 one, whether the LDS serves 8 lanes x 16 B (32 banks) or
// 16 lanes x 16 B (64 banks) per cycle.
__device__ __forceinline__ int dma_swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// L2 prefetch distance of the weight rows (k-steps), and a switch for it.
#ifndef MOE_PFD
#define MOE_PFD 4
#endif
#ifndef MOE_PF_ON
#define MOE_PF_ON 1
#endif

#ifndef MOE_SKEW
#define MOE_SKEW(nt, nk) ((((nt) & 7) * 2) % (nk))
#endif

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Wait until at most BASE + n * STEP vector memory operations are in flight
// (n <= N, wave-uniform; the count must be an immediate).
template <int BASE, int STEP, int N>
__device__ __forceinline__ void wait_vmcnt_groups(int n) {
  if constexpr (N > 0) {
    if (n >= N) wait_vmcnt<BASE + N * STEP>();
    else wait_vmcnt_groups<BASE, STEP, N - 1>(n);
  } else {
    wait_vmcnt<BASE>();
  }
}

// Workgroup barrier for LDS hand-off that does not drain outstanding loads.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt((0x3F & 0xF) | (0x7 << 4) | (0x0 << 8) | ((0x3F >> 4) << 14));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One wave-wide 16-byte-per-lane copy global -> LDS (global_load_lds_dwordx4,
// scalar-base form): lane l reads base + voff_l and its 16 bytes land at LDS
// byte address lds_base + 16 * l.  The base is wave-uniform (SGPRs) and the
// per-lane 32-bit offsets stay fixed for a tile, so advancing a k-step is a
// scalar add and issuing a copy costs no vector instruction (a vector address
// computed per copy would have to wait for the previous copy to read its
// address registers).  Issued from asm so that the compiler does not add its
// own conservative vmcnt(0) before every later LDS read; the instruction
// writes no VGPR, and the kernel's counted vmcnt waits order it before the
// reads of its stage.  The LDS address goes in M0 as an asm operand, so the
// compiler sets M0 itself: a wave's copies into one stage lie a constant
// apart, and each costs one scalar add to M0 from the stage's base register
// (setting M0 inside the asm from a precomputed register per copy took twice
// the scalar instructions and the registers spilled to vector lanes; c4
// GEMM-1 and GEMM-2 ran 2-5% slower).
__device__ __forceinline__ void dma16(const char* base, uint32_t voff, uint32_t lds_base) {
  asm volatile("global_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(base), "{m0}"(lds_base)
               : "memory");
}

// dma16 with the non-temporal hint, for data that is read once (a decode
// batch's fp8 weights: each weight line serves one tile).
__device__ __forceinline__ void dma16_stream(const char* base, uint32_t voff,
                                             uint32_t lds_base) {
  asm volatile("global_load_lds_dwordx4 %0, %1 nt"
               :
               : "v"(voff), "s"(base), "{m0}"(lds_base)
               : "memory");
}

// L2 prefetch: one dword of each lane's line is copied to a scratch LDS
// slot that nothing reads (lane l writes lds_base + 4 * l), which brings the
// lines into L2 ahead of their stage's copy.  Counted by vmcnt like dma16.
__device__ __forceinline__ void prefetch4(const char* base, uint32_t voff, uint32_t lds_base) {
  asm volatile("global_load_lds_dword %0, %1"
               :
               : "v"(voff), "s"(base), "{m0}"(lds_base)
               : "memory");
}

// A pointer the compiler cannot prove uniform, made uniform (its value is
// the same in every lane by construction).
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const char*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// A share of one tile's k-steps.  The workgroup computes k-steps
// [k0, k0 + nk) (of BK each); with parts > 1 it stores its fp32 partial sums
// in its own slot, and the last of the `parts` workgroups to arrive adds all
// slots in part order (so the result does not depend on arrival order) and
// runs the epilogue.  The arrival counter starts at zero and the last
// arriver puts it back to zero, so a workspace zeroed once stays usable
// without a clearing launch before every GEMM.  Part s's slot is slot0 + s * slot_step floats; each
// thread owns a contiguous run of NACC floats in it (the tile's accumulators
// per thread: 256 for a 256x256 tile).
struct KSplit {
  int k0, nk;
  int parts, part;
  float* slot0;
  long long slot_step;
  int* counter;
  int* s_flag;  // one LDS int of the calling kernel
};

// One BM x BN output tile of a grouped GEMM with 16-bit weights (see the
// stage layout above).  A rows come from p.A at row r - a_sub, or, with
// a_gather, at row a_gather[r] (the fused kernel reads token rows of x
// through the layout map instead of a gathered copy).  smem must hold
// SMEM bytes; all threads of the block call it.  K must be a multiple of 64.
template <int DT, int EPI, int BM, int BN, int WM, int WN, int MI = 16>
struct DmaTile {
  typedef MfmaT<DT, MI> MO;
  static constexpr int NW = WM * WN;
  static constexpr int NT = NW * 64;
  static constexpr int BK = 64, NS = 2;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int TM = WTM / MI, TN = WTN / MI;    // MI x MI blocks per wave
  static constexpr int NV = MO::NV;                    // results per lane and block
  static constexpr int KSUB = 512 / MI;                // K of one MFMA: 16 or 32
  static constexpr int NSUB = BK / KSUB;               // substeps per k-step: 4 or 2
  static constexpr int ROWB = BK * 2;  // bytes per staged row
  static constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int A_BLK = BM / 8, B_BLK = BN / 8;  // 1 KB blocks of 8 rows
  static constexpr int BPW = (A_BLK + B_BLK) / NW;       // DMA blocks per wave
  // L2 prefetch: weight (B) rows PFD k-steps ahead, one dword per 128-byte
  // line.  Activation rows are not prefetched: a band's workgroups share
  // them and keep them in L2, while prefetching them too evicts weight lines
  // before their copies (GEMM-1 and GEMM-2 5-15% slower measured with both).
  static constexpr int PFD = MOE_PFD;
  static constexpr bool PF_ON = MOE_PF_ON != 0;
  static constexpr int NPF = (BN + 64 * NW - 1) / (64 * NW);  // prefetches per wave and k-step
  static constexpr int PF_OFS = NS * STAGE;                         // scratch slots
  static constexpr int SMEM = NS * STAGE + NW * 256;
  static_assert(A_BLK % NW == 0 && B_BLK % NW == 0, "blocks per wave");
  static_assert(TM >= 1 && TN >= 1, "tile");
  static_assert(EPI != EPI_SWIGLU || (TN % (MI == 32 ? 2 : 4)) == 0, "swiglu pairs");
  static_assert(PFD >= 3 && BPW + (PFD - 2) * NPF < 64, "vmcnt range");
  static_assert(MI == 32 || MI == 16, "MFMA shape");
  static_assert(A_BYTES == A_BLK * 1024, "B blocks start right after the A blocks");

  static constexpr int NACC = TM * TN * NV;  // accumulators per thread
  static constexpr long long SLOT = (long long)NT * NACC;  // floats per split slot

  // Output staging: the tile's outputs (OES bytes each, OCOLS per row) in
  // the stage buffers, OPITCH bytes per row, 16-byte pieces of row r
  // swizzled by ochunk(r); OCPR pieces per row, ORPP rows per pass of the
  // block.
  static constexpr int OES = 2;
  static constexpr int OCOLS = EPI == EPI_SWIGLU ? BN / 2 : BN;
  static constexpr int OPITCH = OCOLS * OES;
  static constexpr int OCPR = OPITCH / 16;
  static constexpr int ORPP = NT / OCPR;
  static constexpr int OSPAN = MI * OES / 16;  // pieces one row group of a write covers
  static constexpr bool EPI_STAGED = BM * OPITCH <= NS * STAGE && NT % OCPR == 0 &&
                                     BM % ORPP == 0 && OCPR >= (64 / MI) * OSPAN;
  __device__ static __forceinline__ int ochunk(int r) { return ((r >> 2) & (64 / MI - 1)) * OSPAN; }
  __device__ static __forceinline__ int obyte(int r, int c) {
    return r * OPITCH + ((((c * OES) >> 4) ^ ochunk(r)) << 4) + ((c * OES) & 15);
  }

  // nxt_g >= 0: this workgroup's next tile is the full-K tile of group
  // nxt_g, n-tile nxt_nt; the weight lines of its first PFD k-steps are
  // prefetched into L2 before this tile's epilogue, so that its first
  // copies do not wait on HBM.
  __device__ static __forceinline__ void run(const GemmArgs& p, const TileInfo& ti, int nt,
                                             char* smem, const int32_t* a_gather,
                                             const KSplit* ks = nullptr, int nxt_g = -1,
                                             int nxt_nt = 0) {
    typedef typename MO::V V;
    const int tid = (int)threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int lrow = lane & (MI - 1);   // operand row of this lane in a block
    const int kgrp = lane / MI;         // its 8-value group of the substep's K
    const int prow = lane >> 3, pchunk = lane & 7;  // DMA lane -> (row, chunk)
    // MFMA operand read of substep s: logical 16-byte chunk (KSUB / 8) * s +
    // kgrp of a row whose swizzle is that of lrow (blocks start at multiples
    // of MI, and the swizzle depends on the row mod 16).  KSUB / 8 * s has
    // no bits in common with kgrp, so the chunk is (KSUB / 8 * s) ^ sw_row.
    const int sw_row = dma_swz(lrow) ^ kgrp;

    const int a_sub = p.a_local ? ti.base : 0;
    const int c_sub = p.c_local ? ti.base : 0;
    const int n0 = nt * BN;
    const int n0h = nt * (BN / 2);

    // Sources of this wave's DMA blocks: a uniform base per operand and a
    // per-lane 32-bit byte offset, both fixed for the tile; a k-step moves the
    // bases.  A: rows relative to the tile's first row (or token rows of x
    // through a_gather); B: rows of this group's weight matrix.  Blocks
    // j < JA are A blocks (block q = wave + NW * j).
    constexpr int JA = A_BLK / NW;
    int base_row = 0;
    if (!a_gather) {
      base_row = ti.r0 - a_sub;
      if (p.a_local && base_row > p.a_rows - 1) base_row = p.a_rows - 1;
    }
    const char* a_tile = uniform_ptr((const char*)p.A + (long long)base_row * p.lda * 2);
    const char* b_tile = uniform_ptr((const char*)p.B + (long long)ti.g * p.strideB * 2);
    uint32_t voff[BPW];
    int ldsoff[BPW];
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
      const int q = wave + NW * j;
      if (j < JA) {
        const int row = 8 * q + prow;
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
        voff[j] = (uint32_t)(arow - base_row) * (uint32_t)(p.lda * 2) + (uint32_t)(kc * 16);
        ldsoff[j] = q * 1024;
      } else {
        const int row = 8 * (q - A_BLK) + prow;
        const int kc = pchunk ^ dma_swz(row);
        int n;
        if (EPI == EPI_SWIGLU) {
          const int gi = row >> 5;
          n = ((gi & 1) ? p.I : 0) + n0h + (gi >> 1) * 32 + (row & 31);
        } else {
          n = n0 + row;
        }
        voff[j] = (uint32_t)n * (uint32_t)(p.ldb * 2) + (uint32_t)(kc * 16);
        ldsoff[j] = q * 1024;  // the B blocks follow the A_BLK blocks of A
      }
    }

    // L2 prefetch rows: prefetch i covers B rows (i * NW + wave) * 64 + lane
    // (past the end: the last row again).
    uint32_t pfoff[NPF];
#pragma unroll
    for (int i = 0; i < NPF; ++i) {
      int row = (i * NW + wave) * 64 + lane;
      row = row < BN ? row : BN - 1;
      int n;
      if (EPI == EPI_SWIGLU) {
        const int gi = row >> 5;
        n = ((gi & 1) ? p.I : 0) + n0h + (gi >> 1) * 32 + (row & 31);
      } else {
        n = n0 + row;
      }
      pfoff[i] = (uint32_t)n * (uint32_t)(p.ldb * 2);
    }

    typename MO::Acc acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int v = 0; v < NV; ++v) acc[i][j][v] = 0.0f;

    const int nk = ks ? ks->nk : p.K / BK;      // k-steps of this share
    const int kbase = ks ? ks->k0 : 0;          // its first k-step
    const uint32_t lds0 = lds_addr(smem);
    // k-order rotation: tiles of different n-tiles start at different k so
    // that the workgroups of a band (which run in lockstep) do not all read
    // the same column of power-of-two-pitched rows at once, which
    // concentrates the traffic on a few memory channels.  Tiles sharing an
    // n-tile share the rotation (and so their weight reads).
    const int skew = MOE_SKEW(nt, nk);
#define MOE_KOFS(st) ((kbase + (((st) + skew) < nk ? (st) + skew : (st) + skew - nk)) * ROWB)

// Fragments of substep s4 of a stage into FA/FB.
#define MOE_READ(stage, s4, FA, FB)                                                \
do {                                                                             \
    const char* As_ = smem + (stage) * STAGE;                                      \
    const char* Bs_ = As_ + A_BYTES;                                               \
    _Pragma("unroll") for (int i = 0; i < TM; ++i)                                 \
      FA[i] = *(const V*)(As_ + (wm * WTM + i * MI + lrow) * ROWB + ((((KSUB / 8) * (s4)) ^ sw_row) << 4)); \
    _Pragma("unroll") for (int j = 0; j < TN; ++j)                                 \
      FB[j] = *(const V*)(Bs_ + (wn * WTN + j * MI + lrow) * ROWB + ((((KSUB / 8) * (s4)) ^ sw_row) << 4)); \
} while (0)
#define MOE_MFMAS(FA, FB)                                                          \
do {                                                                             \
    _Pragma("unroll") for (int i = 0; i < TM; ++i)                                 \
    _Pragma("unroll") for (int j = 0; j < TN; ++j)                                 \
      acc[i][j] = MO::run(FA[i], FB[j], acc[i][j]);                                \
} while (0)
// Fragment read r of substep s4 of a stage, and the MFMA after which it is
// issued: the TM + TN reads are spread evenly over the TM * TN MFMAs of a
// substep.  MOE_FRAG(r) < TM is A block MOE_FRAG(r), else B block
// MOE_FRAG(r) - TM.  The next substep's MFMAs run A block 0 against every B
// block first, then A blocks 1 .. TM - 1, so the reads follow that order:
// each read then has at least a third of a substep of MFMAs before its
// first use (read in A-then-B order, the last B block had eight MFMAs; 0.5-1%
// faster per GEMM measured, same sums).
#define MOE_FRAG(r) ((r) == 0 ? 0 : (r) <= TN ? TM + (r) - 1 : (r) - TN)
#define MOE_READ1(stage, s4, r, NA, NB)                                            \
do {                                                                             \
    const char* As_ = smem + (stage) * STAGE;                                      \
    const char* Bs_ = As_ + A_BYTES;                                               \
    const int f_ = MOE_FRAG(r);                                                    \
    if (f_ < TM)                                                                   \
      NA[f_] = *(const V*)(As_ + (wm * WTM + f_ * MI + lrow) * ROWB + ((((KSUB / 8) * (s4)) ^ sw_row) << 4)); \
    else                                                                           \
      NB[f_ - TM] = *(const V*)(Bs_ + (wn * WTN + (f_ - TM) * MI + lrow) * ROWB +         \
                                ((((KSUB / 8) * (s4)) ^ sw_row) << 4));            \
} while (0)
#define MOE_READ_AT(r) (((r) + 1) * (TM * TN) / (TM + TN) > 0 ? ((r) + 1) * (TM * TN) / (TM + TN) - 1 : 0)
// The MFMAs of one substep (operands FA, FB) with the fragment reads of
// substep s4 of a stage (into NA, NB) interleaved: a burst of all the reads
// before the MFMAs fills the LDS queue and stalls the wave's issue while the
// matrix pipe waits (measured 1-3% slower per GEMM than this order, same
// sums).
#define MOE_MFMAS_READ(FA, FB, stage, s4, NA, NB)                                  \
do {                                                                             \
    _Pragma("unroll") for (int q_ = 0; q_ < TM * TN; ++q_) {                      \
      acc[q_ / TN][q_ % TN] = MO::run(FA[q_ / TN], FB[q_ % TN], acc[q_ / TN][q_ % TN]); \
      _Pragma("unroll") for (int r_ = 0; r_ < TM + TN; ++r_)                        \
        if (MOE_READ_AT(r_) == q_) MOE_READ1(stage, s4, r_, NA, NB);                \
      __builtin_amdgcn_sched_barrier(0);                                           \
    }                                                                              \
} while (0)
// The next stage becomes readable: this wave's copies of it are done (only
// the n_pf prefetch groups issued after them may be in flight), its LDS
// reads are done, and a barrier covers the other waves' copies and reads.
#define MOE_STAGE_READY(n_pf)                                                      \
do {                                                                             \
    MOE_WAIT_STAGE(n_pf);                                                          \
    __builtin_amdgcn_s_waitcnt((0x3F & 0xF) | (0x7 << 4) | ((0x3F >> 4) << 14));  \
    __builtin_amdgcn_s_barrier();                                                  \
    asm volatile("" ::: "memory");                                                 \
} while (0)
#define MOE_ISSUE(st)                                                              \
do {                                                                             \
    const uint32_t dst_ = lds0 + ((st) % NS) * STAGE;                              \
    const char* ak_ = a_tile + MOE_KOFS(st);                                       \
    const char* bk_ = b_tile + MOE_KOFS(st);                                       \
    _Pragma("unroll") for (int j = 0; j < BPW; ++j)                                \
      dma16(j < JA ? ak_ : bk_, voff[j], dst_ + ldsoff[j]);                        \
} while (0)
#define MOE_PREFETCH(st)                                                           \
do {                                                                             \
    const uint32_t pdst_ = lds0 + PF_OFS + wave * 256;                             \
    if (PF_ON) {                                                                   \
      _Pragma("unroll") for (int i = 0; i < NPF; ++i)                              \
        prefetch4(b_tile + MOE_KOFS(st), pfoff[i], pdst_);                         \
    }                                                                              \
} while (0)
// Wait until at most n_pf prefetch groups (issued after the stage's copies)
// are in flight.
#define MOE_WAIT_STAGE(n_pf) wait_vmcnt_groups<0, NPF, PFD - 2>(PF_ON ? (n_pf) : 0)
// sched_barrier(0) keeps each phase's LDS reads ahead of the MFMAs that
// overlap them (the scheduler would otherwise sink each read to its use).
#define MOE_PHASE() __builtin_amdgcn_sched_barrier(0)

    V xa[TM], xb[TN], ya[TM], yb[TN];
    // Every wave is done with the previous tile's stages: fill both.
    lds_barrier();
    MOE_ISSUE(0);
    if (nk > 1) MOE_ISSUE(1);
#pragma unroll
    for (int s_ = 2; s_ < PFD; ++s_)
      if (s_ < nk) MOE_PREFETCH(s_);
    // stage 0 landed; stage 1 and the npf0 prefetch groups issued after it
    // may be in flight
    const int npf0 = PF_ON && nk > 2 ? (nk < PFD ? nk : PFD) - 2 : 0;
    if (nk <= 1) wait_vmcnt<0>();
    else wait_vmcnt_groups<BPW, NPF, PFD - 2>(npf0);
    __builtin_amdgcn_s_waitcnt((0x3F & 0xF) | (0x7 << 4) | ((0x3F >> 4) << 14));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    MOE_READ(0, 0, xa, xb);

    // Loop invariant at the top of k-step kt: stage kt is visible and its
    // substep 0 is in (xa, xb) (reads possibly in flight); stage kt+1 has
    // been issued.  Substeps 1 .. NSUB-1 are read one substep ahead of their
    // MFMAs, interleaved with them.  Before the MFMAs of the last substep the
    // next stage is made visible; those MFMAs then carry the reads of its
    // substep 0 and the refill of stage kt's buffer (read by every wave by
    // then) with stage kt+2, spread evenly over the MFMAs, so the issue slots
    // overlap the matrix pipe.  The body is straight-line so the compiler's own LDS
    // wait counts stay exact.
    int kt = 0;
    for (; kt < nk - 2; ++kt) {
      const int st = kt & 1;
      // substeps 0 .. NSUB-2, alternating the two fragment sets (NSUB is
      // even, so the last substep's fragments end up in ya, yb)
#pragma unroll
      for (int s4 = 0; s4 + 1 < NSUB; ++s4) {
        if ((s4 & 1) == 0) MOE_MFMAS_READ(xa, xb, st, s4 + 1, ya, yb);
        else MOE_MFMAS_READ(ya, yb, st, s4 + 1, xa, xb);
        MOE_PHASE();
      }
      // prefetch groups issued after stage kt+1's copies: the prologue's
      // npf0 for kt = 0, else the one issued with them (if any)
      MOE_STAGE_READY(kt == 0 ? npf0 : (kt + PFD - 1 < nk));
      {
        const uint32_t dst_ = lds0 + st * STAGE;
        const int kofs_ = MOE_KOFS(kt + 2);
        const char* ak_ = a_tile + kofs_;
        const char* bk_ = b_tile + kofs_;
        constexpr int MF = TM * TN;
        constexpr int EVERY = MF / BPW > 0 ? MF / BPW : 1;
#pragma unroll
        for (int q = 0; q < MF; ++q) {
          acc[q / TN][q % TN] = MO::run(ya[q / TN], yb[q % TN], acc[q / TN][q % TN]);
#pragma unroll
          for (int r_ = 0; r_ < TM + TN; ++r_)
            if (MOE_READ_AT(r_) == q) MOE_READ1(st ^ 1, 0, r_, xa, xb);
#pragma unroll
          for (int r = 0; r < (BPW + MF - 1) / MF; ++r) {
            const int j = (q / EVERY) * ((BPW + MF - 1) / MF) + r;
            if ((q % EVERY) == EVERY - 1 && j < BPW) {
              dma16(j < JA ? ak_ : bk_, voff[j], dst_ + ldsoff[j]);
            }
          }
          MOE_PHASE();
        }
      }
      if (kt + PFD < nk) MOE_PREFETCH(kt + PFD);
      MOE_PHASE();
    }
    // Last two k-steps: no refill.
    for (; kt < nk; ++kt) {
      const int st = kt & 1;
#pragma unroll
      for (int s4 = 0; s4 + 1 < NSUB; ++s4) {
        if ((s4 & 1) == 0) {
          MOE_READ(st, s4 + 1, ya, yb);
          MOE_PHASE();
          MOE_MFMAS(xa, xb);
        } else {
          MOE_READ(st, s4 + 1, xa, xb);
          MOE_PHASE();
          MOE_MFMAS(ya, yb);
        }
        MOE_PHASE();
      }
      if (kt + 1 < nk) {
        MOE_STAGE_READY(kt == 0 ? npf0 : (kt + PFD - 1 < nk));
        MOE_READ(st ^ 1, 0, xa, xb);
        MOE_PHASE();
      }
      MOE_MFMAS(ya, yb);
      MOE_PHASE();
    }
#undef MOE_PHASE
#undef MOE_READ
#undef MOE_MFMAS_READ
#undef MOE_READ1
#undef MOE_FRAG
#undef MOE_READ_AT
#undef MOE_MFMAS
#undef MOE_STAGE_READY
#undef MOE_ISSUE
#undef MOE_PREFETCH
#undef MOE_WAIT_STAGE
#undef MOE_KOFS

    if (PF_ON && nxt_g >= 0) {
      const char* b2 = uniform_ptr((const char*)p.B + (long long)nxt_g * p.strideB * 2);
      const int nk2 = p.K / BK;
      const int skew2 = MOE_SKEW(nxt_nt, nk2);
      const uint32_t pdst = lds0 + PF_OFS + wave * 256;
#pragma unroll
      for (int i = 0; i < NPF; ++i) {
        int row = (i * NW + wave) * 64 + lane;
        row = row < BN ? row : BN - 1;
        int n;
        if (EPI == EPI_SWIGLU) {
          const int gi = row >> 5;
          n = ((gi & 1) ? p.I : 0) + nxt_nt * (BN / 2) + (gi >> 1) * 32 + (row & 31);
        } else {
          n = nxt_nt * BN + row;
        }
        const uint32_t off = (uint32_t)n * (uint32_t)(p.ldb * 2);
#pragma unroll
        for (int s_ = 0; s_ < PFD; ++s_)
          if (s_ < nk2) {
            const int kk = s_ + skew2 < nk2 ? s_ + skew2 : s_ + skew2 - nk2;
            prefetch4(b2 + kk * ROWB, off, pdst);
          }
      }
    }

    // Epilogue (32x32 f32 layout: lane l -> column l % 32, rows
    // 8*(v/4) + 4*(l/32) + v%4; 16x16: column l % 16, rows 4*(l/16) + v).
    // One accumulator block (or SwiGLU pair) at a time; each value is read
    // from the accumulator registers where it is used (acc_read), so the
    // epilogue never holds more than a block of them in vector registers.  The s_nop wait states cover the last MFMAs'
    // results before the first read.
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    if (ks && ks->parts > 1) {
      // Split tile: publish this part's sums; only the last part to arrive
      // goes on, with the sum of all parts in part order.
      // Slot addresses: a uniform base per part plus this thread's 32-bit
      // byte offset (tid * NACC floats), so every load and store folds the
      // accumulator offset into its immediate instead of holding a 64-bit
      // address per value.
      const uint32_t mine_ofs = (uint32_t)tid * (uint32_t)(NACC * 4);
      char* mine = (char*)uniform_ptr((const char*)(ks->slot0 + ks->part * ks->slot_step));
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int v = 0; v < NV; v += 4) {
            f32x4 q;
            q[0] = acc_read(acc[i][j][v]);
            q[1] = acc_read(acc[i][j][v + 1]);
            q[2] = acc_read(acc[i][j][v + 2]);
            q[3] = acc_read(acc[i][j][v + 3]);
            *(f32x4*)(mine + mine_ofs + ((i * TN + j) * NV + v) * 4) = q;
          }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        const int old = __hip_atomic_fetch_add(ks->counter, 1, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
        *ks->s_flag = old == ks->parts - 1;
        if (old == ks->parts - 1) {
          // every part has arrived: the counter goes back to zero for the
          // next launch (the kernel boundary orders it before that launch)
          __hip_atomic_store(ks->counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        }
      }
      __syncthreads();
      if (!*ks->s_flag) return;
      // the sum of all parts in part order, one 16-byte piece at a time
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int v = 0; v < NV; v += 4) {
            const uint32_t off = mine_ofs + ((i * TN + j) * NV + v) * 4;
            const char* b0 = (const char*)uniform_ptr((const char*)ks->slot0);
            f32x4 tot = *(const f32x4*)(b0 + off);
            for (int s2 = 1; s2 < ks->parts; ++s2) {
              const char* bs =
                  (const char*)uniform_ptr((const char*)(ks->slot0 + s2 * ks->slot_step));
              tot += *(const f32x4*)(bs + off);
            }
            acc[i][j][v] = tot[0];
            acc[i][j][v + 1] = tot[1];
            acc[i][j][v + 2] = tot[2];
            acc[i][j][v + 3] = tot[3];
          }
      asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
    }
    const int rsub = kgrp * 4;
    if (EPI_STAGED && ((uintptr_t)p.C & 15) == 0 && ((long long)p.ldc * OES) % 16 == 0) {
      // Staged output: every wave is done with the stage buffers, which now
      // take the finished tile (activation applied, in the output type);
      // then each thread stores whole 16-byte pieces of output rows.  One
      // 16-byte store instead of 8 (16-bit) or 4 (f32) single-value stores,
      // each covering a full row segment, cuts the store instructions and the
      // partial-line writes they caused.  Chunk swizzle (see ochunk): the 64
      // lanes of one staging write cover 64 / MI rows 4 apart, moved to
      // distinct banks.
      __syncthreads();
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        if (EPI == EPI_SWIGLU) {
#pragma unroll
          for (int jp = 0; jp < TN / 2; ++jp) {
            __builtin_amdgcn_sched_barrier(0);
            const int jg = MI == 32 ? 2 * jp : 4 * (jp >> 1) + (jp & 1);
            const int ju = MI == 32 ? jg + 1 : jg + 2;
            const int ocol = MI == 32 ? (wn * (TN / 2) + jp) * 32 + lrow
                                      : (wn * (WTN / 64) + (jp >> 1)) * 32 + (jp & 1) * 16 + lrow;
            // values v and v + 1 sit in rows orow and orow + 1: one packed
            // conversion for both (1 us less per 256 x 256 tile than one per value)
#pragma unroll
            for (int v = 0; v < NV; v += 2) {
              const int orow = wm * WTM + i * MI + (MI == 32 ? (v >> 2) * 8 + (v & 3) : v) + rsub;
              const float h0 = silu_mul(acc_read(acc[i][jg][v]), acc_read(acc[i][ju][v]));
              const float h1 = silu_mul(acc_read(acc[i][jg][v + 1]), acc_read(acc[i][ju][v + 1]));
              const uint32_t pk = Act<DT>::store2(h0, h1);
              *(uint16_t*)(smem + obyte(orow, ocol)) = (uint16_t)pk;
              *(uint16_t*)(smem + obyte(orow + 1, ocol)) = (uint16_t)(pk >> 16);
            }
          }
        } else {
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            __builtin_amdgcn_sched_barrier(0);
            const int ocol = wn * WTN + j * MI + lrow;
#pragma unroll
            for (int v = 0; v < NV; v += 2) {
              const int orow = wm * WTM + i * MI + (MI == 32 ? (v >> 2) * 8 + (v & 3) : v) + rsub;
              float y0 = acc_read(acc[i][j][v]);
              float y1 = acc_read(acc[i][j][v + 1]);
              if (EPI == EPI_GELU) {
                y0 = gelu_erf16(y0);
                y1 = gelu_erf16(y1);
              }
              const uint32_t pk = Act<DT>::store2(y0, y1);
              *(uint16_t*)(smem + obyte(orow, ocol)) = (uint16_t)pk;
              *(uint16_t*)(smem + obyte(orow + 1, ocol)) = (uint16_t)(pk >> 16);
              if (EPI == EPI_GELU) __builtin_amdgcn_sched_barrier(0);
            }
          }
        }
      }
      __syncthreads();
      // Thread t stores 16-byte piece t % OCPR of rows t / OCPR + k * ORPP.
      const int c16 = tid % OCPR;
      const int nrows = ti.r1 - ti.r0;
      char* cbase = (char*)p.C + (long long)(EPI == EPI_SWIGLU ? n0h : n0) * OES + c16 * 16;
      constexpr int NQ = BM / ORPP;
      constexpr int QB = NQ < 4 ? NQ : 4;  // pieces in flight per thread
#pragma unroll 1
      for (int q0 = 0; q0 < NQ; q0 += QB) {
        uint4 val[QB];
#pragma unroll
        for (int u = 0; u < QB; ++u) {
          const int rr = tid / OCPR + (q0 + u) * ORPP;
          val[u] = *(const uint4*)(smem + rr * OPITCH + ((c16 ^ ochunk(rr)) << 4));
        }
#pragma unroll
        for (int u = 0; u < QB; ++u) {
          const int rr = tid / OCPR + (q0 + u) * ORPP;
          const int crow = ti.r0 + rr - c_sub;
          if (rr < nrows && !(p.c_local && crow >= p.c_rows))
            *(uint4*)(cbase + (long long)crow * p.ldc * OES) = val[u];
        }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      int crow[NV];
      bool ok[NV];
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int grow = ti.r0 + wm * WTM + i * MI + (MI == 32 ? (v >> 2) * 8 + (v & 3) : v) + rsub;
        crow[v] = grow - c_sub;
        ok[v] = grow < ti.r1 && !(p.c_local && crow[v] >= p.c_rows);
      }
      if (EPI == EPI_SWIGLU) {
        uint16_t* C = (uint16_t*)p.C;
#pragma unroll
        for (int jp = 0; jp < TN / 2; ++jp) {
          __builtin_amdgcn_sched_barrier(0);
          // B rows alternate 32 gate and 32 up weight rows: MI = 32 pairs
          // blocks (2jp, 2jp+1); MI = 16 pairs (g, g+2), g = 4 (jp/2) + jp%2
          const int jg = MI == 32 ? 2 * jp : 4 * (jp >> 1) + (jp & 1);
          const int ju = MI == 32 ? jg + 1 : jg + 2;
          const int col = MI == 32 ? n0h + (wn * (TN / 2) + jp) * 32 + lrow
                                   : n0h + (wn * (WTN / 64) + (jp >> 1)) * 32 + (jp & 1) * 16 + lrow;
#pragma unroll
          for (int v = 0; v < NV; ++v) {
            if (!ok[v]) continue;
            const float h = silu_mul(acc_read(acc[i][jg][v]), acc_read(acc[i][ju][v]));
            C[(long long)crow[v] * p.ldc + col] = Act<DT>::store(h);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          __builtin_amdgcn_sched_barrier(0);
          const int col = n0 + wn * WTN + j * MI + lrow;
#pragma unroll
          for (int v = 0; v < NV; ++v) {
            if (!ok[v]) continue;
            float y = acc_read(acc[i][j][v]);
            if (EPI == EPI_GELU) y = gelu_erf16(y);
            ((uint16_t*)p.C)[(long long)crow[v] * p.ldc + col] = Act<DT>::store(y);
            // erf is long: one value at a time keeps its temporaries few
            if (EPI == EPI_GELU) __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    }
  }
};

}  // namespace moe
