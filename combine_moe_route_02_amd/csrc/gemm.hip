// Grouped expert GEMMs on MFMA (gfx950) and a plain fp32 path.
//
// The expert FFN of each local expert is a dense contraction over that
// expert's contiguous row segment (GPT-4 MoE page, section 3.1 table: each
// expert is Linear -> activation -> Linear; the segments are the dense
// per-expert layout built at dispatch, DySHARP page, section 3.1 item 3).
// Segment sizes are read on the device from `offsets`, so the grid is sized
// from host-known upper bounds only and surplus workgroups exit at once.
//
// Tile order.  Persistent workgroups; each XCD (hardware dispatches
// workgroup i to XCD i % 8) takes a contiguous slice of the logical tile
// order, which keeps one expert's tiles together: all m-tiles of an expert
// (in bands of at most `gm`) for one n-tile, then the next n-tile.  The
// m-tiles of a band share each weight tile in that XCD's L2, so expert
// weights are read from HBM about once, and a band's activation rows are
// reused across its n-tiles.
//
// 16-bit weights (DmaTile): global -> LDS directly, two stages of BK = 64;
// each wave owns a (BM/WM) x (BN/WN) accumulator block of 16x16 MFMA tiles
// (v_mfma_f32_16x16x32_{bf16,f16}).
// fp8 weights (register-staged kernel below): BK = 64; global -> registers
// -> LDS with a two-buffer ring and one barrier per k-step; 16-byte chunks
// are stored XOR-swizzled (chunk ^ (row & 7)) so that the ds_read_b128 of an
// MFMA operand (32 rows, same k-chunk) touches every bank group once.  Each
// wave owns a (BM/WM) x (BN/WN) accumulator block of 32x32 MFMA tiles
// (v_mfma_f32_32x32x16: 8 values of K per lane per operand).
//
// Epilogues: plain store in the activation dtype, SwiGLU (the B tile
// interleaves 32-row groups of gate and up rows so a wave holds both halves
// of the same h columns), or exact-erf GELU.
// fp8 E4M3 weights are decoded and scaled by their 128x128 tile scale while
// being staged to LDS as bf16.

#include <math.h>

#include "gemm_tile.h"

namespace moe {

enum { W_SAME = 0, W_FP8 = 1 };

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
  const TileInfo ti = band_tile<BM>(p, s_pre, t, p.n_tiles, p.gm, mt, nt);

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
      } else {
        uint16_t* C = (uint16_t*)p.C;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          float y = acc[i][j][v];
          if (EPI == EPI_GELU) y = gelu_erf16(y);
          C[crow * p.ldc + n0 + wn * WTN + j * 32 + lrow] = Act<DT>::store(y);
        }
      }
    }
  }
  }  // tile loop
}

// ---------------------------------------------------------------------------
// fp8 E4M3 weights with few rows per group (decode batches): the weight
// stream is the whole cost, so the tile keeps two 40 KB stages in flight per
// CU and copies whole 128-byte lines.  BM = 32 token rows, BN = 256 weight
// rows, BK = 128: one cache line of each fp8 weight row and exactly one
// 128x128 scale block per 32-row column group per k-step.  Weights stay fp8
// in LDS; each B fragment (8 codes) is decoded exactly to the MFMA input
// type (every E4M3 value is representable in bf16), the k-step's
// products accumulate unscaled, and the block scale multiplies the k-step's
// fp32 partial sums.  Four waves, each 32 x 64 (two 32x32 MFMA columns).
// ---------------------------------------------------------------------------

// 8 E4M3 codes -> 8 bf16, exact (every E4M3 value is a bf16 value): one
// v_cvt_scalef32_pk_bf16_fp8 per two codes, with scale 1 (through f32 with
// v_cvt_pk_f32_fp8 it takes three instructions per two codes; same bits for
// all 256 codes).
__device__ __forceinline__ bf16x8 decode_fp8x8(uint32_t lo, uint32_t hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);  // bytes 0, 1
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);   // bytes 2, 3
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  u32x4 u;
  u[0] = __builtin_bit_cast(uint32_t, a);
  u[1] = __builtin_bit_cast(uint32_t, b);
  u[2] = __builtin_bit_cast(uint32_t, c);
  u[3] = __builtin_bit_cast(uint32_t, d);
  return __builtin_bit_cast(bf16x8, u);
}

// A8: the activations arrive as E4M3 codes with one power-of-two scale per
// row (fp8 dispatch transport).  Both operands then stay fp8 from HBM to the
// MFMA (v_mfma_f32_32x32x16_fp8_fp8, same fragment layout as the 16-bit
// 32x32x16 form, one byte per element); the row scale multiplies the fp32
// sums in the epilogue (exact: a power of two).
__device__ __forceinline__ long fp8x8_as_long(uint32_t lo, uint32_t hi) {
  return (long)(((unsigned long)hi << 32) | lo);
}

template <int DT, int EPI, bool A8 = false, int TN = 2>
struct Fp8SmallTile {
  static_assert(DT == MOE_DTYPE_BF16, "fp8 weights pair with bf16 activations");
  static_assert(TN == 2 || (TN == 1 && EPI != EPI_SWIGLU), "SwiGLU pairs two column groups");
  static constexpr int BM = 32, BN = 128 * TN, BK = 128, NS = 3, NW = 4;
  static constexpr int NT = NW * 64;
  static constexpr int WC = 32 * TN;                  // columns per wave
  static constexpr int A_ROWB = A8 ? BK : BK * 2;     // 128 B (fp8) or 256 B (16-bit)
  static constexpr int B_ROWB = BK;                   // 128 B (fp8)
  static constexpr int A_BYTES = BM * A_ROWB, B_BYTES = BN * B_ROWB;
  static constexpr int STAGE = A_BYTES + B_BYTES;     // 40 KB (24 KB at TN = 1)
  static constexpr int A_BLK = A_BYTES / 1024;        // blocks of 4 (fp8: 8) A rows
  static constexpr int B_BLK = B_BYTES / 1024;        // blocks of 8 B rows
  static constexpr int BPW = (A_BLK + B_BLK) / NW;
  static constexpr int JA = A_BLK / NW;
  static constexpr int SMEM = NS * STAGE;
  static constexpr int SR = 4;  // scale registers per column group: K <= 64 * SR * BK
  static_assert(A_BLK % NW == 0 && B_BLK % NW == 0 && 2 * BPW < 64, "blocks");

  __device__ static __forceinline__ void run(const GemmArgs& p, const TileInfo& ti, int nt,
                                             char* smem) {
    typedef typename MfmaOp<DT>::V V;
    const int tid = (int)threadIdx.x;
    const int lane = tid & 63;
    const int wn = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lrow = lane & 31;
    const int khalf = lane >> 5;
    const int a_sub = p.a_local ? ti.base : 0;
    const int c_sub = p.c_local ? ti.base : 0;
    const int n0 = nt * BN;
    const int n0h = nt * (BN / 2);

    int base_row = ti.r0 - a_sub;
    if (p.a_local && base_row > p.a_rows - 1) base_row = p.a_rows - 1;
    constexpr int AE = A8 ? 1 : 2;  // bytes per A element
    const char* a_tile = uniform_ptr((const char*)p.A + (long long)base_row * p.lda * AE);
    const char* b_tile = uniform_ptr((const char*)p.B + (long long)ti.g * p.strideB);
    uint32_t voff[BPW];
    int ldsoff[BPW];
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
      const int q = wn + NW * j;
      if (j < JA) {
        // 16-bit A: 4 rows x 256 B per block, 16-byte chunk c of row r at
        // c ^ (r & 15); fp8 A: 8 rows x 128 B, chunk c at c ^ ((r >> 1) & 7)
        const int row = A8 ? 8 * q + (lane >> 3) : 4 * q + (lane >> 4);
        const int kc = A8 ? (lane & 7) ^ ((row >> 1) & 7) : (lane & 15) ^ (row & 15);
        int grow = ti.r0 + row;
        grow = grow < ti.r1 ? grow : ti.r1 - 1;
        int arow = grow - a_sub;
        if (p.a_local && arow >= p.a_rows) arow = p.a_rows - 1;
        voff[j] = (uint32_t)(arow - base_row) * (uint32_t)(p.lda * AE) + (uint32_t)(kc * 16);
        ldsoff[j] = q * 1024;
      } else {
        // B: 8 rows x 128 B per block; 16-byte chunk c of row r at c ^ ((r >> 1) & 7)
        const int qb = q - A_BLK;
        const int row = 8 * qb + (lane >> 3);
        const int kc = (lane & 7) ^ ((row >> 1) & 7);
        int n;
        if (EPI == EPI_SWIGLU) {
          const int gi = row >> 5;
          n = ((gi & 1) ? p.I : 0) + n0h + (gi >> 1) * 32 + (row & 31);
        } else {
          n = n0 + row;
        }
        voff[j] = (uint32_t)n * (uint32_t)p.ldb + (uint32_t)(kc * 16);
        ldsoff[j] = A_BYTES + qb * 1024;
      }
    }
    // scale rows of this wave's two column groups
    const float* srow[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      int n;
      if (EPI == EPI_SWIGLU) n = (j ? p.I : 0) + n0h + wn * 32;
      else n = n0 + wn * WC + j * 32;
      srow[j] = p.Bscale + (long long)ti.g * p.strideS + (long long)(n >> 7) * (p.K >> 7);
    }

    f32x16 acc[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[j][v] = 0.0f;

    const uint32_t lds0 = lds_addr(smem);
#define MOE_ISSUE8(st)                                                             \
do {                                                                             \
    const uint32_t dst_ = lds0 + ((st) % NS) * STAGE;                              \
    const char* ak_ = a_tile + (st) * A_ROWB;                                      \
    const char* bk_ = b_tile + (st) * B_ROWB;                                      \
    _Pragma("unroll") for (int j = 0; j < BPW; ++j) {                              \
      if (j < JA) dma16(ak_, voff[j], dst_ + ldsoff[j]);                           \
      else dma16_stream(bk_, voff[j], dst_ + ldsoff[j]);                           \
    }                                                                            \
} while (0)

    // The k-step scales of this wave's column groups, lane l holding k-step
    // l + 64 q in register q; read per k-step with v_readlane.  Loaded and
    // waited for here, before any copy is in flight: a vector load of the
    // scale inside the k-loop would make the wait for it (vmcnt counts in
    // issue order) also wait for the two stages of copies issued before it,
    // draining the copy pipeline every k-step.
    const int nk = p.K / BK;
    float scr[TN][SR];
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < SR; ++q) {
        const int kk = lane + 64 * q;
        scr[j][q] = kk < nk ? srow[j][kk] : 0.0f;
      }
    wait_vmcnt<0>();
    lds_barrier();  // every wave is done with the previous tile's stages
    MOE_ISSUE8(0);
    if (nk > 1) MOE_ISSUE8(1);
    for (int kt = 0; kt < nk; ++kt) {
      // stage kt landed (stage kt+1 may be in flight), visible to all waves;
      // every wave is done reading stage kt-1, whose buffer takes kt+2
      if (kt + 1 < nk) wait_vmcnt<BPW>(); else wait_vmcnt<0>();
      __builtin_amdgcn_s_waitcnt((0x3F & 0xF) | (0x7 << 4) | ((0x3F >> 4) << 14));
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (kt + 2 < nk) MOE_ISSUE8(kt + 2);
      float sc[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        float r = scr[j][0];
#pragma unroll
        for (int q = 1; q < SR; ++q)
          if ((kt >> 6) == q) r = scr[j][q];
        sc[j] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, r), kt & 63));
      }
      const char* As = smem + (kt % NS) * STAGE;
      const char* Bs = As + A_BYTES;
      f32x16 part[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) part[j][v] = 0.0f;
#pragma unroll
      for (int s8 = 0; s8 < BK / 16; ++s8) {
        if constexpr (A8) {
          const uint2 a8 = *(const uint2*)(As + lrow * A_ROWB +
                                          ((s8 ^ ((lrow >> 1) & 7)) << 4) + khalf * 8);
          const long a = fp8x8_as_long(a8.x, a8.y);
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const int brow = wn * WC + j * 32 + lrow;
            const uint2 q8 = *(const uint2*)(Bs + brow * B_ROWB +
                                            ((s8 ^ ((brow >> 1) & 7)) << 4) + khalf * 8);
            part[j] = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(
                a, fp8x8_as_long(q8.x, q8.y), part[j], 0, 0, 0);
          }
        } else {
          const V a = *(const V*)(As + lrow * A_ROWB + (((2 * s8 + khalf) ^ (lrow & 15)) << 4));
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const int brow = wn * WC + j * 32 + lrow;
            const uint2 q8 = *(const uint2*)(Bs + brow * B_ROWB +
                                            ((s8 ^ ((brow >> 1) & 7)) << 4) + khalf * 8);
            part[j] = MfmaOp<DT>::run(a, decode_fp8x8(q8.x, q8.y), part[j]);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[j][v] += sc[j] * part[j][v];
    }
#undef MOE_ISSUE8

    const int rsub = khalf * 4;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int grow = ti.r0 + (v >> 2) * 8 + rsub + (v & 3);
      if (grow >= ti.r1) continue;
      const long long crow = grow - c_sub;
      if (p.c_local && crow >= p.c_rows) continue;
      if constexpr (A8) {
        const float as = p.Ascale[grow - a_sub];  // the row's power-of-two scale
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[j][v] *= as;
      }
      uint16_t* C = (uint16_t*)p.C;
      if (EPI == EPI_SWIGLU) {
        const float h = silu_mul(acc[0][v], acc[1][v]);
        C[crow * p.ldc + n0h + wn * 32 + lrow] = Act<DT>::store(h);
      } else {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          float y = acc[j][v];
          if (EPI == EPI_GELU) y = gelu_erf16(y);
          C[crow * p.ldc + n0 + wn * WC + j * 32 + lrow] = Act<DT>::store(y);
        }
      }
    }
  }
};

template <int DT, int EPI, bool A8 = false, int TN = 2>
__global__ void __launch_bounds__(256) grouped_gemm_fp8s(GemmArgs p) {
  typedef Fp8SmallTile<DT, EPI, A8, TN> Tile;
  __shared__ __attribute__((aligned(1024))) char smem[Tile::SMEM];
  __shared__ int s_pre[1024];
  __shared__ int s_scan[Tile::NT];
  const int total_m = build_mtile_table<Tile::NT, Tile::BM>(p, s_pre, s_scan);
  int t_first, t_end, t_stride;
  xcd_share(total_m * p.n_tiles, t_first, t_end, t_stride);
  for (int t = t_first; t < t_end; t += t_stride) {
    int mt, nt;
    const TileInfo ti = band_tile<Tile::BM>(p, s_pre, t, p.n_tiles, p.gm, mt, nt);
    Tile::run(p, ti, nt, smem);
  }
}

// Parts per tile of a last round of rem tiles on per workgroups (one XCD's
// share): when the round leaves at least half the workgroups idle, each tile
// is split into per / rem parts (at most 8, each of at least 4 k-steps), one
// per workgroup.  Splitting a fuller round does not pay: measured at the
// DeepSeek-V3-like share (a 62%-full round split in 3, two parts per
// workgroup), the partial sums' traffic made GEMM-1 8% slower.
__device__ __forceinline__ int split_parts(int rem, int per, int nk) {
  if (2 * rem > per) return 1;
  int S = per / rem;
  if (S > 8) S = 8;
  if (S > nk / 4) S = nk / 4;
  return S < 1 ? 1 : S;
}

template <int DT, int EPI, int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(WM * WN * 64)
    grouped_gemm_dma(GemmArgs p) {
  typedef DmaTile<DT, EPI, BM, BN, WM, WN> Tile;
  __shared__ __attribute__((aligned(1024))) char smem[Tile::SMEM];
  __shared__ int s_pre[1024];
  __shared__ int s_scan[Tile::NT];
  __shared__ int s_flag;
  const int total_m = build_mtile_table<Tile::NT, BM>(p, s_pre, s_scan);
  // Each XCD takes a contiguous slice of the tile order; its workgroups take
  // whole rounds of tiles.  The last, partial round (rem tiles for per
  // workgroups) is split over k when a workspace is given and split_parts
  // says so: S parts per tile, part s of local tile u on workgroup u * S + s
  // of the XCD.
  const int total = total_m * p.n_tiles;
  const int xcd = (int)blockIdx.x & 7;
  const int per = (int)gridDim.x >> 3;
  const int idx = (int)blockIdx.x >> 3;
  const int lo = (int)((long long)total * xcd / 8);
  const int len = (int)((long long)total * (xcd + 1) / 8) - lo;
  const int full = len / per;
  const int rem = len - full * per;
  const int nk_all = p.K / Tile::BK;
  const int S = rem > 0 && p.split_ws != nullptr ? split_parts(rem, per, nk_all) : 1;
  for (int r = 0; r < full; ++r) {
    int mt, nt;
    const TileInfo ti = band_tile<BM>(p, s_pre, lo + r * per + idx, p.n_tiles, p.gm, mt, nt);
    // the next full-K tile of this workgroup, if any (its weight lines are
    // prefetched during this tile's epilogue)
    int nx = -1;
    if (r + 1 < full) nx = lo + (r + 1) * per + idx;
    else if (rem > 0 && S == 1 && idx < rem) nx = lo + full * per + idx;
    int nx_g = -1, nx_nt = 0;
    if (nx >= 0) {
      int mt2;
      nx_g = band_tile<BM>(p, s_pre, nx, p.n_tiles, p.gm, mt2, nx_nt).g;
    }
    Tile::run(p, ti, nt, smem, nullptr, nullptr, nx_g, nx_nt);
  }
  if (rem == 0) return;
  if (S == 1) {
    if (idx < rem) {
      int mt, nt;
      const TileInfo ti = band_tile<BM>(p, s_pre, lo + full * per + idx, p.n_tiles, p.gm, mt, nt);
      Tile::run(p, ti, nt, smem, nullptr);
    }
    return;
  }
  if (idx < rem * S) {
    const int u = idx / S, part = idx % S;
    int mt, nt;
    const TileInfo ti = band_tile<BM>(p, s_pre, lo + full * per + u, p.n_tiles, p.gm, mt, nt);
    KSplit ks;
    ks.k0 = (int)((long long)part * nk_all / S);
    ks.nk = (int)((long long)(part + 1) * nk_all / S) - ks.k0;
    ks.parts = S;
    ks.part = part;
    ks.slot0 = p.split_ws + (long long)(((u * S) << 3) | xcd) * Tile::SLOT;
    ks.slot_step = 8 * Tile::SLOT;
    ks.counter = p.split_cnt + ((u << 3) | xcd);
    ks.s_flag = &s_flag;
    Tile::run(p, ti, nt, smem, nullptr, &ks);
  }
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
  const TileInfo ti = band_tile<BM>(p, s_pre, t, p.n_tiles, p.gm, mt, nt);

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
// occ: the caller's cache of the kernel's occupancy (one per kernel: every
// kernel here has the same function type, so a cache keyed on the type would
// be shared between them).
template <typename Kern>
dim3 persistent_grid(Kern kernel, int threads, GemmArgs& a, int max_rows, int BM, int BN,
                     int gm, int& occ) {
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
  static int occ = 0;
  const dim3 grid = persistent_grid(kern, WM * WN * 64, a, max_rows, BM, BN, gm, occ);
  hipLaunchKernelGGL(kern, grid, dim3(WM * WN * 64), 0, s, a);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

template <int DT, int EPI, int BM, int BN, int WM, int WN>
dim3 dma_grid(GemmArgs& a, int max_rows, int gm) {
  static int occ = 0;
  return persistent_grid(grouped_gemm_dma<DT, EPI, BM, BN, WM, WN>, WM * WN * 64, a, max_rows,
                         BM, BN, gm, occ);
}

template <int DT, int EPI, int BM, int BN, int WM, int WN>
int run_dma(GemmArgs a, int max_rows, int gm, hipStream_t s) {
  if (a.Nb % BN || a.K % 64) return MOE_ERR_UNSUPPORTED;
  // per-lane DMA offsets are 32-bit: one group's weight matrix must span < 4 GiB
  if ((long long)a.Nb * a.ldb * 2 >= (1ll << 32)) return MOE_ERR_UNSUPPORTED;
  if (a.offsets && a.n_groups > 1024) return MOE_ERR_UNSUPPORTED;
  auto kern = grouped_gemm_dma<DT, EPI, BM, BN, WM, WN>;
  const dim3 grid = dma_grid<DT, EPI, BM, BN, WM, WN>(a, max_rows, gm);
  // the k-split needs one slot per workgroup and one counter per tile slot
  typedef DmaTile<DT, EPI, BM, BN, WM, WN> Tile;
  // (slots are counted in units of a 256x256 tile's accumulators)
  if (a.split_ws && ((long long)grid.x * Tile::SLOT > a.split_slots * 65536ll ||
                     (long long)grid.x * 4 > kSplitCounterBytes))
    a.split_ws = nullptr;
  hipLaunchKernelGGL(kern, grid, dim3(WM * WN * 64), 0, s, a);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

template <int DT, int EPI, bool A8, int TN>
int launch_fp8s(GemmArgs a, int max_rows, hipStream_t s) {
  auto kern = grouped_gemm_fp8s<DT, EPI, A8, TN>;
  static int occ = 0;
  const dim3 grid = persistent_grid(kern, 256, a, max_rows, 32, 128 * TN, 1, occ);
  hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// Tiles of 256 columns, or of 128 where that fills the last round: with one
// 32-row tile per group (the decode regime), t tiles of 256 columns take
// ceil(t / G) rounds on G workgroups and 2t tiles of 128 columns half as long
// each (SwiGLU keeps 256: a wave pairs gate and up columns).
template <int DT, int EPI, bool A8 = false>
int run_fp8s(GemmArgs a, int max_rows, hipStream_t s) {
  // K: whole 128-wide scale blocks, at most 64 * SR of them in the scale registers
  if (a.Nb % 256 || a.K % 128 || a.K > 64 * 4 * 128) return MOE_ERR_UNSUPPORTED;
  if ((long long)a.Nb * a.ldb >= (1ll << 32)) return MOE_ERR_UNSUPPORTED;
  if (a.offsets && a.n_groups > 1024) return MOE_ERR_UNSUPPORTED;
  if constexpr (EPI != EPI_SWIGLU) {
    const long long G = device_cus();
    const long long t = (long long)(a.offsets ? a.n_groups : 1) * (a.Nb / 256);
    if ((2 * t + G - 1) / G < 2 * ((t + G - 1) / G))
      return launch_fp8s<DT, EPI, A8, 1>(a, max_rows, s);
  }
  return launch_fp8s<DT, EPI, A8, 2>(a, max_rows, s);
}

// Relative MFMA efficiency of each tile shape (larger wave tiles need fewer
// LDS reads per MFMA) used to pick a shape; rounds of 256 workgroups model the
// tail of the last wave of tiles.
struct TileShape {
  int BM, BN;
  float eff;
};

// Tile height of the many-rows path (256 or 128): a cost model that counts
// rounds of workgroups, with the last partial round split over k when a
// workspace is attached and it is at most half full.
template <int WK>
int choose_bm(const GemmArgs& a, int max_rows) {
  const int groups = a.offsets ? a.n_groups : 1;
  const int rows = a.offsets ? max_rows : a.dense_M;
  const double avg = (double)rows / (groups > 0 ? groups : 1);
  const TileShape shapes[2] = {{256, 256, 1.0f}, {128, 256, 0.8f}};
  int best = 0;
  double best_t = 1e300;
  for (int c = 0; c < 2; ++c) {
    const TileShape& t = shapes[c];
    if (a.Nb % t.BN) continue;
    // expected m-tiles: a segment's ragged tail costs half a tile on average
    const double mtiles = groups * (avg / t.BM + (a.offsets ? 0.5 : 1.0));
    const double tiles = mtiles * (a.Nb / t.BN);
    const double G = device_cus();
    double rounds = ceil(tiles / G);
    if (WK == W_SAME && a.split_ws) {
      // the last partial round is split over k when at most half full
      const double full = floor(tiles / G), rem = tiles - full * G;
      if (rem > 0 && 2 * rem <= G) rounds = full + 1.15 * rem / G;
    }
    const double tm = rounds * (double)t.BM * t.BN / t.eff;
    if (tm < best_t) {
      best_t = tm;
      best = c;
    }
  }
  return shapes[best].BM;
}

// Few rows per group (decode batches) take the 32-row tiles.
inline bool few_rows(const GemmArgs& a, int max_rows) {
  const int groups = a.offsets ? a.n_groups : 1;
  const int rows = a.offsets ? max_rows : a.dense_M;
  return (double)rows / (groups > 0 ? groups : 1) <= 48.0;
}

// m-tiles per band of the expert-band tile order (weight tiles shared by a
// band's m-tiles close together in time)
#ifndef MOE_BAND_GM
#define MOE_BAND_GM 8
#endif

template <int DT, int WK, int EPI>
int pick_tile(GemmArgs a, int max_rows, hipStream_t s) {
  if (few_rows(a, max_rows)) {
    if constexpr (WK == W_FP8 && DT == MOE_DTYPE_BF16) {
      const int st = run_fp8s<DT, EPI>(a, max_rows, s);
      if (st != MOE_ERR_UNSUPPORTED) return st;  // else the register-staged tile below
    }
    return run_mfma<DT, WK, EPI, 32, 256, 1, 4>(a, max_rows, 1, s);
  }
  if constexpr (WK == W_SAME) {
    if (choose_bm<WK>(a, max_rows) == 256)
      return run_dma<DT, EPI, 256, 256, 2, 2>(a, max_rows, MOE_BAND_GM, s);
    return run_dma<DT, EPI, 128, 256, 2, 2>(a, max_rows, MOE_BAND_GM, s);
  } else {
    return run_mfma<DT, WK, EPI, 128, 256, 2, 2>(a, max_rows, 8, s);
  }
}

template <int EPI>
int run_f32(GemmArgs a, int max_rows, hipStream_t s) {
  if (a.Nb % 64 || a.K % 16) return MOE_ERR_UNSUPPORTED;
  if (a.offsets && a.n_groups > 1024) return MOE_ERR_UNSUPPORTED;
  auto kern = grouped_gemm_f32<EPI>;
  static int occ = 0;
  const dim3 grid = persistent_grid(kern, 256, a, max_rows, 64, 64, 4, occ);
  hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

template <int DT, int WK>
int by_epi(int epi, GemmArgs a, int max_rows, hipStream_t s) {
  switch (epi) {
    case EPI_STORE: return pick_tile<DT, WK, EPI_STORE>(a, max_rows, s);
    case EPI_SWIGLU: return pick_tile<DT, WK, EPI_SWIGLU>(a, max_rows, s);
    case EPI_GELU: return pick_tile<DT, WK, EPI_GELU>(a, max_rows, s);
  }
  return MOE_ERR_ARG;
}

}  // namespace

int launch_gemm_fp8_act(int epi, GemmArgs a, int max_rows, hipStream_t stream) {
  // every row count runs on the 32-row tile: the fp8 transport serves the
  // weight-streaming decode regime
  switch (epi) {
    case EPI_SWIGLU: return run_fp8s<MOE_DTYPE_BF16, EPI_SWIGLU, true>(a, max_rows, stream);
    case EPI_GELU: return run_fp8s<MOE_DTYPE_BF16, EPI_GELU, true>(a, max_rows, stream);
  }
  return MOE_ERR_ARG;
}

int launch_grouped_gemm(int act_dtype, int w_dtype, int epi, GemmArgs a,
                        int max_rows, hipStream_t stream) {
  if (act_dtype == MOE_DTYPE_F32) {
    if (w_dtype != MOE_DTYPE_F32) return MOE_ERR_UNSUPPORTED;
    switch (epi) {
      case EPI_STORE: return run_f32<EPI_STORE>(a, max_rows, stream);
      case EPI_SWIGLU: return run_f32<EPI_SWIGLU>(a, max_rows, stream);
      case EPI_GELU: return run_f32<EPI_GELU>(a, max_rows, stream);
    }
    return MOE_ERR_ARG;
  }
  if (act_dtype == MOE_DTYPE_BF16) {
    if (w_dtype == MOE_DTYPE_BF16) return by_epi<MOE_DTYPE_BF16, W_SAME>(epi, a, max_rows, stream);
    if (w_dtype == MOE_DTYPE_FP8_E4M3)
      return by_epi<MOE_DTYPE_BF16, W_FP8>(epi, a, max_rows, stream);
    return MOE_ERR_UNSUPPORTED;
  }
  if (act_dtype == MOE_DTYPE_F16) {
    if (w_dtype == MOE_DTYPE_F16) return by_epi<MOE_DTYPE_F16, W_SAME>(epi, a, max_rows, stream);
    return MOE_ERR_UNSUPPORTED;
  }
  return MOE_ERR_UNSUPPORTED;
}

// One 256x256 tile's accumulators per workgroup of a one-per-CU grid.
size_t ffn_ws_bytes() {
  return (size_t)kSplitCounterBytes + (size_t)device_cus() * 65536 * sizeof(float);
}

void ffn_ws_attach(GemmArgs& a, void* ws, size_t ws_bytes) {
  a.split_ws = nullptr;
  a.split_cnt = nullptr;
  a.split_slots = 0;
  if (ws == nullptr || ws_bytes <= (size_t)kSplitCounterBytes) return;
  a.split_cnt = (int*)ws;
  a.split_ws = (float*)((char*)ws + kSplitCounterBytes);
  a.split_slots = (long long)((ws_bytes - kSplitCounterBytes) / (65536 * sizeof(float)));
}

}  // namespace moe
