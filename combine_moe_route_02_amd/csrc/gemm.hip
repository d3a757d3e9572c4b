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

// Finds the group and row range of global m-tile `mt` from the device-side
// offsets.  Every thread of the block must call it; returns false (for the
// whole block) when the slot is beyond the last tile.
template <int NT, int BM>
__device__ bool locate_mtile(const GemmArgs& p, int mt, int* s_scan, int* s_res,
                             TileInfo& ti) {
  if (p.offsets == nullptr) {
    const int tiles = (p.dense_M + BM - 1) / BM;
    if (mt >= tiles) return false;
    ti.g = 0;
    ti.r0 = mt * BM;
    ti.r1 = p.dense_M;
    ti.base = 0;
    return true;
  }
  if (threadIdx.x == 0) s_res[0] = -1;
  int carry = 0;
  for (int b = 0; b < p.n_groups; b += NT) {
    const int g = b + (int)threadIdx.x;
    int o0 = 0, o1 = 0, tiles = 0;
    if (g < p.n_groups) {
      o0 = p.offsets[p.e_begin + g];
      o1 = p.offsets[p.e_begin + g + 1];
      tiles = (o1 - o0 + BM - 1) / BM;
    }
    const int incl = block_incl_scan<NT>(tiles, s_scan) + carry;
    const int excl = incl - tiles;
    if (tiles > 0 && mt >= excl && mt < incl) {
      s_res[0] = g;
      s_res[1] = o0 + (mt - excl) * BM;
      s_res[2] = o1;
    }
    carry += s_scan[NT - 1];
    __syncthreads();
    if (s_res[0] >= 0) break;
  }
  if (s_res[0] < 0) return false;
  ti.g = s_res[0];
  ti.r0 = s_res[1];
  ti.r1 = s_res[2];
  ti.base = p.offsets[p.e_begin];
  return true;
}

// logical tile id -> (m-tile slot, n-tile), XCD-aware and banded.
__device__ __forceinline__ void tile_coords(const GemmArgs& p, int& mt, int& nt) {
  const int G8 = (int)gridDim.x >> 3;
  const int bid = (int)blockIdx.x;
  const int logical = (bid & 7) * G8 + (bid >> 3);
  const int band = p.gm * p.n_tiles;
  const int within = logical % band;
  nt = within / p.gm;
  mt = (logical / band) * p.gm + within % p.gm;
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
__device__ __forceinline__ void fp8x16_to_bf16(const uint4& q, float s, uint4& lo,
                                               uint4& hi) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
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
  lo = make_uint4(o[0], o[1], o[2], o[3]);
  hi = make_uint4(o[4], o[5], o[6], o[7]);
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
  __shared__ int s_scan[NT];
  __shared__ int s_res[3];

  int mt, nt;
  tile_coords(p, mt, nt);
  if (mt >= p.mt_slots) return;
  TileInfo ti;
  if (!locate_mtile<NT, BM>(p, mt, s_scan, s_res, ti)) return;

  const int tid = (int)threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const long long a_sub = p.a_local ? ti.base : 0;
  const long long c_sub = p.c_local ? ti.base : 0;
  const int n0 = nt * BN;
  const int n0h = nt * (BN / 2);

  // Source addresses and LDS slots of this thread's chunks.
  const uint16_t* Ag = (const uint16_t*)p.A;
  const uint16_t* a_src[ACH];
  int a_lds[ACH];
#pragma unroll
  for (int i = 0; i < ACH; ++i) {
    const int c = tid + i * NT;
    const int row = c >> 3, kc = c & 7;
    int grow = ti.r0 + row;
    grow = grow < ti.r1 ? grow : ti.r1 - 1;
    long long arow = grow - a_sub;
    if (p.a_local && arow >= p.a_rows) arow = p.a_rows - 1;
    a_src[i] = Ag + arow * p.lda + kc * 8;
    a_lds[i] = row * BK + ((kc ^ (row & 7)) << 3);
  }
  const uint8_t* b_src[BCH];
  int b_lds[BCH];
  const float* s_src[BCH];
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
    const long long eoff = (long long)ti.g * p.strideB + (long long)n * p.ldb;
    if (WK == W_FP8) {
      b_src[i] = (const uint8_t*)p.B + eoff + kc * 8;
      s_src[i] = p.Bscale + (long long)ti.g * p.strideS +
                 (long long)(n >> 7) * (p.K >> 7);
    } else {
      b_src[i] = (const uint8_t*)p.B + (eoff + kc * 8) * 2;
      s_src[i] = nullptr;
    }
    b_lds[i] = row * BK + ((kc ^ (row & 7)) << 3);
  }

  uint4 ra[ACH], rb[BCH];
  float rs[BCH];
  auto load_tiles = [&](int k0) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) ra[i] = *(const uint4*)(a_src[i] + k0);
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
      if (WK == W_FP8) {
        rb[i] = *(const uint4*)(b_src[i] + k0);
        rs[i] = s_src[i][k0 >> 7];
      } else {
        rb[i] = *(const uint4*)(b_src[i] + (long long)k0 * 2);
      }
    }
  };
  auto store_tiles = [&](int buf) {
    uint16_t* As = sA[buf];
    uint16_t* Bs = sB[buf];
#pragma unroll
    for (int i = 0; i < ACH; ++i) *(uint4*)(As + a_lds[i]) = ra[i];
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
      if (WK == W_FP8) {
        uint4 lo, hi;
        fp8x16_to_bf16(rb[i], rs[i], lo, hi);
        const int row = b_lds[i] / BK;
        const int kc = ((b_lds[i] % BK) >> 3) ^ (row & 7);
        *(uint4*)(Bs + b_lds[i]) = lo;
        *(uint4*)(Bs + row * BK + (((kc + 1) ^ (row & 7)) << 3)) = hi;
      } else {
        *(uint4*)(Bs + b_lds[i]) = rb[i];
      }
    }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int nk = p.K / BK;
  load_tiles(0);
  store_tiles(0);
  __syncthreads();

  const int lrow = lane & 31;
  const int khalf = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_tiles((kt + 1) * BK);
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
    if (kt + 1 < nk) store_tiles(cur ^ 1);
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
}

// Plain fp32 grouped GEMM (64x64 tiles, 4x4 outputs per thread).
template <int EPI>
__global__ void __launch_bounds__(256) grouped_gemm_f32(GemmArgs p) {
  constexpr int BM = 64, BN = 64, BK = 16, NT = 256;
  __shared__ float sA[BM][BK + 1];
  __shared__ float sB[BN][BK + 1];
  __shared__ int s_scan[NT];
  __shared__ int s_res[3];

  int mt, nt;
  tile_coords(p, mt, nt);
  if (mt >= p.mt_slots) return;
  TileInfo ti;
  if (!locate_mtile<NT, BM>(p, mt, s_scan, s_res, ti)) return;

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
}

// ---------------------------------------------------------------------------
// Host launcher
// ---------------------------------------------------------------------------

namespace {

template <int BM>
void size_grid(GemmArgs& a, int max_rows, int BN, int gm, dim3& grid) {
  int slots;
  if (a.offsets == nullptr)
    slots = (a.dense_M + BM - 1) / BM;
  else
    slots = (max_rows + BM - 1) / BM + a.n_groups;
  if (gm > slots) gm = slots;
  if (gm < 1) gm = 1;
  slots = (slots + gm - 1) / gm * gm;
  a.mt_slots = slots;
  a.n_tiles = a.Nb / BN;
  a.gm = gm;
  long long total = (long long)slots * a.n_tiles;
  total = (total + 7) / 8 * 8;
  grid = dim3((unsigned)total);
}

template <int DT, int WK, int EPI, int BM, int BN, int WM, int WN>
int run_mfma(GemmArgs a, int max_rows, int gm, hipStream_t s) {
  if (a.Nb % BN || a.K % 64) return MOE_ERR_UNSUPPORTED;
  if (WK == W_FP8 && (a.K % 128 || a.Nb % 128)) return MOE_ERR_UNSUPPORTED;
  dim3 grid;
  size_grid<BM>(a, max_rows, BN, gm, grid);
  if (grid.x == 0) return MOE_OK;
  hipLaunchKernelGGL((grouped_gemm_mfma<DT, WK, EPI, BM, BN, WM, WN>), grid,
                     dim3(WM * WN * 64), 0, s, a);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

template <int DT, int WK, int EPI>
int pick_tile(GemmArgs a, int max_rows, hipStream_t s) {
  const int groups = a.offsets ? a.n_groups : 1;
  const int rows = a.offsets ? max_rows : a.dense_M;
  const int avg = rows / (groups > 0 ? groups : 1);
  if (EPI == EPI_F32) return run_mfma<DT, WK, EPI, 64, 128, 2, 2>(a, max_rows, 4, s);
  if (avg <= 64) return run_mfma<DT, WK, EPI, 32, 256, 1, 4>(a, max_rows, 1, s);
  return run_mfma<DT, WK, EPI, 128, 256, 2, 2>(a, max_rows, 4, s);
}

template <int EPI>
int run_f32(GemmArgs a, int max_rows, hipStream_t s) {
  if (a.Nb % 64 || a.K % 16) return MOE_ERR_UNSUPPORTED;
  dim3 grid;
  size_grid<64>(a, max_rows, 64, 4, grid);
  if (grid.x == 0) return MOE_OK;
  hipLaunchKernelGGL((grouped_gemm_f32<EPI>), grid, dim3(256), 0, s, a);
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
