// Host-side launchers shared between the translation units of the library.
#pragma once

#include "moe_common.h"

namespace moe {

enum Epilogue { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_GELU = 2 };

// One grouped GEMM  C[r, n] = epi( sum_k A[r, k] * B_g[n', k] )  over the
// row segments of groups g = 0..n_groups-1.
struct GemmArgs {
  const void* A;          // activations, 16-bit or f32 (E4M3 codes: launch_gemm_fp8_act)
  long long lda;
  const float* Ascale;    // E4M3 activations: one scale per A row
  const void* B;          // weights of group 0; group g at B + g * strideB
  long long strideB;      // elements (bytes for fp8)
  long long ldb;
  const float* Bscale;    // fp8: [G][rows/128][K/128]
  long long strideS;
  void* C;
  long long ldc;
  const int32_t* offsets; // device: rows of group g = [offsets[e_begin+g], offsets[e_begin+g+1])
  int e_begin;
  int n_groups;
  int dense_M;            // offsets == nullptr: one group of dense_M rows
  int a_local;            // A row index = r - offsets[e_begin] (else r)
  int c_local;            // C row index = r - offsets[e_begin] (else r)
  int a_rows;             // a_local: rows of A (reads are clamped below it)
  int c_rows;             // c_local: rows of C (rows at or past it are not written)
  int Nb;                 // weight rows used by the tile grid (2I for SwiGLU)
  int I;                  // SwiGLU split: gate rows [0, I), up rows [I, 2I)
  int K;
  int mt_slots;           // m-tile slots in the grid
  int n_tiles;
  int gm;                 // m-tiles per band in the tile order
  // Optional k-split of the last, partial round of tiles (16-bit weights):
  // fp32 partial-sum slots and arrival counters in the caller's workspace,
  // or nullptr.
  float* split_ws;
  int* split_cnt;
  long long split_slots;  // slots available (slot = one tile's accumulators)
};

// FFN workspace: arrival counters, then partial-sum slots of split tiles.
constexpr long long kSplitCounterBytes = 16384;
size_t ffn_ws_bytes();
void ffn_ws_attach(GemmArgs& a, void* ws, size_t ws_bytes);

// Column slices for the one-wave-per-token row kernels (gather, combine):
// a batch of few tokens is cut into slices of whole 64-chunk groups so that
// about 2048 waves are in flight; cps = 16-byte chunks per slice.
inline void row_slices(int T, int nch, int& slices, int& cps) {
  const int groups = (nch + 63) / 64;
  int want = T > 0 ? (2048 + T - 1) / T : 1;
  if (want > groups) want = groups;
  if (want < 1) want = 1;
  const int gps = (groups + want - 1) / want;  // 64-chunk groups per slice
  cps = gps * 64;
  slices = (nch + cps - 1) / cps;
}

// GEMM launchers; return MOE_OK / MOE_ERR_UNSUPPORTED / MOE_ERR_HIP.
int launch_grouped_gemm(int act_dtype, int w_dtype, int epi, GemmArgs a,
                        int max_rows, hipStream_t stream);
// E4M3 activations (per-row scales) times E4M3 weights (128x128 block
// scales) on fp8 MFMA, bf16 output.
int launch_gemm_fp8_act(int epi, GemmArgs a, int max_rows, hipStream_t stream);

}  // namespace moe
