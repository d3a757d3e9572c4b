// Router scores and top-k gating.
//
// A router scores each token against every expert and the top-k experts are
// kept (ThunderEP page, section 1.1; GPT-4 MoE page, section 2.3 stage 1).
// Gate weights are either the softmax over all experts, evaluated at the
// picks, with an optional temperature (GPT-4 MoE page, section 4.1 step 2;
// xDeepServe diary, section 5.3), or a sigmoid of each picked score, and
// may be renormalised to sum 1.  A minimum-probability threshold (GPT-4 MoE
// page, section 2.3 stage 2 and its section 4.1 sketch) drops every pick
// whose gate value is not above it: index -1, weight 0.  Gate values fall
// with the selection order, so dropped picks are the last of a token's k.
//
// Selection key.  s = logit + bias (one float32 add), -0.0 made +0.0, mapped
// to an order-preserving uint32 and placed above the complement of the
// expert index: the largest 64-bit key is the largest score and, among equal
// scores, the lowest index.  A 16-lane row of a wave owns a token (E <= 256,
// k <= 16; otherwise a whole wave does); k rounds of a uint64 max over the
// row pick the experts in descending order.

#include "gemm_tile.h"

namespace moe {

__device__ __forceinline__ uint64_t select_key(float s, int e) {
  if (s == 0.0f) s = 0.0f;  // -0.0 ties with +0.0
  const uint32_t b = __float_as_uint(s);
  const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)ord << 32) | (uint32_t)(~(uint32_t)e);
}

__device__ __forceinline__ float key_score(uint64_t key) {
  const uint32_t ord = (uint32_t)(key >> 32);
  const uint32_t b = (ord & 0x80000000u) ? (ord & 0x7fffffffu) : ~ord;
  return __uint_as_float(b);
}

// Max and sum over the 16 lanes of this lane's DPP row (lanes 16 r .. 16 r +
// 15), every lane receiving the result: four row rotations by 1, 2, 4 and 8
// lanes (v_mov_b32_dpp row_ror), no LDS permute.  The max is exact; the sum's
// association depends on the lane, so lanes may differ in the last bit.
__device__ __forceinline__ uint64_t row16_max_u64(uint64_t v) {
#define MOE_ROW_MAX(CTRL)                                                                  \
  do {                                                                                     \
    const uint32_t lo_ = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)v, CTRL, 0xf,  \
                                                            0xf, false);                  \
    const uint32_t hi_ = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), CTRL, \
                                                            0xf, 0xf, false);             \
    const uint64_t w_ = ((uint64_t)hi_ << 32) | lo_;                                       \
    v = w_ > v ? w_ : v;                                                                   \
  } while (0)
  MOE_ROW_MAX(0x121);
  MOE_ROW_MAX(0x122);
  MOE_ROW_MAX(0x124);
  MOE_ROW_MAX(0x128);
#undef MOE_ROW_MAX
  return v;
}

__device__ __forceinline__ float row16_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x121, 0xf, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x122, 0xf, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x124, 0xf, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xf, 0xf, false));
  return v;
}

// Top-k gating of one token by one wave: lane l holds the scores s[i] (bias
// added) of experts e = l + 64 i, i < EPL (experts past E must not count).
// k rounds of a wave-wide uint64 max pick the experts in descending order;
// lane j < k writes the j-th pick and its gate weight.
template <int EPL>
__device__ __forceinline__ void topk_token(const float (&s)[EPL], int E, int k, int gate,
                                           int renorm, float inv_temp, float min_prob,
                                           int32_t* __restrict__ idx_row,
                                           float* __restrict__ w_row) {
  const int lane = lane_id();
  uint64_t key[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    key[i] = e < E ? select_key(s[i], e) : 0;  // 0: below every real key
  }
  uint64_t mine = 0;  // lane j keeps the j-th pick
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (key[i] == best) key[i] = 0;
    if (lane == j) mine = best;
  }
  const uint64_t top = __shfl(mine, 0, MOE_WAVE);
  const float smax = key_score(top);
  float w = 0.0f;
  const float sj = key_score(mine);
  // With k <= 16 the two sums are taken in the order of the 16-lane
  // selection (topk_token16): lane r < 16 adds the terms of experts r + 16 i
  // in i order, then the lanes 0..15 combine by the same row rotations, so a
  // token gets the same weights, bit for bit, from either kernel (which one
  // runs depends on the batch size).  Expert r + 16 i is held by lane
  // r + 16 (i % 4), slot i / 4.
  const bool rows16 = k <= 16;
  if (gate == MOE_GATE_SOFTMAX) {
    float x[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      x[i] = lane + 64 * i < E ? expf((s[i] - smax) * inv_temp) : 0.0f;
    float denom;
    if (rows16) {
      float y[3][EPL];
#pragma unroll
      for (int q = 1; q < 4; ++q)
#pragma unroll
        for (int i = 0; i < EPL; ++i) y[q - 1][i] = __shfl(x[i], (lane + 16 * q) & 63, MOE_WAVE);
      float part = 0.0f;
#pragma unroll
      for (int i = 0; i < 4 * EPL; ++i) {
        const int q = i & 3, slot = i >> 2;
        if ((lane & 15) + 16 * i < E) part += q == 0 ? x[slot] : y[q - 1][slot];
      }
      denom = row16_sum(part);
    } else {
      float part = 0.0f;
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (lane + 64 * i < E) part += x[i];
      denom = wave_sum(part);
    }
    w = expf((sj - smax) * inv_temp) / denom;
  } else {
    w = 1.0f / (1.0f + expf(-sj));
  }
  // threshold on the gate value before renormalisation (min_prob 0: off)
  const bool keep = !(min_prob > 0.0f) || w > min_prob;
  if (!keep) w = 0.0f;
  if (renorm) {
    const float tot = rows16 ? row16_sum(lane < k ? w : 0.0f) : wave_sum(lane < k ? w : 0.0f);
    w = tot > 0.0f ? w / tot : 0.0f;
  }
  if (lane < k) {
    idx_row[lane] = keep ? (int32_t)(~(uint32_t)mine) : -1;
    w_row[lane] = w;
  }
}

// Top-k gating of four tokens at once, one 16-lane row of the wave each:
// lane 16 g + r holds the scores s[i] (bias added) of experts e = r + 16 i,
// i < EPL, of the row's token (experts past E must not count).  The same
// selection as topk_token, with the k rounds' maxima taken over the row by
// DPP rotations, so the four tokens' dependency chains interleave and no
// round waits on an LDS permute.  Lane r < k of a row writes that token's
// r-th pick when `valid`; k <= 16.
template <int EPL>
__device__ __forceinline__ void topk_token16(const float (&s)[EPL], int E, int k, int gate,
                                             int renorm, float inv_temp, float min_prob,
                                             bool valid, int32_t* __restrict__ idx_row,
                                             float* __restrict__ w_row) {
  const int r = lane_id() & 15;
  uint64_t key[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = r + 16 * i;
    key[i] = e < E ? select_key(s[i], e) : 0;  // 0: below every real key
  }
  uint64_t mine = 0, top = 0;  // lane r keeps the r-th pick; top is the first
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) best = key[i] > best ? key[i] : best;
    best = row16_max_u64(best);
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (key[i] == best) key[i] = 0;
    if (r == j) mine = best;
    if (j == 0) top = best;
  }
  const float smax = key_score(top);
  float w = 0.0f;
  const float sj = key_score(mine);
  if (gate == MOE_GATE_SOFTMAX) {
    float part = 0.0f;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (r + 16 * i < E) part += expf((s[i] - smax) * inv_temp);
    const float denom = row16_sum(part);
    w = expf((sj - smax) * inv_temp) / denom;
  } else {
    w = 1.0f / (1.0f + expf(-sj));
  }
  // threshold on the gate value before renormalisation (min_prob 0: off)
  const bool keep = !(min_prob > 0.0f) || w > min_prob;
  if (!keep) w = 0.0f;
  if (renorm) {
    const float tot = row16_sum(r < k ? w : 0.0f);
    w = tot > 0.0f ? w / tot : 0.0f;
  }
  if (valid && r < k) {
    idx_row[r] = keep ? (int32_t)(~(uint32_t)mine) : -1;
    w_row[r] = w;
  }
}

// Four tokens per wave, one per 16-lane row (E <= 256, k <= 16).
template <int EPL>
__global__ void __launch_bounds__(256)
    topk_gate16_kernel(const float* __restrict__ logits, const float* __restrict__ bias,
                       int T, int E, int k, int gate, int renorm, float inv_temp,
                       float min_prob, int32_t* __restrict__ topk_idx,
                       float* __restrict__ topk_w) {
  const int lane = lane_id();
  const int t0 = __builtin_amdgcn_readfirstlane(
      (int)(blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)) * 4);
  if (t0 >= T) return;
  const int t = t0 + (lane >> 4), r = lane & 15;
  const bool valid = t < T;
  const float* lg = logits + (long long)(valid ? t : T - 1) * E;
  float s[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = r + 16 * i;
    s[i] = 0.0f;
    if (e < E) s[i] = bias ? lg[e] + bias[e] : lg[e];
  }
  topk_token16<EPL>(s, E, k, gate, renorm, inv_temp, min_prob, valid,
                    topk_idx + (long long)t * k, topk_w + (long long)t * k);
}

// One wave per token; EPL = experts per lane (lane l holds e = l + 64*i).
template <int EPL>
__global__ void __launch_bounds__(256)
    topk_gate_kernel(const float* __restrict__ logits, const float* __restrict__ bias,
                     int T, int E, int k, int gate, int renorm, float inv_temp,
                     float min_prob, int32_t* __restrict__ topk_idx,
                     float* __restrict__ topk_w) {
  const int lane = lane_id();
  const int t = (int)(blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6));
  if (t >= T) return;
  const float* lg = logits + (long long)t * E;
  float s[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    s[i] = 0.0f;
    if (e < E) s[i] = bias ? lg[e] + bias[e] : lg[e];
  }
  topk_token<EPL>(s, E, k, gate, renorm, inv_temp, min_prob, topk_idx + (long long)t * k,
                  topk_w + (long long)t * k);
}

// 8 consecutive activations -> float (one or two 16-byte loads).
template <int DT>
__device__ __forceinline__ void load8(const typename Act<DT>::T* p, float* f) {
  if (DT == MOE_DTYPE_F32) {
    const float4 a = *(const float4*)p, b = *(const float4*)((const float*)p + 4);
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  } else {
    unpack8<DT>(*(const uint4*)p, f);
  }
}

// acc + a.lo * b.lo + a.hi * b.hi for two packed 16-bit values
// (v_dot2_f32_bf16 / v_dot2_f32_f16).
template <int DT>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  if constexpr (DT == MOE_DTYPE_BF16)
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), acc, false);
  else
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b),
                                  acc, false);
}

// Router projection on the vector ALUs: a block computes TPW tokens x EB
// experts (token block blockIdx.x, expert block blockIdx.y).  Its four waves
// split H: wave w takes the 8-element chunks c with (c / 64) % 4 == w, two
// chunks per step whose loads (kept packed until use) are all issued before
// the arithmetic, so each wave keeps 2 * (TPW + EB) 16-byte loads in flight
// and a row is covered in a quarter of the dependent load steps.  16-bit
// inputs go through packed dot products, two multiply-adds per instruction.  The four partial
// sums of each dot product are added in wave order through LDS (a fixed
// order: the result does not depend on timing).  Used for float32
// activations and for 16-bit rows whose length is not a multiple of 32.
template <int DT, int TPW, int EB>
__global__ void __launch_bounds__(256)
    router_valu_kernel(const void* __restrict__ x, const void* __restrict__ wr, int T,
                       int H, int E, float* __restrict__ logits) {
  typedef typename Act<DT>::T ST;
  constexpr int CPE = DT == MOE_DTYPE_F32 ? 2 : 1;  // 16-byte loads per 8 elements
  __shared__ float part[4][TPW][EB];
  const int lane = lane_id();
  const int wave = (int)threadIdx.x >> 6;
  const int t0 = (int)blockIdx.x * TPW;
  const int e0 = (int)blockIdx.y * EB;
  float acc[TPW][EB];
#pragma unroll
  for (int a = 0; a < TPW; ++a)
#pragma unroll
    for (int e = 0; e < EB; ++e) acc[a][e] = 0.0f;
  const ST* X = (const ST*)x;
  const ST* W = (const ST*)wr;
  const uint4* xrow[TPW];
  const uint4* wrow[EB];
#pragma unroll
  for (int a = 0; a < TPW; ++a) xrow[a] = (const uint4*)(X + (long long)min(t0 + a, T - 1) * H);
#pragma unroll
  for (int e = 0; e < EB; ++e) wrow[e] = (const uint4*)(W + (long long)min(e0 + e, E - 1) * H);
  const int nch = H >> 3;
  for (int c = wave * 64 + lane; c < nch; c += 512) {
    const bool two = c + 256 < nch;
    uint4 xq[2][TPW][CPE], wq[2][EB][CPE];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int cc = (u == 0 || two) ? c + 256 * u : c;
#pragma unroll
      for (int a = 0; a < TPW; ++a)
#pragma unroll
        for (int h = 0; h < CPE; ++h) xq[u][a][h] = xrow[a][cc * CPE + h];
#pragma unroll
      for (int e = 0; e < EB; ++e)
#pragma unroll
        for (int h = 0; h < CPE; ++h) wq[u][e][h] = wrow[e][cc * CPE + h];
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (u == 1 && !two) break;
      if constexpr (DT == MOE_DTYPE_F32) {
        float xf[TPW][8];
#pragma unroll
        for (int a = 0; a < TPW; ++a) load8<DT>((const ST*)xq[u][a], xf[a]);
#pragma unroll
        for (int e = 0; e < EB; ++e) {
          float wf[8];
          load8<DT>((const ST*)wq[u][e], wf);
#pragma unroll
          for (int a = 0; a < TPW; ++a)
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[a][e] = fmaf(xf[a][q], wf[q], acc[a][e]);
        }
      } else {
        // 16-bit pairs straight into the packed dot product (two products
        // and the float32 sum per instruction, no unpacking)
#pragma unroll
        for (int e = 0; e < EB; ++e) {
          const uint32_t wv[4] = {wq[u][e][0].x, wq[u][e][0].y, wq[u][e][0].z, wq[u][e][0].w};
#pragma unroll
          for (int a = 0; a < TPW; ++a) {
            const uint32_t xv[4] = {xq[u][a][0].x, xq[u][a][0].y, xq[u][a][0].z,
                                    xq[u][a][0].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[a][e] = dot2<DT>(xv[q], wv[q], acc[a][e]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int a = 0; a < TPW; ++a) {
#pragma unroll
    for (int e = 0; e < EB; ++e) {
      const float v = wave_sum(acc[a][e]);
      if (lane == 0) part[wave][a][e] = v;
    }
  }
  __syncthreads();
  const int i = (int)threadIdx.x;
  if (i < TPW * EB) {
    const int a = i / EB, e = i % EB;
    const float v = ((part[0][a][e] + part[1][a][e]) + part[2][a][e]) + part[3][a][e];
    if (t0 + a < T && e0 + e < E) logits[(long long)(t0 + a) * E + e0 + e] = v;
  }
}

// Router projection on the matrix cores for batches the staged GEMM tiles
// do not fit (few experts, or a decode batch): one block computes a tile of
// 16 tokens x 16 experts with v_mfma_f32_16x16x32_{bf16,f16}.  Each lane
// loads its operands straight from memory, 16 bytes per load: lane l reads
// row l % 16 (a token of x, an expert of Wr) at the 8-element chunk l / 16
// of every 32-wide k step, so each activation is read once per expert tile
// and one tile covers all experts when there are at most 16.  The NW waves
// of the block take consecutive ranges of k steps and issue the loads of up
// to U k steps at once (the block's time is a few load round trips), and
// their partial 16x16 sums are added in wave order through LDS (a fixed
// order: the result does not depend on timing).
// Expert rows past E are replaced by zeros and not written.

template <int DT, int NW, int U>
__global__ void __launch_bounds__(NW * 64)
    router_mfma_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
                       int T, int H, int E, float* __restrict__ logits) {
  typedef typename MfmaT<DT, 16>::V V;
  __shared__ f32x4 part[NW][64];
  const int lane = lane_id();
  const int wave = (int)threadIdx.x >> 6;
  const int t0 = (int)blockIdx.x * 16, e0 = (int)blockIdx.y * 16;
  const int r = lane & 15, q = lane >> 4;
  const bool ev = e0 + r < E;
  const uint4* xa = (const uint4*)(x + (long long)min(t0 + r, T - 1) * H) + q;
  const uint4* wb = (const uint4*)(wr + (long long)min(e0 + r, E - 1) * H) + q;
  const int nks = H >> 5;  // 32-wide k steps
  const int ks0 = nks * wave / NW, ks1 = nks * (wave + 1) / NW;
  const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  // batches of U k steps, all U loads of a batch in flight at once (past
  // ks1: the last k step again, with zero operands so it adds nothing)
  for (int ks = ks0; ks < ks1; ks += U) {
    uint4 a[U], b[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kk = min(ks + u, ks1 - 1);
      a[u] = xa[kk * 4];
      b[u] = wb[kk * 4];
    }
    __builtin_amdgcn_sched_barrier(0);  // every load of the batch issued first
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool in = ks + u < ks1;
      const uint4 av = in ? a[u] : zero;
      const uint4 bv = (in && ev) ? b[u] : zero;
      acc = MfmaT<DT, 16>::run(__builtin_bit_cast(V, av), __builtin_bit_cast(V, bv), acc);
    }
  }
  part[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    f32x4 s = part[0][lane];
#pragma unroll
    for (int w = 1; w < NW; ++w) s += part[w][lane];
    // 16x16 result layout: lane l holds column l % 16, rows 4 * (l / 16) + v
    if (ev) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = t0 + 4 * q + v;
        if (t < T) logits[(long long)t * E + e0 + r] = s[v];
      }
    }
  }
}

namespace {

template <int DT>
int launch_router_valu(const void* x, const void* wr, int T, int H, int E,
                       float* logits, hipStream_t s) {
#define MOE_ROUTER(TPW, EB)                                                          \
  do {                                                                               \
    hipLaunchKernelGGL((router_valu_kernel<DT, TPW, EB>),                            \
                       dim3((T + (TPW) - 1) / (TPW), (E + (EB) - 1) / (EB)),         \
                       dim3(256), 0, s, x, wr, T, H, E, logits);                     \
  } while (0)
  MOE_ROUTER(4, 8);
#undef MOE_ROUTER
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

template <int DT>
int launch_router_mfma(const void* x, const void* wr, int T, int H, int E, float* logits,
                       hipStream_t s) {
  const dim3 grid((T + 15) / 16, (E + 15) / 16);
  hipLaunchKernelGGL((router_mfma_kernel<DT, 8, 16>), grid, dim3(512), 0, s,
                     (const uint16_t*)x, (const uint16_t*)wr, T, H, E, logits);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// Router projection for many experts and large batches, paired tiles: a
// workgroup scores 128 tokens against 128 experts, and the E / 128
// workgroups that share a token tile run on one XCD at about the same time
// (block b is XCD b % 8), so the tile's activation rows come from HBM once
// and from that XCD's L2 for the others.  Against one workgroup per 64
// tokens x 256 experts this moves 32 KB instead of 40 KB into a compute
// unit per k-step and keeps the same LDS traffic.  Both operands go through
// LDS rings of NR 16 KB stages (128-byte rows by global_load_lds,
// XOR-swizzled chunks; a k-step's A and B copies are issued together); four
// waves of 64 x 64 (2 x 2 tiles of v_mfma_f32_32x32x16), float32 scores.
template <int DT>
__global__ void __launch_bounds__(256)
    router_pair_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
                       int T, int H, int E, int n_mt, float* __restrict__ logits) {
  constexpr int BM = 128, BN = 128, ROWB = 128, NW = 4, NR = 4;
  constexpr int A_STAGE = BM * ROWB, STAGE = (BM + BN) * ROWB;
  constexpr int JA = BM / 8 / NW, JB = BN / 8 / NW;  // 1 KB copies per wave and stage
  typedef typename MfmaOp<DT>::V V;
  __shared__ __attribute__((aligned(1024))) char smem[NR * STAGE];
  const int nn = E / BN;
  const int bid = (int)blockIdx.x;
  const int slot = bid >> 3;
  const int mt = (slot / nn) * 8 + (bid & 7), nt = slot % nn;
  if (mt >= n_mt) return;
  const int tid = (int)threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int lrow = lane & 31, khalf = lane >> 5;
  const int prow = lane >> 3, pchunk = lane & 7;
  const int sw_row = dma_swz(lrow) ^ khalf;
  const int m0 = mt * BM, n0 = nt * BN;
  const char* a_tile = uniform_ptr((const char*)(x + (long long)m0 * H));
  const char* b_tile = uniform_ptr((const char*)(wr + (long long)n0 * H));
  // copy j of a wave fills rows 8 (wave + NW j) .. + 7 of its operand (1 KB)
  uint32_t voffA[JA], voffB[JB];
#pragma unroll
  for (int j = 0; j < JA; ++j) {
    const int row = 8 * (wave + NW * j) + prow;
    const int grow = min(m0 + row, T - 1);
    voffA[j] = (uint32_t)(grow - m0) * (uint32_t)(H * 2) + (uint32_t)((pchunk ^ dma_swz(row)) * 16);
  }
#pragma unroll
  for (int j = 0; j < JB; ++j) {
    const int row = 8 * (wave + NW * j) + prow;
    voffB[j] = (uint32_t)row * (uint32_t)(H * 2) + (uint32_t)((pchunk ^ dma_swz(row)) * 16);
  }
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  const int nk = H / 64;
  const uint32_t lds0 = lds_addr(smem);
#define MOE_ISSUE(st)                                                           \
  do {                                                                          \
    const uint32_t dst_ = lds0 + ((st) % NR) * STAGE;                           \
    _Pragma("unroll") for (int j = 0; j < JA; ++j)                              \
      dma16(a_tile + (st) * ROWB, voffA[j], dst_ + (wave + NW * j) * 1024);     \
    _Pragma("unroll") for (int j = 0; j < JB; ++j)                              \
      dma16(b_tile + (st) * ROWB, voffB[j], dst_ + A_STAGE + (wave + NW * j) * 1024); \
  } while (0)
#define MOE_RREAD(As, Bs, s4, FA, FB)                                           \
  do {                                                                          \
    _Pragma("unroll") for (int i = 0; i < 2; ++i)                               \
      FA[i] = *(const V*)((As) + (wm * 64 + i * 32 + lrow) * ROWB + (((2 * (s4)) ^ sw_row) << 4)); \
    _Pragma("unroll") for (int j = 0; j < 2; ++j)                               \
      FB[j] = *(const V*)((Bs) + (wn * 64 + j * 32 + lrow) * ROWB +             \
                          (((2 * (s4)) ^ sw_row) << 4));                        \
  } while (0)
#pragma unroll
  for (int st = 0; st < NR - 1; ++st)
    if (st < nk) MOE_ISSUE(st);
  for (int kt = 0; kt < nk; ++kt) {
    // Stage kt has landed once at most the stages issued after it are in
    // flight: kt + 1 .. min(kt + NR - 2, nk - 1), JA + JB copies each.  The
    // barrier then covers every wave's copies and frees the slot read in
    // iteration kt - 1, which the next issue refills.
    const int later = min(kt + NR - 2, nk - 1) - kt;
    if (later >= 2) wait_vmcnt<2 * (JA + JB)>();
    else if (later == 1) wait_vmcnt<JA + JB>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_waitcnt((0x3F & 0xF) | (0x7 << 4) | ((0x3F >> 4) << 14));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (kt + NR - 1 < nk) MOE_ISSUE(kt + NR - 1);
    const char* As = smem + (kt % NR) * STAGE;
    const char* Bs = As + A_STAGE;
    V fa0[2], fb0[2], fa1[2], fb1[2];
    MOE_RREAD(As, Bs, 0, fa0, fb0);
#pragma unroll
    for (int s4 = 0; s4 < 4; s4 += 2) {
      MOE_RREAD(As, Bs, s4 + 1, fa1, fb1);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = MfmaOp<DT>::run(fa0[i], fb0[j], acc[i][j]);
      if (s4 + 2 < 4) MOE_RREAD(As, Bs, s4 + 2, fa0, fb0);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = MfmaOp<DT>::run(fa1[i], fb1[j], acc[i][j]);
    }
  }
#undef MOE_ISSUE
#undef MOE_RREAD
  // 32x32 result layout: lane l holds column l % 32, rows 8 * (v / 4) +
  // 4 * (l / 32) + v % 4
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = m0 + wm * 64 + i * 32 + (v >> 2) * 8 + khalf * 4 + (v & 3);
        if (r < T) logits[(long long)r * E + n0 + wn * 64 + j * 32 + lrow] = acc[i][j][v];
      }
}

template <int DT>
int launch_router_pair(const void* x, const void* wr, int T, int H, int E, float* logits,
                       hipStream_t s) {
  // per-lane copy offsets are 32-bit: 128 rows of H values must span < 4 GiB
  if ((long long)128 * H * 2 >= (1ll << 32)) return MOE_ERR_UNSUPPORTED;
  const int n_mt = (T + 127) / 128;
  const int grid = (n_mt + 7) / 8 * 8 * (E / 128);
  hipLaunchKernelGGL((router_pair_kernel<DT>), dim3(grid), dim3(256), 0, s,
                     (const uint16_t*)x, (const uint16_t*)wr, T, H, E, n_mt, logits);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int launch_topk(const float* logits, const float* bias, int T, int E, int k,
                int gate, int renorm, float inv_temp, float min_prob, int32_t* idx,
                float* w, hipStream_t s) {
  // Sixteen lanes per token pay off once there are enough tokens to fill the
  // chip; below that the selection's dependency chain is the latency, and a
  // wave per token (a quarter of the experts per lane) is shorter: route
  // step 32 -> 26 us at 128 tokens x 256 experts, 3-6 us less up to 4096
  // tokens, 2-12 us more from 8192 (256 experts; with 128 or fewer experts
  // the wave kernel is ahead only up to about 256 tokens).
  const bool wide = E > 128 ? T > 4096 : T > 512;
  if (E <= 256 && k <= 16 && wide) {
    // four tokens per wave, sixteen per block
    const dim3 grid16((T + 15) / 16), block16(256);
#define MOE_TOPK16(EPL)                                                              \
  hipLaunchKernelGGL((topk_gate16_kernel<EPL>), grid16, block16, 0, s, logits, bias, T, E, \
                     k, gate, renorm, inv_temp, min_prob, idx, w)
    if (E <= 64) MOE_TOPK16(4);
    else if (E <= 128) MOE_TOPK16(8);
    else MOE_TOPK16(16);
#undef MOE_TOPK16
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
  }
  const dim3 grid((T + 3) / 4), block(256);
#define MOE_TOPK(EPL)                                                         \
  hipLaunchKernelGGL((topk_gate_kernel<EPL>), grid, block, 0, s, logits, bias, \
                     T, E, k, gate, renorm, inv_temp, min_prob, idx, w)
  if (E <= 64) MOE_TOPK(1);
  else if (E <= 128) MOE_TOPK(2);
  else if (E <= 256) MOE_TOPK(4);
  else if (E <= 512) MOE_TOPK(8);
  else MOE_TOPK(16);
#undef MOE_TOPK
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace

int route_impl(const void* x, const void* w_router, int act_dtype, const float* bias,
               int T, int H, int E, int k, int gate, int renorm, float inv_temp,
               float min_prob, float* logits, int32_t* topk_idx, float* topk_w,
               hipStream_t s) {
  if (T == 0) return MOE_OK;
  if (w_router) {
    int st;
    // staged matrix tiles for many experts and enough tokens to fill the
    // chip; otherwise 16x16 matrix tiles with operands loaded per lane (few
    // experts, or a small decode batch), or the vector kernel (float32)
    const bool mfma = act_dtype != MOE_DTYPE_F32 && E >= 128 && E % 128 == 0 &&
                      H % 64 == 0 && T >= 1024;
    if (mfma) {
      st = act_dtype == MOE_DTYPE_F16
               ? launch_router_pair<MOE_DTYPE_F16>(x, w_router, T, H, E, logits, s)
               : launch_router_pair<MOE_DTYPE_BF16>(x, w_router, T, H, E, logits, s);
    } else if (act_dtype != MOE_DTYPE_F32 && H % 32 == 0) {
      st = act_dtype == MOE_DTYPE_F16
               ? launch_router_mfma<MOE_DTYPE_F16>(x, w_router, T, H, E, logits, s)
               : launch_router_mfma<MOE_DTYPE_BF16>(x, w_router, T, H, E, logits, s);
    } else if (act_dtype == MOE_DTYPE_F32) {
      st = launch_router_valu<MOE_DTYPE_F32>(x, w_router, T, H, E, logits, s);
    } else if (act_dtype == MOE_DTYPE_F16) {
      st = launch_router_valu<MOE_DTYPE_F16>(x, w_router, T, H, E, logits, s);
    } else {
      st = launch_router_valu<MOE_DTYPE_BF16>(x, w_router, T, H, E, logits, s);
    }
    if (st != MOE_OK) return st;
  }
  return launch_topk(logits, bias, T, E, k, gate, renorm, inv_temp, min_prob, topk_idx,
                     topk_w, s);
}

}  // namespace moe
