// extern "C" entry points: argument validation, then kernel launches.
// Every check happens before the first launch, so an error return means
// nothing was enqueued.

#include "moe_internal.h"

namespace moe {
int route_impl(const void* x, const void* w_router, int act_dtype, const float* bias,
               int T, int H, int E, int k, int gate, int renorm, float inv_temp,
               float min_prob, float* logits, int32_t* topk_idx, float* topk_w,
               hipStream_t s);
int dispatch_impl(const void* x, int act_dtype, const int32_t* idx, int T, int H,
                  int E, int k, int e_begin, int e_end, int32_t* counts,
                  int32_t* offsets, int32_t* slot_of, int32_t* row_token,
                  void* x_perm, float* x_scale, void* ws, hipStream_t s);
size_t dispatch_ws_bytes(int T, int E);
int place_impl(const int32_t* idx, int T, int k, int E_log, int E_phys,
               const int32_t* rep_offsets, const int32_t* rep_phys, int32_t* phys,
               hipStream_t s);
int load_stats_impl(const int32_t* idx, int T, int k, int E, unsigned long long* stats,
                    hipStream_t s);
int combine_impl(const void* y_perm, const int32_t* slot_of, const float* w,
                 int act_dtype, int T, int H, int k, void* out, hipStream_t s);
int fused_impl(const void* x, const int32_t* offsets, const int32_t* slot_of,
               const int32_t* row_token, const float* topk_w, int act_dtype, int T,
               int H, int E, int k, int I, int e_begin, int e_end, int act,
               const void* w13, const void* w2, void* h_ws, void* y_perm, void* out,
               void* ws, size_t ws_bytes, hipStream_t s);
size_t fused_ws_bytes(int T, int H, int E, int k, int I);
}  // namespace moe

using namespace moe;

namespace {

bool act_ok(int dt) {
  return dt == MOE_DTYPE_F32 || dt == MOE_DTYPE_F16 || dt == MOE_DTYPE_BF16;
}
int elem_bytes(int dt) { return dt == MOE_DTYPE_F32 ? 4 : 2; }
bool pairs_fit(long long T, long long k) { return T * k < (1ll << 31); }

// Row buffers are copied in 16-byte pieces (and staged to LDS by DMA), so
// their bases must be 16-byte aligned; a null pointer passes here and is
// rejected (or allowed) by the caller's own checks.
bool al16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Weight format accepted for a given activation format.
bool weights_ok(int act_dtype, int w_dtype) {
  if (w_dtype == act_dtype) return true;
  return w_dtype == MOE_DTYPE_FP8_E4M3 && act_dtype == MOE_DTYPE_BF16;
}

}  // namespace

extern "C" {

int moe_route(const void* x, const void* w_router, int act_dtype, const float* bias,
              int T, int H, int E, int k, int gate, int renorm, float inv_temperature,
              float min_prob, float* logits, int32_t* topk_idx, float* topk_w,
              hipStream_t stream) {
  if (!act_ok(act_dtype)) return MOE_ERR_UNSUPPORTED;
  if (T < 0 || E < 1 || E > 1024 || k < 1 || k > E || k > 32) return MOE_ERR_ARG;
  if (!pairs_fit(T, k) || !pairs_fit(T, E)) return MOE_ERR_ARG;
  if (gate != MOE_GATE_SOFTMAX && gate != MOE_GATE_SIGMOID) return MOE_ERR_ARG;
  if (!(inv_temperature >= 0.0f) || inv_temperature > 3.0e38f) return MOE_ERR_ARG;
  if (!(min_prob >= 0.0f && min_prob <= 1.0f)) return MOE_ERR_ARG;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_idx || !topk_w) return MOE_ERR_ARG;
  if (w_router && (!x || H < 1 || H % 8)) return MOE_ERR_ARG;
  if (w_router && (!al16(x) || !al16(w_router))) return MOE_ERR_ARG;
  return route_impl(x, w_router, act_dtype, bias, T, H, E, k, gate, renorm,
                    inv_temperature, min_prob, logits, topk_idx, topk_w, stream);
}

int moe_dispatch(const void* x, int act_dtype, const int32_t* topk_idx, int T, int H,
                 int E, int k, int e_begin, int e_end, int32_t* counts,
                 int32_t* offsets, int32_t* slot_of, int32_t* row_token, void* x_perm,
                 void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!act_ok(act_dtype)) return MOE_ERR_UNSUPPORTED;
  if (T < 0 || H < 1 || E < 1 || E > 1024 || k < 1 || k > E || k > 32)
    return MOE_ERR_ARG;
  if (!pairs_fit(T, k)) return MOE_ERR_ARG;
  if (e_begin < 0 || e_end < e_begin || e_end > E) return MOE_ERR_ARG;
  if ((H * elem_bytes(act_dtype)) % 16) return MOE_ERR_ARG;
  if (!counts || !offsets) return MOE_ERR_ARG;
  if (T > 0 && (!x || !topk_idx || !slot_of || !row_token)) return MOE_ERR_ARG;
  if (T > 0 && e_end > e_begin && !x_perm) return MOE_ERR_ARG;
  if (!al16(x) || !al16(x_perm)) return MOE_ERR_ARG;
  if (!ws || ws_bytes < dispatch_ws_bytes(T, E)) return MOE_ERR_WORKSPACE;
  return dispatch_impl(x, act_dtype, topk_idx, T, H, E, k, e_begin, e_end, counts,
                       offsets, slot_of, row_token, x_perm, nullptr, ws, stream);
}

int moe_dispatch_fp8(const void* x, int act_dtype, const int32_t* topk_idx, int T, int H,
                     int E, int k, int e_begin, int e_end, int32_t* counts,
                     int32_t* offsets, int32_t* slot_of, int32_t* row_token,
                     void* x_perm_q, float* x_scale, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
  if (act_dtype != MOE_DTYPE_BF16) return MOE_ERR_UNSUPPORTED;
  if (T < 0 || H < 1 || E < 1 || E > 1024 || k < 1 || k > E || k > 32)
    return MOE_ERR_ARG;
  if (!pairs_fit(T, k)) return MOE_ERR_ARG;
  if (e_begin < 0 || e_end < e_begin || e_end > E) return MOE_ERR_ARG;
  if (H % 8) return MOE_ERR_ARG;
  if (!counts || !offsets) return MOE_ERR_ARG;
  if (T > 0 && (!x || !topk_idx || !slot_of || !row_token)) return MOE_ERR_ARG;
  if (T > 0 && e_end > e_begin && (!x_perm_q || !x_scale)) return MOE_ERR_ARG;
  if (!al16(x) || !al16(x_perm_q)) return MOE_ERR_ARG;
  if (!ws || ws_bytes < dispatch_ws_bytes(T, E)) return MOE_ERR_WORKSPACE;
  return dispatch_impl(x, act_dtype, topk_idx, T, H, E, k, e_begin, e_end, counts,
                       offsets, slot_of, row_token, x_perm_q,
                       x_scale ? x_scale : nullptr, ws, stream);
}

int moe_expert_ffn_up(const void* x_perm, const int32_t* offsets, int act_dtype, int H,
                      int I, int e_begin, int e_end, int max_rows, int act,
                      const void* w13, const float* w13_scale, int w_dtype, void* h_ws,
                      void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!act_ok(act_dtype) || !weights_ok(act_dtype, w_dtype)) return MOE_ERR_UNSUPPORTED;
  if (act != MOE_ACT_SWIGLU && act != MOE_ACT_GELU) return MOE_ERR_ARG;
  if (H < 1 || I < 1 || e_begin < 0 || e_end < e_begin || max_rows < 0)
    return MOE_ERR_ARG;
  if (e_end == e_begin || max_rows == 0) return MOE_OK;
  if (!x_perm || !offsets || !w13 || !h_ws) return MOE_ERR_ARG;
  if (!al16(x_perm) || !al16(w13) || !al16(h_ws)) return MOE_ERR_ARG;
  if (w_dtype == MOE_DTYPE_FP8_E4M3 && !w13_scale) return MOE_ERR_ARG;
  if (ws && ws_bytes < ffn_ws_bytes()) return MOE_ERR_WORKSPACE;
  const int Nb = act == MOE_ACT_SWIGLU ? 2 * I : I;
  // 16-bit tiles cut the weight rows (2I for SwiGLU, I for GELU) into 256s
  if (act_dtype != MOE_DTYPE_F32 && (H % 256 || Nb % 256)) return MOE_ERR_UNSUPPORTED;
  GemmArgs a{};
  ffn_ws_attach(a, ws, ws_bytes);
  a.A = x_perm;
  a.lda = H;
  a.B = w13;
  a.strideB = (long long)Nb * H;
  a.ldb = H;
  a.Bscale = w13_scale;
  a.strideS = (long long)(Nb / 128) * (H / 128);
  a.C = h_ws;
  a.ldc = I;
  a.offsets = offsets;
  a.e_begin = e_begin;
  a.n_groups = e_end - e_begin;
  a.a_local = 0;
  a.c_local = 1;
  a.c_rows = max_rows;
  a.Nb = Nb;
  a.I = I;
  a.K = H;
  return launch_grouped_gemm(act_dtype, w_dtype,
                             act == MOE_ACT_SWIGLU ? EPI_SWIGLU : EPI_GELU, a, max_rows,
                             stream);
}

int moe_expert_ffn_up_fp8(const void* x_perm_q, const float* x_scale,
                          const int32_t* offsets, int H, int I, int e_begin, int e_end,
                          int max_rows, int act, const void* w13, const float* w13_scale,
                          void* h_ws, hipStream_t stream) {
  if (act != MOE_ACT_SWIGLU && act != MOE_ACT_GELU) return MOE_ERR_ARG;
  if (H < 1 || I < 1 || e_begin < 0 || e_end < e_begin || max_rows < 0)
    return MOE_ERR_ARG;
  if (e_end == e_begin || max_rows == 0) return MOE_OK;
  if (!x_perm_q || !x_scale || !offsets || !w13 || !w13_scale || !h_ws) return MOE_ERR_ARG;
  if (!al16(x_perm_q) || !al16(w13) || !al16(h_ws)) return MOE_ERR_ARG;
  const int Nb = act == MOE_ACT_SWIGLU ? 2 * I : I;
  if (H % 128 || I % 128 || Nb % 256) return MOE_ERR_UNSUPPORTED;
  GemmArgs a{};
  a.A = x_perm_q;
  a.lda = H;
  a.Ascale = x_scale;
  a.B = w13;
  a.strideB = (long long)Nb * H;
  a.ldb = H;
  a.Bscale = w13_scale;
  a.strideS = (long long)(Nb / 128) * (H / 128);
  a.C = h_ws;
  a.ldc = I;
  a.offsets = offsets;
  a.e_begin = e_begin;
  a.n_groups = e_end - e_begin;
  a.a_local = 0;
  a.c_local = 1;
  a.c_rows = max_rows;
  a.Nb = Nb;
  a.I = I;
  a.K = H;
  return launch_gemm_fp8_act(act == MOE_ACT_SWIGLU ? EPI_SWIGLU : EPI_GELU, a, max_rows,
                             stream);
}

int moe_expert_ffn_down(const int32_t* offsets, int act_dtype, int H, int I, int e_begin,
                        int e_end, int max_rows, const void* w2, const float* w2_scale,
                        int w_dtype, const void* h_ws, void* y_perm, void* ws,
                        size_t ws_bytes, hipStream_t stream) {
  if (!act_ok(act_dtype) || !weights_ok(act_dtype, w_dtype)) return MOE_ERR_UNSUPPORTED;
  if (H < 1 || I < 1 || e_begin < 0 || e_end < e_begin || max_rows < 0)
    return MOE_ERR_ARG;
  if (e_end == e_begin || max_rows == 0) return MOE_OK;
  if (!offsets || !w2 || !h_ws || !y_perm) return MOE_ERR_ARG;
  if (!al16(w2) || !al16(h_ws) || !al16(y_perm)) return MOE_ERR_ARG;
  if (w_dtype == MOE_DTYPE_FP8_E4M3 && !w2_scale) return MOE_ERR_ARG;
  if (ws && ws_bytes < ffn_ws_bytes()) return MOE_ERR_WORKSPACE;
  GemmArgs a{};
  ffn_ws_attach(a, ws, ws_bytes);
  a.A = h_ws;
  a.lda = I;
  a.B = w2;
  a.strideB = (long long)H * I;
  a.ldb = I;
  a.Bscale = w2_scale;
  a.strideS = (long long)(H / 128) * (I / 128);
  a.C = y_perm;
  a.ldc = H;
  a.offsets = offsets;
  a.e_begin = e_begin;
  a.n_groups = e_end - e_begin;
  a.a_local = 1;
  a.c_local = 0;
  a.a_rows = max_rows;
  a.Nb = H;
  a.I = 0;
  a.K = I;
  return launch_grouped_gemm(act_dtype, w_dtype, EPI_STORE, a, max_rows, stream);
}

int moe_expert_ffn(const void* x_perm, const int32_t* offsets, int act_dtype, int H,
                   int I, int e_begin, int e_end, int max_rows, int act, const void* w13,
                   const float* w13_scale, const void* w2, const float* w2_scale,
                   int w_dtype, void* h_ws, void* y_perm, void* ws, size_t ws_bytes,
                   hipStream_t stream) {
  if (!act_ok(act_dtype) || !weights_ok(act_dtype, w_dtype)) return MOE_ERR_UNSUPPORTED;
  if (act != MOE_ACT_SWIGLU && act != MOE_ACT_GELU) return MOE_ERR_ARG;
  if (e_end > e_begin && max_rows > 0 && (!y_perm || !w2)) return MOE_ERR_ARG;
  if (!al16(x_perm) || !al16(w13) || !al16(w2) || !al16(h_ws) || !al16(y_perm))
    return MOE_ERR_ARG;
  if (ws && ws_bytes < ffn_ws_bytes()) return MOE_ERR_WORKSPACE;
  // Shape checks of both halves happen before either launches.
  const int Nb = act == MOE_ACT_SWIGLU ? 2 * I : I;
  if (act_dtype == MOE_DTYPE_F32) {
    if (H % 64 || I % 64 || Nb % 64) return MOE_ERR_UNSUPPORTED;
  } else {
    if (H % 256 || I % 64 || Nb % 256) return MOE_ERR_UNSUPPORTED;
    if (w_dtype == MOE_DTYPE_FP8_E4M3 && (H % 128 || I % 128)) return MOE_ERR_UNSUPPORTED;
  }
  int st = moe_expert_ffn_up(x_perm, offsets, act_dtype, H, I, e_begin, e_end, max_rows,
                             act, w13, w13_scale, w_dtype, h_ws, ws, ws_bytes, stream);
  if (st != MOE_OK) return st;
  return moe_expert_ffn_down(offsets, act_dtype, H, I, e_begin, e_end, max_rows, w2,
                             w2_scale, w_dtype, h_ws, y_perm, ws, ws_bytes, stream);
}

int moe_place_experts(const int32_t* topk_idx, int T, int k, int E_log, int E_phys,
                      const int32_t* rep_offsets, const int32_t* rep_phys,
                      int32_t* topk_phys, hipStream_t stream) {
  if (T < 0 || k < 1 || k > 32 || E_log < 1 || E_phys < 1 || E_phys > 1024)
    return MOE_ERR_ARG;
  if (!pairs_fit(T, k)) return MOE_ERR_ARG;
  if (T == 0) return MOE_OK;
  if (!topk_idx || !rep_offsets || !rep_phys || !topk_phys) return MOE_ERR_ARG;
  return place_impl(topk_idx, T, k, E_log, E_phys, rep_offsets, rep_phys, topk_phys, stream);
}

int moe_expert_load_stats(const int32_t* topk_idx, int T, int k, int E, uint64_t* stats,
                          hipStream_t stream) {
  if (T < 0 || k < 1 || k > 32 || E < 1 || E > 1024) return MOE_ERR_ARG;
  if (!pairs_fit(T, k)) return MOE_ERR_ARG;
  if (T == 0) return MOE_OK;
  if (!topk_idx || !stats) return MOE_ERR_ARG;
  return load_stats_impl(topk_idx, T, k, E, (unsigned long long*)stats, stream);
}

int moe_combine(const void* y_perm, const int32_t* slot_of, const float* topk_w,
                int act_dtype, int T, int H, int k, void* out, hipStream_t stream) {
  if (!act_ok(act_dtype)) return MOE_ERR_UNSUPPORTED;
  if (T < 0 || H < 1 || k < 1 || k > 32 || !pairs_fit(T, k)) return MOE_ERR_ARG;
  if ((H * elem_bytes(act_dtype)) % 16) return MOE_ERR_ARG;
  if (T == 0) return MOE_OK;
  if (!y_perm || !slot_of || !topk_w || !out) return MOE_ERR_ARG;
  if (!al16(y_perm) || !al16(out)) return MOE_ERR_ARG;
  return combine_impl(y_perm, slot_of, topk_w, act_dtype, T, H, k, out, stream);
}

int moe_layer_fused(const void* x, const int32_t* offsets, const int32_t* slot_of,
                    const int32_t* row_token, const float* topk_w, int act_dtype, int T,
                    int H, int E, int k, int I, int e_begin, int e_end, int act,
                    const void* w13, const void* w2, void* h_ws, void* y_perm, void* out,
                    void* ws, size_t ws_bytes, hipStream_t stream) {
  if (act_dtype != MOE_DTYPE_F16 && act_dtype != MOE_DTYPE_BF16) return MOE_ERR_UNSUPPORTED;
  if (act != MOE_ACT_SWIGLU) return MOE_ERR_UNSUPPORTED;
  if (T < 0 || H < 1 || I < 1 || E < 1 || E > 1024 || k < 1 || k > E || k > 32)
    return MOE_ERR_ARG;
  if (!pairs_fit(T, k)) return MOE_ERR_ARG;
  if (e_begin < 0 || e_end < e_begin || e_end > E) return MOE_ERR_ARG;
  if (H % 256 || I % 128) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !offsets || !slot_of || !row_token || !topk_w || !y_perm || !out)
    return MOE_ERR_ARG;
  if (e_end > e_begin && (!w13 || !w2 || !h_ws)) return MOE_ERR_ARG;
  if (!al16(x) || !al16(w13) || !al16(w2) || !al16(h_ws) || !al16(y_perm) || !al16(out))
    return MOE_ERR_ARG;
  if (!ws || ws_bytes < fused_ws_bytes(T, H, E, k, I)) return MOE_ERR_WORKSPACE;
  return fused_impl(x, offsets, slot_of, row_token, topk_w, act_dtype, T, H, E, k, I,
                    e_begin, e_end, act, w13, w2, h_ws, y_perm, out, ws, ws_bytes, stream);
}

size_t moe_workspace_bytes(int which, int T, int H, int E, int k, int I) {
  if (T < 0 || E < 1) return 0;
  switch (which) {
    case MOE_WS_DISPATCH: return dispatch_ws_bytes(T, E);
    case MOE_WS_FFN: return ffn_ws_bytes();
    case MOE_WS_FUSED: return fused_ws_bytes(T, H, E, k, I);
  }
  return 0;
}

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported dtype or shape";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "kernel launch failed";
    case MOE_ERR_TOO_LARGE: return "sizes exceed the fixed internal scratch";
  }
  return "unknown status";
}

}  // extern "C"
