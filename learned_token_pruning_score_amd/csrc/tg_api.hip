// C ABI of the gated-prefill library: argument checks on the host, then
// asynchronous launches on the caller's stream.  The declarations, with the
// meaning, layout, ownership and error behaviour of every argument, are in
// include/tg.h.
#include <limits.h>
#include <math.h>
#include <stdint.h>

#include "../../include/tg.h"
#include "tg_common.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int elem_bytes(int dtype) { return dtype == TG_BF16 ? 2 : (dtype == TG_F32 ? 4 : 0); }

int from_hip(hipError_t e) { return e == hipSuccess ? TG_OK : TG_ERR_HIP; }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Largest second and third launch-grid dimension.
constexpr int kMaxGridYZ = 65535;

}  // namespace

extern "C" {

int tg_abi_version(void) { return TG_ABI_VERSION; }

const char* tg_status_string(int status) {
  switch (status) {
    case TG_OK: return "ok";
    case TG_ERR_NULL: return "a required pointer is NULL";
    case TG_ERR_SHAPE: return "a size or stride is negative or inconsistent";
    case TG_ERR_DTYPE: return "unknown dtype code";
    case TG_ERR_RANGE: return "a scalar argument is out of range";
    case TG_ERR_ALIGN: return "a pointer or stride is misaligned";
    case TG_ERR_UNSUPPORTED: return "shape not supported by the library's kernels";
    case TG_ERR_WORKSPACE: return "workspace missing or too small";
    case TG_ERR_HIP: return "HIP runtime error at launch";
    default: return "unknown status";
  }
}

int tg_plan(int B, const int32_t* cu_seqlens_h, const int32_t* doc_begin_h,
            const int32_t* doc_end_h, const int32_t* budget_h, int32_t* cu_kept_h,
            int32_t* max_kept_len_h) {
  if (B < 0) return TG_ERR_SHAPE;
  if (!cu_seqlens_h || !cu_kept_h || !max_kept_len_h) return TG_ERR_NULL;
  if (B > 0 && (!doc_begin_h || !doc_end_h || !budget_h)) return TG_ERR_NULL;
  if (cu_seqlens_h[0] != 0) return TG_ERR_SHAPE;
  int64_t acc = 0;
  int32_t longest = 0;
  for (int b = 0; b < B; ++b) {
    const int64_t len = (int64_t)cu_seqlens_h[b + 1] - cu_seqlens_h[b];
    if (len < 0) return TG_ERR_SHAPE;
    if (doc_begin_h[b] < 0 || doc_end_h[b] < doc_begin_h[b] || doc_end_h[b] > len)
      return TG_ERR_SHAPE;
    if (budget_h[b] < 0) return TG_ERR_SHAPE;
    const int64_t doc = (int64_t)doc_end_h[b] - doc_begin_h[b];
    const int64_t kept = (budget_h[b] < doc ? budget_h[b] : doc) + (len - doc);
    acc += kept;
    if (acc > INT32_MAX) return TG_ERR_SHAPE;
    if (kept > longest) longest = (int32_t)kept;
  }
  // outputs only after every check passed
  cu_kept_h[0] = 0;
  acc = 0;
  for (int b = 0; b < B; ++b) {
    const int64_t len = (int64_t)cu_seqlens_h[b + 1] - cu_seqlens_h[b];
    const int64_t doc = (int64_t)doc_end_h[b] - doc_begin_h[b];
    acc += (budget_h[b] < doc ? budget_h[b] : doc) + (len - doc);
    cu_kept_h[b + 1] = (int32_t)acc;
  }
  *max_kept_len_h = longest;
  return TG_OK;
}

int tg_sample_budgets(int B, const int32_t* doc_begin_h, const int32_t* doc_end_h,
                      const float* u_h, float min_frac, float max_frac, int32_t* budget_h) {
  if (B < 0) return TG_ERR_SHAPE;
  if (B > 0 && (!doc_begin_h || !doc_end_h || !u_h || !budget_h)) return TG_ERR_NULL;
  if (!isfinite(min_frac) || !isfinite(max_frac) || !(min_frac >= 0.0f) || !(max_frac <= 1.0f) ||
      min_frac > max_frac)
    return TG_ERR_RANGE;
  for (int b = 0; b < B; ++b) {
    if (doc_end_h[b] < doc_begin_h[b] || doc_begin_h[b] < 0) return TG_ERR_SHAPE;
    if (!(u_h[b] >= 0.0f && u_h[b] < 1.0f)) return TG_ERR_RANGE;
  }
  for (int b = 0; b < B; ++b) {
    const double f = (double)min_frac + ((double)max_frac - (double)min_frac) * (double)u_h[b];
    budget_h[b] = (int32_t)floor(f * (double)(doc_end_h[b] - doc_begin_h[b]));
  }
  return TG_OK;
}

int tg_gate_score(const void* hidden, int64_t ld_hidden, int64_t T, int D, const void* W1,
                  const float* b1, const float* w2, float b2, int F, int dtype, float* scores,
                  void* stream) {
  const int eb = elem_bytes(dtype);
  if (!eb) return TG_ERR_DTYPE;
  if (T < 0 || D <= 0 || F <= 0 || ld_hidden < D) return TG_ERR_SHAPE;
  if (T > INT32_MAX) return TG_ERR_SHAPE;
  if (!isfinite(b2)) return TG_ERR_RANGE;
  if (T == 0) return TG_OK;
  if (!hidden || !W1 || !w2 || !scores) return TG_ERR_NULL;
  if (dtype == TG_BF16) {
    if (D % 8 != 0 || !(F == 64 || F == 128 || F == 256)) return TG_ERR_UNSUPPORTED;
    // a 256-row tile of hidden is addressed with 32-bit byte offsets
    if (ld_hidden >= (1 << 22) || (int64_t)F * D > (1 << 29)) return TG_ERR_UNSUPPORTED;
    if (!aligned16(hidden) || !aligned16(W1) || (ld_hidden * 2) % 16 != 0) return TG_ERR_ALIGN;
    return from_hip(tg::launch_gate_bf16(hidden, ld_hidden, T, D, W1, b1, w2, b2, F, scores,
                                         as_stream(stream)));
  }
  if (F > 1024) return TG_ERR_UNSUPPORTED;
  return from_hip(tg::launch_gate_f32(static_cast<const float*>(hidden), ld_hidden, T, D,
                                      static_cast<const float*>(W1), b1, w2, b2, F, scores,
                                      as_stream(stream)));
}

int tg_select_topk_workspace(int B, int64_t T, size_t* bytes) {
  if (!bytes) return TG_ERR_NULL;
  if (B < 0 || T < 0) return TG_ERR_SHAPE;
  *bytes = tg::select_workspace_bytes(B, T);
  return TG_OK;
}

int tg_select_topk(const float* scores, const int32_t* cu_seqlens, const int32_t* doc_begin,
                   const int32_t* doc_end, const int32_t* budget, int B, int64_t T, uint8_t* keep,
                   void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 0 || T < 0 || T > INT32_MAX) return TG_ERR_SHAPE;
  if (B == 0 && T != 0) return TG_ERR_SHAPE;
  if (T == 0 && B == 0) return TG_OK;
  if (!cu_seqlens || !doc_begin || !doc_end || !budget) return TG_ERR_NULL;
  if (T > 0 && (!scores || !keep)) return TG_ERR_NULL;
  if (B > kMaxGridYZ) return TG_ERR_UNSUPPORTED;  // one launch row per prompt
  if (!workspace || workspace_bytes < tg::select_workspace_bytes(B, T)) return TG_ERR_WORKSPACE;
  if (!aligned16(workspace)) return TG_ERR_ALIGN;
  if (T == 0) return TG_OK;
  return from_hip(tg::launch_select(scores, cu_seqlens, doc_begin, doc_end, budget, B, T, keep,
                                    workspace, as_stream(stream)));
}

int tg_select_topk_noalloc(const float* scores, const int32_t* cu_seqlens,
                           const int32_t* doc_begin, const int32_t* doc_end,
                           const int32_t* budget, int B, int64_t T, uint8_t* keep,
                           void* stream) {
  if (B < 0 || T < 0 || T > INT32_MAX) return TG_ERR_SHAPE;
  if (B == 0 && T != 0) return TG_ERR_SHAPE;
  if (T == 0 && B == 0) return TG_OK;
  if (!cu_seqlens || !doc_begin || !doc_end || !budget) return TG_ERR_NULL;
  if (T > 0 && (!scores || !keep)) return TG_ERR_NULL;
  if (B > kMaxGridYZ) return TG_ERR_UNSUPPORTED;
  const size_t need = tg::select_scratch_bytes_needed(B, T);
  if (need > tg::select_static_scratch_capacity()) return TG_ERR_WORKSPACE;
  if (T == 0) return TG_OK;
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = tg::select_static_scratch(as_stream(stream), &ws);
    if (e != hipSuccess) return TG_ERR_HIP;
  }
  return from_hip(tg::launch_select(scores, cu_seqlens, doc_begin, doc_end, budget, B, T, keep, ws,
                                    as_stream(stream)));
}

int tg_compact_workspace(int B, int64_t T, size_t* bytes) {
  if (!bytes) return TG_ERR_NULL;
  if (B < 0 || T < 0) return TG_ERR_SHAPE;
  *bytes = tg::compact_workspace_bytes(B, T);
  return TG_OK;
}

int tg_compact(const void* hidden, int64_t ld_hidden, int D, int dtype, const int32_t* pos,
               const float* scores, const uint8_t* keep, const int32_t* cu_seqlens,
               const int32_t* doc_begin, const int32_t* doc_end, int B, int64_t T, int64_t Kt,
               void* hidden_out, int32_t* pos_out, float* bias_out, int32_t* kept_idx_out,
               void* workspace, size_t workspace_bytes, void* stream) {
  const int eb = elem_bytes(dtype);
  if (!eb) return TG_ERR_DTYPE;
  if (B < 0 || T < 0 || Kt < 0 || Kt > T || D <= 0 || ld_hidden < D || T > INT32_MAX)
    return TG_ERR_SHAPE;
  if (B == 0 && T != 0) return TG_ERR_SHAPE;
  if (T == 0) return TG_OK;
  if (!hidden || !scores || !keep || !cu_seqlens || !doc_begin || !doc_end) return TG_ERR_NULL;
  if (Kt > 0 && (!hidden_out || !pos_out || !bias_out)) return TG_ERR_NULL;
  if (!workspace || workspace_bytes < tg::compact_workspace_bytes(B, T)) return TG_ERR_WORKSPACE;
  if (!aligned16(workspace)) return TG_ERR_ALIGN;
  // element alignment only; the copy widens to 16-byte units when rows allow
  if ((reinterpret_cast<uintptr_t>(hidden) % eb) != 0 ||
      (Kt > 0 && (reinterpret_cast<uintptr_t>(hidden_out) % eb) != 0))
    return TG_ERR_ALIGN;
  return from_hip(tg::launch_compact(hidden, ld_hidden, D, eb, pos, scores, keep, cu_seqlens,
                                     doc_begin, doc_end, B, T, Kt, hidden_out, pos_out, bias_out,
                                     kept_idx_out, workspace, as_stream(stream)));
}

int tg_gated_attn_fwd(const void* q, const void* k, const void* v, int64_t q_tok_stride,
                      int64_t k_tok_stride, int64_t v_tok_stride, const float* bias_s,
                      const float* gain, float tau, const int32_t* cu_kept, int B,
                      int max_kept_len, int64_t Kt, int Hq, int Hkv, int d, int dtype, void* out,
                      float* lse, void* stream) {
  const int eb = elem_bytes(dtype);
  if (!eb) return TG_ERR_DTYPE;
  if (B < 0 || Kt < 0 || Kt > INT32_MAX || max_kept_len < 0 || max_kept_len > Kt || Hq <= 0 ||
      Hkv <= 0 || d <= 0)
    return TG_ERR_SHAPE;
  if (Hq % Hkv != 0) return TG_ERR_SHAPE;
  if (q_tok_stride < (int64_t)Hq * d || k_tok_stride < (int64_t)Hkv * d ||
      v_tok_stride < (int64_t)Hkv * d)
    return TG_ERR_SHAPE;
  if (!isfinite(tau) || !(tau > 0.0f)) return TG_ERR_RANGE;
  if (d != 64 && d != 128) return TG_ERR_UNSUPPORTED;
  // a 64-key tile of k or v is addressed with 32-bit byte offsets
  if (k_tok_stride > (1 << 23) || v_tok_stride > (1 << 23)) return TG_ERR_UNSUPPORTED;
  // launch grids: one row per prompt; 256-row query tiles (bf16) or one
  // plane per head (fp32) in the third dimension
  if (B > kMaxGridYZ) return TG_ERR_UNSUPPORTED;
  if (dtype == TG_BF16 && (max_kept_len + 255) / 256 > kMaxGridYZ) return TG_ERR_UNSUPPORTED;
  if (dtype == TG_F32 && Hq > kMaxGridYZ) return TG_ERR_UNSUPPORTED;
  if (B == 0 || Kt == 0) return TG_OK;
  if (!q || !k || !v || !cu_kept || !out) return TG_ERR_NULL;
  if (gain && !bias_s) return TG_ERR_NULL;
  if (dtype == TG_BF16) {
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
        (q_tok_stride * 2) % 16 != 0 || (k_tok_stride * 2) % 16 != 0 ||
        (v_tok_stride * 2) % 16 != 0)
      return TG_ERR_ALIGN;
    return from_hip(tg::launch_attn_bf16(q, k, v, q_tok_stride, k_tok_stride, v_tok_stride,
                                         bias_s, gain, tau, cu_kept, B, max_kept_len, Kt, Hq,
                                         Hkv, d, out, lse, as_stream(stream)));
  }
  return from_hip(tg::launch_attn_f32(static_cast<const float*>(q), static_cast<const float*>(k),
                                      static_cast<const float*>(v), q_tok_stride, k_tok_stride,
                                      v_tok_stride, bias_s, gain, tau, cu_kept, B, max_kept_len,
                                      Kt, Hq, Hkv, d, static_cast<float*>(out), lse,
                                      as_stream(stream)));
}

int tg_rope_table(const int32_t* pos, int64_t Kt, int d, double rope_theta, float* table,
                  void* stream) {
  if (Kt < 0 || Kt > INT32_MAX || d <= 0 || d % 2 != 0) return TG_ERR_SHAPE;
  if (!isfinite(rope_theta) || !(rope_theta > 1.0)) return TG_ERR_RANGE;
  if (d != 64 && d != 128) return TG_ERR_UNSUPPORTED;
  if (Kt == 0) return TG_OK;
  if (!pos || !table) return TG_ERR_NULL;
  if (!aligned16(table)) return TG_ERR_ALIGN;
  return from_hip(tg::launch_rope_table(pos, Kt, d, rope_theta, table, as_stream(stream)));
}

int tg_qkv_rope(const void* x, int64_t ld_x, int64_t Kt, int D, const void* w_qkv,
                const float* rope_table, int Hq, int Hkv, int d, int dtype, void* qkv,
                int64_t ld_qkv, void* stream) {
  const int eb = elem_bytes(dtype);
  if (!eb) return TG_ERR_DTYPE;
  if (Kt < 0 || Kt > INT32_MAX || D <= 0 || ld_x < D || Hq <= 0 || Hkv <= 0 || d <= 0)
    return TG_ERR_SHAPE;
  const int64_t N = ((int64_t)Hq + 2 * (int64_t)Hkv) * d;
  if (N > INT32_MAX / 2 || ld_qkv < N) return TG_ERR_SHAPE;
  if (d != 64 && d != 128) return TG_ERR_UNSUPPORTED;
  if (dtype == TG_BF16) {
    if (D % 64 != 0) return TG_ERR_UNSUPPORTED;
    // a 256-row stage of x or W_qkv is addressed with 32-bit byte offsets;
    // tiles are counted in int
    if (ld_x >= (1 << 22) || D >= (1 << 22)) return TG_ERR_UNSUPPORTED;
    if (((Kt + 255) / 256) * ((N + 255) / 256) > INT32_MAX) return TG_ERR_UNSUPPORTED;
  } else if (Kt * N > INT32_MAX) {
    return TG_ERR_UNSUPPORTED;  // one thread per output element
  }
  if (Kt == 0) return TG_OK;
  if (!x || !w_qkv || !rope_table || !qkv) return TG_ERR_NULL;
  if (!aligned16(rope_table)) return TG_ERR_ALIGN;
  if (dtype == TG_BF16) {
    if (!aligned16(x) || !aligned16(w_qkv) || !aligned16(qkv) || (ld_x * 2) % 16 != 0 ||
        (ld_qkv * 2) % 16 != 0)
      return TG_ERR_ALIGN;
    return from_hip(tg::launch_qkv_rope_bf16(x, ld_x, Kt, D, w_qkv, rope_table, Hq, Hkv, d, qkv,
                                             ld_qkv, as_stream(stream)));
  }
  return from_hip(tg::launch_qkv_rope_f32(static_cast<const float*>(x), ld_x, Kt, D,
                                          static_cast<const float*>(w_qkv), rope_table, Hq, Hkv,
                                          d, static_cast<float*>(qkv), ld_qkv, as_stream(stream)));
}

int tg_rms_norm(const void* x, int64_t ld_x, int64_t n, int D, const float* weight, float eps,
                int dtype, void* out, int64_t ld_out, void* stream) {
  const int eb = elem_bytes(dtype);
  if (!eb) return TG_ERR_DTYPE;
  if (n < 0 || n > INT32_MAX || D <= 0 || ld_x < D || ld_out < D) return TG_ERR_SHAPE;
  if (!isfinite(eps) || eps < 0.0f) return TG_ERR_RANGE;
  if (D % 8 != 0) return TG_ERR_UNSUPPORTED;
  if (n == 0) return TG_OK;
  if (!x || !weight || !out) return TG_ERR_NULL;
  if (out == x && ld_out != ld_x) return TG_ERR_SHAPE;  // in place only row for row
  if (!aligned16(x) || !aligned16(out) || !aligned16(weight) || (ld_x * eb) % 16 != 0 ||
      (ld_out * eb) % 16 != 0)
    return TG_ERR_ALIGN;
  return from_hip(tg::launch_rms_norm(x, ld_x, n, D, weight, eps, eb, out, ld_out, as_stream(stream)));
}

namespace {
// Shape limits shared by the bf16 projections: K a multiple of the 64-column
// stage, 32-bit byte offsets inside a 256-row stage, tile count in int.
int check_bf16_proj(int64_t n, int K, int64_t ld, int N) {
  if (K % 64 != 0) return TG_ERR_UNSUPPORTED;
  if (ld >= (1 << 22) || K >= (1 << 22)) return TG_ERR_UNSUPPORTED;
  if (((n + 255) / 256) * (((int64_t)N + 127) / 128) > INT32_MAX) return TG_ERR_UNSUPPORTED;
  return TG_OK;
}
}  // namespace

int tg_linear_residual(const void* a, int64_t ld_a, int64_t n, int K, const void* W, int N,
                       const void* residual, int64_t ld_res, int dtype, void* out, int64_t ld_out,
                       void* stream) {
  const int eb = elem_bytes(dtype);
  if (!eb) return TG_ERR_DTYPE;
  if (n < 0 || n > INT32_MAX || K <= 0 || N <= 0 || ld_a < K || ld_res < N || ld_out < N)
    return TG_ERR_SHAPE;
  if (dtype == TG_BF16) {
    if (N % 64 != 0) return TG_ERR_UNSUPPORTED;
    const int st = check_bf16_proj(n, K, ld_a, N);
    if (st != TG_OK) return st;
  } else if (n * N > INT32_MAX) {
    return TG_ERR_UNSUPPORTED;  // one thread per output element
  }
  if (n == 0) return TG_OK;
  if (!a || !W || !residual || !out) return TG_ERR_NULL;
  if (out == residual && ld_out != ld_res) return TG_ERR_SHAPE;  // in place only row for row
  if (dtype == TG_BF16 &&
      (!aligned16(a) || !aligned16(W) || !aligned16(residual) || !aligned16(out) ||
       (ld_a * eb) % 16 != 0 || (ld_res * eb) % 16 != 0 || (ld_out * eb) % 16 != 0))
    return TG_ERR_ALIGN;
  if (!aligned4(a) || !aligned4(W) || !aligned4(residual) || !aligned4(out)) return TG_ERR_ALIGN;
  return from_hip(tg::launch_linear_residual(a, ld_a, n, K, W, N, residual, ld_res, eb, out, ld_out,
                                             as_stream(stream)));
}

int tg_swiglu(const void* h, int64_t ld_h, int64_t n, int D, const void* w_gate, const void* w_up,
              int I, int dtype, void* out, int64_t ld_out, void* stream) {
  const int eb = elem_bytes(dtype);
  if (!eb) return TG_ERR_DTYPE;
  if (n < 0 || n > INT32_MAX || D <= 0 || I <= 0 || ld_h < D || ld_out < I) return TG_ERR_SHAPE;
  if (dtype == TG_BF16) {
    if (I % 32 != 0) return TG_ERR_UNSUPPORTED;
    const int st = check_bf16_proj(n, D, ld_h, I);
    if (st != TG_OK) return st;
  } else if (n * I > INT32_MAX) {
    return TG_ERR_UNSUPPORTED;
  }
  if (n == 0) return TG_OK;
  if (!h || !w_gate || !w_up || !out) return TG_ERR_NULL;
  if (dtype == TG_BF16 && (!aligned16(h) || !aligned16(w_gate) || !aligned16(w_up) ||
                           !aligned16(out) || (ld_h * eb) % 16 != 0 || (ld_out * eb) % 16 != 0))
    return TG_ERR_ALIGN;
  if (!aligned4(h) || !aligned4(w_gate) || !aligned4(w_up) || !aligned4(out)) return TG_ERR_ALIGN;
  return from_hip(tg::launch_swiglu(h, ld_h, n, D, w_gate, w_up, I, eb, out, ld_out,
                                    as_stream(stream)));
}

int tg_gated_attn_bwd_workspace(int B, int64_t Kt, int Hq, int Hkv, int d, int dtype, int max_kept_len,
                                size_t* bytes) {
  if (!bytes) return TG_ERR_NULL;
  const int eb = elem_bytes(dtype);
  if (!eb) return TG_ERR_DTYPE;
  if (B < 0 || Kt < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || d <= 0 || max_kept_len < 0) return TG_ERR_SHAPE;
  *bytes = tg::attn_bwd_workspace_bytes(B, Kt, Hq, Hkv, d, eb, max_kept_len);
  return TG_OK;
}

int tg_gated_attn_bwd(const void* q, const void* k, const void* v, int64_t q_tok_stride,
                      int64_t k_tok_stride, int64_t v_tok_stride, const float* bias_s,
                      const float* gain, float tau, const int32_t* cu_kept, int B,
                      int max_kept_len, int64_t Kt, int Hq, int Hkv, int d, int dtype,
                      const void* out, const float* lse, const void* dout, void* dq, void* dk,
                      void* dv, float* dbias, float* dgain, float* dtau, void* workspace,
                      size_t workspace_bytes, void* stream) {
  const int eb = elem_bytes(dtype);
  if (!eb) return TG_ERR_DTYPE;
  if (B < 0 || Kt < 0 || Kt > INT32_MAX || max_kept_len < 0 || max_kept_len > Kt || Hq <= 0 ||
      Hkv <= 0 || d <= 0)
    return TG_ERR_SHAPE;
  if (Hq % Hkv != 0) return TG_ERR_SHAPE;
  if (q_tok_stride < (int64_t)Hq * d || k_tok_stride < (int64_t)Hkv * d ||
      v_tok_stride < (int64_t)Hkv * d)
    return TG_ERR_SHAPE;
  if (!isfinite(tau) || !(tau > 0.0f)) return TG_ERR_RANGE;
  if (d != 64 && d != 128) return TG_ERR_UNSUPPORTED;
  // 64-row tiles of q, k, v and dout are addressed with 32-bit byte offsets;
  // launch grids: prompts and 128-row tiles in the second and third dimension
  if (q_tok_stride > (1 << 23) || k_tok_stride > (1 << 23) || v_tok_stride > (1 << 23) ||
      (int64_t)Hq * d > (1 << 23))
    return TG_ERR_UNSUPPORTED;
  if (B > kMaxGridYZ || (max_kept_len + 127) / 128 > kMaxGridYZ) return TG_ERR_UNSUPPORTED;
  if (dtype == TG_F32 && (Kt * Hq > INT32_MAX)) return TG_ERR_UNSUPPORTED;
  if (B == 0 || Kt == 0) return TG_OK;
  if (!q || !k || !v || !cu_kept || !out || !lse || !dout || !dq || !dk || !dv) return TG_ERR_NULL;
  if (gain && !bias_s) return TG_ERR_NULL;
  const size_t need = tg::attn_bwd_workspace_bytes(B, Kt, Hq, Hkv, d, eb, max_kept_len);
  if (!workspace || workspace_bytes < need) return TG_ERR_WORKSPACE;
  if (!aligned16(workspace)) return TG_ERR_ALIGN;
  if (dtype == TG_BF16) {
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(dout) ||
        !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || (q_tok_stride * 2) % 16 != 0 ||
        (k_tok_stride * 2) % 16 != 0 || (v_tok_stride * 2) % 16 != 0)
      return TG_ERR_ALIGN;
  }
  return from_hip(tg::launch_attn_bwd(q, k, v, q_tok_stride, k_tok_stride, v_tok_stride, bias_s,
                                      gain, tau, cu_kept, B, max_kept_len, Kt, Hq, Hkv, d, eb, out,
                                      lse, dout, dq, dk, dv, dbias, dgain, dtau, workspace,
                                      as_stream(stream)));
}

int tg_gate_bwd_workspace(int64_t Kt, int D, int F, int dtype, size_t* bytes) {
  if (!bytes) return TG_ERR_NULL;
  const int eb = elem_bytes(dtype);
  if (!eb) return TG_ERR_DTYPE;
  if (Kt < 0 || D <= 0 || F <= 0) return TG_ERR_SHAPE;
  *bytes = tg::gate_bwd_workspace_bytes(Kt, D, F, eb);
  return TG_OK;
}

int tg_gate_bwd(const void* hidden_k, int64_t ld_hidden, int64_t Kt, int D, const void* W1,
                const float* b1, const float* w2, int F, const float* dbias,
                const int32_t* kept_idx, const int32_t* cu_seqlens, const int32_t* doc_begin,
                const int32_t* doc_end, int B, int dtype, void* dhidden_k, float* dW1, float* db1,
                float* dw2, float* db2, void* workspace, size_t workspace_bytes, void* stream) {
  const int eb = elem_bytes(dtype);
  if (!eb) return TG_ERR_DTYPE;
  if (Kt < 0 || Kt > INT32_MAX || D <= 0 || F <= 0 || ld_hidden < D || B < 0) return TG_ERR_SHAPE;
  if (Kt > 0 && B == 0) return TG_ERR_SHAPE;
  if (!(F == 64 || F == 128 || F == 256)) return TG_ERR_UNSUPPORTED;
  if (dtype == TG_BF16) {
    if (D % 64 != 0 || ld_hidden >= (1 << 22) || D >= (1 << 22)) return TG_ERR_UNSUPPORTED;
  } else if (Kt * F > INT32_MAX || Kt * D > INT32_MAX) {
    return TG_ERR_UNSUPPORTED;
  }
  if ((int64_t)F * D > INT32_MAX / 2) return TG_ERR_UNSUPPORTED;
  if (!W1 || !w2 || !dW1 || !dw2 || !db2) return TG_ERR_NULL;
  const size_t need = tg::gate_bwd_workspace_bytes(Kt, D, F, eb);
  if (!workspace || workspace_bytes < need) return TG_ERR_WORKSPACE;
  if (Kt > 0 && (!hidden_k || !dbias || !kept_idx || !cu_seqlens || !doc_begin || !doc_end ||
                 !dhidden_k))
    return TG_ERR_NULL;
  if (!aligned16(workspace) || !aligned16(w2) || (b1 && !aligned16(b1))) return TG_ERR_ALIGN;
  if (dtype == TG_BF16 && (!aligned16(hidden_k) || !aligned16(W1) || !aligned16(dhidden_k) ||
                           (ld_hidden * 2) % 16 != 0))
    return TG_ERR_ALIGN;
  return from_hip(tg::launch_gate_bwd(hidden_k, ld_hidden, Kt, D, W1, b1, w2, F, dbias, kept_idx,
                                      cu_seqlens, doc_begin, doc_end, B, eb, dhidden_k, dW1, db1,
                                      dw2, db2, workspace, as_stream(stream)));
}

int tg_kv_scatter(const void* k, const void* v, int64_t k_tok_stride, int64_t v_tok_stride,
                  const float* bias_s, const int32_t* cu_kept, int B, int64_t Kt, int Hkv, int d,
                  int dtype, void* k_cache, void* v_cache, int64_t cache_k_stride,
                  int64_t cache_v_stride, float* bias_cache, const int32_t* start, void* stream) {
  const int eb = elem_bytes(dtype);
  if (!eb) return TG_ERR_DTYPE;
  if (B < 0 || Kt < 0 || Hkv <= 0 || d <= 0 || k_tok_stride < (int64_t)Hkv * d ||
      v_tok_stride < (int64_t)Hkv * d || cache_k_stride < (int64_t)Hkv * d ||
      cache_v_stride < (int64_t)Hkv * d)
    return TG_ERR_SHAPE;
  if (Kt > 0 && B == 0) return TG_ERR_SHAPE;
  if (B == 0 || Kt == 0) return TG_OK;
  if (!k || !v || !cu_kept || !k_cache || !v_cache || !bias_cache || !start) return TG_ERR_NULL;
  return from_hip(tg::launch_kv_scatter(k, v, k_tok_stride, v_tok_stride, bias_s, cu_kept, B, Kt, Hkv,
                                        d, eb, k_cache, v_cache, cache_k_stride, cache_v_stride,
                                        bias_cache, start, as_stream(stream)));
}

int tg_kv_append(const void* k_new, const void* v_new, int B, int Hkv, int d, int dtype,
                 void* k_cache, void* v_cache, int64_t cache_k_stride, int64_t cache_v_stride,
                 float* bias_cache, const int32_t* start, const int32_t* pos, void* stream) {
  const int eb = elem_bytes(dtype);
  if (!eb) return TG_ERR_DTYPE;
  if (B < 0 || Hkv <= 0 || d <= 0 || cache_k_stride < (int64_t)Hkv * d ||
      cache_v_stride < (int64_t)Hkv * d)
    return TG_ERR_SHAPE;
  if (B == 0) return TG_OK;
  if (!k_new || !v_new || !k_cache || !v_cache || !bias_cache || !start || !pos) return TG_ERR_NULL;
  return from_hip(tg::launch_kv_append(k_new, v_new, B, Hkv, d, eb, k_cache, v_cache, cache_k_stride,
                                       cache_v_stride, bias_cache, start, pos, as_stream(stream)));
}

int tg_decode_attn_workspace(int B, int Hq, int d, int max_len, size_t* bytes) {
  if (!bytes) return TG_ERR_NULL;
  if (B < 0 || Hq <= 0 || d <= 0 || max_len < 0) return TG_ERR_SHAPE;
  *bytes = tg::decode_workspace_bytes(B, Hq, d, max_len);
  return TG_OK;
}

int tg_decode_attn(const void* q, const void* k_cache, const void* v_cache, int64_t cache_k_stride,
                   int64_t cache_v_stride, const float* bias_cache, const float* gain, float tau,
                   const int32_t* start, const int32_t* lens, int B, int max_len, int Hq, int Hkv,
                   int d, int dtype, void* out, float* lse, void* workspace,
                   size_t workspace_bytes, void* stream) {
  const int eb = elem_bytes(dtype);
  if (!eb) return TG_ERR_DTYPE;
  if (B < 0 || max_len < 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || Hq % Hkv != 0 ||
      cache_k_stride < (int64_t)Hkv * d || cache_v_stride < (int64_t)Hkv * d)
    return TG_ERR_SHAPE;
  if (!isfinite(tau) || !(tau > 0.0f)) return TG_ERR_RANGE;
  if (d != 64 && d != 128) return TG_ERR_UNSUPPORTED;
  if (Hq / Hkv > 8) return TG_ERR_UNSUPPORTED;  // query heads per KV head held in registers
  if ((int64_t)B * Hkv > INT32_MAX || (max_len + 127) / 128 > kMaxGridYZ) return TG_ERR_UNSUPPORTED;
  if (B == 0) return TG_OK;
  if (!q || !k_cache || !v_cache || !start || !lens || !out) return TG_ERR_NULL;
  if (gain && !bias_cache) return TG_ERR_NULL;
  const size_t need = tg::decode_workspace_bytes(B, Hq, d, max_len);
  if (!workspace || workspace_bytes < need) return TG_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(workspace) ||
      (cache_k_stride * eb) % 16 != 0 || (cache_v_stride * eb) % 16 != 0)
    return TG_ERR_ALIGN;
  return from_hip(tg::launch_decode_attn(q, k_cache, v_cache, cache_k_stride, cache_v_stride,
                                         bias_cache, gain, tau, start, lens, B, max_len, Hq, Hkv, d,
                                         eb, out, lse, workspace, as_stream(stream)));
}

}  // extern "C"
