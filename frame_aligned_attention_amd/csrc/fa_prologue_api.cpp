// fa_prologue_api.cpp -- C ABI of the QK prologue (RMSNorm + RoPE, optionally fused with the
// low-bit quantiser): host checks, then the launches of fa_prologue.hip.
#include <cmath>
#include <string>

#include "fa_layout_impl.h"

using namespace fa;

namespace {

fa_status check_common(const fa_tensor *in, const fa_tensor *out, const float *gamma,
                       const int32_t *pos, float eps, float base, int32_t tokens, int32_t batch,
                       int32_t heads, int32_t head_dim, int out_es) {
  if (!in || !out || !gamma || !pos) return fail(FA_ERR_INVALID, "NULL argument");
  if (tokens < 0 || batch < 1 || heads < 1) return fail(FA_ERR_INVALID, "bad geometry");
  if (head_dim != 64 && head_dim != 128) return fail(FA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return fail(FA_ERR_INVALID, "eps must be finite, >= 0");
  if (!(base > 1.0f) || !std::isfinite(base)) return fail(FA_ERR_INVALID, "rope base must be > 1");
  const fa_tensor *t[2] = {in, out};
  const int es[2] = {2, out_es};
  for (int i = 0; i < 2; ++i) {
    if (!t[i]->data) return fail(FA_ERR_INVALID, "tensor data is NULL");
    if ((uintptr_t)t[i]->data % 16 || (t[i]->stride_n * es[i]) % 16 ||
        (t[i]->stride_h * es[i]) % 16 || (batch > 1 && (t[i]->stride_b * es[i]) % 16))
      return fail(FA_ERR_INVALID, "rows must be 16-byte aligned");
    if (t[i]->stride_n < 0 || t[i]->stride_h < 0 || t[i]->stride_b < 0)
      return fail(FA_ERR_INVALID, "negative stride");
  }
  return FA_OK;
}

ProArgs args_of(const fa_tensor *in, const fa_tensor *out, const float *gamma,
                const int32_t *pos, float eps, float base, int32_t tokens, int32_t batch,
                int32_t heads) {
  ProArgs a{};
  a.in = in->data;
  a.isb = in->stride_b; a.isn = in->stride_n; a.ish = in->stride_h;
  a.out = out->data;
  a.osb = out->stride_b; a.osn = out->stride_n; a.osh = out->stride_h;
  a.gamma = gamma;
  a.pos = pos;
  a.eps = eps;
  a.base_log2 = std::log2(base);
  a.n = tokens;
  a.batch = batch;
  a.H = heads;
  return a;
}

}  // namespace

extern "C" fa_status fa_qk_norm_rope(const fa_tensor *in, const fa_tensor *out, const float *gamma,
                                     float eps, const int32_t *pos, float rope_base,
                                     int32_t tokens, int32_t batch, int32_t heads,
                                     int32_t head_dim, fa_hip_stream stream) {
  fa_status st = check_common(in, out, gamma, pos, eps, rope_base, tokens, batch, heads,
                              head_dim, 2);
  if (st != FA_OK) return st;
  ProArgs a = args_of(in, out, gamma, pos, eps, rope_base, tokens, batch, heads);
  hipError_t e = launch_norm_rope(a, head_dim, (hipStream_t)stream);
  if (e != hipSuccess) return fail(FA_ERR_HIP, std::string("launch: ") + hipGetErrorString(e));
  return FA_OK;
}

extern "C" fa_status fa_qk_norm_rope_quant(const fa_tensor *in, const fa_tensor *codes,
                                           const float *gamma, float eps, const int32_t *pos,
                                           float rope_base, int32_t is_key,
                                           const float *k_mean, float *lse_shift,
                                           float softmax_scale, int32_t tokens, int32_t batch,
                                           int32_t heads, int32_t head_dim,
                                           fa_hip_stream stream) {
  fa_status st = check_common(in, codes, gamma, pos, eps, rope_base, tokens, batch, heads,
                              head_dim, 1);
  if (st != FA_OK) return st;
  if (head_dim != 128) return fail(FA_ERR_UNSUPPORTED, "the low-bit format is built for head_dim 128");
  if (!codes->scale) return fail(FA_ERR_INVALID, "codes->scale (per-block scales) is NULL");
  if (is_key && !k_mean) return fail(FA_ERR_INVALID, "keys need k_mean");
  if (lse_shift && (is_key || !k_mean))
    return fail(FA_ERR_INVALID, "lse_shift is for queries with a key mean");
  ProArgs a = args_of(in, codes, gamma, pos, eps, rope_base, tokens, batch, heads);
  a.kind = is_key ? 1 : 0;
  a.mean = k_mean;
  a.lse = lse_shift;
  a.softmax_scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / std::sqrt((float)head_dim);
  a.scale = codes->scale;
  hipError_t e = launch_norm_rope_quant(a, (hipStream_t)stream);
  if (e != hipSuccess) return fail(FA_ERR_HIP, std::string("launch: ") + hipGetErrorString(e));
  return FA_OK;
}
