// fa_w8a8_api.cpp -- C ABI of the per-block W8A8 linear layer: argument checks on the host,
// then the launches of fa_w8a8.hip.
#include <string>

#include "fa_layout_impl.h"

using namespace fa;

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p % 16) == 0; }

fa_status check_shape(int32_t rows, int32_t cols, const char *what) {
  if (rows < 0 || cols < 0) return fail(FA_ERR_INVALID, std::string(what) + ": negative size");
  if (cols % 128) return fail(FA_ERR_INVALID, std::string(what) + ": columns must be a multiple of 128");
  return FA_OK;
}

// leading dimension in elements of size es: at least cols, rows 16-byte aligned, offsets of a
// 256-row tile within 2^31 bytes
fa_status check_ld(int64_t ld, int32_t cols, int es, const char *what) {
  if (ld < cols) return fail(FA_ERR_INVALID, std::string(what) + ": leading dimension < columns");
  if ((ld * es) % 16) return fail(FA_ERR_INVALID, std::string(what) + ": rows not 16-byte aligned");
  // the GEMM addresses a 256-row operand tile with 32-bit offsets: 256 rows stay below 2^31 bytes
  if (ld * es >= (int64_t(1) << 23))
    return fail(FA_ERR_UNSUPPORTED, std::string(what) + ": leading dimension of 2^23 bytes or more");
  return FA_OK;
}

}  // namespace

extern "C" fa_status fa_w8a8_quantize_act(const void *x, int64_t ld_x, int32_t m, int32_t k,
                                          int8_t *xq, int64_t ld_xq, float *sx, int64_t ld_sx,
                                          fa_hip_stream stream) {
  fa_status st = check_shape(m, k, "activations");
  if (st != FA_OK) return st;
  if (m == 0 || k == 0) return FA_OK;
  if (!x || !xq || !sx) return fail(FA_ERR_INVALID, "NULL argument");
  if (!aligned16(x) || !aligned16(xq) || ((uintptr_t)sx % 4))
    return fail(FA_ERR_INVALID, "x and xq must be 16-byte aligned, sx 4-byte aligned");
  if ((st = check_ld(ld_x, k, 2, "x")) != FA_OK) return st;
  if ((st = check_ld(ld_xq, k, 1, "xq")) != FA_OK) return st;
  if (ld_sx < m) return fail(FA_ERR_INVALID, "ld_sx must be >= m");
  W8QuantArgs a{};
  a.in = x;
  a.ld_in = ld_x;
  a.out = xq;
  a.ld_out = ld_xq;
  a.scale = sx;
  a.ld_scale = ld_sx;
  a.rows = m;
  a.cols = k;
  hipError_t e = launch_w8a8_quant_act(a, (hipStream_t)stream);
  if (e != hipSuccess) return fail(FA_ERR_HIP, std::string("launch: ") + hipGetErrorString(e));
  return FA_OK;
}

extern "C" fa_status fa_w8a8_quantize_weight(const void *w, int64_t ld_w, int32_t n, int32_t k,
                                             int8_t *wq, int64_t ld_wq, float *sw,
                                             fa_hip_stream stream) {
  fa_status st = check_shape(n, k, "weights");
  if (st != FA_OK) return st;
  if (n % 128) return fail(FA_ERR_INVALID, "weights: rows must be a multiple of 128");
  if (n == 0 || k == 0) return FA_OK;
  if (!w || !wq || !sw) return fail(FA_ERR_INVALID, "NULL argument");
  if (!aligned16(w) || !aligned16(wq) || ((uintptr_t)sw % 4))
    return fail(FA_ERR_INVALID, "w and wq must be 16-byte aligned, sw 4-byte aligned");
  if ((st = check_ld(ld_w, k, 2, "w")) != FA_OK) return st;
  if ((st = check_ld(ld_wq, k, 1, "wq")) != FA_OK) return st;
  W8QuantArgs a{};
  a.in = w;
  a.ld_in = ld_w;
  a.out = wq;
  a.ld_out = ld_wq;
  a.scale = sw;
  a.ld_scale = k / 128;
  a.rows = n;
  a.cols = k;
  hipError_t e = launch_w8a8_quant_weight(a, (hipStream_t)stream);
  if (e != hipSuccess) return fail(FA_ERR_HIP, std::string("launch: ") + hipGetErrorString(e));
  return FA_OK;
}

extern "C" fa_status fa_w8a8_gemm(const int8_t *xq, int64_t ld_xq, const float *sx, int64_t ld_sx,
                                  const int8_t *wq, int64_t ld_wq, const float *sw, int32_t m,
                                  int32_t n, int32_t k, void *y, int64_t ld_y,
                                  fa_hip_stream stream) {
  fa_status st = check_shape(m, k, "activations");
  if (st != FA_OK) return st;
  if (n < 0 || n % 128) return fail(FA_ERR_INVALID, "n must be a multiple of 128");
  if (m == 0 || n == 0) return FA_OK;
  if (k == 0) return fail(FA_ERR_INVALID, "k must be >= 128");
  if (!xq || !sx || !wq || !sw || !y) return fail(FA_ERR_INVALID, "NULL argument");
  if (!aligned16(xq) || !aligned16(wq) || !aligned16(y) || ((uintptr_t)sx % 4) ||
      ((uintptr_t)sw % 4))
    return fail(FA_ERR_INVALID, "xq, wq and y must be 16-byte aligned, sx and sw 4-byte aligned");
  if ((st = check_ld(ld_xq, k, 1, "xq")) != FA_OK) return st;
  if ((st = check_ld(ld_wq, k, 1, "wq")) != FA_OK) return st;
  if ((st = check_ld(ld_y, n, 2, "y")) != FA_OK) return st;
  if (ld_sx < m) return fail(FA_ERR_INVALID, "ld_sx must be >= m");
  if ((int64_t)(k / 128) * ld_sx >= (int64_t(1) << 29))
    return fail(FA_ERR_UNSUPPORTED, "the activation scales span 2^31 bytes or more");
  W8GemmArgs a{};
  a.xq = xq;
  a.sx = sx;
  a.wq = wq;
  a.sw = sw;
  a.y = y;
  a.ld_xq = ld_xq;
  a.ld_wq = ld_wq;
  a.ld_y = ld_y;
  a.ld_sx = (int32_t)ld_sx;
  a.m = m;
  a.n = n;
  a.k = k;
  hipError_t e = launch_w8a8_gemm(a, (hipStream_t)stream);
  if (e != hipSuccess) return fail(FA_ERR_HIP, std::string("launch: ") + hipGetErrorString(e));
  return FA_OK;
}
