// fa_prologue.hip -- the attention prologue on Q and K: RMSNorm over head_dim, then rotary
// position embedding over three axes (t, y, x), fused into one pass; and the same fused with
// the low-bit path's per-128-token-block int8 quantisation.
//
// The tech report's kernel-fusion paragraph fuses RMSNorm with elementwise work, and the
// structured summary gives each token stream condition-specific RoPE positions; neither gives
// formulas.  What is computed here (a stated reading):
//   y = x / sqrt(mean_d x^2 + eps) * gamma[d]                 (gamma [D], shared by the heads)
//   the D/2 rotation pairs (d, d + D/2) split into t, y, x groups of D/2 - 2*floor(D/6),
//   floor(D/6), floor(D/6) pairs; pair j of a g-pair group turns by pos_axis * base^(-j/g):
//   (a, b) -> (a cos - b sin, a sin + b cos).
// Positions are the caller's, per token (target and source tokens of a frame may share them,
// references take their own), so the same kernel serves every token stream.
//
// Layout: D/8 lanes cover a (token, head) row, 8 channels each; the lanes of the first half of
// the row hold the "a" of every pair, lane l ^ (D/16) holds its "b".
#include "fa_device.h"

namespace fa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

namespace pro {

// per-lane rotation frequencies of its 8 channels' pairs, in turns per position step
// (theta / 2 pi), and the axis of each
template <int D>
__device__ __forceinline__ void lane_freqs(int lanec, float base_log2, float (&theta)[8],
                                           int (&axis)[8]) {
  constexpr int P = D / 2, PY = D / 6, PT = P - 2 * PY;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int c = lanec * 8 + k;
    const int i = c < P ? c : c - P;  // pair index
    const int g = i < PT ? 0 : (i < PT + PY ? 1 : 2);
    const int j = i - (g == 0 ? 0 : (g == 1 ? PT : PT + PY));
    const int gs = g == 0 ? PT : PY;
    axis[k] = g;
    theta[k] = exp2f(-(float)j / (float)gs * base_log2) * 0.15915494309189535f;
  }
}

// sine and cosine of the lane's 8 rotation angles at token position pos3 (angle in turns,
// reduced to [0, 1): v_sin_f32 / v_cos_f32 take turns)
__device__ __forceinline__ void lane_angles(const int *pos3, const float (&theta)[8],
                                            const int (&axis)[8], float (&sn)[8], float (&cs)[8]) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    float rev = (float)pos3[axis[k]] * theta[k];
    rev -= floorf(rev);
    sn[k] = __builtin_amdgcn_sinf(rev);
    cs[k] = __builtin_amdgcn_cosf(rev);
  }
}

// RMSNorm + RoPE of one row held as 8 values per lane (LPR lanes per row) with the lane's 8
// norm weights and the row's rotation sines and cosines; leaves the result rounded to bf16 (as a
// tensor written by the unfused kernel would hold it), as floats.
template <int D>
__device__ __forceinline__ void norm_rope_row(float (&x)[8], int lanec, const float (&gamma)[8],
                                             float eps, const float (&sn)[8],
                                             const float (&cs)[8]) {
  constexpr int LPR = D / 8, HALF = LPR / 2;
  float ss = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) ss = fmaf(x[k], x[k], ss);
#pragma unroll
  for (int o = HALF; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  const float r = 1.0f / sqrtf(ss / (float)D + eps);
  float y[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) y[k] = x[k] * r * gamma[k];
  const bool first = lanec < HALF;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float other = __shfl_xor(y[k], HALF);
    const float a = first ? y[k] : other, b = first ? other : y[k];
    const float v = first ? a * cs[k] - b * sn[k] : a * sn[k] + b * cs[k];
    x[k] = (float)(__bf16)v;
  }
}

}  // namespace pro

// bf16 -> bf16.  One workgroup per (batch, token): 256/LPR rows (heads) per pass; the rotation
// angles depend on the token and the lane only, so their sines and cosines are taken once and
// serve every head.
template <int D>
__global__ void __launch_bounds__(256) norm_rope_kernel(const ProArgs a) {
  constexpr int LPR = D / 8, RPW = 256 / LPR;
  const int t = blockIdx.x % a.n, b = blockIdx.x / a.n;
  const int lanec = threadIdx.x % LPR, rsub = threadIdx.x / LPR;
  float theta[8], sn[8], cs[8];
  int axis[8];
  pro::lane_freqs<D>(lanec, a.base_log2, theta, axis);
  pro::lane_angles(a.pos + 3 * t, theta, axis, sn, cs);
  float gam[8];  // the lane's norm weights, loaded once for every row
#pragma unroll
  for (int k = 0; k < 8; ++k) gam[k] = a.gamma[lanec * 8 + k];
  const __bf16 *in_t = (const __bf16 *)a.in + b * a.isb + (int64_t)t * a.isn + lanec * 8;
  __bf16 *out_t = (__bf16 *)a.out + b * a.osb + (int64_t)t * a.osn + lanec * 8;
  // One pass of RPW heads at a time: with 256-thread workgroups per token the CU holds enough
  // of them to cover the load latency (batching the passes' loads was slower).
  for (int h = rsub; h < a.H; h += RPW) {  // a row's lanes share h
    const bf16x8_t v = *(const bf16x8_t *)(in_t + h * a.ish);
    float x[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = (float)v[k];
    pro::norm_rope_row<D>(x, lanec, gam, a.eps, sn, cs);
    bf16x8_t o;
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] = (__bf16)x[k];
    *(bf16x8_t *)(out_t + h * a.osh) = o;
  }
}

// bf16 -> int8 codes per (batch, head, 128-token block), head_dim 128, the low-bit path's format:
// one workgroup per (block, b, h); 16 lanes per row, 16 rows per pass, 8 passes.  The rotated
// values are rounded to bf16 first, then (K) reduced by the given per-head mean, then quantised
// with scale absmax/127 and round-half-even codes; for Q the per-row shift scale * q.m goes to
// `lse` when a mean is given.
__global__ void __launch_bounds__(256) norm_rope_quant_kernel(const ProArgs a) {
  constexpr int D = 128;
  const int nblk = (a.n + 127) / 128;
  const int bh = blockIdx.x % (a.batch * a.H), blk = blockIdx.x / (a.batch * a.H);
  const int b = bh / a.H, h = bh % a.H;
  const int t = threadIdx.x, lanec = t & 15, rsub = t >> 4;
  float theta[8];
  int axis[8];
  pro::lane_freqs<D>(lanec, a.base_log2, theta, axis);
  float m[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) m[k] = a.mean ? a.mean[(int64_t)bh * D + lanec * 8 + k] : 0.0f;
  float gam[8];  // the lane's norm weights, loaded once for every row
#pragma unroll
  for (int k = 0; k < 8; ++k) gam[k] = a.gamma[lanec * 8 + k];
  float x[8][8];
  bool live[8];
  float amax = 0.0f;
  // The eight row loads go out together: a row past the last token reads the last token's row
  // (and its position) and is zeroed after the rotation.
  const __bf16 *in_bh = (const __bf16 *)a.in + b * a.isb + h * a.ish + lanec * 8;
  bf16x8_t v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    v[j] = *(const bf16x8_t *)(in_bh + (int64_t)min(blk * 128 + j * 16 + rsub, a.n - 1) * a.isn);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int tok = blk * 128 + j * 16 + rsub;
    live[j] = tok < a.n;  // a row's 16 lanes agree
#pragma unroll
    for (int k = 0; k < 8; ++k) x[j][k] = (float)v[j][k];
    float sn[8], cs[8];
    pro::lane_angles(a.pos + 3 * min(tok, a.n - 1), theta, axis, sn, cs);
    pro::norm_rope_row<D>(x[j], lanec, gam, a.eps, sn, cs);
    if (a.kind == 1) {
#pragma unroll
      for (int k = 0; k < 8; ++k) x[j][k] -= m[k];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      x[j][k] = live[j] ? x[j][k] : 0.0f;
      amax = fmaxf(amax, fabsf(x[j][k]));
    }
  }
  if (a.kind == 0 && a.lse && a.mean) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float dot = 0.0f;
#pragma unroll
      for (int k = 0; k < 8; ++k) dot = fmaf(x[j][k], m[k], dot);
      dot += __shfl_xor(dot, 8);
      dot += __shfl_xor(dot, 4);
      dot += __shfl_xor(dot, 2);
      dot += __shfl_xor(dot, 1);
      if (live[j] && lanec == 0)
        a.lse[(int64_t)bh * a.n + blk * 128 + j * 16 + rsub] = a.softmax_scale * dot;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  __shared__ float red[4];
  if ((t & 63) == 0) red[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
  if (t == 0) a.scale[(int64_t)bh * nblk + blk] = amax / 127.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (!live[j]) continue;
    uint32_t w32[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      uint32_t u = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float r = fminf(fmaxf(__builtin_rintf(x[j][4 * q + i] * inv), -127.0f), 127.0f);
        u |= ((uint32_t)(int)r & 0xffu) << (8 * i);
      }
      w32[q] = u;
    }
    const int tok = blk * 128 + j * 16 + rsub;
    *(uint2 *)((char *)a.out + b * a.osb + (int64_t)tok * a.osn + h * a.osh + lanec * 8) =
        uint2{w32[0], w32[1]};
  }
}

hipError_t launch_norm_rope(const ProArgs &a, int head_dim, hipStream_t s) {
  const int64_t grid = (int64_t)a.batch * a.n;
  if (grid == 0 || a.H == 0) return hipSuccess;
  if (head_dim == 64)
    hipLaunchKernelGGL(norm_rope_kernel<64>, dim3((unsigned)grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(norm_rope_kernel<128>, dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_norm_rope_quant(const ProArgs &a, hipStream_t s) {
  const int64_t grid = (int64_t)a.batch * a.H * ((a.n + 127) / 128);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(norm_rope_quant_kernel, dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace fa
