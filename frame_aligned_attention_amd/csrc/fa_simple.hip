// fa_simple.hip -- the ring-buffer append and the fp32 attention kernel.
//
// Ring append: the streaming KV cache ("Vidu S2" structured summary, section
// 4.3: sliding-window context; section 5.2: source frames are not kept).
// Absolute frame g of the target stream lives in ring slot g mod capacity.
//
// fp32 kernel: exact-arithmetic path (one query row per lane, fp32 online
// softmax with expf) over the same block map as the bf16 kernel.  It is the
// path for fp32 inputs; it makes no attempt at speed.
#include "fa_internal.h"

namespace fa {

// One thread per 16-byte piece of a (token, head) row: blockIdx.y = 2*batch + tensor (K, V),
// blockIdx.x a run of 256 / chunks16 rows of that tensor's chunk, rows in (token, head) order, so
// a workgroup reads and writes contiguous spans.  32-bit index arithmetic (rows per tensor and
// batch stay far below 2^31); the byte offsets are 64-bit.
__global__ void __launch_bounds__(256) ring_append_kernel(const RingArgs a) {
  const int lg = __builtin_ctz(a.chunks16);  // chunks16 is 8, 16 or 32
  const int rows = a.frames * a.T * a.H;
  const int row = (int)blockIdx.x * (256 >> lg) + ((int)threadIdx.x >> lg);
  if (row >= rows) return;
  const int c = (int)threadIdx.x & (a.chunks16 - 1);
  const int i = (int)blockIdx.y & 1, b = (int)blockIdx.y >> 1;  // i 0: K, 1: V
  const int tok = row / a.H, h = row - tok * a.H;
  const int fi = tok / a.T, t = tok - fi * a.T;
  const int slot = ring_slot(a.first_frame + fi, a.sink, a.cache_frames);
  const char *src = (const char *)a.src[i] + b * a.ssb[i] + tok * a.ssn[i] + h * a.ssh[i] + c * 16;
  char *dst = (char *)a.dst[i] + b * a.dsb[i] + ((int64_t)slot * a.T + t) * a.dsn[i] +
              h * a.dsh[i] + c * 16;
  *(uint4 *)dst = *(const uint4 *)src;
}

hipError_t launch_ring_append(const RingArgs &a, hipStream_t s) {
  if (a.chunks16 != 8 && a.chunks16 != 16 && a.chunks16 != 32) return hipErrorInvalidValue;
  const int64_t rows = (int64_t)a.frames * a.T * a.H;
  if (rows < 1 || a.batch < 1) return hipSuccess;
  if (rows > INT32_MAX || 2LL * a.batch > 65535) return hipErrorInvalidValue;
  const int per_block = 256 / a.chunks16;
  const int64_t blocks = (rows + per_block - 1) / per_block;
  hipLaunchKernelGGL(ring_append_kernel, dim3((unsigned)blocks, (unsigned)(2 * a.batch)), dim3(256),
                     0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------------ fp32 attention

template <int D>
__global__ void __launch_bounds__(64) attn_f32_kernel(const AttnArgs a) {
  constexpr int KT = 32;  // keys staged per step
  __shared__ float Ks[KT][D];
  __shared__ float Vs[KT][D];
  const DevWork w = a.work[blockIdx.x];
  if (w.tile < 0) return;
  const DevTile tile = a.tiles[w.tile];
  const int b = w.bh / a.H, h = w.bh - (w.bh / a.H) * a.H;
  const int tid = threadIdx.x;
  const int row = tile.row0 + tid;
  const bool valid = tid < tile.rows;
  const Seg qs = a.q[tile.q_kind];
  const float *qp = (const float *)qs.p + b * qs.sb + (int64_t)row * qs.sn + h * qs.sh;
  float q[D], acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = valid ? qp[d] * a.scale : 0.0f;
    acc[d] = 0.0f;
  }
  const int fq = row / a.T;  // frame of the row relative to the chunk (target/source rows)
  float m = -__builtin_inff(), l = 0.0f;
  for (int ri = 0; ri < tile.r_count; ++ri) {
    const DevRange R = a.ranges[tile.r_begin + ri];
    const Seg ks = a.k[R.seg], vs = a.v[R.seg];
    const float *kb = (const float *)ks.p + b * ks.sb + h * ks.sh;
    const float *vb = (const float *)vs.p + b * vs.sb + h * vs.sh;
    int klo = R.begin, khi = R.end;
    if (R.mask == FA_MASK_SAME_FRAME) {
      klo = max(klo, fq * a.T);
      khi = min(khi, (fq + 1) * a.T);
    } else if (R.mask == FA_MASK_GATE && fq < R.param) {
      khi = klo;
    }
    for (int k0 = R.begin; k0 < R.end; k0 += KT) {
      __syncthreads();
      {
        const int j = tid & (KT - 1);
        const int kk = k0 + j;
        const bool in = kk < R.end;
        if (tid < KT) {
          const float *src = kb + (int64_t)kk * ks.sn;
#pragma unroll 8
          for (int d = 0; d < D; ++d) Ks[j][d] = in ? src[d] : 0.0f;
        } else {
          const float *src = vb + (int64_t)kk * vs.sn;
#pragma unroll 8
          for (int d = 0; d < D; ++d) Vs[j][d] = in ? src[d] : 0.0f;
        }
      }
      __syncthreads();
      const int n = min(KT, R.end - k0);
      for (int j = 0; j < n; ++j) {
        const int kidx = k0 + j;
        if (kidx < klo || kidx >= khi) continue;
        float s = 0.0f;
#pragma unroll
        for (int d = 0; d < D; ++d) s = fmaf(q[d], Ks[j][d], s);
        if (s > m) {
          const float alpha = expf(m - s);
          l *= alpha;
#pragma unroll
          for (int d = 0; d < D; ++d) acc[d] *= alpha;
          m = s;
        }
        const float p = expf(s - m);
        l += p;
#pragma unroll
        for (int d = 0; d < D; ++d) acc[d] = fmaf(p, Vs[j][d], acc[d]);
      }
    }
  }
  if (!valid) return;
  const Seg os = a.o[tile.q_kind];
  float *op = (float *)os.p + b * os.sb + (int64_t)row * os.sn + h * os.sh;
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
  for (int d = 0; d < D; ++d) op[d] = acc[d] * inv;
  float *lse = a.lse[tile.q_kind];
  if (lse) lse[(int64_t)w.bh * a.q_rows[tile.q_kind] + row] = l > 0.0f ? m + logf(l) : -__builtin_inff();
}

hipError_t launch_attn_f32(const AttnArgs &a, int head_dim, int grid, hipStream_t s) {
  if (head_dim == 64)
    hipLaunchKernelGGL(attn_f32_kernel<64>, dim3(grid), dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL(attn_f32_kernel<128>, dim3(grid), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace fa
