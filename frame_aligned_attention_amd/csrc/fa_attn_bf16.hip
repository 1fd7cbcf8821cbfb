// fa_attn_bf16.hip -- frame-aligned attention forward, bf16 in/out, gfx950.
//
// The visibility rule ("Vidu S2" tech report, frame-aligned attention and
// causal streaming paragraphs) arrives as a block map: per tile of 128 query
// rows a short list of key ranges (ring runs, chunk, source frames of the
// tile, visible reference images), each with the mask it needs.  The kernel
// walks those ranges in 64-key tiles; keys outside them are never loaded.
//
// Work split.  One workgroup = 4 waves = one query tile of one (batch, head).
// Each wave owns 32 query rows and computes, per key tile,
//   S^T (64 keys x 32 queries) = K_tile . Q^T   with v_mfma_f32_32x32x16_bf16,
// so every lane holds one query column and 32 of its scores: the row max and
// row sum are in-lane, plus one v_permlane32_swap between the two lane halves.
// Then O^T (D x 32) += V^T_tile . P^T, again 32x32x16 MFMAs; P never leaves
// registers because the S^T accumulator already has the B-operand layout of
// the second product, provided V^T is laid out in LDS in the matching key
// order (done when the V tile is staged).
//
// Memory.  K and V tiles are double-buffered in LDS (one barrier per tile);
// the next tile's global loads are issued before the current tile's MFMAs.
// K rows are padded to keep the 16-byte MFMA-operand reads conflict-free;
// V is stored transposed (rows = head_dim channels).  Q stays in VGPRs.
//
// Softmax.  Base-2 online softmax with scale*log2(e) folded into one FMA
// before v_exp_f32.  The running max is only raised when a tile's max
// exceeds it by more than 8 (so p <= 2^8): the O/l rescale is then rare.
#include "fa_internal.h"

namespace fa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float xhalf_max(float x) {
  // v_permlane32_swap exchanges lanes 32..63 of one operand with lanes 0..31 of the other;
  // with both operands = x, the pair holds the two halves' values in every lane.
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xffff0000u);
}

template <int D>
struct Bf16Cfg {
  static constexpr int BM = kBf16BlockM;        // 128 rows, 4 waves
  static constexpr int BN = kBf16BlockN;        // 64 keys per tile
  static constexpr int KSTR = D * 2 + 16;       // LDS bytes per K row
  static constexpr int VSTR = BN * 2 + 16;      // LDS bytes per V^T row
  static constexpr int KBYTES = BN * KSTR;
  static constexpr int BUF = KBYTES + D * VSTR; // one K+V^T buffer
  static constexpr int KCH = BN * D / 8 / 256;  // 16-byte K chunks per thread
  static constexpr int VTASKS = (D / 4) * 8;    // V staging tasks (4 channels x 8 keys each)
};

template <int D>
__global__ void __launch_bounds__(256, 2) attn_bf16_kernel(const AttnArgs a) {
  using Cfg = Bf16Cfg<D>;
  constexpr int BN = Cfg::BN, KSTR = Cfg::KSTR, VSTR = Cfg::VSTR, BUF = Cfg::BUF;
  constexpr float kThr = 8.0f;
  __shared__ __attribute__((aligned(16))) char smem[2 * BUF];

  const DevWork w = a.work[blockIdx.x];
  if (w.tile < 0) return;
  const DevTile tile = a.tiles[w.tile];
  const int b = w.bh / a.H, h = w.bh - (w.bh / a.H) * a.H;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int T = a.T;

  // ---- Q (B operand of S^T): lane holds query row l32 of its wave, channels ds*16 + 8*hl + 0..7
  const int qloc = wave * 32 + l32;
  const bool qvalid = qloc < tile.rows;
  const int qrow = tile.row0 + qloc;
  const Seg qs = a.q[tile.q_kind];
  bf16x8_t qreg[D / 16];
  {
    const __bf16 *qp = (const __bf16 *)qs.p + b * qs.sb + (int64_t)qrow * qs.sn + h * qs.sh;
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
      if (qvalid)
        qreg[ds] = *(const bf16x8_t *)(qp + ds * 16 + 8 * hl);
      else
        qreg[ds] = bf16x8_t{};
    }
  }
  const int fq = qrow / T;  // row frame relative to the chunk (target and source rows)

  // ---- flattened walk over (range, key tile)
  const DevRange *rng = a.ranges + tile.r_begin;
  const int nr = tile.r_count;
  int lr = 0;
  while (lr < nr && rng[lr].begin >= rng[lr].end) ++lr;
  int lk = lr < nr ? rng[lr].begin : 0;

  // staging registers
  uint4 kreg[Cfg::KCH];
  uint2 vreg[8];
  const int dq = tid % (D / 4), vcombo = tid / (D / 4);
  const int vks = vcombo >> 1, vhh = vcombo & 1;

  auto load_tile = [&](int r, int k0) {
    const DevRange R = rng[r];
    const Seg ks = a.k[R.seg], vs = a.v[R.seg];
    const __bf16 *kb = (const __bf16 *)ks.p + b * ks.sb + h * ks.sh;
    const __bf16 *vb = (const __bf16 *)vs.p + b * vs.sb + h * vs.sh;
#pragma unroll
    for (int i = 0; i < Cfg::KCH; ++i) {
      const int c = tid + 256 * i;
      const int key = c / (D / 8), col = c % (D / 8);
      const int kidx = k0 + key;
      if (kidx < R.end)
        kreg[i] = *(const uint4 *)(kb + (int64_t)kidx * ks.sn + col * 8);
      else
        kreg[i] = uint4{0, 0, 0, 0};
    }
    if (tid < Cfg::VTASKS) {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int key = vks * 16 + (s >> 2) * 8 + 4 * vhh + (s & 3);
        const int kidx = k0 + key;
        if (kidx < R.end)
          vreg[s] = *(const uint2 *)(vb + (int64_t)kidx * vs.sn + dq * 4);
        else
          vreg[s] = uint2{0, 0};
      }
    }
  };

  auto store_tile = [&](int buf) {
    char *Kl = smem + buf * BUF;
    char *Vl = Kl + Cfg::KBYTES;
#pragma unroll
    for (int i = 0; i < Cfg::KCH; ++i) {
      const int c = tid + 256 * i;
      const int key = c / (D / 8), col = c % (D / 8);
      *(uint4 *)(Kl + key * KSTR + col * 16) = kreg[i];
    }
    if (tid < Cfg::VTASKS) {
      // V^T row d holds, at positions ks*16 + 8*hh + s, the keys ks*16 + (s/4)*8 + 4*hh + s%4:
      // exactly the keys lane half hh holds in P^T slots s for key slice ks.
      char *dst = Vl + (dq * 4) * VSTR + (vks * 16 + 8 * vhh) * 2;
      uint4 o0, o1, o2, o3;
      o0.x = pack_lo(vreg[0].x, vreg[1].x); o0.y = pack_lo(vreg[2].x, vreg[3].x);
      o0.z = pack_lo(vreg[4].x, vreg[5].x); o0.w = pack_lo(vreg[6].x, vreg[7].x);
      o1.x = pack_hi(vreg[0].x, vreg[1].x); o1.y = pack_hi(vreg[2].x, vreg[3].x);
      o1.z = pack_hi(vreg[4].x, vreg[5].x); o1.w = pack_hi(vreg[6].x, vreg[7].x);
      o2.x = pack_lo(vreg[0].y, vreg[1].y); o2.y = pack_lo(vreg[2].y, vreg[3].y);
      o2.z = pack_lo(vreg[4].y, vreg[5].y); o2.w = pack_lo(vreg[6].y, vreg[7].y);
      o3.x = pack_hi(vreg[0].y, vreg[1].y); o3.y = pack_hi(vreg[2].y, vreg[3].y);
      o3.z = pack_hi(vreg[4].y, vreg[5].y); o3.w = pack_hi(vreg[6].y, vreg[7].y);
      *(uint4 *)(dst + 0 * VSTR) = o0;
      *(uint4 *)(dst + 1 * VSTR) = o1;
      *(uint4 *)(dst + 2 * VSTR) = o2;
      *(uint4 *)(dst + 3 * VSTR) = o3;
    }
  };

  auto advance = [&](int &r, int &k) {
    k += BN;
    if (k >= rng[r].end) {
      ++r;
      while (r < nr && rng[r].begin >= rng[r].end) ++r;
      k = r < nr ? rng[r].begin : 0;
    }
  };

  f32x16_t oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16_t{};
  float m_run = -__builtin_inff();
  float l_part = 0.0f;
  const float c = a.c;

  if (lr < nr) {
    load_tile(lr, lk);
    store_tile(0);
    __syncthreads();
    int cr = lr, ck = lk;
    advance(lr, lk);
    int buf = 0;
    while (true) {
      const bool has_next = lr < nr;
      if (has_next) load_tile(lr, lk);

      // ---- S^T = K . Q^T for 64 keys (two 32-key blocks)
      const char *Kl = smem + buf * BUF;
      const char *Vl = Kl + Cfg::KBYTES;
      f32x16_t s0 = f32x16_t{}, s1 = f32x16_t{};
#pragma unroll
      for (int ds = 0; ds < D / 16; ++ds) {
        const bf16x8_t a0 = *(const bf16x8_t *)(Kl + l32 * KSTR + (ds * 16 + 8 * hl) * 2);
        const bf16x8_t a1 = *(const bf16x8_t *)(Kl + (32 + l32) * KSTR + (ds * 16 + 8 * hl) * 2);
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qreg[ds], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qreg[ds], s1, 0, 0, 0);
      }

      // ---- mask (partial tiles and masked ranges only).  s{kb}[r] is key
      // ck + kb*32 + (r/4)*8 + 4*hl + r%4 for this lane's query.
      const DevRange R = rng[cr];
      if (R.mask != FA_MASK_NONE || ck + BN > R.end) {
        int klo = R.begin, khi = R.end;
        if (R.mask == FA_MASK_SAME_FRAME) {
          klo = max(klo, fq * T);
          khi = min(khi, (fq + 1) * T);
        } else if (R.mask == FA_MASK_GATE && fq < R.param) {
          khi = klo;
        }
        const int base = ck + 4 * hl;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int k0i = base + (r >> 2) * 8 + (r & 3);
          const int k1i = k0i + 32;
          if (k0i < klo || k0i >= khi) s0[r] = -__builtin_inff();
          if (k1i < klo || k1i >= khi) s1[r] = -__builtin_inff();
        }
      }

      // ---- online softmax (base 2, lazy rescale)
      float mx = s0[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s0[r]);
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s1[r]);
      mx = xhalf_max(mx);
      const float mt = mx * c;
      const bool need = mt > m_run + kThr;
      if (__builtin_amdgcn_ballot_w64(need) != 0) {
        const float alpha = need ? __builtin_amdgcn_exp2f(m_run - mt) : 1.0f;
        if (need) m_run = mt;
        l_part *= alpha;
#pragma unroll
        for (int i = 0; i < D / 32; ++i) oacc[i] *= alpha;
      }
      const float mneg = m_run == -__builtin_inff() ? 0.0f : -m_run;
      bf16x8_t p[4];  // P^T operands for the four 16-key slices
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e0 = __builtin_amdgcn_exp2f(fmaf(s0[r], c, mneg));
        const float e1 = __builtin_amdgcn_exp2f(fmaf(s1[r], c, mneg));
        l_part += e0 + e1;
        p[r >> 3][r & 7] = (__bf16)e0;
        p[2 + (r >> 3)][r & 7] = (__bf16)e1;
      }

      // ---- O^T += V^T . P^T
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const bf16x8_t av =
              *(const bf16x8_t *)(Vl + (db * 32 + l32) * VSTR + (ks * 16 + 8 * hl) * 2);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, p[ks], oacc[db], 0, 0, 0);
        }
      }

      if (has_next) store_tile(buf ^ 1);
      __syncthreads();
      if (!has_next) break;
      cr = lr;
      ck = lk;
      advance(lr, lk);
      buf ^= 1;
    }
  }

  // ---- epilogue: O = O^T / l, LSE = (m + log2 l) * ln 2
  const float l_tot = xhalf_sum(l_part);
  if (!qvalid) return;
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  const Seg os = a.o[tile.q_kind];
  __bf16 *op = (__bf16 *)os.p + b * os.sb + (int64_t)qrow * os.sn + h * os.sh;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
      bf16x4_t v;
      v[0] = (__bf16)(oacc[db][g * 4 + 0] * inv);
      v[1] = (__bf16)(oacc[db][g * 4 + 1] * inv);
      v[2] = (__bf16)(oacc[db][g * 4 + 2] * inv);
      v[3] = (__bf16)(oacc[db][g * 4 + 3] * inv);
      *(bf16x4_t *)(op + db * 32 + g * 8 + 4 * hl) = v;
    }
  }
  float *lse = a.lse[tile.q_kind];
  if (lse && hl == 0)
    lse[(int64_t)w.bh * a.q_rows[tile.q_kind] + qrow] =
        l_tot > 0.0f ? (m_run + __log2f(l_tot)) * 0.6931471805599453f : -__builtin_inff();
}

hipError_t launch_attn_bf16(const AttnArgs &a, int head_dim, int grid, hipStream_t s) {
  if (head_dim == 64)
    hipLaunchKernelGGL(attn_bf16_kernel<64>, dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(attn_bf16_kernel<128>, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace fa
