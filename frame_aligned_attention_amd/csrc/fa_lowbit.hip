// fa_lowbit.hip -- the low-bit frame-aligned attention path for gfx950: the
// quantiser (per-head key mean, per-128-token-block int8 Q/K and e4m3 V) and the
// attention kernel with int8 Q.K^T (v_mfma_i32_32x32x32_i8) and e4m3 P.V
// (v_mfma_scale_f32_32x32x64_f8f6f4), fp32 online softmax.
// build-flags: -fno-honor-nans
// (Finite inputs give no NaN here; without the flag every row max first quiets the
// scores it compares, 4 more VALU instructions per tile.)
//
// The pages name low-bit attention only ("Vidu S2" launch article, technical
// stack section; tech report, hybrid-attention paragraph).  What it computes here:
//  - K is reduced by one per-(batch, head) channel mean m of the call's keys;
//    the softmax does not change (q.m is constant along a row);
//  - Q and K: symmetric int8 per (batch, head, 128-token block), scale
//    absmax/127, code = round_half_even(x * (127/absmax));
//  - V: OCP e4m3 per block with a power-of-two scale 2^e, the smallest with
//    448 * 2^e >= absmax (so the largest code lies in (224, 448]), codes
//    x * 2^-e rounded to nearest even by v_cvt_pk_fp8_f32;
//  - scores s = (q8 . k8) * sq * sk * softmax_scale, online softmax in fp32
//    with p = 2^(s*log2e - m);
//  - P.V in e4m3: p' = p * 2^8 <= 256 (exact running max), and
//    each tile's V block scale 2^e is applied by the MFMA's e8m0 scale of V;
//    O = sum(2^e p' v8) / l with l = sum(p') taken by an MFMA on the same e4m3
//    p' (numerator and denominator weigh every key alike).
// Key tiles never straddle a 128-token block (a range's first tile ends at the
// next 64-key boundary), so K and V scales are uniform per tile.
#include "fa_device.h"

namespace fa {

typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// ============================================================== quantiser

__global__ void __launch_bounds__(64) quant_init_kernel(float *v_absmax, int n) {
  const int i = blockIdx.x * 64 + threadIdx.x;
  if (i < n) v_absmax[i] = 0.0f;
}

// Per-(batch, head) channel mean of the keys in view.  kMeanSplit workgroups of 1024 threads
// per (b, h), each over 128/kMeanSplit channels: LPR lanes read a token row's slice (16 bytes
// each), SLOTS row slots walk the tokens with four loads in flight per lane, each lane sums its
// 8 channels in fp32 in a fixed order, then a fixed-order tree over the row slots:
// deterministic.
constexpr int kMeanThreads = 1024;
constexpr int kMeanSplit = 4;
__global__ void __launch_bounds__(kMeanThreads) kmean_kernel(const QuantArgs a) {
  constexpr int CPW = 128 / kMeanSplit;  // channels per workgroup
  constexpr int LPR = CPW / 8;           // lanes per token row
  constexpr int SLOTS = kMeanThreads / LPR;
  const int bh = blockIdx.x / kMeanSplit, c0 = (blockIdx.x % kMeanSplit) * CPW;
  const int b = bh / a.H, h = bh % a.H;
  const int t = threadIdx.x, lanec = t % LPR, slot = t / LPR;
  const int ch = c0 + lanec * 8;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int count = 0;
  for (int si = 0; si < a.nseg; ++si) {
    const QSeg &g = a.seg[si];
    if (g.kind != 1) continue;
    for (int run = 0; run < 2; ++run) {
      const int lo = run ? g.lo1 : g.lo0, hi = run ? g.hi1 : g.hi0;
      if (hi <= lo) continue;
      count += hi - lo;
      const __bf16 *base = (const __bf16 *)g.in + b * g.isb + h * g.ish + ch;
      int tok = lo + slot;
      for (; tok + 3 * SLOTS < hi; tok += 4 * SLOTS) {
        bf16x8_t v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          v[u] = *(const bf16x8_t *)(base + (int64_t)(tok + u * SLOTS) * g.isn);
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] += (float)v[u][i];
      }
      for (; tok < hi; tok += SLOTS) {
        const bf16x8_t v = *(const bf16x8_t *)(base + (int64_t)tok * g.isn);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += (float)v[i];
      }
    }
  }
  // red[slot][channel of the slice]; slots summed pairwise in a fixed order
  __shared__ float red[SLOTS][CPW + 1];
#pragma unroll
  for (int i = 0; i < 8; ++i) red[slot][lanec * 8 + i] = acc[i];
  __syncthreads();
  for (int w = SLOTS / 2; w > 0; w >>= 1) {
    for (int e = t; e < w * CPW; e += kMeanThreads) {
      const int s_ = e / CPW, c = e % CPW;
      red[s_][c] += red[s_ + w][c];
    }
    __syncthreads();
  }
  if (t < CPW) a.k_mean[(int64_t)bh * a.D + c0 + t] = count ? red[0][t] / (float)count : 0.0f;
}

__device__ __forceinline__ bool in_runs(const QSeg &g, int tok) {
  return (tok >= g.lo0 && tok < g.hi0) || (tok >= g.lo1 && tok < g.hi1);
}

// One workgroup per (tensor, 128-token block, batch, head).  16 lanes cover the 256 bytes of a
// token row (8 channels each), so a wave reads 4 whole rows per load; 16 rows per pass, 8
// passes per block.
__global__ void __launch_bounds__(256) quant_kernel(const QuantArgs a) {
  // heads vary fastest along the grid: workgroups running together read neighbouring pieces of
  // the same token rows
  const int nbh = a.batch * a.H;
  const int bh = blockIdx.x % nbh, flat = blockIdx.x / nbh;
  const int b = bh / a.H, h = bh % a.H;
  int si = 0;
  while (si + 1 < a.nseg && a.seg[si + 1].blk_begin <= flat) ++si;
  const QSeg &g = a.seg[si];
  const int blk = g.blk0 + (flat - g.blk_begin);
  const int t = threadIdx.x, lane16 = t & 15, rsub = t >> 4;
  if (g.kind == 3) {  // codes made earlier: only their scale counts towards v_absmax
    if (t == 0)
      atomicMax((unsigned int *)(a.v_absmax + bh),
                __float_as_uint(g.scale[(int64_t)bh * g.nblk + blk]));
    return;
  }
  const int c0 = lane16 * 8;
  const bool need_m = g.kind == 1 || (g.kind == 0 && g.lse);
  float m[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) m[i] = need_m ? a.k_mean[(int64_t)bh * a.D + c0 + i] : 0.0f;
  float x[8][8];
  bool live[8];
  float amax = 0.0f;
  // The eight row loads go out together: a row outside the runs reads row min(tok, n - 1), which
  // lies inside the tensor, and its values are dropped.  (Loads under a per-row branch were
  // issued one at a time, each waited for before the next.)
  const __bf16 *in_bh = (const __bf16 *)g.in + b * g.isb + h * g.ish + c0;
  bf16x8_t v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int tok = blk * 128 + j * 16 + rsub;
    live[j] = in_runs(g, tok);
    v[j] = *(const bf16x8_t *)(in_bh + (int64_t)min(tok, g.n - 1) * g.isn);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float e = g.kind == 1 ? (float)v[j][i] - m[i] : (float)v[j][i];
      x[j][i] = live[j] ? e : 0.0f;
      amax = fmaxf(amax, fabsf(x[j][i]));
    }
  }
  if (g.kind == 0 && g.lse) {
    // the LSE the kernel computes is that of the smoothed scores q.(k - m); record the
    // per-row shift scale * q.m, which the attention kernel adds back
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float dot = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) dot = fmaf(x[j][i], m[i], dot);
      dot += __shfl_xor(dot, 8);
      dot += __shfl_xor(dot, 4);
      dot += __shfl_xor(dot, 2);
      dot += __shfl_xor(dot, 1);
      if (live[j] && lane16 == 0)
        g.lse[(int64_t)bh * g.n + blk * 128 + j * 16 + rsub] = a.softmax_scale * dot;
    }
  }
  // block absmax: across the wave, then across the four waves
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  __shared__ float red[4];
  if ((t & 63) == 0) red[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float scale, inv;
  if (g.kind == 2) {
    // V: the smallest power of two 2^e (e >= -126) with 448 * 2^e >= amax.  For amax =
    // 1.f * 2^(E - 127) that is e = E - 135, plus one when 1.f > 1.75; a subnormal amax takes
    // the floor.  Codes x * 2^-e are exact scalings before the e4m3 rounding.
    const uint32_t bits = __float_as_uint(amax);
    const int e = max((int)(bits >> 23) - 135 + ((bits & 0x7fffffu) > 0x600000u ? 1 : 0), -126);
    scale = amax > 0.0f ? __uint_as_float((uint32_t)(e + 127) << 23) : 0.0f;
    inv = amax > 0.0f ? __uint_as_float((uint32_t)(127 - e) << 23) : 0.0f;
  } else {
    scale = amax / 127.0f;
    inv = amax > 0.0f ? 127.0f / amax : 0.0f;
  }
  if (t == 0) {
    g.scale[(int64_t)bh * g.nblk + blk] = scale;
    if (g.kind == 2 && a.v_absmax)
      atomicMax((unsigned int *)(a.v_absmax + bh), __float_as_uint(scale));
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (!live[j]) continue;
    uint32_t w32[2];
    if (g.kind == 2) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        int v = __builtin_amdgcn_cvt_pk_fp8_f32(x[j][4 * k] * inv, x[j][4 * k + 1] * inv, 0, false);
        v = __builtin_amdgcn_cvt_pk_fp8_f32(x[j][4 * k + 2] * inv, x[j][4 * k + 3] * inv, v, true);
        w32[k] = (uint32_t)v;
      }
    } else {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        uint32_t v = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float r = fminf(fmaxf(__builtin_rintf(x[j][4 * k + i] * inv), -127.0f), 127.0f);
          v |= ((uint32_t)(int)r & 0xffu) << (8 * i);
        }
        w32[k] = v;
      }
    }
    const int tok = blk * 128 + j * 16 + rsub;
    char *o = (char *)g.out + b * g.osb + (int64_t)tok * g.osn + h * g.osh + c0;
    *(uint2 *)o = uint2{w32[0], w32[1]};
  }
}

hipError_t launch_quant_lowbit(const QuantArgs &a, bool mean_given, hipStream_t s) {
  const int nbh = a.batch * a.H;
  if (a.v_absmax)
    hipLaunchKernelGGL(quant_init_kernel, dim3((nbh + 63) / 64), dim3(64), 0, s, a.v_absmax, nbh);
  if (!mean_given)
    hipLaunchKernelGGL(kmean_kernel, dim3(nbh * kMeanSplit), dim3(kMeanThreads), 0, s, a);
  if (a.total_blocks > 0)
    hipLaunchKernelGGL(quant_kernel, dim3(nbh * a.total_blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ============================================================== attention

namespace lb {
constexpr int D = 128;
constexpr int BN = 64;                          // keys per tile
constexpr int ROWB = D;                         // bytes per K/V row (1-byte codes)
constexpr int CH = ROWB / 16;                   // 16-byte chunks per row (8)
constexpr int TILEB = BN * ROWB;                // 8 KB
constexpr int LOADS = TILEB / (256 * 16);       // 2 direct loads per thread per tile
// Chunk c of row r lives at chunk c ^ sw(r), sw(r) = (bit 2, bit 1, bit 3 of r) as bits 0..2.
// LDS serves 256 bytes a cycle (64 banks): 16 lanes of a ds_read_b128, 32 lanes of a ds_read_b64.
// A K read (16 lanes = 16 consecutive rows, one chunk each) needs sw to be one-to-one on the 8
// rows of each parity, which holds as it is one-to-one on bits 1..3.  A transposing V read (32
// lanes = rows {a, a+2, a+8, a+10} for two row parities, chunk pairs c, c^1) needs sw >> 1 to be
// one-to-one on bits 1 and 3, which it is.  Both reads are then free of bank conflicts.
__device__ __forceinline__ int sw(int r) { return ((r >> 2) & 1) | (r & 2) | ((r >> 1) & 4); }
}  // namespace lb

// Work split as in the bf16 kernels: 4 waves of 32 query rows per 128-row work item, keys as the M
// dimension.  Per 64-key tile: S^T = K Q^T on 8 int8 MFMAs, softmax, O^T += V^T P^T on 4 e4m3
// MFMAs and the row sums on one more.  The loads of tile j+1 go out at the start of step j into
// the other LDS buffers; the step itself runs S, softmax and PV of tile j in order.  Two
// workgroups share a CU (32 KB of LDS each); the waves of the other one fill each wave's
// dependency gaps.
//
// Most of what a wave issues per tile is the softmax's VALU work, so three things cut it:
//  - the int32 score accumulators start at the bits of the float kBias = 1.5 * 2^23: |q.k| <=
//    128 * 127^2 < 2^22, so the sum's bits read as the float kBias + q.k exactly and no integer
//    to float conversion is needed; kBias * fk is folded into the exp FMA (that term rounds
//    once per tile, to under one unit of the integer score, far below the int8 rounding of q.k);
//  - V block scales are powers of two, applied by the PV MFMA's own e8m0 block scale, so every
//    tile takes p' = p * 2^8 with no per-tile weight;
//  - the row sums of p' come from a 16x16x128 e4m3 MFMA of a ones pattern against P^T (the same
//    e4m3 values the PV product uses), not from 32 adds.
// The running max is raised only when a row's max passes it by more than kThr = 0.75, so p' stays
// below 2^8.75 ~ 430, under e4m3's 448, and most tiles past the first skip the rescale (with an
// exact max some row of the wave sets a new one on a large share of tiles).  Values only get
// larger than under the exact max, never closer to e4m3's subnormals; a lazier max with a
// smaller shift (p' = p 2^6, raised past +2) cost accuracy on small rows.
__global__ void __launch_bounds__(256, 2) attn_lowbit_kernel(const AttnArgs a) {
  using namespace lb;
  constexpr int kBiasBits = 0x4B400000;
  constexpr float kBias = 12582912.0f;
  constexpr float kThr = 0.75f;
  constexpr float kPShift = 8.0f;  // p' = p * 2^kPShift < 2^(8 + kThr) ~ 430 < 448
  __shared__ __attribute__((aligned(1024))) char kbuf0[TILEB];
  __shared__ __attribute__((aligned(1024))) char kbuf1[TILEB];
  __shared__ __attribute__((aligned(1024))) char vbuf0[TILEB];
  __shared__ __attribute__((aligned(1024))) char vbuf1[TILEB];

  const DevWork w = cload<DevWork>((const cWork *)a.work + blockIdx.x);
  if (w.tile < 0) return;
  const DevTile tile = cload<DevTile>((const cTile *)a.tiles + w.tile);
  const int b = w.bh / a.H, h = w.bh - (w.bh / a.H) * a.H;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int T = a.T;

  // ---- Q codes (B operand of S^T): lane holds row l32 of its wave, channels ds*32 + 16*hl + 0..15
  const int qloc = wave * 32 + l32;
  const bool qvalid = qloc < tile.rows;
  const int qrow = tile.row0 + qloc;
  const Seg qs = a.q[tile.q_kind];
  i32x4_t qreg[4];
  {
    const char *qp = (const char *)qs.p + b * qs.sb + (int64_t)qrow * qs.sn + h * qs.sh;
#pragma unroll
    for (int ds = 0; ds < 4; ++ds)
      qreg[ds] = qvalid ? *(const i32x4_t *)(qp + ds * 32 + 16 * hl) : i32x4_t{0, 0, 0, 0};
  }
  // Q tiles are 128-row aligned: one Q block per workgroup
  const float sq = *((const cFloat *)qs.scale + (int64_t)w.bh * qs.nblk + tile.row0 / 128);
  const float cq = sq * a.c;  // times sk gives the log2-domain scale of an int score
  const int fq = qrow / T;

  // ---- LDS read offsets
  const int koff0 = l32 * ROWB + ((hl ^ sw(l32)) * 16);  // k-step ds at koff0 ^ (ds << 5)
  // V^T operand via ds_read_b64_tr_b8: in 16-lane group g, lane i reads 8 bytes of row
  // key(g/2, 8t + i/2), channels db*32 + (g%2)*16 + 8*(i%2) .. +7, for t = 0..3.
  int voff0;  // block db, key slice t at (voff0 ^ (db << 5)) + 16 t rows
  {
    const int i = lane & 15, g = lane >> 4;
    const int hv = g >> 1, gh = g & 1, sp = i >> 1, u = i & 1;
    const int row = (sp >> 2) * 8 + 4 * hv + (sp & 3);
    voff0 = row * ROWB + ((gh ^ sw(row)) * 16) + 8 * u;
  }
  int lrow[LOADS], lcb[LOADS];
#pragma unroll
  for (int j = 0; j < LOADS; ++j) {
    const int p = (4 * j + wave) * 64 + lane;
    lrow[j] = p / CH;
    lcb[j] = ((p % CH) ^ sw(lrow[j])) * 16;
  }

  // ---- cursors: tiles never straddle a 128-token block; a range's first tile runs to the next
  // 64-key boundary, the following ones are aligned
  const cRange *rng = (const cRange *)a.ranges + tile.r_begin;
  const int nr = tile.r_count;
  struct Cur {
    int r, k, kend, begin, end, mask, param, seg;
    uint64_t base, vbase;  // byte addresses of (b, key 0, h) of the range's K and V codes
    uint32_t sn, vsn;      // bytes between consecutive keys of K and of V
  };
  auto set_end = [&](Cur &c) { c.kend = min(c.end, (c.k & ~(BN - 1)) + BN); };
  auto enter = [&](Cur &c, int r) {
    while (r < nr && rng[r].begin >= rng[r].end) ++r;
    c.r = r;
    if (r >= nr) return;
    const DevRange R = cload<DevRange>(rng + r);
    c.k = c.begin = R.begin;
    c.end = R.end;
    c.mask = R.mask;
    c.param = R.param;
    c.seg = R.seg;
    set_end(c);
    const Seg ks = a.k[R.seg], vs = a.v[R.seg];
    c.base = (uint64_t)ks.p + (uint64_t)((int64_t)b * ks.sb + (int64_t)h * ks.sh);
    c.sn = (uint32_t)ks.sn;
    c.vbase = (uint64_t)vs.p + (uint64_t)((int64_t)b * vs.sb + (int64_t)h * vs.sh);
    c.vsn = (uint32_t)vs.sn;
  };
  auto next = [&](Cur &c) {
    if (c.r >= nr) return;
    c.k = c.kend;
    if (c.k >= c.end)
      enter(c, c.r + 1);
    else
      set_end(c);
  };
  // buffer descriptors of the K and V codes of the tile at cursor c; past the last range they
  // are empty (their loads return zeros into a buffer nobody reads again)
  auto tile_rsrc = [&](const Cur &c, uint64_t base, uint32_t sn) {
    const bool live = c.r < nr;
    const uint64_t ub = base + (uint64_t)(uint32_t)c.k * sn;
    return make_rsrc(ub, live ? (int)((c.kend - c.k) * sn) : 0);
  };
  auto load_one = [&](__amdgpu_buffer_rsrc_t rs, uint32_t sn, char *buf, int j) {
    const uint32_t off = (uint32_t)lrow[j] * sn + lcb[j];
    lds_char *dst = (lds_char *)buf + (4 * j + wave) * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)dst, 16,
                                             (int)off, 0, 0, 0);
  };
  auto issue = [&](const Cur &c, char *kbuf, char *vbuf) {
    const __amdgpu_buffer_rsrc_t rk = tile_rsrc(c, c.base, c.sn), rv = tile_rsrc(c, c.vbase, c.vsn);
#pragma unroll
    for (int j = 0; j < LOADS; ++j) load_one(rk, c.sn, kbuf, j);
#pragma unroll
    for (int j = 0; j < LOADS; ++j) load_one(rv, c.vsn, vbuf, j);
  };
  // per-tile scales of the tile at cursor c: log2-domain score factor, and the V block scale
  // 2^e as its e8m0 code e + 127 (the float's exponent field; 0 for an all-zero block, whose
  // codes are 0)
  auto tile_scales = [&](const Cur &c, float &fk, int &ve8) {
    const Seg ks = a.k[c.seg], vs = a.v[c.seg];
    const int blk = c.k >> 7;
    const float sk = *((const cFloat *)ks.scale + (int64_t)w.bh * ks.nblk + blk);
    const float sv = *((const cFloat *)vs.scale + (int64_t)w.bh * vs.nblk + blk);
    fk = fmaxf(cq * sk, 1e-30f);  // an all-zero Q or K block: scores 0, masks stay -inf
    ve8 = (int)((__float_as_uint(sv) >> 23) & 0xffu);
  };

  f32x16_t oacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) oacc[i] = f32x16_t{};
  // finite start: the first tile with a visible key always raises it (a row with none keeps
  // l = 0, its exp arguments all -inf)
  float m_run = -1e30f;
  // Row sums: D of v_mfma_scale_f32_16x16x128_f8f6f4 with A = a ones pattern and B = P^T.  Lane l
  // of P^T holds query l % 32 (32 of its 64 keys; lane l + 32 the others), and a 16x16x128
  // product pairs lane 16g + i of A with lane 16g + j of B over the same 32 bytes.  A row 0 of
  // ones on the lanes of groups g = 0, 2 and a row 1 on groups 1, 3 make D[0][j] the sum of
  // query j and D[1][j] that of query j + 16: lanes 0-15 hold them in lacc[0] and lacc[1].
  f32x4_t lacc = f32x4_t{};
  i32x8_t ones;
  {
    const int g16 = lane >> 4, i16 = lane & 15;
    const int ov = i16 == (g16 & 1) ? 0x38383838 : 0;  // e4m3 1.0 = 0x38
#pragma unroll
    for (int i = 0; i < 8; ++i) ones[i] = ov;
  }
  i32x16_t sbias;
#pragma unroll
  for (int i = 0; i < 16; ++i) sbias[i] = kBiasBits;

  auto qk = [&](const char *kbuf, i32x16_t &s0, i32x16_t &s1) {
    const lds_char *Kl = (const lds_char *)kbuf;
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) {
      const i32x4_t a0 = *(const i32x4_t *)(Kl + (koff0 ^ (ds << 5)));
      const i32x4_t a1 = *(const i32x4_t *)(Kl + 32 * ROWB + (koff0 ^ (ds << 5)));
      s0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, qreg[ds], ds == 0 ? sbias : s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, qreg[ds], ds == 0 ? sbias : s1, 0, 0, 0);
    }
  };

  // softmax + PV of the tile at cursor c with scores (s0, s1) and V in `vbuf`
  auto softmax_pv = [&](const Cur &c, const i32x16_t &s0, const i32x16_t &s1, const char *vbuf) {
    float fk;
    int ve8;
    tile_scales(c, fk, ve8);
    float x0[16], x1[16];  // kBias + score, exactly
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      x0[i] = __builtin_bit_cast(float, (int)s0[i]);
      x1[i] = __builtin_bit_cast(float, (int)s1[i]);
    }
    if (c.mask != FA_MASK_NONE || c.kend - c.k < BN) {
      int klo = c.begin, khi = c.kend;
      if (c.mask == FA_MASK_SAME_FRAME) {
        klo = max(klo, fq * T);
        khi = min(khi, (fq + 1) * T);
      } else if (c.mask == FA_MASK_GATE && fq < c.param) {
        khi = klo;
      }
      const int base = c.k + 4 * hl;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int k0i = base + (i >> 2) * 8 + (i & 3);
        const int k1i = k0i + 32;
        if (k0i < klo || k0i >= khi) x0[i] = -__builtin_inff();
        if (k1i < klo || k1i >= khi) x1[i] = -__builtin_inff();
      }
    }
    float mx = fmaxf(x0[0], x0[1]);
#pragma unroll
    for (int i = 2; i < 16; ++i) mx = fmaxf(mx, x0[i]);
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, x1[i]);
    mx = xhalf_max(mx);
    const float mt = (mx - kBias) * fk;  // the difference is exact; fk > 0; -inf stays -inf
    // the new max, the exp of alpha and the rescale only in the branch, taken when some row's
    // max grew
    const bool need = mt > m_run + kThr;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      const float alpha = need ? __builtin_amdgcn_exp2f(m_run - mt) : 1.0f;
      m_run = need ? mt : m_run;
#pragma unroll
      for (int i = 0; i < 4; ++i) oacc[i] *= alpha;
      // lanes 0-15 hold the sums of queries l and l + 16: the latter's alpha from lane l + 16
      const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(alpha), __float_as_uint(alpha),
                                                      false, false);
      lacc[0] *= alpha;
      lacc[1] *= __uint_as_float(r[1]);
    }
    // exp2 argument s fk - m + kPShift, with s fk = (kBias + s) fk - kBias fk
    const float mneg = (kPShift - m_run) - kBias * fk;
    i32x8_t pw;  // P^T: byte kb*16 + r of the lane's 32 keys
#pragma unroll
    for (int i = 0; i < 16; i += 4) {
      float e[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        e[j] = __builtin_amdgcn_exp2f(fmaf(x0[i + j], fk, mneg));
        e[4 + j] = __builtin_amdgcn_exp2f(fmaf(x1[i + j], fk, mneg));
      }
      // each packing writes one half of its word and keeps the other: the first of a pair is
      // seeded with a dead register instead of a zero
      const int o0 = __builtin_bit_cast(int, e[0]), o1 = __builtin_bit_cast(int, e[4]);
      int v = __builtin_amdgcn_cvt_pk_fp8_f32(e[0], e[1], o0, false);
      pw[i / 4] = __builtin_amdgcn_cvt_pk_fp8_f32(e[2], e[3], v, true);
      v = __builtin_amdgcn_cvt_pk_fp8_f32(e[4], e[5], o1, false);
      pw[4 + i / 4] = __builtin_amdgcn_cvt_pk_fp8_f32(e[6], e[7], v, true);
    }
    const lds_char *Vl = (const lds_char *)vbuf;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      i32x8_t av;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const i32x2_t r2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) i32x2_t *)(Vl + (voff0 ^ (db << 5)) + t * 16 * ROWB));
        av[2 * t] = r2[0];
        av[2 * t + 1] = r2[1];
      }
      // V's block scale rides on the A operand's e8m0 scale
      oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, pw, oacc[db], 0, 0, 0, ve8, 0,
                                                                 127);
    }
    lacc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones, pw, lacc, 0, 0, 0, 127, 0, 127);
  };

  auto end_step = [&]() {
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };

  // One cursor walks the tiles for the loads (tile j+1 during step j); the tile of the step
  // itself (mask, scales) is a copy taken before each advance.
  Cur cc, ck;
  enter(ck, 0);
  if (ck.r < nr) {
    cc = ck;
    issue(ck, kbuf0, vbuf0);
    next(ck);
    end_step();
    i32x16_t s0, s1;
    while (true) {
      if (ck.r < nr) issue(ck, kbuf1, vbuf1);
      qk(kbuf0, s0, s1);
      softmax_pv(cc, s0, s1, vbuf0);
      end_step();
      if (ck.r >= nr) break;
      cc = ck;
      next(ck);
      if (ck.r < nr) issue(ck, kbuf0, vbuf0);
      qk(kbuf1, s0, s1);
      softmax_pv(cc, s0, s1, vbuf1);
      end_step();
      if (ck.r >= nr) break;
      cc = ck;
      next(ck);
    }
  }

  // ---- epilogue: O = O^T / l, LSE = (m + log2 l - kPShift) * ln 2, l = sum p' of the query
  const float ls0 = __shfl(lacc[0], l32 & 15), ls1 = __shfl(lacc[1], l32 & 15);
  const float l_tot = l32 < 16 ? ls0 : ls1;
  if (!qvalid) return;
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  const Seg os = a.o[tile.q_kind];
  __bf16 *op = (__bf16 *)os.p + b * os.sb + (int64_t)qrow * os.sn + h * os.sh;
#pragma unroll
  for (int db = 0; db < 4; ++db) {
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
  if (lse && hl == 0) {
    // lse holds the smoothing shift scale * q.m written by the quantiser
    float *lp = lse + (int64_t)w.bh * a.q_rows[tile.q_kind] + qrow;
    *lp = l_tot > 0.0f ? (m_run + __log2f(l_tot) - kPShift) * 0.6931471805599453f + *lp
                       : -__builtin_inff();
  }
}

hipError_t launch_attn_lowbit(const AttnArgs &a, int head_dim, int grid, hipStream_t s) {
  if (head_dim != 128) return hipErrorInvalidValue;
  hipLaunchKernelGGL(attn_lowbit_kernel, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace fa
