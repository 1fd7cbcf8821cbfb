// fa_w8a8.hip -- per-block W8A8 linear layer for gfx950: y = x . w^T with int8 activations
// (one fp32 scale per row and 128-column block) and int8 weights (one fp32 scale per 128 x 128
// block), as the tech report's paragraph on linear layers describes (fine-grained block scales
// keep an outlier from setting the range of a whole tensor or channel).
//
// Quantisers: scale = absmax/127, code = round_half_even(x * (127/absmax)) clamped to +-127,
// the same arithmetic as the attention path's quantiser.
//
// GEMM.  One workgroup (8 waves, one per CU) per 256 (m) x 128 (n) output tile.  Every
// 128-column K-block is one quantisation block: the int32 products of its four 32-deep k-steps
// accumulate in the MFMA (v_mfma_i32_32x32x32_i8, exact), then are dequantised into fp32
// accumulators with the block's two scales.  The product is computed as y^T = w . x^T (weights
// as the A operand), so each lane's output column is one activation row: the activation scale
// is one register per 32-row tile and the weight scale is uniform per workgroup.  Operand tiles
// go straight from HBM into a 3-stage LDS ring (direct loads, bounds-checked descriptors
// zero-fill rows past m), rows XOR-swizzled in 16-byte chunks for conflict-free MFMA operand
// reads; a K-block's loads have two steps to land.  The two waves on each SIMD ping-pong: one
// multiplies a block while the other dequantises.
#include "fa_device.h"

namespace fa {

typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

// ============================================================== quantisers

// Activations: 16 lanes per (row, 128-column block), 8 values each; 16 blocks per workgroup.
__global__ void __launch_bounds__(256) w8a8_quant_act_kernel(const W8QuantArgs a) {
  const int grp = blockIdx.x * 16 + (threadIdx.x >> 4), l16 = threadIdx.x & 15;
  const int kbt = a.cols / 128;
  const int row = grp / kbt, kb = grp - (grp / kbt) * kbt;
  if (row >= a.rows) return;  // whole 16-lane groups leave together
  const bf16x8_t v =
      *(const bf16x8_t *)((const __bf16 *)a.in + (int64_t)row * a.ld_in + kb * 128 + l16 * 8);
  float x[8], amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[i] = (float)v[i];
    amax = fmaxf(amax, fabsf(x[i]));
  }
  amax = fmaxf(amax, __shfl_xor(amax, 8));
  amax = fmaxf(amax, __shfl_xor(amax, 4));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
  uint32_t w32[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    uint32_t u = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float r = fminf(fmaxf(__builtin_rintf(x[4 * k + i] * inv), -127.0f), 127.0f);
      u |= ((uint32_t)(int)r & 0xffu) << (8 * i);
    }
    w32[k] = u;
  }
  *(uint2 *)((int8_t *)a.out + (int64_t)row * a.ld_out + kb * 128 + l16 * 8) = uint2{w32[0], w32[1]};
  if (l16 == 0) a.scale[(int64_t)kb * a.ld_scale + row] = amax / 127.0f;
}

// Weights: one workgroup per 128 x 128 block; thread t covers half a row (64 values).
__global__ void __launch_bounds__(256) w8a8_quant_weight_kernel(const W8QuantArgs a) {
  const int kbt = a.cols / 128;
  const int nb = blockIdx.x / kbt, kb = blockIdx.x - (blockIdx.x / kbt) * kbt;
  const int t = threadIdx.x, row = nb * 128 + (t >> 1), c0 = kb * 128 + (t & 1) * 64;
  const __bf16 *p = (const __bf16 *)a.in + (int64_t)row * a.ld_in + c0;
  float x[64], amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const bf16x8_t v = *(const bf16x8_t *)(p + 8 * j);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[8 * j + i] = (float)v[i];
      amax = fmaxf(amax, fabsf(x[8 * j + i]));
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  __shared__ float red[4];
  if ((t & 63) == 0) red[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
  int8_t *o = (int8_t *)a.out + (int64_t)row * a.ld_out + c0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t w32[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t u = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float r = fminf(fmaxf(__builtin_rintf(x[16 * j + 4 * k + i] * inv), -127.0f), 127.0f);
        u |= ((uint32_t)(int)r & 0xffu) << (8 * i);
      }
      w32[k] = u;
    }
    *(uint4 *)(o + 16 * j) = uint4{w32[0], w32[1], w32[2], w32[3]};
  }
  if (t == 0) a.scale[(int64_t)nb * kbt + kb] = amax / 127.0f;
}

// ============================================================== GEMM

// Grid slot -> (m tile, n tile).  Workgroups are handed to the 8 XCDs round robin (slot j*8 + x
// runs on XCD x).  With 8 or more n tiles, XCD x owns the n tiles [x*NT/8, (x+1)*NT/8) and walks
// them in groups of 8 m tiles: the ~64 workgroups an XCD runs at once then cover about 8 m tiles
// x 8 n tiles, so each K-block slice of an activation or weight tile is read from HBM or the
// last-level cache once and reused about 8 times from the XCD's L2.  Fewer n tiles: plain order.
__host__ __device__ inline int w8a8_grid(int mt_count, int nt_count) {
  if (nt_count < 8) return mt_count * nt_count;
  return 8 * ((nt_count + 7) / 8) * mt_count;
}
__device__ inline bool w8a8_item(int slot, int mt_count, int nt_count, int &mt, int &nt) {
  if (nt_count < 8) {
    if (slot >= mt_count * nt_count) return false;
    mt = slot / nt_count;
    nt = slot - mt * nt_count;
    return true;
  }
  const int x = slot % 8, j = slot / 8;
  const int nt_lo = x * nt_count / 8, ntx = (x + 1) * nt_count / 8 - nt_lo;
  if (j >= ntx * mt_count) return false;
  const int full = (mt_count / 8) * 8;  // m tiles in complete groups of 8
  int ntl;
  if (j < full * ntx) {
    const int g = j / (8 * ntx), r = j - g * (8 * ntx);
    ntl = r / 8;
    mt = g * 8 + (r % 8);
  } else {
    const int r = j - full * ntx, rem = mt_count - full;
    ntl = r / rem;
    mt = full + (r % rem);
  }
  nt = nt_lo + ntl;
  return true;
}

namespace w8 {
constexpr int BM = 256, BN = 128, BK = 128;  // output tile (m, n); K-block = quantisation block
constexpr int NTHR = 512;                   // 8 waves, each a 64 (n) x 64 (m) corner
constexpr int XTILE = BM * BK;              // bytes of one activation stage (32 KB)
constexpr int WTILE = BN * BK;              // bytes of one weight stage (16 KB)
constexpr int XLOADS = XTILE / (NTHR * 16); // 16-byte direct loads per thread per stage (4)
constexpr int WLOADS = WTILE / (NTHR * 16); // (2)
constexpr int RSTEP = NTHR * 16 / BK;       // rows covered by one load of all lanes (64)
// chunk c of row r lives at chunk c ^ ((r >> 1) & 7): a ds_read_b128 of 16 lanes (16 rows at
// one logical chunk) then touches 16 distinct (row parity, chunk) bank groups
__device__ __forceinline__ int sw(int r) { return (r >> 1) & 7; }
}  // namespace w8

// 256 (m) x 128 (n) output tile per workgroup, one workgroup per CU, K-blocks through a 3-stage
// LDS ring (48 KB a stage): block kb+2 is loaded while block kb is multiplied, so a load has two
// steps to land.
__global__ void __launch_bounds__(512, 1) w8a8_gemm_kernel(const W8GemmArgs a) {
  using namespace w8;
  __shared__ __attribute__((aligned(1024))) char xs0[XTILE];
  __shared__ __attribute__((aligned(1024))) char xs1[XTILE];
  __shared__ __attribute__((aligned(1024))) char xs2[XTILE];
  __shared__ __attribute__((aligned(1024))) char ws0[WTILE];
  __shared__ __attribute__((aligned(1024))) char ws1[WTILE];
  __shared__ __attribute__((aligned(1024))) char ws2[WTILE];

  const int mt_count = (a.m + BM - 1) / BM, nt_count = a.n / BN;
  int mt, nt;
  if (!w8a8_item((int)blockIdx.x, mt_count, nt_count, mt, nt)) return;
  const int m0 = mt * BM, n0 = nt * BN;
  const int kbt = a.k / BK;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int wn = wave >> 2, wm = wave & 3;  // wave's corner: n rows wn*64.., m rows wm*64..

  // direct loads: load j of wave w fills LDS chunks (8j + w)*64 + lane = row lrow0 + j*RSTEP,
  // logical chunk lc (the swizzle is the same for every j since RSTEP is a multiple of 16)
  const int p0 = wave * 64 + lane;
  const int lrow0 = p0 / 8;
  const int lcol = ((p0 % 8) ^ sw(lrow0)) * 16;
  const uint32_t xoff0 = (uint32_t)lrow0 * (uint32_t)a.ld_xq + lcol;
  const uint32_t woff0 = (uint32_t)lrow0 * (uint32_t)a.ld_wq + lcol;
  const int xrows = min(BM, a.m - m0);
  const __amdgpu_buffer_rsrc_t xrs =
      make_rsrc((uint64_t)a.xq + (uint64_t)m0 * a.ld_xq, (int)((int64_t)xrows * a.ld_xq));
  const __amdgpu_buffer_rsrc_t wrs =
      make_rsrc((uint64_t)a.wq + (uint64_t)n0 * a.ld_wq, (int)((int64_t)BN * a.ld_wq));
  // Loads of K-block kb into one stage.  Steps issue them unconditionally (a fixed count of
  // vector loads per step keeps the waits exact); past the last block they read columns beyond
  // k of the same rows, or zeros past the descriptor's end, into a stage nobody multiplies.
  auto issue = [&](int kb, char *xdst, char *wdst) {
#pragma unroll
    for (int j = 0; j < XLOADS; ++j) {
      lds_char *dx = (lds_char *)xdst + (8 * j + wave) * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xrs, (__attribute__((address_space(3))) void *)dx, 16,
          (int)(xoff0 + (uint32_t)(j * RSTEP) * (uint32_t)a.ld_xq + kb * BK), 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < WLOADS; ++j) {
      lds_char *dw = (lds_char *)wdst + (8 * j + wave) * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          wrs, (__attribute__((address_space(3))) void *)dw, 16,
          (int)(woff0 + (uint32_t)(j * RSTEP) * (uint32_t)a.ld_wq + kb * BK), 0, 0, 0);
    }
  };

  // operand reads: lane reads row (tile base + l32), logical chunk 2*ks + hl of the K-block
  int coff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) coff[ks] = (((2 * ks + hl) ^ sw(l32)) * 16);

  // activation scales: lane's row is m0 + wm*64 + tm*32 + l32; rows past m and blocks past the
  // last read 0 (bounds)
  const __amdgpu_buffer_rsrc_t srs =
      make_rsrc((uint64_t)a.sx, (int)((int64_t)kbt * a.ld_sx * 4));
  auto load_sx = [&](int kb, float (&s)[2]) {
#pragma unroll
    for (int tm = 0; tm < 2; ++tm) {
      const int row = m0 + wm * 64 + tm * 32 + l32;
      s[tm] = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(srs, (kb * a.ld_sx + row) * 4, 0, 0));
    }
  };
  const cFloat *swp = (const cFloat *)a.sw + (int64_t)nt * kbt;

  f32x16_t acc[2][2];
#pragma unroll
  for (int tn = 0; tn < 2; ++tn)
#pragma unroll
    for (int tm = 0; tm < 2; ++tm) acc[tn][tm] = f32x16_t{};

  // the 16 MFMAs of one K-block: int32 products of its four 32-deep k-steps, per 32x32 tile
  auto mfmas = [&](const char *xbuf, const char *wbuf, i32x16_t (&part)[2][2]) {
    const lds_char *X = (const lds_char *)xbuf, *W = (const lds_char *)wbuf;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      i32x4_t wf[2], xf[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        wf[t] = *(const i32x4_t *)(W + (wn * 64 + t * 32 + l32) * BK + coff[ks]);
        xf[t] = *(const i32x4_t *)(X + (wm * 64 + t * 32 + l32) * BK + coff[ks]);
      }
#pragma unroll
      for (int tn = 0; tn < 2; ++tn)
#pragma unroll
        for (int tm = 0; tm < 2; ++tm)
          part[tn][tm] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
              wf[tn], xf[tm], ks == 0 ? i32x16_t{} : part[tn][tm], 0, 0, 0);
    }
  };
  // fold one K-block's products into the fp32 accumulators with its two scales
  auto dequant = [&](const i32x16_t (&part)[2][2], const float (&sx)[2], float swk) {
#pragma unroll
    for (int tm = 0; tm < 2; ++tm) {
      const float s = sx[tm] * swk;
#pragma unroll
      for (int tn = 0; tn < 2; ++tn)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[tn][tm][i] = fmaf((float)part[tn][tm][i], s, acc[tn][tm][i]);
    }
  };
  // Each wave has waited for its own loads of the block to publish; the barrier (no fence: a
  // fence would wait for every load in flight) then makes them visible, and since a wave's LDS
  // reads of a stage are consumed by MFMAs issued before it, the stage is free afterwards.
  auto publish = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  // Ping-pong.  Waves 0-3 (group A, n rows 0..63) and 4-7 (group B, n rows 64..127) pair up
  // on the four SIMDs.  Step kb has two slots: in the first, A multiplies block kb while B
  // dequantises block kb-1; in the second, A dequantises kb while B multiplies it.  A barrier
  // (no fence) hands the slots over; the step's last barrier publishes block kb+1.  Each group
  // keeps one set of int32 products; A's live within a step, B's across the publish.
  // At the start of a step every wave issues the scales of its block; its share of the tiles of
  // block kb+2 follows once its MFMAs of the step are issued (group A: after its MFMA slot,
  // group B: after the publish), so the direct loads' LDS writes do not meet the operand reads
  // of the MFMA slots (loads at the start of A's step were 2% slower).  At
  // the step's end each wave waits for all but the newest six loads (block kb+1 has landed).  The
  // waits are s_waitcnt builtins, which the compiler's own wait counting sees (an inline-asm
  // wait is opaque to it, and it then inserts full waits).
  i32x16_t part[2][2];
  const bool grp_a = wn == 0;
  auto handover = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  auto mfma_slot = [&](const char *xbuf, const char *wbuf) {
    mfmas(xbuf, wbuf, part);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // DS: operands of k-step 0
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      if (i % 4 == 0 && i < 12) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // DS
    }
  };
  auto end_step = [&]() {
    static_assert(XLOADS + WLOADS == 6, "wait count below");
    __builtin_amdgcn_s_waitcnt(0xF76);  // vmcnt(6), a wait the compiler's counter sees
    publish();
  };
  // Group A, step kb: MFMAs of block kb (stage kb % 3), then their dequantisation.
  auto stepA = [&](int kb, const char *xbuf, const char *wbuf, char *xnext, char *wnext) {
    float s[2];
    load_sx(kb, s);
    __builtin_amdgcn_sched_barrier(0);
    const float swk = swp[kb];
    mfma_slot(xbuf, wbuf);
    handover();
    issue(kb + 2, xnext, wnext);
    __builtin_amdgcn_sched_barrier(0);
    dequant(part, s, swk);
    end_step();
  };
  // Group B, iteration kb: the second slot of step kb (MFMAs of block kb), its publish, the start
  // of step kb+1 (scales of block kb+1 into sn; tiles of block kb+3 into the stage just
  // multiplied) and the first slot of step kb+1 (dequantisation of block kb with scales sc).
  // Products made and consumed in one iteration keep one register set.
  auto iterB = [&](int kb, char *xbuf, char *wbuf, const float (&sc)[2], float (&sn)[2]) {
    mfma_slot(xbuf, wbuf);
    end_step();
    load_sx(kb + 1, sn);
    __builtin_amdgcn_sched_barrier(0);
    issue(kb + 3, xbuf, wbuf);
    dequant(part, sc, swp[kb]);
  };

  issue(0, xs0, ws0);
  issue(1, xs1, ws1);
  __builtin_amdgcn_s_waitcnt(0xF76);  // vmcnt(6): block 0
  publish();
  // Both loops are unrolled so every stage is a compile-time name (the compiler then knows which
  // LDS array a load in flight writes; at a loop head it still waits for the newest loads, so
  // six steps per iteration rather than three halve that cost).  Both pass the same barriers:
  // 1 + 2 kbt.
  if (grp_a) {
    for (int kb = 0;;) {
      stepA(kb, xs0, ws0, xs2, ws2);
      if (++kb >= kbt) break;
      stepA(kb, xs1, ws1, xs0, ws0);
      if (++kb >= kbt) break;
      stepA(kb, xs2, ws2, xs1, ws1);
      if (++kb >= kbt) break;
      stepA(kb, xs0, ws0, xs2, ws2);
      if (++kb >= kbt) break;
      stepA(kb, xs1, ws1, xs0, ws0);
      if (++kb >= kbt) break;
      stepA(kb, xs2, ws2, xs1, ws1);
      if (++kb >= kbt) break;
    }
  } else {
    float sa[2], sb[2];
    // start of step 0: scales of block 0, tiles of block 2; nothing to dequantise in its first
    // slot
    load_sx(0, sa);
    __builtin_amdgcn_sched_barrier(0);
    issue(2, xs2, ws2);
    handover();
    for (int kb = 0;;) {
      iterB(kb, xs0, ws0, sa, sb);
      if (++kb >= kbt) break;
      handover();
      iterB(kb, xs1, ws1, sb, sa);
      if (++kb >= kbt) break;
      handover();
      iterB(kb, xs2, ws2, sa, sb);
      if (++kb >= kbt) break;
      handover();
      iterB(kb, xs0, ws0, sb, sa);
      if (++kb >= kbt) break;
      handover();
      iterB(kb, xs1, ws1, sa, sb);
      if (++kb >= kbt) break;
      handover();
      iterB(kb, xs2, ws2, sb, sa);
      if (++kb >= kbt) break;
      handover();
    }
  }
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no load outlives the workgroup

  // epilogue: y[m][n] bf16; lane's m = m0 + wm*64 + tm*32 + l32, n = n0 + wn*64 + tn*32 +
  // (i/4)*8 + 4*hl + i%4 (four consecutive columns per group of four accumulator registers)
#pragma unroll
  for (int tm = 0; tm < 2; ++tm) {
    const int row = m0 + wm * 64 + tm * 32 + l32;
    if (row >= a.m) continue;
    __bf16 *yr = (__bf16 *)a.y + (int64_t)row * a.ld_y + n0 + wn * 64 + 4 * hl;
#pragma unroll
    for (int tn = 0; tn < 2; ++tn)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4_t v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = (__bf16)acc[tn][tm][4 * g + i];
        *(bf16x4_t *)(yr + tn * 32 + g * 8) = v;
      }
  }
}

hipError_t launch_w8a8_quant_act(const W8QuantArgs &a, hipStream_t s) {
  const int64_t groups = (int64_t)a.rows * (a.cols / 128);
  if (groups == 0) return hipSuccess;
  hipLaunchKernelGGL(w8a8_quant_act_kernel, dim3((unsigned)((groups + 15) / 16)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_w8a8_quant_weight(const W8QuantArgs &a, hipStream_t s) {
  const int blocks = (a.rows / 128) * (a.cols / 128);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(w8a8_quant_weight_kernel, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_w8a8_gemm(const W8GemmArgs &a, hipStream_t s) {
  const int grid = w8a8_grid((a.m + w8::BM - 1) / w8::BM, a.n / w8::BN);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(w8a8_gemm_kernel, dim3(grid), dim3(w8::NTHR), 0, s, a);
  return hipGetLastError();
}

}  // namespace fa
