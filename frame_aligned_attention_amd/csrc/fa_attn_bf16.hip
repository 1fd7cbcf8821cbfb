// fa_attn_bf16.hip -- frame-aligned attention forward, bf16 in/out, gfx950.
// build-flags: -fno-honor-nans
// (No NaN arises from finite inputs here: masked scores are -inf and every exp
// argument is -inf or finite.  Without the flag each row-max reduction first
// canonicalises the MFMA results it compares, 8 more VALU instructions per tile.)
//
// The visibility rule ("Vidu S2" tech report, frame-aligned attention and
// causal streaming paragraphs) arrives as a block map: per work item of 128
// or 256 query rows a short list of key ranges (ring runs, chunk, source
// frames of the rows, visible reference images), each with the mask it
// needs.  The kernels walk those ranges in 64-key tiles; keys outside them
// are never loaded.
//
// Two kernels share the arithmetic and the LDS layout:
//  * attn_bf16_kernel: 4 waves, 128 rows, two workgroups per CU, each wave
//    interleaving its softmax with its MFMAs;
//  * attn_bf16_pp_kernel: 8 waves, 256 rows, one workgroup per CU, the two
//    waves of each SIMD alternating a matrix phase and a softmax phase
//    ("ping-pong", below).  Each K/V tile then serves twice the rows.
// The block map picks the work-item height (the ping-pong kernel unless its
// workgroups need more rounds over the chip than the 128-row ones).
//
// Per wave and key tile: 32 query rows and keys as the M dimension,
//   S^T (64 keys x 32 queries) = K_tile . Q^T,  then  O^T (D x 32) += V^T_tile . P^T.
// The 4-wave kernel uses v_mfma_f32_32x32x16_bf16: every lane holds one query
// column and 32 of its scores, so the row max and row sum are in-lane plus one
// v_permlane32_swap between the lane halves.  The ping-pong kernel uses
// v_mfma_f32_16x16x32_bf16 (a higher share of the matrix core's peak on gfx950):
// a query's 64 scores sit in four lanes, reduced in-lane and by two lane swaps
// (its layout is described at the kernel).  In both, P never leaves registers:
// the S^T accumulator already is the B operand of the second product once V^T's
// key order matches it.
//
// Memory.  K and V tiles go from HBM straight into LDS (buffer loads with
// the LDS bit, 16 bytes per lane, no VGPR staging); the buffer descriptor of
// a tile covers only the keys of its range, so the hardware's bounds check
// returns zeros for the tail of a partial tile and nothing outside a range
// is read.  Rows are XOR-swizzled in 16-byte chunks so the MFMA operand
// reads are free of bank conflicts.  V stays row-major (keys x channels) in
// LDS and is read with the gfx950 transposing LDS load (ds_read_b64_tr_b16),
// which hands each lane the 4 keys of one channel its A operand needs.
//
// Pipeline (4-wave kernel).  K tile j+2 and V tile j+1 load while the waves
// compute softmax(S_j), S_{j+1} = K_{j+1} Q^T and O += V_j P_j; one barrier
// per tile.  The MFMAs of S_{j+1} do not depend on the softmax of tile j, so
// the instruction stream interleaves them (matrix core and VALU overlap).
//
// Softmax.  Base-2 online softmax with scale*log2(e) folded into one FMA
// before v_exp_f32.  The running max is raised only when a tile's max
// exceeds it by more than 8 (so p <= 2^8): the O/l rescale is then rare.
// The ping-pong kernel goes further in a first, fast pass over a work item:
// a wave takes the row max only until each of its rows has seen a key, and
// that first max stays the exp offset.  The offset cancels in O = sum p v /
// sum p and is added back in the LSE, so any value that keeps p finite gives
// the same result up to rounding.  A workgroup vote after the pass reruns the
// item with the lazy rule on every tile if some row sum reached 2^64 or
// overflowed, i.e. if a later score rose far above the first maximum.
// Row sums are taken on the bf16-rounded p that feed the PV product: the
// 4-wave kernel with v_dot2c_f32_bf16 against ones, the ping-pong kernel on
// the matrix core (a ones operand times P^T, in its matrix phase).
#include <type_traits>

#include "fa_device.h"

namespace fa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
template <int D>
struct Bf16Cfg {
  static constexpr int BN = kBf16BlockN;        // keys per tile
  static constexpr int ROWB = D * 2;            // bytes per K/V row in LDS
  static constexpr int CH = ROWB / 16;          // 16-byte chunks per row
  static constexpr int TILEB = BN * ROWB;       // bytes per K (or V) tile
  static constexpr int LOADS = TILEB / (256 * 16);  // 16-byte direct loads per thread per tile
  static constexpr int RSTEP = 256 * 16 / ROWB;     // rows covered by one load of all lanes
  static constexpr int DS = D / 16;             // k-steps of S^T = K Q^T
  static constexpr int DB = D / 32;             // 32-channel blocks of O^T
  // K: chunk c of row r lives at chunk c ^ (r % CH): a ds_read_b128 of 16 lanes (16 rows, one
  // logical chunk) hits 16 distinct chunk slots.  V: at c ^ ((4r) % CH): a transposing read of
  // a half wave (4 rows x 4 logical chunks x 2 halves, rows differing in their low 2 bits)
  // again hits 16 distinct slots (with D = 64 two rows share a slot).
  __device__ static int ksw(int r) { return r & (CH - 1); }
  __device__ static int vsw(int r) { return (4 * r) & (CH - 1); }
  // V in the ping-pong kernel (16x16x32 products): a transposing read group of 16 lanes takes
  // rows 4g..4g+3 at two consecutive logical chunks; chunk c of row r lives at c ^ 2(r % 8),
  // so the eight rows a half wave reads land on eight distinct chunk pairs (with D = 64, rows
  // r and r + 4 share a pair).
  __device__ static int vsw16(int r) { return (2 * r) & (CH - 1) & 14; }
};

// Where each lane's direct loads of a tile land and which bytes of the tile's rows they fetch:
// load j of wave w writes LDS chunks [(4j + w)*64, +64) of the tile, lane i chunk
// (4j + w)*64 + i, i.e. row row0 + j*RSTEP at logical chunk lcb/16 of that row.  RSTEP is a
// multiple of CH, so the swizzle (a function of the row modulo CH) is the same for every j.
// SW: 0 = K, 1 = V of the 4-wave kernel, 2 = V of the ping-pong kernel.
template <int D, int SW>
__device__ __forceinline__ void load_map(int w, int lane, int &row0, int &lcb) {
  using Cfg = Bf16Cfg<D>;
  static_assert(Cfg::RSTEP % Cfg::CH == 0 && Cfg::RSTEP % 8 == 0,
                "swizzle must not depend on the load index");
  const int p = w * 64 + lane;
  row0 = p / Cfg::CH;
  const int pc = p % Cfg::CH;
  const int lc = pc ^ (SW == 2 ? Cfg::vsw16(row0) : SW == 1 ? Cfg::vsw(row0) : Cfg::ksw(row0));
  lcb = lc * 16;
}

template <int D>
__global__ void __launch_bounds__(256, 2) attn_bf16_kernel(const AttnArgs a) {
  using Cfg = Bf16Cfg<D>;
  constexpr int BN = Cfg::BN, ROWB = Cfg::ROWB, TILEB = Cfg::TILEB;
  constexpr float kThr = 8.0f;
  // LDS: two K and two V tile buffers.  Separate arrays (not one array indexed by buffer) let
  // the compiler see that direct loads into one buffer never alias reads of another, so it
  // does not wait for in-flight prefetches before every LDS read.
  __shared__ __attribute__((aligned(1024))) char kbuf0[TILEB];
  __shared__ __attribute__((aligned(1024))) char kbuf1[TILEB];
  __shared__ __attribute__((aligned(1024))) char vbuf0[TILEB];
  __shared__ __attribute__((aligned(1024))) char vbuf1[TILEB];

  const DevWork w = cload<DevWork>((const cWork *)a.work + blockIdx.x);
  if (w.tile < 0) return;
  const DevTile tile = cload<DevTile>((const cTile *)a.tiles + w.tile);
  const int b = w.bh / a.H, h = w.bh - (w.bh / a.H) * a.H;
  const int tid = threadIdx.x;
  // the wave index is uniform per wave; say so, since it feeds M0 (LDS address of direct loads)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int T = a.T;

  // ---- Q (B operand of S^T): lane holds query row l32 of its wave, channels ds*16 + 8*hl + 0..7
  const int qloc = wave * 32 + l32;
  const bool qvalid = qloc < tile.rows;
  const int qrow = tile.row0 + qloc;
  bf16x8_t qreg[Cfg::DS];
  {
    const Seg qs = a.q[tile.q_kind];
    const __bf16 *qp = (const __bf16 *)qs.p + b * qs.sb + (int64_t)qrow * qs.sn + h * qs.sh;
#pragma unroll
    for (int ds = 0; ds < Cfg::DS; ++ds)
      qreg[ds] = qvalid ? *(const bf16x8_t *)(qp + ds * 16 + 8 * hl) : bf16x8_t{};
  }
  const int fq = qrow / T;  // row frame relative to the chunk (target and source rows)

  // ---- per-lane constants of the LDS reads
  // K (A operand of S^T): row kb*32 + l32, logical chunk 2*ds + hl.
  int koff[Cfg::DS];
#pragma unroll
  for (int ds = 0; ds < Cfg::DS; ++ds)
    koff[ds] = l32 * ROWB + (((2 * ds + hl) ^ Cfg::ksw(l32)) * 16);
  // V (A operand of O^T via the transposing read): lane i = 4s + av of 16-lane group g reads
  // row ks*16 + r*8 + 4*(g/2) + s, channels db*32 + (g%2)*16 + 4*av .. +3.
  int voff[Cfg::DB];
  {
    const int i = lane & 15, g = lane >> 4;
    const int s = i >> 2, av = i & 3, hv = g >> 1, gh = g & 1;
    const int vrow = 4 * hv + s;
#pragma unroll
    for (int db = 0; db < Cfg::DB; ++db) {
      const int lc = db * 4 + gh * 2 + (av >> 1);
      voff[db] = vrow * ROWB + ((lc ^ Cfg::vsw(vrow)) * 16) + (av & 1) * 8;
    }
  }
  // direct-load row and column of this lane's first load (K and V layouts differ)
  int krow0, kcb0, vrow0, vcb0;
  load_map<D, 0>(wave, lane, krow0, kcb0);
  load_map<D, 1>(wave, lane, vrow0, vcb0);

  // ---- tile cursors over the flattened (range, 64-key tile) sequence.  Each cursor keeps the
  // fields of its current range (and, for the load cursors, the (batch, head) base of the
  // range's tensor) in scalar registers; the block map is only read again when a cursor
  // crosses into the next range, a few times per work item.
  const cRange *rng = (const cRange *)a.ranges + tile.r_begin;
  const int nr = tile.r_count;
  struct Cur {
    int r, k, begin, end, mask, param;
    uint64_t base;  // byte address of (b, key 0, h) of the range's K or V tensor
    uint32_t sn2;   // bytes between consecutive keys
  };
  // kind: 0 = no tensor (mask cursor), 1 = K, 2 = V
  auto enter = [&](Cur &c, int r, int kind) {
    while (r < nr && rng[r].begin >= rng[r].end) ++r;
    c.r = r;
    if (r >= nr) return;
    const DevRange R = cload<DevRange>(rng + r);
    c.k = c.begin = R.begin;
    c.end = R.end;
    c.mask = R.mask;
    c.param = R.param;
    if (kind) {
      const Seg sg = kind == 2 ? a.v[R.seg] : a.k[R.seg];
      c.base = (uint64_t)sg.p + (uint64_t)((int64_t)b * sg.sb + (int64_t)h * sg.sh) * 2u;
      c.sn2 = (uint32_t)sg.sn * 2u;
    }
  };
  auto next = [&](Cur &c, int kind) {
    if (c.r >= nr) return;
    c.k += BN;
    if (c.k >= c.end) enter(c, c.r + 1, kind);
  };

  // Buffer descriptor of the tile at cursor c (K or V).  It covers only the keys of the range,
  // so the hardware returns zeros past its end; a cursor past the last range gets an empty
  // descriptor (its loads return zeros into a buffer nobody reads).
  auto tile_rsrc = [&](const Cur &c) {
    const bool live = c.r < nr;
    const uint64_t ub = c.base + (uint64_t)(uint32_t)c.k * c.sn2;
    const int nvalid = live ? min(BN, c.end - c.k) : 0;
    return make_rsrc(ub, (int)(nvalid * c.sn2));
  };
  // Direct load j of this lane's share of a tile into LDS buffer `buf`; voff0 is the lane's
  // byte offset of its first load within the tile (row0 * sn2 + column).
  auto load_one = [&](__amdgpu_buffer_rsrc_t rs, uint32_t voff0, uint32_t sn2, char *buf, int j) {
    const uint32_t off = voff0 + (uint32_t)(j * Cfg::RSTEP) * sn2;
    lds_char *dst = (lds_char *)buf + (4 * j + wave) * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)dst, 16,
                                             (int)off, 0, 0, 0);
  };
  auto lane_off = [&](const Cur &c, bool is_v) {
    return (uint32_t)(is_v ? vrow0 : krow0) * c.sn2 + (uint32_t)(is_v ? vcb0 : kcb0);
  };
  auto issue = [&](const Cur &c, bool is_v, char *buf) {
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(c);
    const uint32_t o = lane_off(c, is_v);
#pragma unroll
    for (int j = 0; j < Cfg::LOADS; ++j) load_one(rs, o, c.sn2, buf, j);
  };

  f32x16_t oacc[Cfg::DB];
#pragma unroll
  for (int i = 0; i < Cfg::DB; ++i) oacc[i] = f32x16_t{};
  float m_run = -__builtin_inff();
  float l_part = 0.0f;
  const float c = a.c;
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};

  // S^T = K . Q^T for the K tile in LDS buffer `kb_off`
  auto qk_step = [&](const lds_char *Kl, int ds, f32x16_t &s0, f32x16_t &s1) {
    const bf16x8_t a0 = *(const bf16x8_t *)(Kl + koff[ds]);
    const bf16x8_t a1 = *(const bf16x8_t *)(Kl + 32 * ROWB + koff[ds]);
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qreg[ds], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qreg[ds], s1, 0, 0, 0);
  };

  // Masks the scores of the tile at cursor c: s{kb}[i] is key c.k + kb*32 + (i/4)*8 + 4*hl + i%4
  // of this lane's query.  Only partial tiles and masked ranges come here.
  auto apply_mask = [&](const Cur &c, f32x16_t &s0, f32x16_t &s1) {
    if (c.mask == FA_MASK_NONE && c.k + BN <= c.end) return;
    int klo = c.begin, khi = c.end;
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
      if (k0i < klo || k0i >= khi) s0[i] = -__builtin_inff();
      if (k1i < klo || k1i >= khi) s1[i] = -__builtin_inff();
    }
  };

  // One pipeline step: softmax and PV of the tile whose scores are in (s0, s1) and whose V
  // sits in LDS buffer `vbuf`, while S of the next tile (K in LDS buffer `kbuf`) accumulates in
  // (n0, n1) and the direct loads of K (two tiles ahead, cursor kc -> kdst) and V (one tile
  // ahead, cursor vc -> vdst) are issued.  The row max and the (rare) O rescale come first;
  // the rest is one branch-free region whose instruction order the scheduling hints set:
  // operand reads run a few MFMAs ahead, the exp work of this tile hides under the MFMAs of
  // the next S, and the direct loads trickle in one every other MFMA.
  auto step = [&](f32x16_t &s0, f32x16_t &s1, f32x16_t &n0, f32x16_t &n1, const char *kbuf,
                  const char *vbuf, const Cur &kc, char *kdst, const Cur &vc, char *vdst) {
    // ---- row max of this tile (in-lane over 32 scores, then across the lane halves)
    float mx = fmaxf(fmaxf(s0[0], s0[1]), s0[2]);
#pragma unroll
    for (int i = 3; i < 15; i += 2) mx = fmaxf(fmaxf(mx, s0[i]), s0[i + 1]);
    mx = fmaxf(fmaxf(mx, s0[15]), s1[0]);
#pragma unroll
    for (int i = 1; i < 15; i += 2) mx = fmaxf(fmaxf(mx, s1[i]), s1[i + 1]);
    mx = fmaxf(mx, s1[15]);
    mx = xhalf_max(mx);
    // lazy max update: raised only past m_run + 8 (values stay <= 2^8)
    const float mt = mx * c;
    const bool need = mt > m_run + kThr;
    const float alpha = need ? __builtin_amdgcn_exp2f(m_run - mt) : 1.0f;
    m_run = need ? mt : m_run;
    l_part *= alpha;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
      for (int i = 0; i < Cfg::DB; ++i) oacc[i] *= alpha;
    }
    const float mneg = m_run == -__builtin_inff() ? 0.0f : -m_run;

    // ---- one region.  While a wave is in it, raise its priority: of the two waves sharing
    // a SIMD the one in its MFMA-dense region wins issue, and the other's row-max / barrier
    // work fills the gaps.
    __builtin_amdgcn_s_setprio(1);
    const lds_char *Kl = (const lds_char *)kbuf;
    const __amdgpu_buffer_rsrc_t krs = tile_rsrc(kc), vrs = tile_rsrc(vc);
    const uint32_t kof = lane_off(kc, false), vof = lane_off(vc, true);
    auto prefetch = [&](int ds) {
#pragma unroll
      for (int li = ds * 2 * Cfg::LOADS / Cfg::DS; li < (ds + 1) * 2 * Cfg::LOADS / Cfg::DS; ++li) {
        if (li < Cfg::LOADS)
          load_one(krs, kof, kc.sn2, kdst, li);
        else
          load_one(vrs, vof, vc.sn2, vdst, li - Cfg::LOADS);
      }
    };
    u32x4_t pw[4];  // P^T operands of the four 16-key slices, as packed bf16 pairs
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      const bf16x2_t e0 = {(__bf16)__builtin_amdgcn_exp2f(fmaf(s0[i], c, mneg)),
                           (__bf16)__builtin_amdgcn_exp2f(fmaf(s0[i + 1], c, mneg))};
      const bf16x2_t e1 = {(__bf16)__builtin_amdgcn_exp2f(fmaf(s1[i], c, mneg)),
                           (__bf16)__builtin_amdgcn_exp2f(fmaf(s1[i + 1], c, mneg))};
      l_part = __builtin_amdgcn_fdot2_f32_bf16(e0, ones, l_part, false);
      l_part = __builtin_amdgcn_fdot2_f32_bf16(e1, ones, l_part, false);
      pw[i >> 3][(i & 7) >> 1] = __builtin_bit_cast(uint32_t, e0);
      pw[2 + (i >> 3)][(i & 7) >> 1] = __builtin_bit_cast(uint32_t, e1);
    }
    n0 = f32x16_t{};
    n1 = f32x16_t{};
#pragma unroll
    for (int ds = 0; ds < Cfg::DS; ++ds) {
      qk_step(Kl, ds, n0, n1);
      prefetch(ds);
    }
    // O^T += V^T . P^T
    const lds_char *Vl = (const lds_char *)vbuf;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int db = 0; db < Cfg::DB; ++db) {
        const lds_char *src = Vl + ks * 16 * ROWB + voff[db];
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4_t *)(src));
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4_t *)(src + 8 * ROWB));
        const s16x4_t both[2] = {lo, hi};
        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, both);
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            av, __builtin_bit_cast(bf16x8_t, pw[ks]), oacc[db], 0, 0, 0);
      }
    }
    // schedule of the region (groups are filled in order, dependencies permitting):
    // K operand reads two k-steps ahead; per QK MFMA a share of the exp VALU and every other
    // MFMA one direct load; V operand reads four PV MFMAs ahead.
    constexpr int NQK = 2 * Cfg::DS, NPV = 4 * Cfg::DB;
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // DS read: K operands of k-steps 0, 1
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA (QK)
      if (i + 4 < NQK) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
      if (i % 2 == 0) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // VALU
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // DS read: V operands of PV 0..3
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA (PV)
      if (i + 4 < NPV) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS read
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // VALU (rest of the softmax)
    }
  };

  // Every wave waits for its own direct loads, then the barrier publishes all of them (and
  // frees the buffers read in this step).
  auto end_step = [&]() {
    __builtin_amdgcn_s_setprio(0);
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };

  Cur cc, cv, ck;  // tile j (mask, softmax, PV); tile j+1 (V loads); tile j+2 (K loads)
  enter(cc, 0, 0);
  if (cc.r < nr) {
    enter(cv, cc.r, 2);
    Cur k0c, k1c;  // prologue K tiles 0 and 1
    enter(k0c, cc.r, 1);
    k1c = k0c;
    next(k1c, 1);
    // prologue: K_0 -> kbuf0, V_0 -> vbuf0, K_1 -> kbuf1; S_0
    issue(k0c, false, kbuf0);
    issue(cv, true, vbuf0);
    if (k1c.r < nr) issue(k1c, false, kbuf1);
    next(cv, 2);       // now tile 1
    ck = k1c;
    next(ck, 1);       // now tile 2
    end_step();
    f32x16_t sa0 = f32x16_t{}, sa1 = f32x16_t{}, sb0, sb1;
    {
      const lds_char *K0 = (const lds_char *)kbuf0;
#pragma unroll
      for (int ds = 0; ds < Cfg::DS; ++ds) qk_step(K0, ds, sa0, sa1);
    }
    __syncthreads();  // every wave has read kbuf0 before step 0 loads K_2 into it
    // Steps alternate buffers: even steps read kbuf1 / vbuf0 and load K into kbuf0 / V into
    // vbuf1; odd steps the other way round.  Unrolled by two so the score registers swap roles
    // instead of being copied.
    while (true) {
      // even step j: S_j in (sa), next S into (sb)
      apply_mask(cc, sa0, sa1);
      step(sa0, sa1, sb0, sb1, kbuf1, vbuf0, ck, kbuf0, cv, vbuf1);
      end_step();
      if (cv.r >= nr) break;
      next(cc, 0); next(cv, 2); next(ck, 1);
      // odd step
      apply_mask(cc, sb0, sb1);
      step(sb0, sb1, sa0, sa1, kbuf0, vbuf1, ck, kbuf1, cv, vbuf0);
      end_step();
      if (cv.r >= nr) break;
      next(cc, 0); next(cv, 2); next(ck, 1);
    }
  }

  // ---- epilogue: O = O^T / l, LSE = (m + log2 l) * ln 2
  const float l_tot = xhalf_sum(l_part);
  if (!qvalid) return;
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  const Seg os = a.o[tile.q_kind];
  __bf16 *op = (__bf16 *)os.p + b * os.sb + (int64_t)qrow * os.sn + h * os.sh;
#pragma unroll
  for (int db = 0; db < Cfg::DB; ++db) {
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

// Ping-pong kernel.  Waves 0-3 (group A) and 4-7 (group B) share the four
// SIMDs, one of each per SIMD (waves are dealt to SIMDs round robin).  Each
// key tile is a pair of phases per wave: group A runs its matrix phase (S of
// the next tile and O += V P of this one: MFMAs and LDS reads only) and then
// its softmax phase (VALU only), group B the other way round, so each SIMD's
// matrix core is fed by one wave while the other wave's exp work issues beside
// it.  One workgroup barrier per tile publishes the next tiles' direct loads;
// between two of them the waves of a SIMD swap roles on their own (a barrier
// at the swap, holding all four SIMDs in step, made the kernel 2-3% slower).
// Group A issues the direct loads of the pair's K and V tiles at the start of
// its matrix phase; they have the whole pair to land.
//
// Its products run on v_mfma_f32_16x16x32_bf16 (16x16 outputs, 32-deep), which
// sustains a higher share of the matrix core's peak on gfx950 than the 32x32x16
// form.  Per wave, 32 query rows in two 16-row blocks qb and 64 keys in four
// 16-key blocks kb:
//   S^T[kb][qb] (16 keys x 16 queries) = K_kb . Q_qb^T, four 32-channel k-steps;
//     lane l holds query qb*16 + l%16 and keys kb*16 + 4*(l/16) + r, r = 0..3,
//     so a query's 64 scores sit in the four lanes l%16 + {0,16,32,48}: 16 in
//     each, reduced in-lane, then by v_permlane32_swap and v_permlane16_swap.
//   O^T[cb][qb] (16 channels x 16 queries) += V^T . P^T over two 32-key steps t;
//     the B operand of step t is lane l's p of key blocks 2t and 2t+1 (keys
//     32t + 4g + r and 32t + 16 + 4g + r, g = l/16), so P never leaves its
//     lane; the A operand takes the same keys of channel cb*16 + l%16 from two
//     transposing LDS reads.
//   Row sums: L[qb] (16 x 16) += ones (16 x 32 keys) . P^T with the same B
//     operands, so every row of L holds the 16 queries' sums and lane l reads
//     its query's in place.  The softmax phase, which sets the pace, then has no
//     row-sum arithmetic; the matrix phase has room for the four extra MFMAs.
// max(a, b) for values that are never NaN, without the quieting of signalling NaNs an IEEE-mode
// v_max_f32 asks of inputs it cannot prove canonical (lane exchanges and pinned MFMA results):
// the middle of (a, b, +inf) is the larger of a and b, -inf included.
__device__ __forceinline__ float max_nn(float a, float b) {
  return __builtin_amdgcn_fmed3f(a, b, __builtin_inff());
}

// Row maxima of both 16-row query blocks across the four lanes of a query (l16 + {0, 16, 32,
// 48}), given each lane's partial maxima m0 (block 0) and m1 (block 1).  The first exchange
// swaps m0 of lanes 32-63 with m1 of lanes 0-31, so one max leaves block 0's half-reduced value
// in lanes 0-31 and block 1's in lanes 32-63; one 16-lane exchange finishes each, and a last
// 32-lane exchange hands every lane both blocks' maxima.
__device__ __forceinline__ void rows_max2(float &m0, float &m1) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(m0), __float_as_uint(m1), false, false);
  float h = max_nn(__uint_as_float(r[0]), __uint_as_float(r[1]));
  auto r2 = __builtin_amdgcn_permlane16_swap(__float_as_uint(h), __float_as_uint(h), false, false);
  h = max_nn(__uint_as_float(r2[0]), __uint_as_float(r2[1]));
  auto r3 = __builtin_amdgcn_permlane32_swap(__float_as_uint(h), __float_as_uint(h), false, false);
  m0 = __uint_as_float(r3[0]);
  m1 = __uint_as_float(r3[1]);
}

template <int D>
__global__ void __launch_bounds__(512, 1) attn_bf16_pp_kernel(const AttnArgs a) {
  using Cfg = Bf16Cfg<D>;
  constexpr int BN = Cfg::BN, ROWB = Cfg::ROWB, TILEB = Cfg::TILEB;
  constexpr int KS = D / 32;   // 32-channel k-steps of S^T
  constexpr int CB = D / 16;   // 16-channel blocks of O^T
  constexpr float kThr = 8.0f;
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  // LDS: two K and two V tile buffers.  Separate arrays (not one array indexed by buffer) let
  // the compiler see that direct loads into one buffer never alias reads of another, so it
  // does not wait for in-flight prefetches before every LDS read.
  __shared__ __attribute__((aligned(1024))) char kbuf0[TILEB];
  __shared__ __attribute__((aligned(1024))) char kbuf1[TILEB];
  __shared__ __attribute__((aligned(1024))) char vbuf0[TILEB];
  __shared__ __attribute__((aligned(1024))) char vbuf1[TILEB];

  const DevWork w = cload<DevWork>((const cWork *)a.work + blockIdx.x);
  if (w.tile < 0) return;
  const DevTile tile = cload<DevTile>((const cTile *)a.tiles + w.tile);
  const int b = w.bh / a.H, h = w.bh - (w.bh / a.H) * a.H;
  const int tid = threadIdx.x;
  // the wave index is uniform per wave; say so, since it feeds M0 (LDS address of direct loads)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool grp_a = wave < 4;  // group A: matrix phase first in every pair
  const int lane = tid & 63, g4 = lane >> 4, l16 = lane & 15;
  const int T = a.T;
  // a wave whose 32 rows all lie past the tile's end only loads and keeps step
  const bool wlive = wave * 32 < tile.rows;

  // ---- Q (B operand of S^T): lane holds query row l16 of block qb, channels ks*32 + 8*g4 + 0..7
  bf16x8_t qreg[2][KS];
  int fq[2];  // row frame relative to the chunk (target and source rows)
  bool qvalid[2];
  int qrow[2];
  {
    const Seg qs = a.q[tile.q_kind];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qloc = wave * 32 + qb * 16 + l16;
      qvalid[qb] = qloc < tile.rows;
      qrow[qb] = tile.row0 + qloc;
      fq[qb] = qrow[qb] / T;
      const __bf16 *qp =
          (const __bf16 *)qs.p + b * qs.sb + (int64_t)qrow[qb] * qs.sn + h * qs.sh;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qreg[qb][ks] = qvalid[qb] ? *(const bf16x8_t *)(qp + ks * 32 + 8 * g4) : bf16x8_t{};
    }
  }

  // ---- per-lane constants of the LDS reads
  // K (A operand of S^T): row kb*16 + l16, logical chunk 4*ks + g4 (kb moves the row by 16,
  // which leaves the swizzle alone: an immediate offset).
  int koff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = l16 * ROWB + (((4 * ks + g4) ^ Cfg::ksw(l16)) * 16);
  // V (A operand of O^T via the transposing read): the 16 lanes of group g4 read key rows
  // 4*g4 + (l16 >> 2) (+ 32t, + 16 for the second read) at channels cb*16 + 4*(l16 & 3) .. +3;
  // lane l16 of the group then holds those four keys of channel cb*16 + l16.
  int voff[CB];
  {
    const int vrow = 4 * g4 + (l16 >> 2);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int lc = 2 * cb + ((l16 & 3) >> 1);
      voff[cb] = vrow * ROWB + ((lc ^ Cfg::vsw16(vrow)) * 16) + (l16 & 1) * 8;
    }
  }
  // direct-load row and column of this lane's first load (K and V layouts differ)
  int krow0, kcb0, vrow0, vcb0;
  load_map<D, 0>(wave, lane, krow0, kcb0);
  load_map<D, 2>(wave, lane, vrow0, vcb0);

  // ---- tile cursors over the flattened (range, 64-key tile) sequence.  Each cursor keeps the
  // fields of its current range (and, for the load cursors, the (batch, head) base of the
  // range's tensor) in scalar registers; the block map is only read again when a cursor
  // crosses into the next range, a few times per work item.
  const cRange *rng = (const cRange *)a.ranges + tile.r_begin;
  const int nr = tile.r_count;
  struct Cur {
    int r, k, begin, end, mask, param;
    uint64_t base;  // byte address of (b, key 0, h) of the range's K or V tensor
    uint32_t sn2;   // bytes between consecutive keys
  };
  // kind: 0 = no tensor (mask cursor), 1 = K, 2 = V
  auto enter = [&](Cur &c, int r, int kind) {
    while (r < nr && rng[r].begin >= rng[r].end) ++r;
    c.r = r;
    if (r >= nr) return;
    const DevRange R = cload<DevRange>(rng + r);
    c.k = c.begin = R.begin;
    c.end = R.end;
    c.mask = R.mask;
    c.param = R.param;
    if (kind) {
      const Seg sg = kind == 2 ? a.v[R.seg] : a.k[R.seg];
      c.base = (uint64_t)sg.p + (uint64_t)((int64_t)b * sg.sb + (int64_t)h * sg.sh) * 2u;
      c.sn2 = (uint32_t)sg.sn * 2u;
    }
  };
  auto next = [&](Cur &c, int kind) {
    if (c.r >= nr) return;
    c.k += BN;
    if (c.k >= c.end) enter(c, c.r + 1, kind);
  };

  // Buffer descriptor of the tile at cursor c (K or V).  It covers only the keys of the range,
  // so the hardware returns zeros past its end; a cursor past the last range gets an empty
  // descriptor (its loads return zeros into a buffer nobody reads again).
  auto tile_rsrc = [&](const Cur &c) {
    const bool live = c.r < nr;
    const uint64_t ub = c.base + (uint64_t)(uint32_t)c.k * c.sn2;
    const int nvalid = live ? min(BN, c.end - c.k) : 0;
    return make_rsrc(ub, (int)(nvalid * c.sn2));
  };
  auto lane_off = [&](const Cur &c, bool is_v) {
    return (uint32_t)(is_v ? vrow0 : krow0) * c.sn2 + (uint32_t)(is_v ? vcb0 : kcb0);
  };
  // Direct load j of this lane's share of a tile into LDS buffer `buf` (group A waves only).
  auto load_one = [&](__amdgpu_buffer_rsrc_t rs, uint32_t off0, uint32_t sn2, char *buf, int j) {
    const uint32_t off = off0 + (uint32_t)(j * Cfg::RSTEP) * sn2;
    lds_char *dst = (lds_char *)buf + (4 * j + wave) * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)dst, 16,
                                             (int)off, 0, 0, 0);
  };
  auto issue = [&](const Cur &c, bool is_v, char *buf) {
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(c);
    const uint32_t o = lane_off(c, is_v);
#pragma unroll
    for (int j = 0; j < Cfg::LOADS; ++j) load_one(rs, o, c.sn2, buf, j);
  };

  f32x4_t oacc[CB][2];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) oacc[cb][0] = oacc[cb][1] = f32x4_t{};
  // finite start: the first tile with any visible key always raises it, so -m_run is the exp
  // offset from then on with no test for -inf (a row with no visible key keeps l = 0)
  float m_run[2] = {-1e30f, -1e30f};
  bool exact = false;  // pass with the row max on every tile (after a failed fast pass)
  bool seeded = false;  // fast pass: every row of the wave has seen a key (wave-uniform)
  // row sums on the matrix core: D (16x16) += ones (16 x 32 keys) . P^T (32 keys x 16 queries)
  // makes every row of D the row sums of the 16 queries, so lane l's lsum[qb] holds the sum of
  // query qb*16 + l%16 (in all four elements)
  f32x4_t lsum[2] = {f32x4_t{}, f32x4_t{}};
  const bf16x8_t ones8 = {(__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f,
                          (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f};
  const float c = a.c;
  const float cinv = 1.0f / a.c;
  f32x4_t s[4][2];  // S^T of the tile awaiting its softmax, [kb][qb]
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) s[kb][0] = s[kb][1] = f32x4_t{};
  u32x4_t pw[2][2];  // P^T operands [t][qb], as packed bf16 pairs
#pragma unroll
  for (int t = 0; t < 2; ++t) pw[t][0] = pw[t][1] = u32x4_t{};

  // S^T += K . Q^T for key block kb and k-step ks, both query blocks
  auto qk_step = [&](const lds_char *Kl, int kb, int ks) {
    const bf16x8_t ka = *(const bf16x8_t *)(Kl + kb * 16 * ROWB + koff[ks]);
    s[kb][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qreg[0][ks], s[kb][0], 0, 0, 0);
    s[kb][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qreg[1][ks], s[kb][1], 0, 0, 0);
  };
  // O^T += V^T . P^T for channel block cb and key step t, both query blocks
  auto pv_step = [&](const lds_char *Vl, int t, int cb) {
    const lds_char *src = Vl + t * 32 * ROWB + voff[cb];
    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_t *)(src));
    const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_t *)(src + 16 * ROWB));
    const s16x4_t both[2] = {lo, hi};
    const bf16x8_t av = __builtin_bit_cast(bf16x8_t, both);
    oacc[cb][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
        av, __builtin_bit_cast(bf16x8_t, pw[t][0]), oacc[cb][0], 0, 0, 0);
    oacc[cb][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
        av, __builtin_bit_cast(bf16x8_t, pw[t][1]), oacc[cb][1], 0, 0, 0);
  };
  auto rowsum_step = [&](int t) {
    lsum[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones8, __builtin_bit_cast(bf16x8_t, pw[t][0]),
                                                      lsum[0], 0, 0, 0);
    lsum[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones8, __builtin_bit_cast(bf16x8_t, pw[t][1]),
                                                      lsum[1], 0, 0, 0);
  };

  // Matrix phase: S of the next tile (K in `kbuf`) and O += V P of this one (V in `vbuf`, P in
  // pw).  After the last tile the S product runs on whatever `kbuf` holds and is dropped: one
  // straight-line block, so the accumulators keep their registers.  Operand reads run a few
  // MFMAs ahead.  In group A the phase also issues the pair's direct loads (K at cursor ck
  // into `kw`, V at cursor cv into `vw`), one per MFMA pair over the phase's last pairs (the
  // PV products, whose operand reads are behind them by then): spread over the whole phase
  // they competed with its K reads and were 0.4-1.8% slower.
  auto matrix_phase = [&](const char *kbuf, const char *vbuf, auto with_loads, const Cur &kc,
                          char *kw, const Cur &vc, char *vw) {
    const lds_char *Kl = (const lds_char *)kbuf, *Vl = (const lds_char *)vbuf;
    constexpr int NQK = 4 * KS, NPV = 2 * CB, NL = 2 * Cfg::LOADS;  // in pairs of MFMAs
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) s[kb][0] = s[kb][1] = f32x4_t{};
    if constexpr (decltype(with_loads)::value) {
      const __amdgpu_buffer_rsrc_t krs = tile_rsrc(kc), vrs = tile_rsrc(vc);
      const uint32_t kof = lane_off(kc, false), vof = lane_off(vc, true);
#pragma unroll
      for (int j = 0; j < Cfg::LOADS; ++j) load_one(krs, kof, kc.sn2, kw, j);
#pragma unroll
      for (int j = 0; j < Cfg::LOADS; ++j) load_one(vrs, vof, vc.sn2, vw, j);
    }
    // k-step major, so the four S accumulators of a query block are never needed back to back
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) qk_step(Kl, kb, ks);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) pv_step(Vl, t, cb);
    rowsum_step(0);
    rowsum_step(1);
    // operands five MFMA pairs ahead (~160 cycles of matrix work, the LDS latency under this
    // load): K reads (one per QK pair), then V reads (two per PV pair).  Three pairs ahead was
    // 2-3% slower, six level; seven and more leave too few registers, and more reads in flight
    // only add LDS contention.
    constexpr int LA = 5;
    __builtin_amdgcn_sched_group_barrier(0x100, LA, 0);  // DS read: K operands of pairs 0..LA-1
#pragma unroll
    for (int i = 0; i < NQK + NPV + 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA pair (QK, then PV, then sums)
      if constexpr (decltype(with_loads)::value)
        if (i >= NQK + NPV + 2 - NL)  // the loads, one per pair of the last NL pairs
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM
      if (i + LA < NQK)
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      else if (i + LA < NQK + NPV)
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  };

  // Softmax phase of the tile at mask cursor cc, whose scores are in s: mask, row max, (rare)
  // O rescale, P = exp2(c s - m) into pw, row sums.  Advances cc to the next tile.
  auto softmax_phase = [&](Cur &cc) {
    {
      // mask: s[kb][qb][r] is key cc.k + kb*16 + 4*g4 + r of query block qb's row; only
      // partial tiles and masked ranges come here
      if (cc.mask != FA_MASK_NONE || cc.k + BN > cc.end) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          int klo = cc.begin, khi = cc.end;
          if (cc.mask == FA_MASK_SAME_FRAME) {
            klo = max(klo, fq[qb] * T);
            khi = min(khi, (fq[qb] + 1) * T);
          } else if (cc.mask == FA_MASK_GATE && fq[qb] < cc.param) {
            khi = klo;
          }
          // one key at a time (the empty asm keeps the compares from being batched, which
          // would hold dozens of 64-bit lane masks in scalar registers at once)
          const uint32_t span = (uint32_t)max(khi - klo, 0);
          const int base = cc.k + 4 * g4 - klo;
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const uint32_t rel = (uint32_t)(base + kb * 16 + r);
              float v = s[kb][qb][r];
              v = rel < span ? v : -__builtin_inff();
              s[kb][qb][r] = v;
            }
        }
      }
      // Row max and lazy test.  The exact pass takes them on every tile.  The fast pass takes
      // them only until every row of the wave has seen a key (`seeded`, a wave-uniform flag):
      // from then on the first max stays the exp offset (any offset gives the same softmax;
      // this one only has to keep p finite, which the vote after the pass checks).
      float rmax[2] = {-__builtin_inff(), -__builtin_inff()};
      if (exact || !seeded) {
        // row max: in-lane over the 16 scores of each query block as three-way maxima, then
        // across the four lanes that share the query (l16 + {0, 16, 32, 48}), both blocks at once
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const float m0 = fmaxf(fmaxf(s[0][qb][0], s[0][qb][1]), s[0][qb][2]);
          const float m1 = fmaxf(fmaxf(s[0][qb][3], s[1][qb][0]), s[1][qb][1]);
          const float m2 = fmaxf(fmaxf(s[1][qb][2], s[1][qb][3]), s[2][qb][0]);
          const float m3 = fmaxf(fmaxf(s[2][qb][1], s[2][qb][2]), s[2][qb][3]);
          const float m4 = fmaxf(fmaxf(s[3][qb][0], s[3][qb][1]), s[3][qb][2]);
          rmax[qb] = fmaxf(fmaxf(fmaxf(m0, m1), m2), fmaxf(fmaxf(m3, m4), s[3][qb][3]));
        }
        rows_max2(rmax[0], rmax[1]);
      }
      // lazy max update: raised only when a row's max passes m_run + 8 (values stay <= 2^8),
      // tested on the raw scores against (m_run + 8) / c; the update and the O rescale of both
      // query blocks sit in one rare branch (a separate branch on the same flag: inside the
      // row-max branch the kernel spilled)
      if (exact || !seeded) {
        const bool need0 = rmax[0] > fmaf(m_run[0], cinv, kThr * cinv);
        const bool need1 = rmax[1] > fmaf(m_run[1], cinv, kThr * cinv);
        if (__builtin_amdgcn_ballot_w64(need0 || need1) != 0) {
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            const bool need = qb == 0 ? need0 : need1;
            const float mt = rmax[qb] * c;
            const float alpha = need ? __builtin_amdgcn_exp2f(m_run[qb] - mt) : 1.0f;
            m_run[qb] = need ? mt : m_run[qb];
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) oacc[cb][qb] *= alpha;
            lsum[qb] *= alpha;
          }
        }
      }
      if (!exact && !seeded)
        seeded = __builtin_amdgcn_ballot_w64(m_run[0] == -1e30f || m_run[1] == -1e30f) == 0;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const float mneg = -m_run[qb];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {  // key block 2t + h2
            const f32x4_t &sv = s[2 * t + h2][qb];
            const bf16x2_t e0 = {(__bf16)__builtin_amdgcn_exp2f(fmaf(sv[0], c, mneg)),
                                 (__bf16)__builtin_amdgcn_exp2f(fmaf(sv[1], c, mneg))};
            const bf16x2_t e1 = {(__bf16)__builtin_amdgcn_exp2f(fmaf(sv[2], c, mneg)),
                                 (__bf16)__builtin_amdgcn_exp2f(fmaf(sv[3], c, mneg))};
            pw[t][qb][2 * h2] = __builtin_bit_cast(uint32_t, e0);
            pw[t][qb][2 * h2 + 1] = __builtin_bit_cast(uint32_t, e1);
          }
        }
      }
    }
    next(cc, 0);
  };

  // Phase ends.  Between the two phases of a pair no data changes hands (the buffers both
  // phases read were filled before the pair began), so the swap is only a scheduling fence.
  // The pair's end publishes its direct loads: every wave waits for its own, then the barrier
  // (its fence also completes every LDS read of the pair, freeing those buffers for the next
  // pair's loads).
  // A phase's results are pinned before the fence that ends it: the instruction selector
  // orders only side-effecting nodes, so without the pins it may place pure arithmetic of one
  // phase after the fence, in the next.
  auto pin_softmax = [&]() {
#pragma unroll
    for (int t = 0; t < 2; ++t) __asm__ volatile("" : "+v"(pw[t][0]), "+v"(pw[t][1]));
    __asm__ volatile("" : "+v"(m_run[0]), "+v"(m_run[1]));
  };
  auto pin_matrix = [&]() {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) __asm__ volatile("" : "+v"(s[kb][0]), "+v"(s[kb][1]));
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) __asm__ volatile("" : "+v"(oacc[cb][0]), "+v"(oacc[cb][1]));
    __asm__ volatile("" : "+v"(lsum[0]), "+v"(lsum[1]));
  };
  // No arithmetic may be moved across a phase end (the machine scheduler would otherwise pull
  // the exp work of a softmax phase into the neighbouring matrix phase).
  auto handover = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  auto publish = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };

  // One pass over the work item's tiles.  The fast pass runs first; the exact pass runs only
  // if the fast one let a row sum reach 2^64 or overflow, i.e. a later score far above the
  // row's first max (p <= 2^(c (max - first max)), l <= that times the key count; inputs of
  // ordinary scale stay far below).  The exact pass keeps p <= 2^8 by the lazy rule.  The vote
  // is workgroup-wide, since every wave takes part in the loads and barriers of a pass.  The
  // lambda is inlined at both calls, so each pass has its own schedule (one loop around a
  // single copy, with the vote inside it, made the fast pass 12% slower).
  auto run_pass = [&]() {
    seeded = false;
    Cur cc, cv, ck;  // mask cursor (tile awaiting softmax); V loads; K loads
    enter(cc, 0, 0);
    if (cc.r < nr) {
      enter(cv, cc.r, 2);
      Cur k0c, k1c;  // prologue K tiles 0 and 1
      enter(k0c, cc.r, 1);
      k1c = k0c;
      next(k1c, 1);
      // prologue: K_0 -> kbuf0, V_0 -> vbuf0, K_1 -> kbuf1; S_0 everywhere, softmax of S_0 in
      // group A (group B takes it in the first pair)
      if (grp_a) {
        issue(k0c, false, kbuf0);
        issue(cv, true, vbuf0);
        issue(k1c, false, kbuf1);
      }
      next(cv, 2);  // now tile 1
      ck = k1c;
      next(ck, 1);  // now tile 2
      publish();
      auto advance = [&]() {
        const bool more = cv.r < nr;  // tile j+1 exists (every wave agrees)
        next(ck, 1);
        next(cv, 2);
        return more;
      };
      using yes = std::integral_constant<bool, true>;
      using no = std::integral_constant<bool, false>;
      // Pair j: loads of K_{j+2} and V_{j+1} (by group A, at its matrix phase); the
      // matrix phase reads K_{j+1} and V_j.  Even pairs read kbuf1 / vbuf0 and load into kbuf0 /
      // vbuf1, odd pairs the other way round; unrolled by two so the buffers are compile-time
      // names.  Group A, group B and the waves without rows run separate copies of the loop
      // (same barriers), so no copy carries another's register assignment.
      if (!wlive) {
        __syncthreads();
        auto pair = [&](char *kw, char *vw) {
          if (grp_a) {
            issue(ck, false, kw);
            issue(cv, true, vw);
          }
          const bool more = advance();
          handover();
          publish();
          return more;
        };
        while (pair(kbuf0, vbuf1) && pair(kbuf1, vbuf0)) {
        }
      } else {
        {
          const lds_char *K0 = (const lds_char *)kbuf0;
  #pragma unroll
          for (int ks = 0; ks < KS; ++ks)
  #pragma unroll
            for (int kb = 0; kb < 4; ++kb) qk_step(K0, kb, ks);
        }
        if (grp_a) {
          softmax_phase(cc);
          __syncthreads();  // every wave has read kbuf0 before the first pair loads K_2 into it
          auto pair = [&](const char *kr, const char *vr, char *kw, char *vw) {
            matrix_phase(kr, vr, yes{}, ck, kw, cv, vw);
            pin_matrix();
            const bool more = advance();
            handover();
            if (more) {
              softmax_phase(cc);
              pin_softmax();
            }
            publish();
            return more;
          };
          while (pair(kbuf1, vbuf0, kbuf0, vbuf1) && pair(kbuf0, vbuf1, kbuf1, vbuf0)) {
          }
        } else {
          __syncthreads();
          auto pair = [&](const char *kr, const char *vr, char *kw, char *vw) {
            const bool more = advance();
            softmax_phase(cc);
            pin_softmax();
            handover();
            matrix_phase(kr, vr, no{}, ck, kw, cv, vw);
            pin_matrix();
            publish();
            return more;
          };
          while (pair(kbuf1, vbuf0, kbuf0, vbuf1) && pair(kbuf0, vbuf1, kbuf1, vbuf0)) {
          }
        }
      }
    }
  };
  run_pass();
  bool bad = false;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) bad = bad || !(lsum[qb][0] < 0x1p64f);
  if (__syncthreads_or(bad)) {
    exact = true;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) oacc[cb][0] = oacc[cb][1] = f32x4_t{};
    m_run[0] = m_run[1] = -1e30f;
    lsum[0] = lsum[1] = f32x4_t{};
    run_pass();
  }

  // ---- epilogue: O = O^T / l, LSE = (m + log2 l) * ln 2.  A query's row sum is spread over
  // its four lanes; lane l16 + 16*g4 stores channels cb*16 + 4*g4 .. +3 of its query.
  if (tile.ws) {
    // One key part of a split work item: its normalised O in fp32, rows of D floats, and its
    // LSE go to workspace slot ws - 1; merge_parts_kernel writes the item's O and LSE.
    float *slot = a.ws + (int64_t)(tile.ws - 1) * ws_slot_floats(D);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float l_tot = lsum[qb][0];
      if (!qvalid[qb]) continue;
      const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
      const int qloc = qrow[qb] - tile.row0;
      float *op = slot + qloc * D;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        f32x4_t v;
        v[0] = oacc[cb][qb][0] * inv;
        v[1] = oacc[cb][qb][1] * inv;
        v[2] = oacc[cb][qb][2] * inv;
        v[3] = oacc[cb][qb][3] * inv;
        *(f32x4_t *)(op + cb * 16 + 4 * g4) = v;
      }
      if (g4 == 0)
        slot[kBf16PPBlockM * D + qloc] =
            l_tot > 0.0f ? (m_run[qb] + __log2f(l_tot)) * 0.6931471805599453f : -__builtin_inff();
    }
    return;
  }
  const Seg os = a.o[tile.q_kind];
  float *lse = a.lse[tile.q_kind];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float l_tot = lsum[qb][0];
    if (!qvalid[qb]) continue;
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    __bf16 *op = (__bf16 *)os.p + b * os.sb + (int64_t)qrow[qb] * os.sn + h * os.sh;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
      bf16x4_t v;
      v[0] = (__bf16)(oacc[cb][qb][0] * inv);
      v[1] = (__bf16)(oacc[cb][qb][1] * inv);
      v[2] = (__bf16)(oacc[cb][qb][2] * inv);
      v[3] = (__bf16)(oacc[cb][qb][3] * inv);
      *(bf16x4_t *)(op + cb * 16 + 4 * g4) = v;
    }
    if (lse && g4 == 0)
      lse[(int64_t)w.bh * a.q_rows[tile.q_kind] + qrow[qb]] =
          l_tot > 0.0f ? (m_run[qb] + __log2f(l_tot)) * 0.6931471805599453f : -__builtin_inff();
  }
}

// Merge of a split work item's key parts.  Part i left, for each row, its normalised O_i and
// LSE_i over its own keys; over all the item's keys LSE = log sum_i exp(LSE_i) and
// O = sum_i exp(LSE_i - LSE) O_i (parts in which a row sees no key have LSE_i = -inf and
// weigh nothing).  D/4 threads share a row, four channels each; a workgroup covers 1024/D rows
// and D/4 workgroups one item's 256 rows.
template <int D>
__global__ void __launch_bounds__(256) merge_parts_kernel(const AttnArgs a) {
  constexpr int TPR = D / 4, RPB = 256 / TPR, BPI = kBf16PPBlockM / RPB;
  constexpr int64_t SF = ws_slot_floats(D);
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  const int s = blockIdx.x / BPI;
  const DevSplit sp = a.splits[s];
  const DevTile tile = a.tiles[sp.tile];
  const int r = (blockIdx.x - s * BPI) * RPB + (int)threadIdx.x / TPR;
  const int c = ((int)threadIdx.x % TPR) * 4;
  if (r >= tile.rows) return;
  const float *base = a.ws + (int64_t)sp.slot0 * SF;
  float m = -__builtin_inff();
  for (int p = 0; p < sp.parts; ++p) m = fmaxf(m, base[p * SF + kBf16PPBlockM * D + r]);
  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  float l = 0.0f;
  if (m > -__builtin_inff()) {
    for (int p = 0; p < sp.parts; ++p) {
      const float wgt = __expf(base[p * SF + kBf16PPBlockM * D + r] - m);
      const f32x4_t o = *(const f32x4_t *)(base + p * SF + (int64_t)r * D + c);
      l += wgt;
      acc += wgt * o;
    }
  }
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  const int b = sp.bh / a.H, h = sp.bh - (sp.bh / a.H) * a.H;
  const int qrow = tile.row0 + r;
  const Seg os = a.o[tile.q_kind];
  bf16x4_t v;
  v[0] = (__bf16)(acc[0] * inv);
  v[1] = (__bf16)(acc[1] * inv);
  v[2] = (__bf16)(acc[2] * inv);
  v[3] = (__bf16)(acc[3] * inv);
  *(bf16x4_t *)((__bf16 *)os.p + b * os.sb + (int64_t)qrow * os.sn + h * os.sh + c) = v;
  float *lse = a.lse[tile.q_kind];
  if (lse && c == 0)
    lse[(int64_t)sp.bh * a.q_rows[tile.q_kind] + qrow] = l > 0.0f ? m + __logf(l) : -__builtin_inff();
}

hipError_t launch_merge_parts(const AttnArgs &a, int head_dim, int n_split, hipStream_t s) {
  if (head_dim == 64)
    hipLaunchKernelGGL(merge_parts_kernel<64>, dim3(n_split * 16), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(merge_parts_kernel<128>, dim3(n_split * 32), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attn_bf16(const AttnArgs &a, int head_dim, int block_m, int grid,
                            hipStream_t s) {
  if (block_m == kBf16PPBlockM) {
    if (head_dim == 64)
      hipLaunchKernelGGL(attn_bf16_pp_kernel<64>, dim3(grid), dim3(512), 0, s, a);
    else
      hipLaunchKernelGGL(attn_bf16_pp_kernel<128>, dim3(grid), dim3(512), 0, s, a);
  } else {
    if (head_dim == 64)
      hipLaunchKernelGGL(attn_bf16_kernel<64>, dim3(grid), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(attn_bf16_kernel<128>, dim3(grid), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace fa
