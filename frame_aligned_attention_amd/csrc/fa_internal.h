// fa_internal.h -- structures shared by the host side of libfa.so and its
// gfx950 kernels: the device form of a layout's block map and the kernel
// argument blocks.  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa.h"

namespace fa {

// Tile sizes of the kernels.  The block map is built for the kernel that
// will consume it: BM query rows per tile, key tiles of BN keys.
constexpr int kBf16BlockM = 128;   // 4 waves x 32 query rows
constexpr int kBf16PPBlockM = 256; // ping-pong kernel: 8 waves x 32 query rows
constexpr int kBf16BlockN = 64;
constexpr int kF32BlockM = 64;     // one wave, one row per lane
constexpr int kF32BlockN = 64;
constexpr int kLowbitBlockM = 128;
constexpr int kLowbitBlockN = 64;
constexpr int kQuantBlock = 128;   // tokens per quantisation block

// One key range of a tile.  seg: FA_SEG_*; mask: FA_MASK_*.
struct DevRange {
  int32_t seg;
  int32_t mask;
  int32_t begin;
  int32_t end;
  int32_t param;
  int32_t pad[3];
};

// One tile of query rows.  Ranges [r_begin, r_begin + r_count) of the map.  ws = 0: the
// kernel writes the tile's O and LSE; ws = s + 1: the tile is one key part of a split work item
// and the kernel writes its normalised fp32 O and its LSE to workspace slot s instead.
struct DevTile {
  int32_t q_kind;
  int32_t row0;
  int32_t rows;
  int32_t r_begin;
  int32_t r_count;
  int32_t ws;
  int32_t pad[2];
};

// A work item whose keys were split: the base tile, its (batch*heads + head), and the `parts`
// workspace slots slot0 .. slot0 + parts - 1 the merge combines into its O and LSE.
struct DevSplit {
  int32_t tile;
  int32_t bh;
  int32_t slot0;
  int32_t parts;
};

// Workspace slot of a key part (ping-pong kernel rows): O as fp32 [256][D], then LSE [256].
constexpr int64_t ws_slot_floats(int head_dim) { return int64_t(256) * (head_dim + 1); }
constexpr int kMaxKeyParts = 16;  // parts per split work item
constexpr int kMaxWsSlots = 256;  // slots per layout (the split parts fill at most one round)

// Grid slot -> (tile, batch*heads + head); tile < 0 marks an idle slot.
struct DevWork {
  int32_t tile;
  int32_t bh;
};

// A device tensor: base pointer and element strides (head_dim contiguous).
struct Seg {
  const void *p;
  int64_t sb, sn, sh;
  const float *scale;  // low-bit per-block scales [b][h][nblk]
  int32_t nblk;
  int32_t pad;
};

struct AttnArgs {
  Seg k[4];          // by FA_SEG_*
  Seg v[4];
  Seg q[3];          // by query kind
  Seg o[3];
  float *lse[3];
  int32_t q_rows[3]; // rows per query kind (LSE row stride)
  int32_t T;
  int32_t H;
  float scale;       // softmax scale
  float c;           // scale * log2(e)
  const DevTile *tiles;
  const DevRange *ranges;
  const DevWork *work;
  float *ws;                 // key-part workspace (slots of ws_slot_floats(D) floats)
  const DevSplit *splits;    // split work items, for the merge
};

struct RingArgs {
  const void *src[2];
  void *dst[2];
  int64_t ssb[2], ssn[2], ssh[2];
  int64_t dsb[2], dsn[2], dsh[2];
  int32_t T, H, frames, first_frame, cache_frames, chunks16;  // 16-byte chunks per (token, head)
  int32_t batch;
  int32_t sink;  // sink frames: slots 0 .. sink-1 for good
};

// Ring slot of absolute frame g: a sink frame keeps its own slot, the others cycle through the
// cache_frames - sink remaining slots (callers make sure there is one when g >= sink).
__host__ __device__ inline int ring_slot(int g, int sink, int cache_frames) {
  return g < sink ? g : sink + (g - sink) % (cache_frames - sink);
}

// Launchers (defined in the .hip files); return hipError_t of the launch.
hipError_t launch_attn_bf16(const AttnArgs &a, int head_dim, int block_m, int grid,
                            hipStream_t s);
// Combines the key parts of n_split split work items into their O and LSE.
hipError_t launch_merge_parts(const AttnArgs &a, int head_dim, int n_split, hipStream_t s);
hipError_t launch_attn_f32(const AttnArgs &a, int head_dim, int grid, hipStream_t s);
hipError_t launch_attn_lowbit(const AttnArgs &a, int head_dim, int grid, hipStream_t s);
hipError_t launch_ring_append(const RingArgs &a, hipStream_t s);

// One tensor for the low-bit quantiser: bf16 input, 1-byte codes out (same token-major layout),
// fp32 scales per (batch, head, 128-token block).  Only tokens in up to two runs
// [lo0, hi0), [lo1, hi1) are read and written (ring frames outside the call's view are not).
struct QSeg {
  const void *in;
  int64_t isb, isn, ish;  // elements
  void *out;
  int64_t osb, osn, osh;  // elements (bytes)
  float *scale;           // [batch][heads][nblk]
  int32_t nblk;           // blocks of the tensor (row length of `scale`)
  int32_t kind;           // 0: Q int8, 1: K int8 after the mean, 2: V e4m3,
                          // 3: V already coded -- only fold its block scales into v_absmax
  int32_t lo0, hi0, lo1, hi1;
  int32_t blk_begin;      // first entry of this tensor in the flat block list
  int32_t blk0, nproc;    // the tensor's blocks blk0 .. blk0 + nproc - 1 are processed
  int32_t n;              // tokens
  float *lse;             // Q tensors: per-row smoothing shift scale*q.m -> [batch][heads][n]
};

constexpr int kMaxQSeg = 12;

struct QuantArgs {
  QSeg seg[kMaxQSeg];
  int32_t nseg;
  int32_t total_blocks;   // sum of nblk
  int32_t H, D, batch;
  float *k_mean;          // [batch][heads][D]
  float *v_absmax;        // [batch][heads]: largest V block scale (atomic max); NULL = not kept
  float softmax_scale;
};

hipError_t launch_quant_lowbit(const QuantArgs &a, bool mean_given, hipStream_t s);

// Per-block W8A8 linear layer.  Quantiser: bf16 [rows][ld_in] -> int8 [rows][ld_out]; scales
// per (row, 128-column block) at scale[block * ld_scale + row] (activations) or per 128 x 128
// block at scale[row_block * (cols/128) + block] (weights).
struct W8QuantArgs {
  const void *in;
  int64_t ld_in;   // elements
  void *out;
  int64_t ld_out;  // bytes
  float *scale;
  int64_t ld_scale;
  int32_t rows, cols;
};

// y [m][ld_y] bf16 = dequant(xq [m][ld_xq] int8, sx [k/128][ld_sx]) . dequant(wq [n][ld_wq] int8,
// sw [n/128][k/128])^T; n and k multiples of 128.
struct W8GemmArgs {
  const void *xq;
  const float *sx;
  const void *wq;
  const float *sw;
  void *y;
  int64_t ld_xq, ld_wq, ld_y;
  int32_t ld_sx;
  int32_t m, n, k;
};

// QK prologue (RMSNorm + three-axis RoPE), optionally fused with the low-bit quantiser.
struct ProArgs {
  const void *in;
  int64_t isb, isn, ish;  // elements
  void *out;
  int64_t osb, osn, osh;  // elements (bf16 out) or bytes (int8 codes out)
  const float *gamma;     // [D]
  const int32_t *pos;     // [n][3]: t, y, x
  float eps, base_log2;
  int32_t n, batch, H;
  int32_t kind;           // quantised output: 0 = Q, 1 = K (reduced by `mean`)
  const float *mean;      // [batch][H][D] or NULL
  float *lse;             // Q with a mean: per-row shift softmax_scale * q.m, [batch][H][n]
  float softmax_scale;
  float *scale;           // quantised output: [batch][H][ceil(n/128)]
};

hipError_t launch_norm_rope(const ProArgs &a, int head_dim, hipStream_t s);
hipError_t launch_norm_rope_quant(const ProArgs &a, hipStream_t s);

hipError_t launch_w8a8_quant_act(const W8QuantArgs &a, hipStream_t s);
hipError_t launch_w8a8_quant_weight(const W8QuantArgs &a, hipStream_t s);
hipError_t launch_w8a8_gemm(const W8GemmArgs &a, hipStream_t s);

}  // namespace fa
