/*
 * fa.h -- C ABI of the MI355X (gfx950) frame-aligned attention library (libfa.so).
 *
 * The operation.  Frame-aligned attention as the "Vidu S2" pages describe it
 * (tech report text, paragraphs on frame-aligned attention and on causal
 * streaming editing; structured summary sections 3.3, 4.3 and 5.2; news
 * clipping point 7).  Three token streams meet in one softmax attention:
 *   target  -- the frames being generated; F frames of T tokens,
 *   source  -- the input video, one frame of T tokens per target frame,
 *   reference images -- n_ref images of ref_tokens[r] tokens.
 * A target row of absolute frame f sees:
 *   - target keys of every frame of the call (bidirectional model), or, when
 *     streaming block-wise causally, of the current chunk plus the `window`
 *     frames before it (history held in a ring-buffer KV cache);
 *   - source keys of frame f only;
 *   - reference image r iff f >= ref_t0[r] (timestamp-aligned reference).
 * Source rows (when asked for) see their own frame's source keys and the
 * gated references; reference rows see all reference keys.  Scores are
 * scale * q.k, the softmax is exact; outputs are O and the natural-log
 * log-sum-exp LSE of the visible scores.
 *
 * Conventions.
 *  - Every call returns fa_status; nothing throws across the ABI.
 *    Descriptor, shape, pointer and alignment checks run on the host before
 *    anything is enqueued; a failed check returns FA_ERR_INVALID /
 *    FA_ERR_UNSUPPORTED / FA_ERR_CAPACITY and enqueues nothing.  A HIP
 *    launch failure returns FA_ERR_HIP.  Faults inside kernels surface at
 *    the caller's next synchronisation.  fa_last_error() gives a
 *    thread-local text for the last failure.
 *  - Device tensors are token-major [batch][tokens][heads][head_dim] with the
 *    head_dim axis contiguous; other strides are free (fa_tensor).  Base
 *    pointers and the b/n/h strides must keep every row 16-byte aligned.
 *  - The caller owns every tensor.  The library owns only what it allocates
 *    for a layout or a stream object (a small device block map) and frees it
 *    in the matching destroy call.  fa_attn_fwd allocates nothing.
 *  - Work is enqueued on the caller's HIP stream (with PyTorch-ROCm, the
 *    current torch stream) and is asynchronous.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *fa_hip_stream; /* hipStream_t; NULL = the default stream */

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID = -1,     /* malformed descriptor, pointer, stride or argument */
  FA_ERR_UNSUPPORTED = -2, /* valid but not built: head_dim, dtype, sizes beyond limits */
  FA_ERR_CAPACITY = -3,    /* the ring cannot hold the history the call needs */
  FA_ERR_HIP = -4,         /* a HIP runtime call failed */
  FA_ERR_NOMEM = -5        /* host or device allocation failed */
} fa_status;

typedef enum {
  FA_F32 = 0,    /* fp32 in, fp32 out, fp32 arithmetic */
  FA_BF16 = 1,   /* bf16 in, bf16 out, fp32 softmax and accumulation */
  FA_LOWBIT = 2  /* int8 Q/K (per-128-token block scales), fp8 e4m3 V and P, fp32 softmax */
} fa_dtype;

enum { FA_Q_TARGET = 1, FA_Q_SOURCE = 2, FA_Q_REF = 4 };

#define FA_WINDOW_ALL (-1)
#define FA_MAX_REF 8

/*
 * One call's geometry.  Bidirectional model: chunk_start = 0, window = 0,
 * cache_frames = 0, frames = F.  Streaming: frames = C (the chunk),
 * chunk_start = absolute frame of the chunk's first frame, window = history
 * frames kept visible before it (block-wise causal: every row of the chunk
 * sees the same history), cache_frames = ring capacity in frames.
 * sink_frames: the first frames of the stream that stay visible to every
 * later chunk beside the window (the sink blocks the tech report's
 * Self-Replay Forcing paragraph and the structured summary's S1/S2 section
 * keep next to the sliding window; how many is the caller's choice).  They
 * occupy ring slots 0 .. sink_frames-1 for good.
 */
typedef struct {
  int32_t frames;           /* query frames in the call (F or C), >= 1 */
  int32_t tokens_per_frame; /* T, target and source alike, >= 1 */
  int32_t n_ref;            /* reference images, 0 .. FA_MAX_REF (the reference is optional) */
  int32_t ref_tokens[FA_MAX_REF]; /* tokens of each image, stored back to back in k_ref/v_ref */
  int32_t ref_t0[FA_MAX_REF];     /* absolute frame from which image r is visible */
  int32_t chunk_start;      /* absolute frame index of query frame 0 */
  int32_t window;           /* history frames visible before chunk_start; FA_WINDOW_ALL = all */
  int32_t cache_frames;     /* ring capacity in frames; 0 = no ring (no history) */
  int32_t query_rows;       /* FA_Q_* bits: which rows are queries */
  int32_t batch, heads, head_dim; /* head_dim 64 or 128; query heads == key heads */
  int32_t dtype;            /* fa_dtype */
  float scale;              /* softmax scale; 0 = 1/sqrt(head_dim) */
  int32_t sink_frames;      /* streaming: frames 0 .. sink_frames-1 stay visible; 0 = none */
  int32_t block_rows;       /* FA_BF16: query rows per work item, 128 or 256 (the 8-wave
                               ping-pong kernel); 0 = chosen from the grid (256 unless it needs
                               more rounds of workgroups over the 256 CUs than 128 does).
                               Other dtypes: 0 only. */
  int32_t key_split;        /* FA_KEY_SPLIT_AUTO: with 256-row bf16 items, the work items of a
                               last round that would leave most CUs idle have their keys split
                               into parts that run side by side, and a merge kernel combines
                               the parts' O and LSE (the result is the same attention up to
                               rounding).  FA_KEY_SPLIT_OFF: never. */
} fa_layout_desc;

enum { FA_KEY_SPLIT_AUTO = 0, FA_KEY_SPLIT_OFF = 1 };

/* A device tensor [batch][tokens][heads][head_dim], head_dim contiguous. */
typedef struct {
  void *data;                           /* element [0][0][0][0]; NULL = absent */
  int64_t stride_b, stride_n, stride_h; /* in elements */
  float *scale;                         /* FA_LOWBIT: per-block scales [batch][heads][ceil(tokens/128)] */
} fa_tensor;

/*
 * Every tensor of one call.  Rows: q_tgt/o_tgt frames*T, q_src/o_src
 * frames*T, q_ref/o_ref sum(ref_tokens).  Keys: k/v_tgt are the call's own
 * target frames (frames*T), k/v_src the same frames' source (frames*T),
 * k/v_ref the references, k/v_ring the ring (cache_frames*T; absolute frame
 * g lives in slot g if g < sink_frames, else in slot
 * sink_frames + (g - sink_frames) mod (cache_frames - sink_frames); tokens
 * [slot*T, slot*T+T)).  With sink_frames = 0: slot g mod cache_frames.
 * lse_*: [batch][heads][rows] fp32, NULL to skip.  Outputs of kinds not in
 * query_rows may be absent.
 */
typedef struct {
  fa_tensor q_tgt, q_src, q_ref;
  fa_tensor k_ring, v_ring;
  fa_tensor k_tgt, v_tgt, k_src, v_src, k_ref, v_ref;
  fa_tensor o_tgt, o_src, o_ref;
  float *lse_tgt, *lse_src, *lse_ref;
  float *k_mean;   /* FA_LOWBIT quantiser: per-head channel mean [batch][heads][head_dim] */
  float *v_absmax; /* FA_LOWBIT quantiser, optional (NULL = not kept): largest V block
                      scale of the call [batch][heads]; fa_attn_fwd does not read it */
  void *workspace; /* optional: device scratch for the partial results of key-split work
                      items (fa_layout_splits), at least fa_layout_workspace_bytes(L) bytes,
                      16-byte aligned, used by no other call while this one runs; NULL = the
                      layout's own (calls with one layout that overlap on a device then race
                      on it) */
  size_t workspace_bytes; /* size of workspace; a smaller one than L needs is FA_ERR_INVALID */
} fa_io;

typedef struct fa_layout fa_layout; /* opaque, immutable after build */

const char *fa_status_str(fa_status s);
/* Text of the last failure on the calling thread ("" if none). */
const char *fa_last_error(void);

/*
 * Validates a descriptor and builds its block map: for every tile of
 * query rows (one query kind, consecutive rows), the list of key ranges the
 * rule above makes visible -- ring runs (split at the wrap), the chunk, the
 * source frames of the tile's rows, the visible reference images -- each
 * with the mask it needs (none, same-frame, or t0 gate).  Keys outside every
 * range are never read.  The work order (longest tiles first, heads grouped
 * per XCD) is fixed here.  Pure host work; the block map goes to the device
 * on first use.
 * ring_first_frame: the ring holds every frame of [ring_first_frame,
 * chunk_start) and every sink frame before chunk_start; -1 = "everything
 * visible is held".  Visible history older than it (sink frames aside)
 * returns FA_ERR_CAPACITY, as does a ring too small for the visible history
 * (cache_frames - sink_frames cycling slots) or for the sink frames.
 * *out receives a new layout owned by the caller (fa_layout_destroy).
 */
fa_status fa_layout_build(const fa_layout_desc *d, int32_t ring_first_frame, fa_layout **out);

/*
 * Puts the layout's block map on the current device now (a synchronous
 * allocation and copy, done once per device), so that later fa_attn_fwd
 * calls with it allocate and copy nothing.  Needed before a stream that
 * launches fa_attn_fwd is captured into a HIP graph (the launch optimisation
 * of the tech report's fusion-and-graphs paragraph and the launch article's
 * technical-stack section): under capture, fa_attn_fwd with a map not yet on
 * the device returns FA_ERR_INVALID instead of allocating.  fa_ring_append
 * and fa_quantize_lowbit need no preparation.  FA_ERR_NOMEM / FA_ERR_HIP on
 * device failures.
 */
fa_status fa_layout_prepare(const fa_layout *L);

/*
 * Work counts of a layout: useful (query, key) pairs and useful FLOPs
 * (4*head_dim per pair, all heads and batches), keys the kernel visits
 * (pairs including masked entries of partial tiles), and the algorithmic
 * HBM bytes (every Q/K/V element read once, O and LSE written once).
 * Any pointer may be NULL.
 */
fa_status fa_layout_stats(const fa_layout *L, double *useful_pairs, double *useful_flops,
                          double *visited_pairs, double *bytes);

/* Block-map inspection (host).  One query tile and its key ranges. */
enum { FA_SEG_RING = 0, FA_SEG_TGT = 1, FA_SEG_SRC = 2, FA_SEG_REF = 3 };
enum { FA_MASK_NONE = 0, FA_MASK_SAME_FRAME = 1, FA_MASK_GATE = 2 };
typedef struct {
  int32_t q_kind;   /* 0 target, 1 source, 2 reference rows */
  int32_t row0;     /* first row of the tile within its query kind */
  int32_t rows;     /* rows in the tile (the last tile of a kind may be short) */
  int32_t n_ranges;
} fa_tile_info;
typedef struct {
  int32_t seg;      /* FA_SEG_*: which key tensor */
  int32_t begin;    /* first key (token index within that tensor) */
  int32_t end;      /* one past the last key */
  int32_t mask;     /* FA_MASK_NONE: every row sees every key;
                       FA_MASK_SAME_FRAME: row of frame f sees keys of frame f only;
                       FA_MASK_GATE: rows of frame f >= param see the range, others none */
  int32_t param;    /* FA_MASK_GATE: t0 - chunk_start */
} fa_range_info;
/* Tiles of the block map: their count, the query rows per tile (block_m: 64 fp32, 128 low-bit,
 * 128 or 256 bf16 as the descriptor's block_rows resolved) and the keys per kernel step
 * (block_n).  Any pointer may be NULL.  FA_ERR_INVALID if L is NULL. */
fa_status fa_layout_tiles(const fa_layout *L, int32_t *n_tiles, int32_t *block_m, int32_t *block_n);
/* Copies tile i and up to cap of its ranges. */
fa_status fa_layout_tile(const fa_layout *L, int32_t i, fa_tile_info *tile, fa_range_info *ranges,
                         int32_t cap);

/* Bytes of key-split scratch a call with L needs (0 when nothing is split): what
 * fa_io.workspace must provide.  FA_ERR_INVALID if L or bytes is NULL. */
fa_status fa_layout_workspace_bytes(const fa_layout *L, size_t *bytes);
/* Work items whose keys are split (key_split): how many there are and their parts in total.
 * The tiles above are the block map proper; a split item's parts cover its tile's keys
 * exactly once between them.  Any pointer may be NULL. */
fa_status fa_layout_splits(const fa_layout *L, int32_t *n_split, int32_t *n_parts);
/* Split item s: its tile index, batch*heads + head, its part count, and part p (0 <= p < parts,
 * or p = -1 for none) with up to cap of its ranges.  FA_ERR_INVALID for an index out of range. */
fa_status fa_layout_split(const fa_layout *L, int32_t s, int32_t *tile, int32_t *bh,
                          int32_t *parts, int32_t p, fa_tile_info *part, fa_range_info *ranges,
                          int32_t cap);

/* Frees a layout (host and device parts).  Work using it must have completed. */
fa_status fa_layout_destroy(fa_layout *L);

/*
 * Frame-aligned attention forward for one call described by L: O and LSE
 * for the rows in L's query_rows, on `stream`.  FA_F32 and FA_BF16 read the
 * tensors directly; FA_LOWBIT reads the codes and scales written by
 * fa_quantize_lowbit (q/k int8, v e4m3) and writes bf16 O.  Rows with no
 * visible key (impossible under the rule unless T = 0) get O = 0, LSE = -inf.
 * The first call with a layout on a device uploads its block map (unless
 * fa_layout_prepare did); after that it allocates and copies nothing.
 * A layout with split work items (fa_layout_splits) also gets, with its
 * block map, a workspace for the parts' partial results (at most 256 slots
 * of 256*(head_dim+1) floats); io->workspace, when given, is used instead.
 * Calls with one such layout that overlap on a device (streams without
 * ordering between them) must each bring their own io->workspace, else they
 * race on the layout's.  FA_ERR_INVALID for a misaligned workspace.
 * Asynchronous.
 */
fa_status fa_attn_fwd(const fa_layout *L, const fa_io *io, fa_hip_stream stream);

/*
 * fa_attn_fwd for callers that cannot allocate (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same operation, outputs and checks as
 * fa_attn_fwd, but the layout's block map is copied on every call (one host-to-device copy on
 * `stream`, from the pinned image fa_layout_prepare makes) into a static device array that
 * the library holds on each GPU until the process ends, and the kernels read it there.  The
 * array has 4 MiB for the map and, after it, 32.25 MiB (256 slots of 256*129 floats, the
 * most any layout asks for) for the partial results of split work items (fa_layout_splits),
 * unless io->workspace brings the caller's.
 * The call allocates and frees nothing.  L must have been prepared on this device
 * (fa_layout_prepare), else FA_ERR_INVALID.  A block map larger than 4 MiB (tiles, ranges,
 * the work list and the split items, each part rounded up to 256 bytes) returns
 * FA_ERR_CAPACITY before anything is enqueued.  Every call on a GPU shares that GPU's array,
 * which keeps the last call's contents: calls ordered on one stream are safe, calls on
 * different streams of one GPU that may overlap race (one call's copy can overwrite the map
 * another call's kernel is reading, and their split parts share the workspace).
 */
fa_status fa_attn_fwd_noalloc(const fa_layout *L, const fa_io *io, fa_hip_stream stream);

/*
 * Low-bit prologue for an FA_LOWBIT layout.  The pages name low-bit attention as part of the
 * serving stack ("Vidu S2：全球领先的实时交互与实时编辑模型，正式发布", section "Vidu S2 背后的技术体系";
 * "Vidu S2: Real-Time Interactive, Editable, and Spatial Video Generation", hybrid-attention
 * paragraph) without fixing its arithmetic; the rules below are this library's reading.
 * From the bf16 tensors of `in`:
 *  - a per-(batch, head) channel mean m of all keys the call reads (ring
 *    frames in view, chunk, source, references) into out->k_mean, or, with
 *    FA_QUANT_MEAN_GIVEN, m read from out->k_mean;
 *  - every Q (query kinds of L) and every key tensor as symmetric int8 per
 *    (batch, head, 128-token block): scale = absmax/127, code =
 *    round_half_even(x * (127/absmax)), keys after subtracting m (exact for
 *    the softmax: q.m is constant along a row);
 *  - every V as OCP e4m3 per block with a power-of-two scale: 2^e for the
 *    smallest integer e >= -126 with 448 * 2^e >= absmax, codes x * 2^-e
 *    rounded to nearest even (the attention kernel applies 2^e as the e8m0
 *    block scale of its PV product); if out->v_absmax is non-NULL, the
 *    largest V block scale per (batch, head) goes there.
 * Codes go to out->{q,k,v}_* .data (same strides as declared there), scales
 * to their .scale arrays.  Ring frames outside the call's view are not read.
 * Smoothing shifts every score of a row by scale*q.m, which leaves O unchanged
 * but not the LSE: for each query kind whose out->lse_* is non-NULL the
 * quantiser writes that per-row shift there, and fa_attn_fwd on the low-bit
 * layout adds it to the LSE it computes.  Pass the same lse_* buffers to both
 * calls (or NULL to both).
 * FA_QUANT_RING_READY (needs FA_QUANT_MEAN_GIVEN): the ring's codes and scales in
 * out->k_ring / out->v_ring are kept up to date by fa_ring_quantize, with the same mean; the ring
 * is then not read or quantised here (with a non-NULL v_absmax the scales of its V blocks in
 * view are still folded into it).  The per-call work is Q, the chunk, its source frames and the references.
 */
enum { FA_QUANT_MEAN_GIVEN = 1, FA_QUANT_RING_READY = 2 };
fa_status fa_quantize_lowbit(const fa_layout *L, const fa_io *in, const fa_io *out, int32_t flags,
                             fa_hip_stream stream);

/*
 * Streaming append (structured summary section 4.3, sliding-window KV cache;
 * section 5.2, source frames are not cached): copies frames [0, frames) of
 * k_chunk/v_chunk -- absolute frames first_frame .. first_frame+frames-1 --
 * into their ring slots (see fa_io; sink frames keep slots 0 ..
 * sink_frames-1).  At most cache_frames - sink_frames non-sink frames per
 * call, else FA_ERR_INVALID.  Batch above 32767, or 2^31 or more (token, head)
 * rows in one append, return FA_ERR_UNSUPPORTED.  Element type from d->dtype
 * (FA_LOWBIT rings hold bf16; fa_ring_quantize keeps a coded copy).  Asynchronous.
 */
fa_status fa_ring_append(const fa_layout_desc *d, const fa_tensor *k_ring, const fa_tensor *v_ring,
                         const fa_tensor *k_chunk, const fa_tensor *v_chunk, int32_t first_frame,
                         int32_t frames, fa_hip_stream stream);

/*
 * Low-bit ring kept coded at append time (the low-bit attention of the launch article's
 * technical-stack section and the tech report's hybrid-attention paragraph, with the
 * sliding-window KV cache of the structured summary's section 4.3): after fa_ring_append has
 * put frames [first_frame, first_frame + frames) into the bf16 ring k_ring / v_ring, this
 * re-quantises every 128-token block of the ring tensor that holds any of their tokens, from
 * the bf16 ring, into k_codes (int8, keys minus k_mean [batch][heads][head_dim]) and v_codes
 * (e4m3) -- the same layout as the ring with 1-byte elements, scales per (batch, head, block)
 * in their .scale arrays, arithmetic as in fa_quantize_lowbit.  A block shared with a
 * neighbouring slot is coded whole from that slot's current bf16 contents, so ring slots never
 * written must hold finite values (zeros).  The codes then serve every later low-bit call with
 * FA_QUANT_RING_READY and the same k_mean.  d: the stream's FA_LOWBIT descriptor (ring geometry,
 * sink frames, heads, batch; head_dim 128).  Argument errors FA_ERR_INVALID before any launch;
 * asynchronous.
 */
fa_status fa_ring_quantize(const fa_layout_desc *d, const fa_tensor *k_ring, const fa_tensor *v_ring,
                           const fa_tensor *k_codes, const fa_tensor *v_codes, const float *k_mean,
                           int32_t first_frame, int32_t frames, fa_hip_stream stream);

/*
 * QK prologue: RMSNorm over head_dim then rotary position embedding over three
 * axes, in one pass (the tech report's kernel-fusion paragraph fuses RMSNorm
 * with elementwise work; the structured summary gives each token stream
 * condition-specific RoPE positions).  Neither gives formulas; computed:
 *   y = x / sqrt(mean_d x^2 + eps) * gamma[d]          (gamma [head_dim], all heads)
 *   the head_dim/2 pairs (d, d + head_dim/2) split into t, y, x groups of
 *   D/2 - 2*floor(D/6), floor(D/6), floor(D/6) pairs; pair j of a g-pair group
 *   turns by pos[axis] * rope_base^(-j/g): (a, b) -> (a cos - b sin, a sin + b cos).
 * pos: int32 [tokens][3] (t, y, x) per token, the caller's choice per stream.
 * in / out: bf16 [batch][tokens][heads][head_dim] (fa_tensor strides); in may
 * equal out.  head_dim 64 or 128.  Asynchronous; allocates nothing; argument
 * errors FA_ERR_INVALID / FA_ERR_UNSUPPORTED before any launch.
 */
fa_status fa_qk_norm_rope(const fa_tensor *in, const fa_tensor *out, const float *gamma, float eps,
                          const int32_t *pos, float rope_base, int32_t tokens, int32_t batch,
                          int32_t heads, int32_t head_dim, fa_hip_stream stream);
/*
 * The same prologue fused with the low-bit quantiser (head_dim 128): writes
 * int8 codes [batch][tokens][heads][head_dim] (codes->data, byte strides) and
 * per-(batch, head, 128-token block) scales (codes->scale) exactly as
 * fa_quantize_lowbit would from the bf16 output of fa_qk_norm_rope: values are
 * rounded to bf16, keys (is_key = 1) reduced by k_mean [batch][heads][head_dim]
 * (required), scale absmax/127, codes round half to even.  For queries with
 * k_mean given, lse_shift [batch][heads][tokens] receives softmax_scale * q.m
 * (0 = 1/sqrt(head_dim)) -- what fa_attn_fwd adds back to the LSE.
 */
fa_status fa_qk_norm_rope_quant(const fa_tensor *in, const fa_tensor *codes, const float *gamma,
                                float eps, const int32_t *pos, float rope_base, int32_t is_key,
                                const float *k_mean, float *lse_shift, float softmax_scale,
                                int32_t tokens, int32_t batch, int32_t heads, int32_t head_dim,
                                fa_hip_stream stream);

/*
 * Per-block W8A8 linear layer (tech report, paragraph on linear layers: a
 * per-block W8A8 GEMM whose fine-grained scales keep an outlier from setting
 * the range of a whole tensor or channel; the launch article's technical-stack
 * section names it beside the attention work).  The projections either side
 * of the attention: y = x . w^T.  int8 codes with one fp32 scale per block:
 * activations per (row, 128-column block), weights per 128 x 128 block;
 * scale = absmax/127, code = round_half_even(x * (127/absmax)) clamped to
 * +-127.  All matrices row-major with K (the reduction dimension) contiguous;
 * ld_* are leading dimensions in elements.  The caller owns every buffer; all
 * calls are asynchronous on `stream` and allocate nothing.  Argument errors
 * (NULL, misaligned base or rows -- bases 16-byte aligned, rows a multiple of
 * 16 bytes --, k or n not multiples of 128, ld < columns) return
 * FA_ERR_INVALID before any launch; a row of 2^23 bytes or more returns
 * FA_ERR_UNSUPPORTED; FA_ERR_HIP on a failed launch.
 *
 * fa_w8a8_quantize_act: x bf16 [m][ld_x] -> xq int8 [m][ld_xq] and sx fp32
 * with the scale of row i, K-block b at sx[b * ld_sx + i] (ld_sx >= m).
 * m may be any size (0 is a no-op); k a multiple of 128.
 */
fa_status fa_w8a8_quantize_act(const void *x, int64_t ld_x, int32_t m, int32_t k, int8_t *xq,
                               int64_t ld_xq, float *sx, int64_t ld_sx, fa_hip_stream stream);
/* fa_w8a8_quantize_weight: w bf16 [n][ld_w] -> wq int8 [n][ld_wq] and sw fp32
 * [n/128][k/128] row-major; n and k multiples of 128 (done once per weight). */
fa_status fa_w8a8_quantize_weight(const void *w, int64_t ld_w, int32_t n, int32_t k, int8_t *wq,
                                  int64_t ld_wq, float *sw, fa_hip_stream stream);
/* fa_w8a8_gemm: y bf16 [m][ld_y] = sum over K-blocks b of sx[b][i] * sw[j/128][b] *
 * (exact int32 dot of the block), accumulated in fp32, rounded to bf16 once.
 * n and k multiples of 128, m any size. */
fa_status fa_w8a8_gemm(const int8_t *xq, int64_t ld_xq, const float *sx, int64_t ld_sx,
                       const int8_t *wq, int64_t ld_wq, const float *sw, int32_t m, int32_t n,
                       int32_t k, void *y, int64_t ld_y, fa_hip_stream stream);

/*
 * Streaming driver: one object per stream of chunks.  It keeps the frame
 * counter and what the ring holds, caches the layout of every distinct
 * chunk position, and per chunk runs attention over (ring history in the
 * window, chunk, its source frames, the references) then appends the
 * chunk's target K/V to the ring.  Source K/V are never kept.
 */
typedef struct fa_stream fa_stream;
/* d gives the chunk geometry; its chunk_start is the first chunk's frame. */
fa_status fa_stream_create(const fa_layout_desc *d, fa_stream **out);
/* Attention for the next chunk (fa_attn_fwd with the stream's layout), then
 * fa_stream_advance.  FA_F32 and FA_BF16 streams. */
fa_status fa_stream_chunk(fa_stream *s, const fa_io *io, fa_hip_stream stream);
/* Appends the chunk's target K/V (io->k_tgt/v_tgt) to the ring (io->k_ring/v_ring)
 * at the next frame position and advances the stream by d->frames.  Low-bit
 * streams call fa_stream_layout, fa_quantize_lowbit and fa_attn_fwd first. */
fa_status fa_stream_advance(fa_stream *s, const fa_io *io, fa_hip_stream stream);
/* The layout the next chunk will use.  Owned by the stream: every layout the stream hands
 * out (here or inside fa_stream_chunk) stays valid, with its device block map, until
 * fa_stream_destroy -- a new reference set (fa_stream_set_refs) only stops reusing the old
 * ones -- so a HIP graph captured with it stays replayable for the stream's lifetime.  Work
 * using a stream's layouts must complete before fa_stream_destroy. */
fa_status fa_stream_layout(fa_stream *s, const fa_layout **out);
/* next_frame: chunk_start of the next chunk; ring_first_frame: the ring holds
 * [ring_first_frame, next_frame) and the sink frames (== next_frame when it
 * holds nothing else). */
fa_status fa_stream_state(const fa_stream *s, int32_t *next_frame, int32_t *ring_first_frame);
/* Resume at a saved state (the ring tensors must hold what that state says). */
fa_status fa_stream_seek(fa_stream *s, int32_t next_frame, int32_t ring_first_frame);
/* Replace the reference set (a reference injected mid-stream with its t0). */
fa_status fa_stream_set_refs(fa_stream *s, int32_t n_ref, const int32_t *ref_tokens,
                             const int32_t *ref_t0);
fa_status fa_stream_destroy(fa_stream *s);

#ifdef __cplusplus
}
#endif
#endif
