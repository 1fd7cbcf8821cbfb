/*
 * fa_oracle.h -- CPU oracle for frame-aligned attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This header and oracle/fa_oracle.c are a plain,
 * slow, obviously-correct reference used by tests/, by the smoke check and by
 * the CPU-baseline leg of bench.py.  The product library never includes,
 * links or calls anything here, and nothing here includes the product's
 * headers.
 *
 * What it computes (the pages' rules, restated):
 *  - "Vidu S2" tech report text, paragraph on frame-aligned attention (the
 *    bidirectional editing model): generated (target) tokens interact
 *    bidirectionally across the target sequence; each generated frame
 *    exchanges information only with the source frame of the same time
 *    step; every generated frame can attend to the reference-image tokens.
 *  - Same report, paragraph on causal streaming editing: temporal attention
 *    over target tokens becomes block-wise causal, conditioned on the valid
 *    historical states up to the current segment; the Vidu S2 structured
 *    summary (section 4.3) adds the sliding-window context.
 *  - Sink frames: the tech report's Self-Replay Forcing paragraph and the
 *    structured summary's S1/S2 section keep "sink blocks" beside the
 *    sliding-window context without saying more; read here as: the first
 *    `sink` frames of the stream stay visible to every later target row, on
 *    top of the window (sink = 0: none).
 *  - Vidu S2 structured summary section 5.2: a source frame leaves the cache
 *    once its target frame is produced (so a chunk only reads its own source
 *    frames).
 *  - News clipping point 7 (timestamp-aligned references): a reference
 *    injected mid-stream takes effect from its timestamp; read here as
 *    "target frame f sees image r iff f >= t0[r]".
 *  - Source rows and reference rows as queries follow a fixed convention:
 *    source rows see their own-frame source tokens and the (gated)
 *    references; reference rows see reference tokens only.
 *
 * Per visible key j of query row i:
 *   s_j = scale * sum_d q_i[d] k_j[d]            (double accumulation)
 *   m = max_j s_j,  l = sum_j exp(s_j - m)
 *   o_i = sum_j exp(s_j - m) v_j / l,  lse_i = m + ln(l)  (natural log)
 * A row with no visible key gets o = 0 and lse = -inf.
 *
 * Per-block quantiser (the low-bit prologue): per (head, 128-token block)
 * symmetric int8 with scale absmax/127, and OCP e4m3 fp8 with a power-of-two
 * scale (the smallest 2^e with 448 * 2^e >= absmax), both round-to-nearest-
 * even; K is first reduced by a per-head, per-channel mean vector.
 */
#ifndef FA_ORACLE_H
#define FA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { FAO_TGT = 0, FAO_SRC = 1, FAO_REF = 2 };

typedef struct {
  int T;            /* tokens per latent frame (target and source alike) */
  int C;            /* query frames in this call (a chunk; bidirectional: all frames) */
  int cs;           /* absolute frame index of query frame 0 (bidirectional: 0) */
  int window;       /* target frames before cs that stay visible; -1 = all history */
  int hist_first;   /* absolute frame of token 0 of k_hist / v_hist */
  int n_ref;        /* reference images */
  const int *ref_tokens;  /* [n_ref] tokens per image, stored back to back in *_ref */
  const int *ref_t0;      /* [n_ref] absolute frame from which the image is visible */
  int H, D;
  double scale;     /* softmax scale; the configs use 1/sqrt(D) */
  /* Inputs: fp32, token-major [tokens][H][D], contiguous. */
  const float *q_tgt, *q_src, *q_ref;   /* C*T, C*T and sum(ref_tokens) rows */
  const float *k_hist, *v_hist;         /* target K/V of absolute frames hist_first .. cs+C-1 */
  const float *k_src, *v_src;           /* source K/V of frames cs .. cs+C-1 */
  const float *k_ref, *v_ref;           /* reference K/V */
  int sink;         /* streaming: frames 0 .. sink-1 stay visible to target rows; 0 = none */
} fa_oracle_problem;

/* Number of threads OpenMP will use (for reporting). */
int fa_oracle_threads(void);

/*
 * All rows of the query kinds in kind_mask (bit FAO_TGT/FAO_SRC/FAO_REF).
 * o_* : [rows][H][D] fp32, lse_* : [H][rows] fp32; a NULL pair skips that kind.
 * Returns 0, or -1 if a visible target frame is older than hist_first, or -2
 * on a malformed problem.
 */
int fa_oracle_attn(const fa_oracle_problem *p, int kind_mask,
                   float *o_tgt, float *lse_tgt, float *o_src, float *lse_src,
                   float *o_ref, float *lse_ref);

/*
 * A list of single rows: (kind[i], head[i], row[i]) -> o[i][D], lse[i].
 * Same return codes.
 */
int fa_oracle_attn_rows(const fa_oracle_problem *p, int n, const int *kind,
                        const int *head, const int *row, float *o, float *lse);

/* Visible-key count of one row, by the same rule (for closed-form checks). */
long fa_oracle_count(const fa_oracle_problem *p, int kind, int row);

/*
 * Quantiser, one tensor [N][H][D] fp32.  For every head h and block
 * b = token/128: x' = x - mean[h][:] (mean may be NULL = zero), absmax over
 * the block's N_b*D values.  int8: scale = absmax/127, code =
 * round_half_even(x' * (127/absmax)) clamped to +-127 (float32, one division
 * for each of scale and its inverse).  e4m3: scale = 2^e for the smallest
 * integer e >= -126 with 448 * 2^e >= absmax (exact, no division), code = the
 * e4m3 encoding of x' * 2^-e, so the largest code lies in (224, 448].  An
 * all-zero block gets scale 0 and codes 0.  A device reproduces the codes bit
 * for bit.
 * codes: [N][H][D]; scales: [H][ceil(N/128)].
 */
void fa_oracle_quant_int8(const float *x, int N, int H, int D, const float *mean,
                          int8_t *codes, float *scales);
void fa_oracle_quant_e4m3(const float *x, int N, int H, int D, const float *mean,
                          uint8_t *codes, float *scales);
/*
 * Per-block W8A8 linear layer (tech report, paragraph on linear layers: a
 * per-block W8A8 GEMM whose fine-grained scales keep outliers from setting
 * the range of a whole tensor or channel).  Reading: int8 codes with one fp32
 * scale per block, activations in blocks of 1 row x 128 columns, weights in
 * blocks of 128 x 128, both quantised like the attention path (scale
 * absmax/127, code = round_half_even(x * (127/absmax)) clamped to +-127).
 *
 * fa_oracle_quant_int8_2d: row-major [rows][cols] in blocks of br x bc (edge
 * blocks partial); scales [ceil(rows/br)][ceil(cols/bc)] row-major.
 */
void fa_oracle_quant_int8_2d(const float *x, int rows, int cols, int br, int bc, int8_t *codes,
                             float *scales);
/*
 * y[i][j] = sum over 128-column blocks b of sx[i][b] * sw[j/128][b] *
 * (sum over k in block b of xq[i][k] * wq[j][k]), the inner sums exact in
 * integers, the rest in double.  xq [m][k], wq [n][k], sx [m][kb],
 * sw [ceil(n/128)][kb] with kb = ceil(k/128); y [m][n].
 */
void fa_oracle_w8a8_gemm(const int8_t *xq, const float *sx, const int8_t *wq, const float *sw,
                         int m, int n, int k, double *y);

/*
 * QK prologue: RMSNorm then rotary position embedding, per (token, head).  The
 * tech report's kernel-fusion paragraph fuses RMSNorm with elementwise work,
 * and the structured summary gives each token stream condition-specific RoPE
 * positions; neither gives formulas, so this is a stated reading:
 *   RMSNorm: y = x / sqrt(mean_d x^2 + eps) * gamma[d]   (gamma [D], all heads)
 *   RoPE over three axes (t, y, x): the D/2 rotation pairs (d, d + D/2) are
 *   split into groups of pt = D/2 - 2*floor(D/6), py = px = floor(D/6) pairs
 *   (t first); pair j of a group of g pairs turns by angle pos_axis * base^(-j/g):
 *   (a, b) -> (a cos - b sin, a sin + b cos) with a = y[d], b = y[d + D/2].
 * x, out [N][H][D]; pos [N][3] (t, y, x) per token; double arithmetic.
 */
void fa_oracle_norm_rope(const float *x, int N, int H, int D, const float *gamma, double eps,
                         const int *pos, double base, float *out);

/* OCP e4m3 (bias 7, no infinities, 0x7f/0xff NaN, max 448): RNE, saturating. */
uint8_t fa_oracle_e4m3_encode(float x);
float fa_oracle_e4m3_decode(uint8_t c);

/* Per-head, per-channel mean of the keys: mean[h][d] over n_seg segments of
 * [n_tok[s]][H][D] fp32 rows, accumulated in double, rounded once to fp32. */
void fa_oracle_kmean(int n_seg, const float *const *seg, const int *n_tok, int H, int D,
                     float *mean);

#ifdef __cplusplus
}
#endif
#endif
