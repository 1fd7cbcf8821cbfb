// fa_layout.cpp -- descriptor validation and the block map.
//
// The visibility rule is the one of the "Vidu S2" pages (tech report,
// paragraphs on frame-aligned attention and on causal streaming editing;
// structured summary sections 4.3 and 5.2; news clipping point 7): a target
// row of frame f reads the target keys of the call's frames (plus, when
// streaming, the `window` history frames before the chunk and the stream's
// first sink_frames frames), the source keys of frame f, and reference image
// r iff f >= t0[r].  Here that rule is
// turned, once per descriptor, into per-tile key ranges so that the kernels
// never build a dense mask and never touch keys outside the ranges.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>

#include "fa_layout_impl.h"

namespace fa {

static fa_status validate(const fa_layout_desc *d, int32_t ring_first, int32_t *hist_lo_out,
                          int32_t *ring_first_out) {
  if (!d) return fail(FA_ERR_INVALID, "descriptor is NULL");
  if (d->frames < 1) return fail(FA_ERR_INVALID, "frames must be >= 1");
  if (d->tokens_per_frame < 1) return fail(FA_ERR_INVALID, "tokens_per_frame must be >= 1");
  if (d->n_ref < 0 || d->n_ref > FA_MAX_REF)
    return fail(FA_ERR_INVALID, "n_ref must be in [0, FA_MAX_REF]");
  int64_t ref_total = 0;
  for (int r = 0; r < d->n_ref; ++r) {
    if (d->ref_tokens[r] < 0) return fail(FA_ERR_INVALID, "ref_tokens must be >= 0");
    ref_total += d->ref_tokens[r];
  }
  if (d->chunk_start < 0) return fail(FA_ERR_INVALID, "chunk_start must be >= 0");
  if (d->window < FA_WINDOW_ALL) return fail(FA_ERR_INVALID, "window must be >= -1");
  if (d->cache_frames < 0) return fail(FA_ERR_INVALID, "cache_frames must be >= 0");
  if (d->sink_frames < 0) return fail(FA_ERR_INVALID, "sink_frames must be >= 0");
  if (d->block_rows != 0 && (d->dtype != FA_BF16 || (d->block_rows != kBf16BlockM &&
                                                      d->block_rows != kBf16PPBlockM)))
    return fail(FA_ERR_INVALID, "block_rows must be 0, or 128 or 256 with FA_BF16");
  if (d->key_split != FA_KEY_SPLIT_AUTO && d->key_split != FA_KEY_SPLIT_OFF)
    return fail(FA_ERR_INVALID, "key_split must be FA_KEY_SPLIT_AUTO or FA_KEY_SPLIT_OFF");
  if (d->query_rows <= 0 || d->query_rows > 7)
    return fail(FA_ERR_INVALID, "query_rows must be a non-empty set of FA_Q_* bits");
  if (d->batch < 1 || d->heads < 1) return fail(FA_ERR_INVALID, "batch and heads must be >= 1");
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(FA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (d->dtype != FA_F32 && d->dtype != FA_BF16 && d->dtype != FA_LOWBIT)
    return fail(FA_ERR_INVALID, "unknown dtype");
  if (d->dtype == FA_LOWBIT && d->head_dim != 128)
    return fail(FA_ERR_UNSUPPORTED, "the low-bit path is built for head_dim 128");
  if (!(d->scale >= 0.0f) || !std::isfinite(d->scale))
    return fail(FA_ERR_INVALID, "scale must be finite and >= 0");
  const int64_t rows = (int64_t)d->frames * d->tokens_per_frame;
  const int64_t ring_tok = (int64_t)d->cache_frames * d->tokens_per_frame;
  const int64_t lim = int64_t(1) << 30;
  if (rows >= lim || ring_tok >= lim || ref_total >= lim)
    return fail(FA_ERR_UNSUPPORTED, "a tensor has 2^30 tokens or more");
  if ((int64_t)d->batch * d->heads * std::max(rows, ref_total) >= (int64_t(1) << 31))
    return fail(FA_ERR_UNSUPPORTED, "batch*heads*rows must stay below 2^31");
  const int64_t cs = d->chunk_start;
  const int64_t lo = d->window < 0 ? 0 : std::max<int64_t>(0, cs - d->window);
  if (cs + d->frames >= lim) return fail(FA_ERR_UNSUPPORTED, "chunk_start too large");
  if (ring_first > cs) return fail(FA_ERR_INVALID, "ring_first_frame is after chunk_start");
  // Visible history: the sink frames before the chunk, [0, min(S, cs)), in slots of their own,
  // and the window [lo, cs); its non-sink part [nlo, cs) cycles through cap - S slots.
  const int64_t S = d->sink_frames, cap = d->cache_frames;
  const int64_t nlo = std::max(lo, S);
  if (std::min(S, cs) > 0 && cap < S)
    return fail(FA_ERR_CAPACITY, "the ring has fewer slots than sink frames");
  if (nlo < cs) {  // some non-sink history is visible
    if (cap - S < cs - nlo)
      return fail(FA_ERR_CAPACITY, "the ring holds fewer frames than the visible history");
    if (ring_first < 0) ring_first = (int32_t)nlo;
    if (ring_first > nlo)
      return fail(FA_ERR_CAPACITY, "visible history is older than the ring's oldest frame");
    if (std::max<int64_t>(ring_first, S) < cs - (cap - S))
      return fail(FA_ERR_INVALID, "ring_first_frame is older than the ring can hold");
  } else {
    if (ring_first < 0) ring_first = (int32_t)cs;
  }
  if (ring_first > cs) return fail(FA_ERR_INVALID, "ring_first_frame is after chunk_start");
  *hist_lo_out = (int32_t)lo;
  *ring_first_out = ring_first;
  return FA_OK;
}

static void add_ref_ranges(const fa_layout_desc *d, int fa_rel, int fb_rel,
                           std::vector<DevRange> &out) {
  // Reference image r occupies tokens [off_r, off_r + n_r) of the reference tensor.  The tile's
  // rows are frames cs+fa .. cs+fb; image r is visible to a row iff its frame >= t0[r].
  const int cs = d->chunk_start;
  int off = 0;
  for (int r = 0; r < d->n_ref; ++r) {
    const int n = d->ref_tokens[r], t0 = d->ref_t0[r];
    const int lo = off, hi = off + n;
    off = hi;
    if (n == 0) continue;
    if (cs + fb_rel < t0) continue;  // no row of the tile sees it yet
    if (cs + fa_rel >= t0) {         // every row sees it
      if (!out.empty() && out.back().seg == FA_SEG_REF && out.back().mask == FA_MASK_NONE &&
          out.back().end == lo) {
        out.back().end = hi;  // merge with the previous fully visible image
        continue;
      }
      out.push_back(DevRange{FA_SEG_REF, FA_MASK_NONE, lo, hi, 0, {0, 0, 0}});
    } else {
      out.push_back(DevRange{FA_SEG_REF, FA_MASK_GATE, lo, hi, t0 - cs, {0, 0, 0}});
    }
  }
}

// Keys of a tile in the kernels' 64-key steps, range by range.
static int64_t tile_steps(const fa_layout *L, const DevTile &t) {
  int64_t n = 0;
  for (int j = 0; j < t.r_count; ++j) {
    const DevRange &r = L->ranges[t.r_begin + j];
    if (r.end > r.begin) n += (r.end - r.begin + kBf16BlockN - 1) / kBf16BlockN;
  }
  return n;
}

// Key split of the ping-pong kernel's last round.  That kernel runs one workgroup per CU, so N
// work items take ceil(N / 256) rounds, and when the last round holds few items as costly as
// the others, most of the chip idles through it.  Each such item is cut into parts along its
// 64-key steps (a part's sub-ranges keep their range's mask, which depends on absolute key and
// row positions only); the parts run on the idle CUs, write normalised O and LSE to workspace
// slots, and a merge kernel combines them with log-sum-exp weights.  Returns the length of the
// last round in rounds as the split leaves it (1 when nothing is split).
static constexpr int64_t kMinPartSteps = 8;  // 512 keys: below that a part's fixed costs dominate
static double split_last_round(fa_layout *L) {
  constexpr int64_t kCUs = 256;
  std::vector<int> live;  // grid slots of work items
  for (int j = 0; j < (int)L->work.size(); ++j)
    if (L->work[j].tile >= 0) live.push_back(j);
  const int64_t n = (int64_t)live.size();
  if (n == 0 || L->d.key_split == FA_KEY_SPLIT_OFF) return 1.0;
  const int64_t rounds = (n + kCUs - 1) / kCUs, tail = n - kCUs * (rounds - 1);
  std::vector<int64_t> steps(L->tiles.size());
  int64_t max_steps = 0;
  for (size_t i = 0; i < L->tiles.size(); ++i) {
    steps[i] = tile_steps(L, L->tiles[i]);
    max_steps = std::max(max_steps, steps[i]);
  }
  // Items of the last round costing half the largest item or more are split; the rest of the
  // round (cheaper kinds of query rows) runs as it is.
  std::vector<int> cut;
  int64_t other = 0;
  for (int64_t i = n - tail; i < n; ++i) {
    const int64_t st = steps[L->work[live[i]].tile];
    if (2 * st >= max_steps && st >= 2 * kMinPartSteps)
      cut.push_back(live[i]);
    else
      other = std::max(other, st);
  }
  if (cut.empty()) return 1.0;
  const int64_t room = kCUs - (tail - (int64_t)cut.size());
  const int64_t P = std::min<int64_t>(kMaxKeyParts, room / (int64_t)cut.size());
  if (P < 2) return 1.0;
  double last = (double)other / (double)max_steps;
  int slot = 0;
  for (int j : cut) {
    const DevWork w = L->work[j];
    const DevTile base = L->tiles[w.tile];  // a copy: `tiles` grows below
    const int64_t nb = steps[w.tile];
    const int64_t parts = std::min<int64_t>(P, nb / kMinPartSteps);
    last = std::max(last, (double)((nb + parts - 1) / parts) / (double)max_steps);
    L->splits.push_back(DevSplit{w.tile, w.bh, slot, (int32_t)parts});
    // part p takes steps [p*nb/parts, (p+1)*nb/parts) of the tile's range sequence
    int r = 0;        // range of the tile being handed out
    int64_t k = 0;    // its steps already handed out
    for (int64_t p = 0; p < parts; ++p) {
      int64_t want = (p + 1) * nb / parts - p * nb / parts;
      DevTile t = base;
      t.r_begin = (int32_t)L->ranges.size();
      t.ws = slot + (int32_t)p + 1;
      while (want > 0 && r < base.r_count) {
        const DevRange src = L->ranges[base.r_begin + r];  // a copy: `ranges` grows below
        const int64_t rs =
            src.end > src.begin ? (src.end - src.begin + kBf16BlockN - 1) / kBf16BlockN : 0;
        if (k >= rs) {
          ++r;
          k = 0;
          continue;
        }
        const int64_t take = std::min(want, rs - k);
        DevRange sub = src;
        sub.begin = (int32_t)(src.begin + k * kBf16BlockN);
        sub.end = (int32_t)std::min<int64_t>(src.end, src.begin + (k + take) * kBf16BlockN);
        L->ranges.push_back(sub);
        k += take;
        want -= take;
      }
      t.r_count = (int32_t)L->ranges.size() - t.r_begin;
      L->work.push_back(DevWork{(int32_t)L->tiles.size(), w.bh});
      L->tiles.push_back(t);
    }
    slot += (int)parts;
    L->work[j] = DevWork{-1, 0};
  }
  L->ws_slots = slot;
  return last;
}

static void fill_map(fa_layout *L, const std::vector<DevRange> &ring_runs);

static fa_status build(const fa_layout_desc *din, int32_t ring_first, fa_layout *L) {
  int32_t hist_lo = 0, rf = 0;
  fa_status st = validate(din, ring_first, &hist_lo, &rf);
  if (st != FA_OK) return st;
  L->d = *din;
  fa_layout_desc &d = L->d;
  if (d.scale == 0.0f) d.scale = 1.0f / std::sqrt((float)d.head_dim);
  for (int r = d.n_ref; r < FA_MAX_REF; ++r) d.ref_tokens[r] = 0, d.ref_t0[r] = 0;
  L->ring_first = rf;
  L->hist_lo = hist_lo;
  const int T = d.tokens_per_frame, F = d.frames, cs = d.chunk_start;
  L->block_m = d.dtype == FA_F32 ? kF32BlockM : d.dtype == FA_BF16 ? kBf16BlockM : kLowbitBlockM;
  if (d.dtype == FA_BF16) L->block_m = d.block_rows ? d.block_rows : kBf16PPBlockM;
  L->block_n = d.dtype == FA_F32 ? kF32BlockN : d.dtype == FA_BF16 ? kBf16BlockN : kLowbitBlockN;
  int ref_total = 0;
  for (int r = 0; r < d.n_ref; ++r) ref_total += d.ref_tokens[r];
  L->ref_total = ref_total;
  L->q_rows[0] = (d.query_rows & FA_Q_TARGET) ? F * T : 0;
  L->q_rows[1] = (d.query_rows & FA_Q_SOURCE) ? F * T : 0;
  L->q_rows[2] = (d.query_rows & FA_Q_REF) ? ref_total : 0;

  // Ring runs: slots of the visible history frames (the sink frames before the chunk and the
  // window [hist_lo, cs)), as maximal runs in slot order (the softmax does not care about key
  // order).
  const int S = d.sink_frames;
  const int hist_frames = (cs - hist_lo) + std::min(S, hist_lo);
  L->hist_frames = hist_frames;
  std::vector<DevRange> ring_runs;
  if (hist_frames > 0) {
    const int cap = d.cache_frames;
    std::vector<char> used(cap, 0);
    for (int g = 0; g < cs; ++g)
      if (g >= hist_lo || g < S) used[ring_slot(g, S, cap)] = 1;
    for (int s = 0; s < cap;) {
      if (!used[s]) { ++s; continue; }
      int e = s;
      while (e < cap && used[e]) ++e;
      ring_runs.push_back(DevRange{FA_SEG_RING, FA_MASK_NONE, s * T, e * T, 0, {0, 0, 0}});
      s = e;
    }
  }

  fill_map(L, ring_runs);
  if (d.dtype == FA_BF16 && L->block_m == kBf16PPBlockM) {
    int64_t live = 0;
    for (const DevWork &w : L->work) live += w.tile >= 0;
    const double last = split_last_round(L);
    if (d.block_rows == 0) {
      // 256 rows unless the 128-row kernel (two workgroups per CU) needs clearly fewer rounds
      // over the chip's 256 CUs, the split part of a last round counting as its fraction of a
      // round.  The 256-row kernel runs a round of the same rows ~9% faster (3600-token chunk:
      // 4 rounds of either), hence the 0.95.
      const int64_t rounds = (live + 255) / 256;
      const double pp = (double)(rounds > 0 ? rounds - 1 : 0) + (rounds > 0 ? last : 0.0);
      int64_t items = 0;
      for (int k = 0; k < 3; ++k) items += (L->q_rows[k] + kBf16BlockM - 1) / kBf16BlockM;
      items *= (int64_t)d.batch * d.heads;
      const int64_t r128 = (items + 511) / 512;
      if (0.95 * pp > (double)r128) {
        L->tiles.clear();
        L->ranges.clear();
        L->work.clear();
        L->splits.clear();
        L->ws_slots = 0;
        L->block_m = kBf16BlockM;
        fill_map(L, ring_runs);
      }
    }
  }
  return FA_OK;
}

// Tiles and key ranges of the block map at L->block_m rows per tile, the work counts, and the
// work order.
static void fill_map(fa_layout *L, const std::vector<DevRange> &ring_runs) {
  const fa_layout_desc &d = L->d;
  const int T = d.tokens_per_frame, F = d.frames, cs = d.chunk_start;
  const int ref_total = L->ref_total, hist_frames = L->hist_frames;
  const int BM = L->block_m;
  for (int kind = 0; kind < 3; ++kind) {
    const int rows = L->q_rows[kind];
    for (int row0 = 0; row0 < rows; row0 += BM) {
      DevTile t{};
      t.q_kind = kind;
      t.row0 = row0;
      t.rows = std::min(BM, rows - row0);
      t.r_begin = (int)L->ranges.size();
      std::vector<DevRange> &R = L->ranges;
      if (kind == 2) {
        if (ref_total > 0) R.push_back(DevRange{FA_SEG_REF, FA_MASK_NONE, 0, ref_total, 0, {0, 0, 0}});
      } else {
        const int fa_rel = row0 / T, fb_rel = (row0 + t.rows - 1) / T;
        if (kind == 0) {
          for (const DevRange &rr : ring_runs) R.push_back(rr);
          R.push_back(DevRange{FA_SEG_TGT, FA_MASK_NONE, 0, F * T, 0, {0, 0, 0}});
        }
        R.push_back(DevRange{FA_SEG_SRC, fa_rel == fb_rel ? FA_MASK_NONE : FA_MASK_SAME_FRAME,
                             fa_rel * T, (fb_rel + 1) * T, 0, {0, 0, 0}});
        add_ref_ranges(&d, fa_rel, fb_rel, R);
      }
      t.r_count = (int)L->ranges.size() - t.r_begin;
      L->tiles.push_back(t);
    }
  }
  L->n_tiles = (int32_t)L->tiles.size();

  // Work counts.
  const double BH = (double)d.batch * d.heads;
  double useful = 0;
  for (int kind = 0; kind < 2; ++kind) {
    if (!L->q_rows[kind]) continue;
    for (int f = 0; f < F; ++f) {
      double keys = T;  // own-frame source
      if (kind == 0) keys += (double)(F + hist_frames) * T;
      for (int r = 0; r < d.n_ref; ++r)
        if (cs + f >= d.ref_t0[r]) keys += d.ref_tokens[r];
      useful += keys * T;
    }
  }
  if (L->q_rows[2]) useful += (double)ref_total * ref_total;
  L->useful_pairs = useful * BH;
  double visited = 0;
  for (const DevTile &t : L->tiles) {
    double keys = 0;
    for (int i = 0; i < t.r_count; ++i)
      keys += L->ranges[t.r_begin + i].end - L->ranges[t.r_begin + i].begin;
    visited += keys * t.rows;
  }
  L->visited_pairs = visited * BH;
  // Algorithmic bytes: each element of Q, of every key segment some range reads, and of V, read
  // once; O and LSE written once.
  const double eq = d.dtype == FA_F32 ? 4 : d.dtype == FA_BF16 ? 2 : 1;
  const double ek = eq, ev = eq, eo = d.dtype == FA_F32 ? 4 : 2;
  bool seg_used[4] = {false, false, false, false};
  double seg_keys[4] = {0, 0, 0, 0};
  for (const DevRange &r : L->ranges) seg_used[r.seg] = true;
  seg_keys[FA_SEG_RING] = (double)hist_frames * T;
  seg_keys[FA_SEG_TGT] = (double)F * T;
  seg_keys[FA_SEG_SRC] = (double)F * T;
  seg_keys[FA_SEG_REF] = ref_total;
  double keys = 0;
  for (int s = 0; s < 4; ++s) keys += seg_used[s] ? seg_keys[s] : 0;
  double qrows = (double)L->q_rows[0] + L->q_rows[1] + L->q_rows[2];
  L->bytes = BH * d.head_dim * (qrows * (eq + eo) + keys * (ek + ev)) + BH * qrows * 4;

  // Work order.  Kinds in decreasing cost (target rows read the most keys), each kind's items
  // in (batch, head, tile) order cut into 8 contiguous parts, part x to XCD x.  Workgroups are
  // handed to the XCDs round robin by grid index, so slot j*8 + x runs on XCD x: the
  // workgroups an XCD runs together share heads, and their K/V reads hit that XCD's L2.
  std::vector<std::vector<DevWork>> per_kind(3);
  std::vector<double> kind_cost(3, 0.0);
  for (int i = 0; i < (int)L->tiles.size(); ++i) {
    const DevTile &t = L->tiles[i];
    double c = 0;
    for (int j = 0; j < t.r_count; ++j)
      c += L->ranges[t.r_begin + j].end - L->ranges[t.r_begin + j].begin;
    kind_cost[t.q_kind] = std::max(kind_cost[t.q_kind], c);
  }
  for (int b = 0; b < d.batch; ++b)
    for (int h = 0; h < d.heads; ++h)
      for (int i = 0; i < (int)L->tiles.size(); ++i)
        per_kind[L->tiles[i].q_kind].push_back(DevWork{i, b * d.heads + h});
  int order[3] = {0, 1, 2};
  std::stable_sort(order, order + 3, [&](int a, int b) { return kind_cost[a] > kind_cost[b]; });
  std::vector<std::vector<DevWork>> xcd(8);
  for (int k : order) {
    const size_t n = per_kind[k].size();
    for (size_t x = 0; x < 8; ++x)
      for (size_t i = x * n / 8; i < (x + 1) * n / 8; ++i) xcd[x].push_back(per_kind[k][i]);
  }
  size_t maxlen = 0;
  for (auto &v : xcd) maxlen = std::max(maxlen, v.size());
  L->work.assign(maxlen * 8, DevWork{-1, 0});
  for (size_t x = 0; x < 8; ++x)
    for (size_t j = 0; j < xcd[x].size(); ++j) L->work[j * 8 + x] = xcd[x][j];
}

fa_status device_map(const fa_layout *L, DeviceMap *out, bool may_upload) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(FA_ERR_HIP, "hipGetDevice failed");
  std::lock_guard<std::mutex> g(L->mu);
  auto it = L->dev.find(dev);
  if (it != L->dev.end()) {
    *out = it->second;
    return FA_OK;
  }
  if (!may_upload)
    return fail(FA_ERR_INVALID,
                "the layout's block map is not on this device yet: call fa_layout_prepare "
                "before capturing the stream");
  DeviceMap m;
  const size_t nt = std::max<size_t>(1, L->tiles.size()), nr = std::max<size_t>(1, L->ranges.size()),
               nw = std::max<size_t>(1, L->work.size()), ns = std::max<size_t>(1, L->splits.size());
  const size_t wsb = ws_bytes(L);
  auto free_all = [&]() {
    if (m.tiles) (void)hipFree(m.tiles);
    if (m.ranges) (void)hipFree(m.ranges);
    if (m.work) (void)hipFree(m.work);
    if (m.splits) (void)hipFree(m.splits);
    if (m.ws) (void)hipFree(m.ws);
  };
  if (hipMalloc(&m.tiles, nt * sizeof(DevTile)) != hipSuccess ||
      hipMalloc(&m.ranges, nr * sizeof(DevRange)) != hipSuccess ||
      hipMalloc(&m.work, nw * sizeof(DevWork)) != hipSuccess ||
      hipMalloc(&m.splits, ns * sizeof(DevSplit)) != hipSuccess ||
      (wsb && hipMalloc(&m.ws, wsb) != hipSuccess)) {
    (void)hipGetLastError();
    free_all();
    return fail(FA_ERR_NOMEM, "device allocation of the block map failed");
  }
  bool ok = true;
  auto put = [&](void *dst, const void *src, size_t bytes) {
    if (bytes) ok &= hipMemcpy(dst, src, bytes, hipMemcpyHostToDevice) == hipSuccess;
  };
  put(m.tiles, L->tiles.data(), L->tiles.size() * sizeof(DevTile));
  put(m.ranges, L->ranges.data(), L->ranges.size() * sizeof(DevRange));
  put(m.work, L->work.data(), L->work.size() * sizeof(DevWork));
  put(m.splits, L->splits.data(), L->splits.size() * sizeof(DevSplit));
  if (!ok) {
    (void)hipGetLastError();
    free_all();
    return fail(FA_ERR_HIP, "uploading the block map failed");
  }
  L->dev[dev] = m;
  *out = m;
  return FA_OK;
}

size_t ws_bytes(const fa_layout *L) {
  return (size_t)L->ws_slots * (size_t)ws_slot_floats(L->d.head_dim) * sizeof(float);
}

}  // namespace fa

using namespace fa;

namespace fa {
size_t map_image_bytes(const fa_layout *L, size_t *off_ranges, size_t *off_work,
                       size_t *off_splits) {
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t r = up(L->tiles.size() * sizeof(DevTile));
  const size_t w = r + up(L->ranges.size() * sizeof(DevRange));
  const size_t sp = w + up(L->work.size() * sizeof(DevWork));
  if (off_ranges) *off_ranges = r;
  if (off_work) *off_work = w;
  if (off_splits) *off_splits = sp;
  return sp + up(L->splits.size() * sizeof(DevSplit));
}
}  // namespace fa

extern "C" fa_status fa_layout_prepare(const fa_layout *L) {
  if (!L) return fail(FA_ERR_INVALID, "layout is NULL");
  if (L->work.empty()) return FA_OK;
  DeviceMap m;
  fa_status st = device_map(L, &m, true);
  if (st != FA_OK) return st;
  // pinned host image of the block map, the source of fa_attn_fwd_noalloc's per-call copy
  std::lock_guard<std::mutex> g(L->mu);
  if (!L->pinned) {
    size_t orr = 0, ow = 0, osp = 0;
    const size_t bytes = map_image_bytes(L, &orr, &ow, &osp);
    char *p = nullptr;
    if (hipHostMalloc((void **)&p, bytes, hipHostMallocDefault) != hipSuccess) {
      (void)hipGetLastError();
      return fail(FA_ERR_NOMEM, "pinned host allocation of the block map image failed");
    }
    std::memset(p, 0, bytes);
    std::memcpy(p, L->tiles.data(), L->tiles.size() * sizeof(DevTile));
    std::memcpy(p + orr, L->ranges.data(), L->ranges.size() * sizeof(DevRange));
    std::memcpy(p + ow, L->work.data(), L->work.size() * sizeof(DevWork));
    if (!L->splits.empty())
      std::memcpy(p + osp, L->splits.data(), L->splits.size() * sizeof(DevSplit));
    fa_layout *M = const_cast<fa_layout *>(L);
    M->off_ranges = orr;
    M->off_work = ow;
    M->off_splits = osp;
    L->pinned_bytes = bytes;
    L->pinned = p;
  }
  return FA_OK;
}

extern "C" fa_status fa_layout_build(const fa_layout_desc *d, int32_t ring_first_frame,
                                     fa_layout **out) {
  if (!out) return fail(FA_ERR_INVALID, "out is NULL");
  *out = nullptr;
  fa_layout *L = new (std::nothrow) fa_layout();
  if (!L) return fail(FA_ERR_NOMEM, "host allocation failed");
  fa_status st;
  try {
    st = build(d, ring_first_frame, L);
  } catch (const std::bad_alloc &) {
    st = fail(FA_ERR_NOMEM, "host allocation failed");
  }
  if (st != FA_OK) {
    delete L;
    return st;
  }
  *out = L;
  return FA_OK;
}

extern "C" fa_status fa_layout_stats(const fa_layout *L, double *useful_pairs, double *useful_flops,
                                     double *visited_pairs, double *bytes) {
  if (!L) return fail(FA_ERR_INVALID, "layout is NULL");
  if (useful_pairs) *useful_pairs = L->useful_pairs;
  if (useful_flops) *useful_flops = L->useful_pairs * 4.0 * L->d.head_dim;
  if (visited_pairs) *visited_pairs = L->visited_pairs;
  if (bytes) *bytes = L->bytes;
  return FA_OK;
}

extern "C" fa_status fa_layout_tiles(const fa_layout *L, int32_t *n_tiles, int32_t *block_m,
                                     int32_t *block_n) {
  if (!L) return fail(FA_ERR_INVALID, "layout is NULL");
  if (n_tiles) *n_tiles = L->n_tiles;
  if (block_m) *block_m = L->block_m;
  if (block_n) *block_n = L->block_n;
  return FA_OK;
}

static void copy_tile(const fa_layout *L, const DevTile &t, fa_tile_info *tile,
                      fa_range_info *ranges, int32_t cap) {
  if (tile) *tile = fa_tile_info{t.q_kind, t.row0, t.rows, t.r_count};
  if (ranges)
    for (int j = 0; j < t.r_count && j < cap; ++j) {
      const DevRange &r = L->ranges[t.r_begin + j];
      ranges[j] = fa_range_info{r.seg, r.begin, r.end, r.mask, r.param};
    }
}

extern "C" fa_status fa_layout_tile(const fa_layout *L, int32_t i, fa_tile_info *tile,
                                    fa_range_info *ranges, int32_t cap) {
  if (!L) return fail(FA_ERR_INVALID, "layout is NULL");
  if (i < 0 || i >= L->n_tiles) return fail(FA_ERR_INVALID, "tile index out of range");
  copy_tile(L, L->tiles[i], tile, ranges, cap);
  return FA_OK;
}

extern "C" fa_status fa_layout_workspace_bytes(const fa_layout *L, size_t *bytes) {
  if (!L) return fail(FA_ERR_INVALID, "layout is NULL");
  if (!bytes) return fail(FA_ERR_INVALID, "bytes is NULL");
  *bytes = ws_bytes(L);
  return FA_OK;
}

extern "C" fa_status fa_layout_splits(const fa_layout *L, int32_t *n_split, int32_t *n_parts) {
  if (!L) return fail(FA_ERR_INVALID, "layout is NULL");
  if (n_split) *n_split = (int32_t)L->splits.size();
  if (n_parts) *n_parts = L->ws_slots;
  return FA_OK;
}

extern "C" fa_status fa_layout_split(const fa_layout *L, int32_t s, int32_t *tile, int32_t *bh,
                                     int32_t *parts, int32_t p, fa_tile_info *part,
                                     fa_range_info *ranges, int32_t cap) {
  if (!L) return fail(FA_ERR_INVALID, "layout is NULL");
  if (s < 0 || s >= (int32_t)L->splits.size())
    return fail(FA_ERR_INVALID, "split index out of range");
  const DevSplit &sp = L->splits[s];
  if (p < -1 || p >= sp.parts) return fail(FA_ERR_INVALID, "part index out of range");
  if (tile) *tile = sp.tile;
  if (bh) *bh = sp.bh;
  if (parts) *parts = sp.parts;
  if (p >= 0) {
    // the part tiles follow the block map's tiles in slot order
    const int32_t ti = L->n_tiles + sp.slot0 + p;
    copy_tile(L, L->tiles[ti], part, ranges, cap);
  }
  return FA_OK;
}

extern "C" fa_status fa_layout_destroy(fa_layout *L) {
  if (!L) return FA_OK;
  {
    std::lock_guard<std::mutex> g(L->mu);
    if (!L->dev.empty()) {
      int cur = 0;
      (void)hipGetDevice(&cur);
      for (auto &kv : L->dev) {
        (void)hipSetDevice(kv.first);
        (void)hipFree(kv.second.tiles);
        (void)hipFree(kv.second.ranges);
        (void)hipFree(kv.second.work);
        (void)hipFree(kv.second.splits);
        if (kv.second.ws) (void)hipFree(kv.second.ws);
      }
      (void)hipSetDevice(cur);
    }
    if (L->pinned) (void)hipHostFree(L->pinned);
  }
  delete L;
  return FA_OK;
}
