// fa_api.cpp -- the C ABI: errors, I/O validation, kernel dispatch, ring
// append and the streaming driver.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "fa_layout_impl.h"

namespace fa {

static thread_local std::string g_last_error;

void set_error(const std::string &msg) { g_last_error = msg; }

fa_status fail(fa_status s, const std::string &msg) {
  g_last_error = msg;
  return s;
}

static int elem_q(int dtype) { return dtype == FA_F32 ? 4 : dtype == FA_BF16 ? 2 : 1; }
static int elem_o(int dtype) { return dtype == FA_F32 ? 4 : 2; }

static fa_status check_tensor(const fa_tensor &t, int esize, int batch, const char *name,
                              bool need_scale) {
  if (!t.data) return fail(FA_ERR_INVALID, std::string(name) + ": data is NULL");
  const uintptr_t p = (uintptr_t)t.data;
  if (p % 16) return fail(FA_ERR_INVALID, std::string(name) + ": base pointer not 16-byte aligned");
  if ((t.stride_n * esize) % 16 || (t.stride_h * esize) % 16 ||
      (batch > 1 && (t.stride_b * esize) % 16))
    return fail(FA_ERR_INVALID, std::string(name) + ": strides keep rows 16-byte aligned only if "
                                                    "stride*element_size is a multiple of 16");
  if (t.stride_n < 0 || t.stride_h < 0 || t.stride_b < 0)
    return fail(FA_ERR_INVALID, std::string(name) + ": negative stride");
  if (need_scale && !t.scale)
    return fail(FA_ERR_INVALID, std::string(name) + ": low-bit scale array is NULL");
  return FA_OK;
}

static Seg seg_of(const fa_tensor &t, int ntok) {
  Seg s{};
  s.p = t.data;
  s.sb = t.stride_b;
  s.sn = t.stride_n;
  s.sh = t.stride_h;
  s.scale = t.scale;
  s.nblk = (ntok + kQuantBlock - 1) / kQuantBlock;
  return s;
}

static const char *kQName[3] = {"q_tgt", "q_src", "q_ref"};
static const char *kOName[3] = {"o_tgt", "o_src", "o_ref"};
static const char *kKName[4] = {"k_ring", "k_tgt", "k_src", "k_ref"};
static const char *kVName[4] = {"v_ring", "v_tgt", "v_src", "v_ref"};

fa_status attn_fwd_map(const fa_layout *L, const fa_io *io, hipStream_t stream,
                       const DeviceMap *map) {
  if (!L) return fail(FA_ERR_INVALID, "layout is NULL");
  if (!io) return fail(FA_ERR_INVALID, "io is NULL");
  const fa_layout_desc &d = L->d;
  const bool low = d.dtype == FA_LOWBIT;
  const int eq = elem_q(d.dtype), eo = elem_o(d.dtype);
  const fa_tensor *qs[3] = {&io->q_tgt, &io->q_src, &io->q_ref};
  const fa_tensor *os[3] = {&io->o_tgt, &io->o_src, &io->o_ref};
  const fa_tensor *ks[4] = {&io->k_ring, &io->k_tgt, &io->k_src, &io->k_ref};
  const fa_tensor *vs[4] = {&io->v_ring, &io->v_tgt, &io->v_src, &io->v_ref};
  float *lses[3] = {io->lse_tgt, io->lse_src, io->lse_ref};
  const int T = d.tokens_per_frame;
  const int seg_tok[4] = {d.cache_frames * T, d.frames * T, d.frames * T, L->ref_total};
  bool used[4] = {false, false, false, false};
  for (const DevRange &r : L->ranges) used[r.seg] = true;
  AttnArgs a{};
  for (int k = 0; k < 3; ++k) {
    if (!L->q_rows[k]) continue;
    fa_status st = check_tensor(*qs[k], eq, d.batch, kQName[k], low);
    if (st != FA_OK) return st;
    st = check_tensor(*os[k], eo, d.batch, kOName[k], false);
    if (st != FA_OK) return st;
    if (lses[k] && ((uintptr_t)lses[k]) % 4) return fail(FA_ERR_INVALID, "lse not 4-byte aligned");
    a.q[k] = seg_of(*qs[k], L->q_rows[k]);
    a.o[k] = seg_of(*os[k], L->q_rows[k]);
    a.lse[k] = lses[k];
    a.q_rows[k] = L->q_rows[k];
  }
  for (int s = 0; s < 4; ++s) {
    if (!used[s]) continue;
    fa_status st = check_tensor(*ks[s], eq, d.batch, kKName[s], low);
    if (st != FA_OK) return st;
    st = check_tensor(*vs[s], eq, d.batch, kVName[s], low);
    if (st != FA_OK) return st;
    if (d.dtype != FA_F32) {
      // the tiled kernels bound each key tile with a buffer descriptor over whole rows
      for (const fa_tensor *t : {ks[s], vs[s]})
        if (t->stride_n < d.head_dim || t->stride_n > (1 << 24))
          return fail(FA_ERR_UNSUPPORTED, std::string(kKName[s]) +
                                              "/v: stride_n must be in [head_dim, 2^24]");
    }
    a.k[s] = seg_of(*ks[s], seg_tok[s]);
    a.v[s] = seg_of(*vs[s], seg_tok[s]);
  }
  a.T = T;
  a.H = d.heads;
  a.scale = d.scale;
  a.c = d.scale * 1.4426950408889634f;
  if (L->work.empty()) return FA_OK;
  DeviceMap m;
  if (map) {
    m = *map;
  } else {
    // Under stream capture the block map must already be on the device (fa_layout_prepare).
    hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &capture) != hipSuccess) {
      (void)hipGetLastError();
      capture = hipStreamCaptureStatusNone;
    }
    fa_status st = device_map(L, &m, capture == hipStreamCaptureStatusNone);
    if (st != FA_OK) return st;
  }
  a.tiles = m.tiles;
  a.ranges = m.ranges;
  a.work = m.work;
  a.ws = io->workspace ? (float *)io->workspace : m.ws;
  a.splits = m.splits;
  if (io->workspace && ((uintptr_t)io->workspace) % 16)
    return fail(FA_ERR_INVALID, "workspace not 16-byte aligned");
  if (io->workspace && io->workspace_bytes < ws_bytes(L))
    return fail(FA_ERR_INVALID, "workspace of " + std::to_string(io->workspace_bytes) +
                                    " bytes; the layout needs " + std::to_string(ws_bytes(L)));
  if (!L->splits.empty() && !a.ws) return fail(FA_ERR_INVALID, "split layout without a workspace");
  const int grid = (int)L->work.size();
  hipError_t e;
  if (d.dtype == FA_F32)
    e = launch_attn_f32(a, d.head_dim, grid, stream);
  else if (d.dtype == FA_BF16)
    e = launch_attn_bf16(a, d.head_dim, L->block_m, grid, stream);
  else
    e = launch_attn_lowbit(a, d.head_dim, grid, stream);
  if (e != hipSuccess) return fail(FA_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(e));
  if (!L->splits.empty()) {
    e = launch_merge_parts(a, d.head_dim, (int)L->splits.size(), stream);
    if (e != hipSuccess)
      return fail(FA_ERR_HIP, std::string("merge launch: ") + hipGetErrorString(e));
  }
  return FA_OK;
}

static fa_status ring_append(const fa_layout_desc *d, const fa_tensor *k_ring,
                             const fa_tensor *v_ring, const fa_tensor *k_chunk,
                             const fa_tensor *v_chunk, int32_t first_frame, int32_t frames,
                             hipStream_t stream) {
  if (!d || !k_ring || !v_ring || !k_chunk || !v_chunk)
    return fail(FA_ERR_INVALID, "NULL argument");
  if (d->cache_frames < 1) return fail(FA_ERR_INVALID, "cache_frames must be >= 1 to append");
  if (d->tokens_per_frame < 1 || d->heads < 1 || d->batch < 1)
    return fail(FA_ERR_INVALID, "bad geometry");
  if (d->head_dim != 64 && d->head_dim != 128) return fail(FA_ERR_UNSUPPORTED, "head_dim");
  if (d->sink_frames < 0 || d->sink_frames > d->cache_frames)
    return fail(FA_ERR_INVALID, "sink_frames must be in [0, cache_frames]");
  if (first_frame < 0) return fail(FA_ERR_INVALID, "first_frame must be >= 0");
  if (frames < 0) return fail(FA_ERR_INVALID, "frames must be >= 0");
  // non-sink frames of this append cycle through cache_frames - sink_frames slots
  const int64_t nonsink =
      (int64_t)first_frame + frames - std::max<int64_t>(first_frame, d->sink_frames);
  if (nonsink > (int64_t)d->cache_frames - d->sink_frames)
    return fail(FA_ERR_INVALID, "more non-sink frames than the ring's cycling slots");
  if (frames == 0) return FA_OK;
  if (d->batch > 32767 || (int64_t)frames * d->tokens_per_frame * d->heads > INT32_MAX)
    return fail(FA_ERR_UNSUPPORTED, "append: batch above 32767 or 2^31 (token, head) rows");
  const int es = d->dtype == FA_F32 ? 4 : 2;
  const fa_tensor *t[4] = {k_ring, v_ring, k_chunk, v_chunk};
  const char *nm[4] = {"k_ring", "v_ring", "k_chunk", "v_chunk"};
  for (int i = 0; i < 4; ++i) {
    fa_status st = check_tensor(*t[i], es, d->batch, nm[i], false);
    if (st != FA_OK) return st;
  }
  RingArgs a{};
  for (int i = 0; i < 2; ++i) {
    const fa_tensor &s = i ? *v_chunk : *k_chunk;
    const fa_tensor &r = i ? *v_ring : *k_ring;
    a.src[i] = s.data;
    a.dst[i] = r.data;
    a.ssb[i] = s.stride_b * es; a.ssn[i] = s.stride_n * es; a.ssh[i] = s.stride_h * es;
    a.dsb[i] = r.stride_b * es; a.dsn[i] = r.stride_n * es; a.dsh[i] = r.stride_h * es;
  }
  a.T = d->tokens_per_frame;
  a.H = d->heads;
  a.frames = frames;
  a.first_frame = first_frame;
  a.cache_frames = d->cache_frames;
  a.sink = d->sink_frames;
  a.chunks16 = d->head_dim * es / 16;
  a.batch = d->batch;
  hipError_t e = launch_ring_append(a, stream);
  if (e != hipSuccess) return fail(FA_ERR_HIP, std::string("ring append: ") + hipGetErrorString(e));
  return FA_OK;
}

static fa_status quantize_lowbit(const fa_layout *L, const fa_io *in, const fa_io *out,
                                 int32_t flags, hipStream_t stream) {
  if (!L || !in || !out) return fail(FA_ERR_INVALID, "NULL argument");
  const fa_layout_desc &d = L->d;
  if (d.dtype != FA_LOWBIT) return fail(FA_ERR_INVALID, "layout is not FA_LOWBIT");
  if (flags & ~(FA_QUANT_MEAN_GIVEN | FA_QUANT_RING_READY))
    return fail(FA_ERR_INVALID, "unknown flags");
  const bool ring_ready = (flags & FA_QUANT_RING_READY) != 0;
  if (ring_ready && !(flags & FA_QUANT_MEAN_GIVEN))
    return fail(FA_ERR_INVALID, "FA_QUANT_RING_READY needs FA_QUANT_MEAN_GIVEN (the ring's key "
                                "codes were made with that mean)");
  if (!out->k_mean) return fail(FA_ERR_INVALID, "k_mean is NULL");
  const int T = d.tokens_per_frame;
  QuantArgs qa{};
  qa.H = d.heads;
  qa.D = d.head_dim;
  qa.batch = d.batch;
  qa.k_mean = out->k_mean;
  qa.v_absmax = out->v_absmax;
  qa.softmax_scale = d.scale;
  int nseg = 0, blocks = 0;
  auto add = [&](const fa_tensor &ti, const fa_tensor &to, int ntok, int kind, int lo0, int hi0,
                 int lo1, int hi1, const char *name) -> fa_status {
    fa_status st = check_tensor(ti, 2, d.batch, name, false);
    if (st != FA_OK) return st;
    st = check_tensor(to, 1, d.batch, name, true);
    if (st != FA_OK) return st;
    if (nseg >= kMaxQSeg) return fail(FA_ERR_UNSUPPORTED, "too many tensors to quantise");
    QSeg &g = qa.seg[nseg++];
    g.in = ti.data; g.isb = ti.stride_b; g.isn = ti.stride_n; g.ish = ti.stride_h;
    g.out = to.data; g.osb = to.stride_b; g.osn = to.stride_n; g.osh = to.stride_h;
    g.scale = to.scale;
    g.nblk = (ntok + kQuantBlock - 1) / kQuantBlock;
    g.kind = kind;
    g.lo0 = lo0; g.hi0 = hi0; g.lo1 = lo1; g.hi1 = hi1;
    g.blk_begin = blocks;
    g.blk0 = 0;
    g.nproc = g.nblk;
    g.n = ntok;
    g.lse = nullptr;
    blocks += g.nproc;
    return FA_OK;
  };
  const fa_tensor *qi[3] = {&in->q_tgt, &in->q_src, &in->q_ref};
  const fa_tensor *qo[3] = {&out->q_tgt, &out->q_src, &out->q_ref};
  fa_status st;
  for (int k = 0; k < 3; ++k) {
    if (!L->q_rows[k]) continue;
    st = add(*qi[k], *qo[k], L->q_rows[k], 0, 0, L->q_rows[k], 0, 0, kQName[k]);
    if (st != FA_OK) return st;
    qa.seg[nseg - 1].lse = k == 0 ? out->lse_tgt : k == 1 ? out->lse_src : out->lse_ref;
  }
  // key tensors the block map reads, and the ring's slot runs in view
  bool used[4] = {false, false, false, false};
  int rlo[2] = {0, 0}, rhi[2] = {0, 0}, nrun = 0;
  for (const DevRange &r : L->ranges) {
    used[r.seg] = true;
    if (r.seg == FA_SEG_RING) {
      bool seen = false;
      for (int i = 0; i < nrun; ++i) seen |= (rlo[i] == r.begin && rhi[i] == r.end);
      if (!seen) {
        if (nrun >= 2) return fail(FA_ERR_UNSUPPORTED, "more than two ring runs");
        rlo[nrun] = r.begin;
        rhi[nrun] = r.end;
        ++nrun;
      }
    }
  }
  const fa_tensor *ki[4] = {&in->k_ring, &in->k_tgt, &in->k_src, &in->k_ref};
  const fa_tensor *ko[4] = {&out->k_ring, &out->k_tgt, &out->k_src, &out->k_ref};
  const fa_tensor *vi[4] = {&in->v_ring, &in->v_tgt, &in->v_src, &in->v_ref};
  const fa_tensor *vo[4] = {&out->v_ring, &out->v_tgt, &out->v_src, &out->v_ref};
  const int seg_tok[4] = {d.cache_frames * T, d.frames * T, d.frames * T, L->ref_total};
  for (int kind = 1; kind <= 2; ++kind)
    for (int sgi = 0; sgi < 4; ++sgi) {
      if (!used[sgi]) continue;
      const int n = seg_tok[sgi];
      if (sgi == FA_SEG_RING && ring_ready) {
        // the ring's codes are kept by fa_ring_quantize; only a requested v_absmax still takes
        // the V scales of the blocks in view
        if (kind == 1 || !out->v_absmax) continue;
        const fa_tensor &vc = *vo[sgi];
        if (!vc.scale) return fail(FA_ERR_INVALID, "v_ring: low-bit scale array is NULL");
        for (int i = 0; i < nrun; ++i) {
          if (rhi[i] <= rlo[i]) continue;
          if (nseg >= kMaxQSeg) return fail(FA_ERR_UNSUPPORTED, "too many tensors to quantise");
          QSeg &g = qa.seg[nseg++];
          g = QSeg{};
          g.scale = vc.scale;
          g.nblk = (n + kQuantBlock - 1) / kQuantBlock;
          g.kind = 3;
          g.blk_begin = blocks;
          g.blk0 = rlo[i] / kQuantBlock;
          g.nproc = (rhi[i] - 1) / kQuantBlock - g.blk0 + 1;
          g.n = n;
          blocks += g.nproc;
        }
        continue;
      }
      const int lo0 = sgi == FA_SEG_RING ? rlo[0] : 0, hi0 = sgi == FA_SEG_RING ? rhi[0] : n;
      const int lo1 = sgi == FA_SEG_RING ? rlo[1] : 0, hi1 = sgi == FA_SEG_RING ? rhi[1] : 0;
      st = add(kind == 1 ? *ki[sgi] : *vi[sgi], kind == 1 ? *ko[sgi] : *vo[sgi], n, kind, lo0,
               hi0, lo1, hi1, kind == 1 ? kKName[sgi] : kVName[sgi]);
      if (st != FA_OK) return st;
    }
  qa.nseg = nseg;
  qa.total_blocks = blocks;
  if ((int64_t)blocks * d.batch * d.heads >= (int64_t(1) << 31))
    return fail(FA_ERR_UNSUPPORTED, "too many quantisation blocks");
  hipError_t e = launch_quant_lowbit(qa, (flags & FA_QUANT_MEAN_GIVEN) != 0, stream);
  if (e != hipSuccess) return fail(FA_ERR_HIP, std::string("quantiser launch: ") + hipGetErrorString(e));
  return FA_OK;
}

// Re-quantises every 128-token block of the ring's code tensors that holds a token of frames
// [first_frame, first_frame + frames), from the bf16 ring (whole blocks, so a block shared with a
// neighbouring slot is coded from that slot's current bf16 contents too).
static fa_status ring_quantize(const fa_layout_desc *d, const fa_tensor *k_ring,
                               const fa_tensor *v_ring, const fa_tensor *k_codes,
                               const fa_tensor *v_codes, const float *k_mean, int32_t first_frame,
                               int32_t frames, hipStream_t stream) {
  if (!d || !k_ring || !v_ring || !k_codes || !v_codes || !k_mean)
    return fail(FA_ERR_INVALID, "NULL argument");
  if (d->dtype != FA_LOWBIT) return fail(FA_ERR_INVALID, "descriptor is not FA_LOWBIT");
  if (d->head_dim != 128) return fail(FA_ERR_UNSUPPORTED, "low-bit head_dim must be 128");
  if (d->cache_frames < 1 || d->tokens_per_frame < 1 || d->heads < 1 || d->batch < 1)
    return fail(FA_ERR_INVALID, "bad geometry");
  if (d->sink_frames < 0 || d->sink_frames > d->cache_frames)
    return fail(FA_ERR_INVALID, "sink_frames must be in [0, cache_frames]");
  if (first_frame < 0 || frames < 0) return fail(FA_ERR_INVALID, "negative frame range");
  const int64_t nonsink =
      (int64_t)first_frame + frames - std::max<int64_t>(first_frame, d->sink_frames);
  if (nonsink > (int64_t)d->cache_frames - d->sink_frames)
    return fail(FA_ERR_INVALID, "more non-sink frames than the ring's cycling slots");
  if (frames == 0) return FA_OK;
  const int T = d->tokens_per_frame;
  const int ntok = d->cache_frames * T;
  if ((int64_t)ntok * d->heads * d->batch >= (int64_t(1) << 31))
    return fail(FA_ERR_UNSUPPORTED, "ring too large");
  for (const fa_tensor *t : {k_ring, v_ring}) {
    fa_status st = check_tensor(*t, 2, d->batch, t == k_ring ? "k_ring" : "v_ring", false);
    if (st != FA_OK) return st;
  }
  for (const fa_tensor *t : {k_codes, v_codes}) {
    fa_status st = check_tensor(*t, 1, d->batch, t == k_codes ? "k_codes" : "v_codes", true);
    if (st != FA_OK) return st;
  }
  // block ranges touched by the frames' slots, merged
  std::vector<std::pair<int, int>> br;  // [b0, b1)
  for (int32_t g = first_frame; g < first_frame + frames; ++g) {
    const int slot = ring_slot(g, d->sink_frames, d->cache_frames);
    const int b0 = slot * T / kQuantBlock, b1 = ((slot + 1) * T + kQuantBlock - 1) / kQuantBlock;
    br.push_back({b0, b1});
  }
  std::sort(br.begin(), br.end());
  std::vector<std::pair<int, int>> merged;
  for (auto &r : br) {
    if (!merged.empty() && r.first <= merged.back().second)
      merged.back().second = std::max(merged.back().second, r.second);
    else
      merged.push_back(r);
  }
  QuantArgs qa{};
  qa.H = d->heads;
  qa.D = d->head_dim;
  qa.batch = d->batch;
  qa.k_mean = const_cast<float *>(k_mean);
  qa.v_absmax = nullptr;
  qa.softmax_scale = d->scale;
  int nseg = 0, blocks = 0;
  for (int kind = 1; kind <= 2; ++kind)
    for (auto &r : merged) {
      if (nseg >= kMaxQSeg) return fail(FA_ERR_UNSUPPORTED, "too many block runs in one call");
      const fa_tensor &ti = kind == 1 ? *k_ring : *v_ring;
      const fa_tensor &to = kind == 1 ? *k_codes : *v_codes;
      QSeg &g = qa.seg[nseg++];
      g = QSeg{};
      g.in = ti.data; g.isb = ti.stride_b; g.isn = ti.stride_n; g.ish = ti.stride_h;
      g.out = to.data; g.osb = to.stride_b; g.osn = to.stride_n; g.osh = to.stride_h;
      g.scale = to.scale;
      g.nblk = (ntok + kQuantBlock - 1) / kQuantBlock;
      g.kind = kind;
      g.lo0 = r.first * kQuantBlock;
      g.hi0 = std::min(r.second * kQuantBlock, ntok);
      g.blk_begin = blocks;
      g.blk0 = r.first;
      g.nproc = r.second - r.first;
      g.n = ntok;
      blocks += g.nproc;
    }
  qa.nseg = nseg;
  qa.total_blocks = blocks;
  hipError_t e = launch_quant_lowbit(qa, true, stream);
  if (e != hipSuccess) return fail(FA_ERR_HIP, std::string("ring quantiser: ") + hipGetErrorString(e));
  return FA_OK;
}

}  // namespace fa

using namespace fa;

extern "C" fa_status fa_ring_quantize(const fa_layout_desc *d, const fa_tensor *k_ring,
                                      const fa_tensor *v_ring, const fa_tensor *k_codes,
                                      const fa_tensor *v_codes, const float *k_mean,
                                      int32_t first_frame, int32_t frames, fa_hip_stream stream) {
  return ring_quantize(d, k_ring, v_ring, k_codes, v_codes, k_mean, first_frame, frames,
                       (hipStream_t)stream);
}

extern "C" fa_status fa_quantize_lowbit(const fa_layout *L, const fa_io *in, const fa_io *out,
                                        int32_t flags, fa_hip_stream stream) {
  return quantize_lowbit(L, in, out, flags, (hipStream_t)stream);
}

extern "C" const char *fa_status_str(fa_status s) {
  switch (s) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID: return "FA_ERR_INVALID";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_CAPACITY: return "FA_ERR_CAPACITY";
    case FA_ERR_HIP: return "FA_ERR_HIP";
    case FA_ERR_NOMEM: return "FA_ERR_NOMEM";
  }
  return "FA_ERR_UNKNOWN";
}

extern "C" const char *fa_last_error(void) { return g_last_error.c_str(); }

extern "C" fa_status fa_attn_fwd(const fa_layout *L, const fa_io *io, fa_hip_stream stream) {
  return attn_fwd_map(L, io, (hipStream_t)stream, nullptr);
}

extern "C" fa_status fa_ring_append(const fa_layout_desc *d, const fa_tensor *k_ring,
                                    const fa_tensor *v_ring, const fa_tensor *k_chunk,
                                    const fa_tensor *v_chunk, int32_t first_frame, int32_t frames,
                                    fa_hip_stream stream) {
  return ring_append(d, k_ring, v_ring, k_chunk, v_chunk, first_frame, frames,
                     (hipStream_t)stream);
}

// ---------------------------------------------------------------- streaming driver

struct fa_stream {
  fa_layout_desc d;
  int32_t next_frame = 0;
  int32_t ring_first = 0;
  std::vector<fa_layout *> cache;    // distinct block maps of the current reference set
  std::vector<fa_layout *> retired;  // layouts handed out earlier, kept until destroy
  fa_layout *current = nullptr;      // layout of the next chunk
};

namespace fa {

static bool same_map(const fa_layout *a, const fa_layout *b) {
  if (a->tiles.size() != b->tiles.size() || a->ranges.size() != b->ranges.size() ||
      a->work.size() != b->work.size() || a->splits.size() != b->splits.size() ||
      a->n_tiles != b->n_tiles || a->block_m != b->block_m)
    return false;
  // descriptors may differ only in chunk_start / ref_t0, both folded into the ranges
  fa_layout_desc x = a->d, y = b->d;
  x.chunk_start = y.chunk_start = 0;
  for (int r = 0; r < FA_MAX_REF; ++r) x.ref_t0[r] = y.ref_t0[r] = 0;
  if (std::memcmp(&x, &y, sizeof(fa_layout_desc)) != 0) return false;
  return std::memcmp(a->tiles.data(), b->tiles.data(), a->tiles.size() * sizeof(DevTile)) == 0 &&
         std::memcmp(a->ranges.data(), b->ranges.data(), a->ranges.size() * sizeof(DevRange)) == 0 &&
         std::memcmp(a->work.data(), b->work.data(), a->work.size() * sizeof(DevWork)) == 0 &&
         (a->splits.empty() ||
          std::memcmp(a->splits.data(), b->splits.data(), a->splits.size() * sizeof(DevSplit)) == 0);
}

// Layout of the chunk at s->next_frame, shared with an earlier chunk when the block map is the
// same (steady state repeats with the ring's period).  Stats of shared layouts are identical
// too, since they are functions of the block map and geometry.
static fa_status stream_layout(fa_stream *s, fa_layout **out) {
  if (s->current) {
    *out = s->current;
    return FA_OK;
  }
  fa_layout_desc d = s->d;
  d.chunk_start = s->next_frame;
  fa_layout *L = nullptr;
  fa_status st = fa_layout_build(&d, s->ring_first, &L);
  if (st != FA_OK) return st;
  for (fa_layout *c : s->cache)
    if (same_map(c, L)) {
      fa_layout_destroy(L);
      s->current = c;
      *out = c;
      return FA_OK;
    }
  if (s->cache.size() >= 64) {  // stop matching against the oldest one; it stays valid
    s->retired.push_back(s->cache.front());
    s->cache.erase(s->cache.begin());
  }
  s->cache.push_back(L);
  s->current = L;
  *out = L;
  return FA_OK;
}

// A layout the stream has handed out (fa_stream_layout, or a chunk still running on the device)
// must stay valid until fa_stream_destroy: a new reference set only retires the cached ones.
static void stream_reset_cache(fa_stream *s) {
  s->retired.insert(s->retired.end(), s->cache.begin(), s->cache.end());
  s->cache.clear();
  s->current = nullptr;
}

static void stream_free_layouts(fa_stream *s) {
  for (fa_layout *c : s->cache) fa_layout_destroy(c);
  for (fa_layout *c : s->retired) fa_layout_destroy(c);
  s->cache.clear();
  s->retired.clear();
  s->current = nullptr;
}

}  // namespace fa

extern "C" fa_status fa_stream_create(const fa_layout_desc *d, fa_stream **out) {
  if (!out) return fail(FA_ERR_INVALID, "out is NULL");
  *out = nullptr;
  if (!d) return fail(FA_ERR_INVALID, "descriptor is NULL");
  if (d->cache_frames < 1) return fail(FA_ERR_INVALID, "a stream needs cache_frames >= 1");
  fa_layout *probe = nullptr;  // validates the geometry at the first chunk position
  fa_status st = fa_layout_build(d, d->chunk_start, &probe);
  if (st == FA_ERR_CAPACITY) st = fa_layout_build(d, -1, &probe);
  if (st != FA_OK) return st;
  fa_layout_destroy(probe);
  fa_stream *s = new (std::nothrow) fa_stream();
  if (!s) return fail(FA_ERR_NOMEM, "host allocation failed");
  s->d = *d;
  s->next_frame = d->chunk_start;
  s->ring_first = d->chunk_start;
  *out = s;
  return FA_OK;
}

extern "C" fa_status fa_stream_layout(fa_stream *s, const fa_layout **out) {
  if (!s || !out) return fail(FA_ERR_INVALID, "NULL argument");
  fa_layout *L = nullptr;
  fa_status st = stream_layout(s, &L);
  *out = L;
  return st;
}

extern "C" fa_status fa_stream_advance(fa_stream *s, const fa_io *io, fa_hip_stream stream) {
  if (!s || !io) return fail(FA_ERR_INVALID, "NULL argument");
  fa_status st = ring_append(&s->d, &io->k_ring, &io->v_ring, &io->k_tgt, &io->v_tgt,
                             s->next_frame, s->d.frames, (hipStream_t)stream);
  if (st != FA_OK) return st;
  s->next_frame += s->d.frames;
  // the cycling part holds the last cache_frames - sink_frames frames; sink frames stay
  s->ring_first = std::max(s->ring_first, s->next_frame - (s->d.cache_frames - s->d.sink_frames));
  s->current = nullptr;
  return FA_OK;
}

extern "C" fa_status fa_stream_chunk(fa_stream *s, const fa_io *io, fa_hip_stream stream) {
  if (!s || !io) return fail(FA_ERR_INVALID, "NULL argument");
  if (s->d.dtype == FA_LOWBIT)
    return fail(FA_ERR_UNSUPPORTED,
                "low-bit streams: fa_stream_layout, fa_quantize_lowbit, fa_attn_fwd, then "
                "fa_stream_advance");
  fa_layout *L = nullptr;
  fa_status st = stream_layout(s, &L);
  if (st != FA_OK) return st;
  st = attn_fwd_map(L, io, (hipStream_t)stream, nullptr);
  if (st != FA_OK) return st;
  return fa_stream_advance(s, io, stream);
}

extern "C" fa_status fa_stream_state(const fa_stream *s, int32_t *next_frame,
                                     int32_t *ring_first_frame) {
  if (!s) return fail(FA_ERR_INVALID, "stream is NULL");
  if (next_frame) *next_frame = s->next_frame;
  if (ring_first_frame) *ring_first_frame = s->ring_first;
  return FA_OK;
}

extern "C" fa_status fa_stream_seek(fa_stream *s, int32_t next_frame, int32_t ring_first_frame) {
  if (!s) return fail(FA_ERR_INVALID, "stream is NULL");
  const int32_t S = s->d.sink_frames;
  if (next_frame < 0 || ring_first_frame < 0 || ring_first_frame > next_frame ||
      (next_frame > S &&
       next_frame - std::max(ring_first_frame, S) > s->d.cache_frames - S))
    return fail(FA_ERR_INVALID, "inconsistent stream state");
  s->next_frame = next_frame;
  s->ring_first = ring_first_frame;
  s->current = nullptr;
  return FA_OK;
}

extern "C" fa_status fa_stream_set_refs(fa_stream *s, int32_t n_ref, const int32_t *ref_tokens,
                                        const int32_t *ref_t0) {
  if (!s) return fail(FA_ERR_INVALID, "stream is NULL");
  if (n_ref < 0 || n_ref > FA_MAX_REF || (n_ref > 0 && (!ref_tokens || !ref_t0)))
    return fail(FA_ERR_INVALID, "bad reference set");
  for (int r = 0; r < n_ref; ++r)
    if (ref_tokens[r] < 0) return fail(FA_ERR_INVALID, "ref_tokens must be >= 0");
  s->d.n_ref = n_ref;
  for (int r = 0; r < FA_MAX_REF; ++r) {
    s->d.ref_tokens[r] = r < n_ref ? ref_tokens[r] : 0;
    s->d.ref_t0[r] = r < n_ref ? ref_t0[r] : 0;
  }
  stream_reset_cache(s);
  return FA_OK;
}

extern "C" fa_status fa_stream_destroy(fa_stream *s) {
  if (!s) return FA_OK;
  stream_free_layouts(s);
  delete s;
  return FA_OK;
}
