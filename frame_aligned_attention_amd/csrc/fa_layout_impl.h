// fa_layout_impl.h -- host representation of a layout (block map + work order).
#pragma once

#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "fa_internal.h"

namespace fa {

void set_error(const std::string &msg);
fa_status fail(fa_status s, const std::string &msg);

struct DeviceMap {
  DevTile *tiles = nullptr;
  DevRange *ranges = nullptr;
  DevWork *work = nullptr;
  DevSplit *splits = nullptr;
  float *ws = nullptr;  // key-part workspace (layouts with split work items only)
};

}  // namespace fa

struct fa_layout {
  fa_layout_desc d;
  int32_t ring_first = 0;   // oldest frame the ring holds (resolved)
  int32_t hist_lo = 0;      // first frame of the visible window
  int32_t hist_frames = 0;  // visible history frames (window and sink frames before the chunk)
  int32_t block_m = 0, block_n = 0;
  int32_t q_rows[3] = {0, 0, 0};
  int32_t ref_total = 0;
  std::vector<fa::DevTile> tiles;   // the n_tiles query tiles, then the key parts of split items
  std::vector<fa::DevRange> ranges;
  std::vector<fa::DevWork> work;    // grid order (XCD-interleaved), key parts last
  std::vector<fa::DevSplit> splits; // split work items (their parts are in `tiles` and `work`)
  int32_t n_tiles = 0;              // query tiles of the block map proper
  int32_t ws_slots = 0;             // workspace slots the key parts use
  double useful_pairs = 0, visited_pairs = 0, bytes = 0;
  mutable std::mutex mu;
  mutable std::map<int, fa::DeviceMap> dev;  // per HIP device id
  // The block map as one pinned host image (tiles | ranges | work | splits, each part 256-byte
  // aligned),
  // made by fa_layout_prepare; fa_attn_fwd_noalloc copies it into its static device array.
  mutable char *pinned = nullptr;
  mutable size_t pinned_bytes = 0;
  size_t off_ranges = 0, off_work = 0, off_splits = 0;
};

namespace fa {
// Device copy of L's block map for the current device (uploaded on first use).
// The layout's block map on the current device.  Uploads it on first use unless may_upload is
// false (a stream being captured into a graph must not allocate or copy synchronously).
fa_status device_map(const fa_layout *L, DeviceMap *out, bool may_upload = true);
// Byte size of the block map as one image with each part 256-byte aligned (sets the offsets).
size_t map_image_bytes(const fa_layout *L, size_t *off_ranges, size_t *off_work,
                       size_t *off_splits);
// Bytes of the key-part workspace L's split work items need (0 if none).
size_t ws_bytes(const fa_layout *L);
// Checks the tensors of `io` against L and launches the attention kernel with the block map
// `map` (or, if NULL, the layout's own device copy, uploaded on first use).
fa_status attn_fwd_map(const fa_layout *L, const fa_io *io, hipStream_t stream,
                       const DeviceMap *map);
}  // namespace fa
