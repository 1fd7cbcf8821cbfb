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
  std::vector<fa::DevTile> tiles;
  std::vector<fa::DevRange> ranges;
  std::vector<fa::DevWork> work;  // grid order (XCD-interleaved)
  double useful_pairs = 0, visited_pairs = 0, bytes = 0;
  mutable std::mutex mu;
  mutable std::map<int, fa::DeviceMap> dev;  // per HIP device id
};

namespace fa {
// Device copy of L's block map for the current device (uploaded on first use).
// The layout's block map on the current device.  Uploads it on first use unless may_upload is
// false (a stream being captured into a graph must not allocate or copy synchronously).
fa_status device_map(const fa_layout *L, DeviceMap *out, bool may_upload = true);
}  // namespace fa
