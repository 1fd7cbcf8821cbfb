// fa_noalloc.hip -- fa_attn_fwd_noalloc: the attention call for callers that cannot allocate
// (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// fa_attn_fwd keeps a layout's block map (and, for layouts with split work items, the parts'
// workspace) in device memory the library allocates on first use.  This entry point instead
// copies the map, every call, into one file-scope device array per GPU (held until the process
// ends) whose first kNoallocMapBytes hold the map and whose remaining kNoallocWsBytes are the
// workspace, and launches the same kernels on it.  The copy's source is the pinned host image
// fa_layout_prepare makes, so the call enqueues one host-to-device copy and the kernels, and
// allocates and frees nothing.  Every call on a GPU shares that GPU's array: calls whose copy or
// kernels overlap on one GPU (different streams without ordering between them) race; calls on
// one stream are ordered.  The workspace needs no clearing: every slot a merge reads was
// written by the same call's attention kernel.
#include <map>
#include <mutex>

#include "fa_layout_impl.h"

namespace fa {

constexpr size_t kNoallocMapBytes = size_t(4) << 20;
// the most workspace a layout asks for: kMaxWsSlots slots at head_dim 128
constexpr size_t kNoallocWsBytes = size_t(kMaxWsSlots) * ws_slot_floats(128) * sizeof(float);

static __device__ __attribute__((aligned(256))) char scratch[kNoallocMapBytes + kNoallocWsBytes];

static std::mutex g_scratch_mu;
static std::map<int, char *> g_scratch_ptr;  // device id -> address of that device's `scratch`

// The current device's address of `scratch`, looked up once per device with the device
// current.  The host-side name of the array is not a device address and is never used as one.
static fa_status scratch_address(char **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return fail(FA_ERR_HIP, "hipGetDevice failed");
  }
  std::lock_guard<std::mutex> g(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it == g_scratch_ptr.end()) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return fail(FA_ERR_HIP, std::string("hipGetSymbolAddress of the static block-map array: ") +
                                  hipGetErrorString(e));
    }
    it = g_scratch_ptr.emplace(dev, (char *)p).first;
  }
  *out = it->second;
  return FA_OK;
}

}  // namespace fa

using namespace fa;

extern "C" fa_status fa_attn_fwd_noalloc(const fa_layout *L, const fa_io *io,
                                         fa_hip_stream stream) {
  if (!L) return fail(FA_ERR_INVALID, "layout is NULL");
  if (!io) return fail(FA_ERR_INVALID, "io is NULL");
  if (L->work.empty()) return FA_OK;
  const size_t bytes = map_image_bytes(L, nullptr, nullptr, nullptr);
  if (bytes > kNoallocMapBytes)
    return fail(FA_ERR_CAPACITY, "block map of " + std::to_string(bytes) +
                                     " bytes exceeds the static array of fa_attn_fwd_noalloc (" +
                                     std::to_string(kNoallocMapBytes) + " bytes); use fa_attn_fwd");
  if (ws_bytes(L) > kNoallocWsBytes)
    return fail(FA_ERR_CAPACITY, "key-part workspace exceeds the static array of "
                                 "fa_attn_fwd_noalloc; use fa_attn_fwd");
  char *src = nullptr;
  size_t orr = 0, ow = 0, osp = 0;
  {
    std::lock_guard<std::mutex> g(L->mu);
    src = L->pinned;
    orr = L->off_ranges;
    ow = L->off_work;
    osp = L->off_splits;
  }
  if (!src)
    return fail(FA_ERR_INVALID, "fa_attn_fwd_noalloc needs a prepared layout (fa_layout_prepare "
                                "makes the pinned block-map image it copies from)");
  char *dst = nullptr;
  fa_status st = scratch_address(&dst);
  if (st != FA_OK) return st;
  const hipError_t e = hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice, (hipStream_t)stream);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(FA_ERR_HIP, std::string("block map copy: ") + hipGetErrorString(e));
  }
  DeviceMap m;
  m.tiles = (DevTile *)dst;
  m.ranges = (DevRange *)(dst + orr);
  m.work = (DevWork *)(dst + ow);
  m.splits = (DevSplit *)(dst + osp);
  m.ws = L->ws_slots ? (float *)(dst + kNoallocMapBytes) : nullptr;
  return attn_fwd_map(L, io, (hipStream_t)stream, &m);
}
