// noalloc.hip -- delta_diff_noalloc: delta_diff for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  The compaction's scratch (tile counts,
// scans, staging slots and arena) lives in a file-scope device array of this
// library instead of a caller workspace.
//
// The array exists once per GPU the library runs on and is held until the
// process ends.  Its device address is taken once per device with
// hipGetSymbolAddress, with that device current, and kept: in host code the
// array's name is only a stand-in and must never reach a kernel.  Every call
// on one GPU uses that GPU's array, so calls that overlap on one GPU (two
// streams, two threads) race; the calls' own kernels clear what must start at
// zero (the staging arena's fill counter, the dense-tile count), and nothing
// else is read before the same call writes it.
#include <atomic>

#include "sbd.h"
#include "sbd_internal.h"

namespace sbd {
namespace {

constexpr size_t kNoAllocScratchBytes = size_t(48) << 20;
// The fixed regions for 2^28 elements take 17.0 MiB; the rest of the array
// is staging arena (tiles that do not fit it are recomputed, same result).
constexpr int64_t kNoAllocMaxElems = int64_t(1) << 28;

__device__ __attribute__((aligned(256))) unsigned char scratch[kNoAllocScratchBytes];

// The device address of `scratch` on the current device, or nullptr with
// the runtime's message in `err`.
void* scratch_address(const char*& err) {
  static std::atomic<void*> ptrs[64];  // per device; zero until first taken
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    err = e != hipSuccess ? hipGetErrorString(e) : "device ordinal out of range";
    return nullptr;
  }
  void* p = ptrs[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      err = e != hipSuccess ? hipGetErrorString(e) : "null symbol address";
      return nullptr;
    }
    ptrs[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace
}  // namespace sbd

extern "C" {

int64_t delta_diff_noalloc_max_elems(void) { return sbd::kNoAllocMaxElems; }

delta_status delta_diff_noalloc(const uint16_t* old_bits, const uint16_t* new_bits, int64_t n,
                                int32_t* idx, uint16_t* val, int64_t capacity, int64_t* nnz,
                                void* stream) {
  using sbd::fail_with;
  if (n < 0 || capacity < 0)
    return fail_with(DELTA_E_INVALID, "delta_diff_noalloc: n=%lld capacity=%lld", (long long)n,
                     (long long)capacity);
  if (n > sbd::kNoAllocMaxElems)
    return fail_with(DELTA_E_RANGE,
                     "delta_diff_noalloc: n=%lld exceeds its static scratch (at most %lld "
                     "elements); use delta_diff with a workspace",
                     (long long)n, (long long)sbd::kNoAllocMaxElems);
  if (nnz == nullptr) return fail_with(DELTA_E_INVALID, "delta_diff_noalloc: nnz is null");
  if (n > 0 && (old_bits == nullptr || new_bits == nullptr))
    return fail_with(DELTA_E_INVALID, "delta_diff_noalloc: null input with n=%lld", (long long)n);
  if (capacity > 0 && (idx == nullptr || val == nullptr))
    return fail_with(DELTA_E_INVALID, "delta_diff_noalloc: null output with capacity=%lld",
                     (long long)capacity);
  const sbd::WsLayout L = sbd::ws_layout(sbd::max_tiles_for(n, 1), 1);
  if (L.wide > sbd::kNoAllocScratchBytes)  // cannot happen for n within the limit
    return fail_with(DELTA_E_WORKSPACE, "delta_diff_noalloc: layout of %zu bytes exceeds the "
                     "static scratch", L.wide);
  // the kernels run on the stream's device and take the current device's
  // array, so the two must be the same device
  if (stream != nullptr) {
    int cur = 0;
    hipDevice_t sdev = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess) e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail_with(DELTA_E_HIP, "delta_diff_noalloc: stream device: %s", hipGetErrorString(e));
    }
    if (static_cast<int>(sdev) != cur)
      return fail_with(DELTA_E_INVALID,
                       "delta_diff_noalloc: the stream belongs to device %d, the current "
                       "device is %d",
                       static_cast<int>(sdev), cur);
  }
  const char* why = nullptr;
  void* ws = sbd::scratch_address(why);
  if (ws == nullptr)
    return fail_with(DELTA_E_HIP, "delta_diff_noalloc: scratch address: %s", why);
  sbd::DiffParam single{old_bits, new_bits, n, 0, 0};
  const int64_t tiles = (n + sbd::kDiffTile - 1) / sbd::kDiffTile;
  sbd::clear_last_error();
  const hipError_t e =
      sbd::launch_diff(nullptr, single, 1, tiles, idx, false, val, capacity, nnz, nullptr, ws, L,
                       sbd::arena_quads_for(L, sbd::kNoAllocScratchBytes),
                       static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return fail_with(DELTA_E_HIP, "delta_diff_noalloc launch: %s", hipGetErrorString(e));
  return DELTA_OK;
}

}  // extern "C"
