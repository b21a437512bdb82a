// abi.hip -- the extern "C" entry points declared in include/sbd.h:
// argument validation, workspace layout, parameter-table upload and launch.
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>
#include <vector>

#include "sbd.h"
#include "sbd_internal.h"

namespace {

thread_local std::string g_error;

delta_status fail(delta_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return s;
}

delta_status ok() { return DELTA_OK; }

delta_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(DELTA_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t kInt32Max = 2147483647LL;
// No buffer holds 2^62 elements: a count above it is refused before any size
// or grid computation could overflow.
constexpr int64_t kMaxCount = int64_t(1) << 62;

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// The workspace regions are laid out at 256-byte offsets and written with
// 16-byte stores, so the workspace itself must start on a 256-byte boundary
// (every hipMalloc and torch allocation does).
bool ws_aligned(const void* ws) { return (reinterpret_cast<uintptr_t>(ws) & 255u) == 0; }

}  // namespace

namespace sbd {

delta_status fail_with(delta_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return s;
}

void clear_last_error() { g_error.clear(); }

int64_t max_tiles_for(int64_t total_elems, int32_t nparams) {
  // each parameter adds at most one partial tile
  return total_elems / kDiffTile + int64_t(nparams) + 1;
}

WsLayout ws_layout(int64_t max_tiles, int32_t nparams) {
  const size_t tiles = size_t(max_tiles);
  const size_t chunks = (tiles + size_t(kScanChunk) - 1) / size_t(kScanChunk);
  WsLayout L;
  const size_t entry = sizeof(DiffParam) > sizeof(SnapParam) ? sizeof(DiffParam) : sizeof(SnapParam);
  L.ndense = 0;
  L.arena_next = 8;
  L.counts = 256;
  L.inpfx = L.counts + align256(sizeof(uint32_t) * tiles);
  L.chunk_tot = L.inpfx + align256(sizeof(uint32_t) * tiles);
  L.chunk_base = L.chunk_tot + align256(sizeof(uint32_t) * chunks);
  L.dense_list = L.chunk_base + align256(sizeof(uint64_t) * (chunks + 1));
  L.tile_desc = L.dense_list + align256(sizeof(int32_t) * tiles);
  L.table = L.tile_desc + align256(sizeof(TileDesc) * tiles);
  L.tile_pos = L.table + align256(entry * size_t(nparams > 0 ? nparams : 1));
  // The slots start a fixed 9472 bytes past a 1 MB boundary of the workspace,
  // whatever the table sizes before them.  Where the compact slots fall
  // relative to HBM's channel interleave measurably changes the cost of the
  // count kernel's slot writes; with 4 KB slots, on the 7B-shaped list
  // (diff_many, ms): 1 MB
  // aligned 4.64, +256 B 4.66, +1280 B 4.56, +2048 B 4.65, +9472 B 4.55
  // (the best of those tried; rotating each tile's start in its slot was
  // worse still).
  constexpr size_t kSlotAlign = size_t(1) << 20, kSlotSkew = 9472;
  L.compact = (L.tile_pos + align256(sizeof(uint64_t) * tiles) + kSlotAlign - 1) /
                  kSlotAlign * kSlotAlign + kSlotSkew;
  L.wide = L.compact + sizeof(uint32_t) * size_t(kCompactWords) * tiles;
  L.total = L.wide + sizeof(uint32_t) * size_t(kWideWords) * tiles;
  return L;
}

uint64_t arena_quads_for(const WsLayout& L, size_t ws_bytes) {
  const size_t have = ws_bytes > L.wide ? ws_bytes - L.wide : 0;
  const size_t most = L.total - L.wide;
  return static_cast<uint64_t>((have < most ? have : most) / 16);
}

}  // namespace sbd

extern "C" {

size_t delta_workspace_size(int64_t total_elems, int32_t nparams) {
  if (total_elems < 0 || nparams < 0) return 0;
  return sbd::ws_layout(sbd::max_tiles_for(total_elems, nparams), nparams).total;
}

size_t delta_workspace_size_for(int64_t total_elems, int32_t nparams, int64_t capacity) {
  if (total_elems < 0 || nparams < 0 || capacity < 0) return 0;
  const int64_t tiles = sbd::max_tiles_for(total_elems, nparams);
  const sbd::WsLayout L = sbd::ws_layout(tiles, nparams);
  const int64_t keep = capacity < total_elems ? capacity : total_elems;
  // 4 bytes per kept entry, plus up to 16 bytes of quad rounding per tile;
  // none at all for capacity 0 (the minimum).  The worst case caps it, and is
  // taken directly where 4 bytes per entry would exceed it (so the product
  // cannot overflow).
  const size_t most = L.total - L.wide;
  size_t arena = 0;
  if (keep > 0)
    arena = size_t(keep) <= most / 4 ? align256(4 * size_t(keep) + 16 * size_t(tiles)) : most;
  return L.wide + (arena < most ? arena : most);
}

const char* delta_last_error(void) { return g_error.c_str(); }

delta_status delta_diff(const uint16_t* old_bits, const uint16_t* new_bits, int64_t n,
                        int32_t* idx, uint16_t* val, int64_t capacity, int64_t* nnz, void* ws,
                        size_t ws_bytes, void* stream) {
  if (n < 0) return fail(DELTA_E_INVALID, "delta_diff: n=%lld < 0", (long long)n);
  if (capacity < 0)
    return fail(DELTA_E_INVALID, "delta_diff: capacity=%lld < 0", (long long)capacity);
  if (n > kInt32Max)
    return fail(DELTA_E_RANGE, "delta_diff: n=%lld exceeds the int32 index range",
                (long long)n);
  if (nnz == nullptr) return fail(DELTA_E_INVALID, "delta_diff: nnz is null");
  if (n > 0 && (old_bits == nullptr || new_bits == nullptr))
    return fail(DELTA_E_INVALID, "delta_diff: null input with n=%lld", (long long)n);
  if (capacity > 0 && (idx == nullptr || val == nullptr))
    return fail(DELTA_E_INVALID, "delta_diff: null output with capacity=%lld",
                (long long)capacity);
  const sbd::WsLayout L = sbd::ws_layout(sbd::max_tiles_for(n, 1), 1);
  if (ws == nullptr || ws_bytes < L.wide)
    return fail(DELTA_E_WORKSPACE, "delta_diff: workspace %zu bytes, need at least %zu",
                ws_bytes, L.wide);
  if (!ws_aligned(ws))
    return fail(DELTA_E_WORKSPACE, "delta_diff: workspace not 256-byte aligned");
  sbd::DiffParam single{old_bits, new_bits, n, 0, 0};
  const int64_t tiles = (n + sbd::kDiffTile - 1) / sbd::kDiffTile;  // < kMaxTiles for n < 2^31
  g_error.clear();
  return hip_status(sbd::launch_diff(nullptr, single, 1, tiles, idx, false, val, capacity, nnz,
                                     nullptr, ws, L, sbd::arena_quads_for(L, ws_bytes),
                                     static_cast<hipStream_t>(stream)),
                    "delta_diff launch");
}

}  // extern "C"

namespace {

// delta_diff_many and delta_diff_many_sharded: validation, table upload and
// launch.  global_idx: int64 indices flat_offsets[p] + local index, else
// parameter-local int32 indices.
delta_status diff_many_impl(const char* fn, bool global_idx, int32_t nparams,
                            const uint16_t* const* old_ptrs, const uint16_t* const* new_ptrs,
                            const int64_t* numels, const int64_t* flat_offsets, void* idx,
                            uint16_t* val,
                            int64_t capacity, int64_t* nnz, int64_t* offsets, void* ws,
                            size_t ws_bytes, void* stream) {
  if (nparams < 0) return fail(DELTA_E_INVALID, "%s: nparams=%d < 0", fn, nparams);
  if (capacity < 0) return fail(DELTA_E_INVALID, "%s: capacity=%lld < 0", fn, (long long)capacity);
  if (offsets == nullptr) return fail(DELTA_E_INVALID, "%s: offsets is null", fn);
  if (nparams > 0 && (old_ptrs == nullptr || new_ptrs == nullptr || numels == nullptr ||
                      nnz == nullptr))
    return fail(DELTA_E_INVALID, "%s: null parameter array", fn);
  if (global_idx && nparams > 0 && flat_offsets == nullptr)
    return fail(DELTA_E_INVALID, "%s: flat_offsets is null", fn);
  std::vector<sbd::DiffParam> table(static_cast<size_t>(nparams > 0 ? nparams : 0));
  int64_t total = 0, tiles = 0;
  for (int32_t p = 0; p < nparams; ++p) {
    const int64_t n = numels[p];
    if (n < 0) return fail(DELTA_E_INVALID, "%s: numels[%d]=%lld < 0", fn, p, (long long)n);
    if (n > kInt32Max)
      return fail(DELTA_E_RANGE, "%s: numels[%d]=%lld exceeds the int32 index range", fn, p,
                  (long long)n);
    if (n > 0 && (old_ptrs[p] == nullptr || new_ptrs[p] == nullptr))
      return fail(DELTA_E_INVALID, "%s: null tensor pointer for parameter %d", fn, p);
    int64_t fo = 0;
    if (global_idx) {
      fo = flat_offsets[p];
      if (fo < 0)
        return fail(DELTA_E_INVALID, "%s: flat_offsets[%d]=%lld < 0", fn, p, (long long)fo);
      if (fo > INT64_MAX - n)
        return fail(DELTA_E_RANGE, "%s: flat_offsets[%d] + numel overflows int64", fn, p);
    }
    table[p] = sbd::DiffParam{old_ptrs[p], new_ptrs[p], n, tiles, fo};
    tiles += (n + sbd::kDiffTile - 1) / sbd::kDiffTile;
    total += n;
  }
  if (capacity > 0 && (idx == nullptr || val == nullptr))
    return fail(DELTA_E_INVALID, "%s: null output with capacity=%lld", fn, (long long)capacity);
  if (tiles >= sbd::kMaxTiles)
    return fail(DELTA_E_RANGE, "%s: %lld tiles exceed one launch (%lld)", fn, (long long)tiles,
                (long long)sbd::kMaxTiles);
  const sbd::WsLayout L = sbd::ws_layout(sbd::max_tiles_for(total, nparams), nparams);
  if (ws == nullptr || ws_bytes < L.wide)
    return fail(DELTA_E_WORKSPACE, "%s: workspace %zu bytes, need at least %zu", fn, ws_bytes,
                L.wide);
  if (!ws_aligned(ws)) return fail(DELTA_E_WORKSPACE, "%s: workspace not 256-byte aligned", fn);
  hipStream_t s = static_cast<hipStream_t>(stream);
  sbd::DiffParam* d_table = reinterpret_cast<sbd::DiffParam*>(static_cast<char*>(ws) + L.table);
  if (nparams > 0) {
    const hipError_t e = hipMemcpyAsync(d_table, table.data(), sizeof(sbd::DiffParam) * table.size(),
                                        hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_status(e, "table copy");
  }
  g_error.clear();
  sbd::DiffParam none{nullptr, nullptr, 0, 0, 0};
  return hip_status(sbd::launch_diff(nparams > 0 ? d_table : nullptr, none, nparams, tiles, idx,
                                     global_idx, val, capacity, nnz, offsets, ws, L,
                                     sbd::arena_quads_for(L, ws_bytes), s),
                    fn);
}

}  // namespace

extern "C" {

delta_status delta_diff_many(int32_t nparams, const uint16_t* const* old_ptrs,
                             const uint16_t* const* new_ptrs, const int64_t* numels,
                             int32_t* idx, uint16_t* val, int64_t capacity, int64_t* nnz,
                             int64_t* offsets, void* ws, size_t ws_bytes, void* stream) {
  return diff_many_impl("delta_diff_many", false, nparams, old_ptrs, new_ptrs, numels, nullptr,
                        idx, val, capacity, nnz, offsets, ws, ws_bytes, stream);
}

delta_status delta_diff_many_sharded(int32_t nparams, const uint16_t* const* old_ptrs,
                                     const uint16_t* const* new_ptrs, const int64_t* numels,
                                     const int64_t* flat_offsets, int64_t* idx, uint16_t* val,
                                     int64_t capacity, int64_t* nnz, int64_t* offsets, void* ws,
                                     size_t ws_bytes, void* stream) {
  return diff_many_impl("delta_diff_many_sharded", true, nparams, old_ptrs, new_ptrs, numels,
                        flat_offsets, idx, val, capacity, nnz, offsets, ws, ws_bytes, stream);
}

}  // extern "C"

namespace {

delta_status apply_one(const char* fn, uint16_t* snapshot, int64_t n, const int32_t* idx,
                       const uint16_t* val, int64_t nnz, int64_t* violations, void* stream) {
  if (n < 0 || nnz < 0)
    return fail(DELTA_E_INVALID, "%s: n=%lld nnz=%lld", fn, (long long)n, (long long)nnz);
  if (n > kInt32Max)
    return fail(DELTA_E_RANGE, "%s: n=%lld exceeds the int32 index range", fn, (long long)n);
  if (nnz > kMaxCount) return fail(DELTA_E_RANGE, "%s: nnz=%lld above 2^62", fn, (long long)nnz);
  if (nnz > 0 && (snapshot == nullptr || idx == nullptr || val == nullptr))
    return fail(DELTA_E_INVALID, "%s: null pointer with nnz=%lld", fn, (long long)nnz);
  sbd::SnapParam single{snapshot, n};
  g_error.clear();
  return hip_status(sbd::launch_apply(nullptr, single, 1, nullptr, idx, val, nnz, n, violations,
                                      static_cast<hipStream_t>(stream)),
                    fn);
}

}  // namespace

extern "C" {

delta_status delta_apply(uint16_t* snapshot, int64_t n, const int32_t* idx, const uint16_t* val,
                         int64_t nnz, void* stream) {
  return apply_one("delta_apply", snapshot, n, idx, val, nnz, nullptr, stream);
}

delta_status delta_apply_checked(uint16_t* snapshot, int64_t n, const int32_t* idx,
                                 const uint16_t* val, int64_t nnz, int64_t* violations,
                                 void* stream) {
  if (violations == nullptr)
    return fail(DELTA_E_INVALID, "delta_apply_checked: violations is null");
  return apply_one("delta_apply_checked", snapshot, n, idx, val, nnz, violations, stream);
}

delta_status delta_apply_many(int32_t nparams, uint16_t* const* snap_ptrs, const int64_t* numels,
                              const int32_t* idx, const uint16_t* val, const int64_t* offsets,
                              int64_t max_nnz, int64_t* violations, void* ws, size_t ws_bytes,
                              void* stream) {
  if (nparams < 0 || max_nnz < 0)
    return fail(DELTA_E_INVALID, "delta_apply_many: nparams=%d max_nnz=%lld", nparams,
                (long long)max_nnz);
  if (max_nnz > kMaxCount)
    return fail(DELTA_E_RANGE, "delta_apply_many: max_nnz=%lld above 2^62", (long long)max_nnz);
  if (nparams == 0 || max_nnz == 0) {
    g_error.clear();
    return hip_status(sbd::launch_apply(nullptr, sbd::SnapParam{nullptr, 0}, 0, nullptr, nullptr,
                                        nullptr, 0, 0, violations, static_cast<hipStream_t>(stream)),
                      "delta_apply_many launch");
  }
  if (snap_ptrs == nullptr || numels == nullptr || offsets == nullptr || idx == nullptr ||
      val == nullptr)
    return fail(DELTA_E_INVALID, "delta_apply_many: null pointer argument");
  std::vector<sbd::SnapParam> table(static_cast<size_t>(nparams));
  int64_t total_elems = 0;
  for (int32_t p = 0; p < nparams; ++p) {
    const int64_t n = numels[p];
    if (n < 0)
      return fail(DELTA_E_INVALID, "delta_apply_many: numels[%d]=%lld < 0", p, (long long)n);
    if (n > kInt32Max)
      return fail(DELTA_E_RANGE,
                  "delta_apply_many: numels[%d]=%lld exceeds the int32 index range", p,
                  (long long)n);
    if (n > 0 && snap_ptrs[p] == nullptr)
      return fail(DELTA_E_INVALID, "delta_apply_many: null snapshot for parameter %d", p);
    table[p] = sbd::SnapParam{snap_ptrs[p], n};
    total_elems += n;
  }
  const size_t need = 256 + align256(sizeof(sbd::SnapParam) * size_t(nparams));
  if (ws == nullptr || ws_bytes < need)
    return fail(DELTA_E_WORKSPACE, "delta_apply_many: workspace %zu bytes, need %zu", ws_bytes,
                need);
  if (!ws_aligned(ws))
    return fail(DELTA_E_WORKSPACE, "delta_apply_many: workspace not 256-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  sbd::SnapParam* d_table = reinterpret_cast<sbd::SnapParam*>(static_cast<char*>(ws) + 256);
  const hipError_t e = hipMemcpyAsync(d_table, table.data(), sizeof(sbd::SnapParam) * table.size(),
                                      hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return hip_status(e, "delta_apply_many table copy");
  g_error.clear();
  return hip_status(sbd::launch_apply(d_table, sbd::SnapParam{nullptr, 0}, nparams, offsets, idx,
                                      val, max_nnz, total_elems, violations, s),
                    "delta_apply_many launch");
}

size_t delta_streamed_staging_size(int32_t nparams, int32_t nchunks, int32_t max_chunk_params,
                                   int64_t max_chunk_nnz) {
  if (nparams < 0 || nchunks < 0 || max_chunk_params < 0 || max_chunk_nnz < 0) return 0;
  return sbd::streamed_staging_size(nparams, nchunks, max_chunk_params, max_chunk_nnz);
}

delta_status delta_apply_streamed(int32_t nparams, uint16_t* const* snap_ptrs,
                                  const int64_t* numels, int32_t nchunks,
                                  const delta_host_chunk* chunks, void* staging,
                                  size_t staging_bytes, void* copy_stream, void* apply_stream) {
  std::string err;
  const delta_status st = sbd::apply_streamed_impl(nparams, snap_ptrs, numels, nchunks, chunks,
                                                   staging, staging_bytes, copy_stream,
                                                   apply_stream, err);
  if (st != DELTA_OK) return fail(st, "%s", err.c_str());
  g_error.clear();
  return DELTA_OK;
}

delta_status delta_apply_many_host(int32_t nparams, uint16_t* const* snap_ptrs,
                                   const int64_t* numels, const int32_t* idx_host,
                                   const uint16_t* val_host, const int64_t* offsets_host,
                                   int64_t max_nnz, int64_t* violations, void* ws,
                                   size_t ws_bytes, void* stream) {
  if (max_nnz > kMaxCount)
    return fail(DELTA_E_RANGE, "delta_apply_many_host: max_nnz=%lld above 2^62",
                (long long)max_nnz);
  std::string err;
  const delta_status st =
      sbd::apply_host_impl(nparams, snap_ptrs, numels, idx_host, val_host, offsets_host, max_nnz,
                           violations, ws, ws_bytes, stream, err);
  if (st != DELTA_OK) return fail(st, "%s", err.c_str());
  g_error.clear();
  return DELTA_OK;
}

size_t xor_streamed_staging_size(int64_t chunk_elems) {
  return chunk_elems <= 0 ? 0 : sbd::xor_streamed_staging_size(chunk_elems);
}

delta_status xor_apply_streamed(uint16_t* snapshot, const uint16_t* mask_host, int64_t n,
                                int64_t chunk_elems, void* staging, size_t staging_bytes,
                                void* copy_stream, void* apply_stream) {
  if (n > kMaxCount) return fail(DELTA_E_RANGE, "xor_apply_streamed: n=%lld above 2^62", (long long)n);
  std::string err;
  const delta_status st = sbd::xor_apply_streamed_impl(snapshot, mask_host, n, chunk_elems,
                                                       staging, staging_bytes, copy_stream,
                                                       apply_stream, err);
  if (st != DELTA_OK) return fail(st, "%s", err.c_str());
  g_error.clear();
  return DELTA_OK;
}

}  // extern "C"

namespace {

// Bytes per position of a parameter in the per-parameter wire format: the
// narrowest of the two widths the pages allow (2 or 4 bytes) that holds every
// parameter-local index.
int wire_width(int64_t numel) { return numel <= 65536 ? 2 : 4; }

// Per-parameter position widths into the workspace's table region.
delta_status upload_widths(const char* fn, int32_t nparams, const int64_t* numels, void* ws,
                           size_t ws_bytes, hipStream_t s, int32_t** d_widths) {
  if (nparams < 0) return fail(DELTA_E_INVALID, "%s: nparams=%d < 0", fn, nparams);
  if (nparams > 0 && numels == nullptr) return fail(DELTA_E_INVALID, "%s: numels is null", fn);
  std::vector<int32_t> widths(static_cast<size_t>(nparams > 0 ? nparams : 1), 2);
  for (int32_t p = 0; p < nparams; ++p) {
    if (numels[p] < 0 || numels[p] > kInt32Max)
      return fail(numels[p] < 0 ? DELTA_E_INVALID : DELTA_E_RANGE,
                  "%s: numels[%d]=%lld outside [0, 2^31-1]", fn, p, (long long)numels[p]);
    widths[p] = wire_width(numels[p]);
  }
  const sbd::WsLayout L = sbd::ws_layout(sbd::max_tiles_for(0, nparams), nparams);
  if (ws == nullptr || ws_bytes < L.total)
    return fail(DELTA_E_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn, ws_bytes, L.total);
  if (!ws_aligned(ws)) return fail(DELTA_E_WORKSPACE, "%s: workspace not 256-byte aligned", fn);
  *d_widths = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + L.table);
  const hipError_t e = hipMemcpyAsync(*d_widths, widths.data(), sizeof(int32_t) * widths.size(),
                                      hipMemcpyHostToDevice, s);
  return e == hipSuccess ? DELTA_OK : hip_status(e, fn);
}

}  // namespace

extern "C" {

delta_status delta_wire_encode(int32_t nparams, const int64_t* numels, const int32_t* idx,
                               const int64_t* offsets, int64_t max_entries, uint8_t* positions,
                               int64_t positions_capacity, int64_t* pos_offsets, void* ws,
                               size_t ws_bytes, void* stream) {
  if (max_entries < 0 || positions_capacity < 0)
    return fail(DELTA_E_INVALID, "delta_wire_encode: negative size");
  if (max_entries > kMaxCount || positions_capacity > kMaxCount)
    return fail(DELTA_E_RANGE, "delta_wire_encode: size above 2^62");
  if (offsets == nullptr || pos_offsets == nullptr)
    return fail(DELTA_E_INVALID, "delta_wire_encode: null offsets");
  if (max_entries > 0 && idx == nullptr)
    return fail(DELTA_E_INVALID, "delta_wire_encode: null idx");
  if (positions_capacity > 0 && positions == nullptr)
    return fail(DELTA_E_INVALID, "delta_wire_encode: null positions");
  if ((reinterpret_cast<uintptr_t>(positions) & 1u) != 0)
    return fail(DELTA_E_INVALID, "delta_wire_encode: positions not 2-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* d_widths = nullptr;
  const delta_status st =
      upload_widths("delta_wire_encode", nparams, numels, ws, ws_bytes, s, &d_widths);
  if (st != DELTA_OK) return st;
  g_error.clear();
  return hip_status(sbd::launch_wire_encode(nparams, d_widths, idx, offsets, max_entries,
                                            positions, positions_capacity, pos_offsets, s),
                    "delta_wire_encode launch");
}

delta_status delta_wire_decode(int32_t nparams, const int64_t* numels, const uint8_t* positions,
                               int64_t positions_bytes, const int64_t* pos_offsets,
                               const int64_t* offsets, int64_t max_entries, int32_t* idx,
                               int64_t* violations, void* ws, size_t ws_bytes, void* stream) {
  if (max_entries < 0 || positions_bytes < 0)
    return fail(DELTA_E_INVALID, "delta_wire_decode: negative size");
  if (max_entries > kMaxCount || positions_bytes > kMaxCount)
    return fail(DELTA_E_RANGE, "delta_wire_decode: size above 2^62");
  if (offsets == nullptr || pos_offsets == nullptr)
    return fail(DELTA_E_INVALID, "delta_wire_decode: null offsets");
  if (max_entries > 0 && idx == nullptr) return fail(DELTA_E_INVALID, "delta_wire_decode: null idx");
  if (positions_bytes > 0 && positions == nullptr)
    return fail(DELTA_E_INVALID, "delta_wire_decode: null positions");
  if ((reinterpret_cast<uintptr_t>(positions) & 1u) != 0)
    return fail(DELTA_E_INVALID, "delta_wire_decode: positions not 2-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* d_widths = nullptr;
  const delta_status st =
      upload_widths("delta_wire_decode", nparams, numels, ws, ws_bytes, s, &d_widths);
  if (st != DELTA_OK) return st;
  g_error.clear();
  return hip_status(sbd::launch_wire_decode(nparams, d_widths, positions, positions_bytes,
                                            pos_offsets, offsets, max_entries, idx, violations,
                                            s),
                    "delta_wire_decode launch");
}

int64_t delta_wire_positions_size(int32_t nparams, const int64_t* numels,
                                  const int64_t* offsets_host) {
  if (nparams < 0 || (nparams > 0 && (numels == nullptr || offsets_host == nullptr))) return -1;
  int64_t bytes = 0;
  for (int32_t p = 0; p < nparams; ++p) {
    if (offsets_host[p] < 0 || offsets_host[p + 1] < offsets_host[p]) return -1;
    const int64_t count = offsets_host[p + 1] - offsets_host[p];
    if (numels[p] < 0 || numels[p] > kInt32Max) return -1;
    const int w = wire_width(numels[p]);
    if (count > (INT64_MAX - bytes) / w) return -1;  // the size would not fit int64
    bytes += count * w;
  }
  return bytes;
}

delta_status delta_wire_hash(const uint8_t* positions, int64_t npos, const uint16_t* values,
                             int64_t nval, uint64_t* hashes, void* stream) {
  if (npos < 0 || nval < 0) return fail(DELTA_E_INVALID, "delta_wire_hash: negative size");
  if (npos > kMaxCount || nval > kMaxCount)
    return fail(DELTA_E_RANGE, "delta_wire_hash: size above 2^62");
  if (hashes == nullptr || (npos > 0 && positions == nullptr) || (nval > 0 && values == nullptr))
    return fail(DELTA_E_INVALID, "delta_wire_hash: null pointer");
  g_error.clear();
  return hip_status(sbd::launch_wire_hash(positions, npos, values, nval, hashes,
                                          static_cast<hipStream_t>(stream)),
                    "delta_wire_hash launch");
}

delta_status delta_wire_checksum(const uint8_t* positions, int64_t npos, const uint16_t* values,
                                 int64_t nval, uint64_t* checksum, void* stream) {
  if (npos < 0 || nval < 0) return fail(DELTA_E_INVALID, "delta_wire_checksum: negative size");
  if (npos > kMaxCount || nval > kMaxCount)
    return fail(DELTA_E_RANGE, "delta_wire_checksum: size above 2^62");
  if (checksum == nullptr || (npos > 0 && positions == nullptr) ||
      (nval > 0 && values == nullptr))
    return fail(DELTA_E_INVALID, "delta_wire_checksum: null pointer");
  g_error.clear();
  return hip_status(sbd::launch_wire_checksum(positions, npos, values, nval, checksum,
                                              static_cast<hipStream_t>(stream)),
                    "delta_wire_checksum launch");
}

}  // extern "C"

namespace {

// The blocked-positions parameter table (size, first block) into the
// workspace's table region; the total block count in *nblocks.  A decode
// passes the received byte count: fewer bytes than the tables is rejected
// before anything is copied or launched.
delta_status upload_blocked(const char* fn, int32_t nparams, const int64_t* numels, void* ws,
                            size_t ws_bytes, hipStream_t s, sbd::BlockedParam** d_table,
                            int64_t* nblocks, int64_t in_bytes = -1) {
  if (nparams < 0) return fail(DELTA_E_INVALID, "%s: nparams=%d < 0", fn, nparams);
  if (nparams > 0 && numels == nullptr) return fail(DELTA_E_INVALID, "%s: numels is null", fn);
  std::vector<sbd::BlockedParam> table(static_cast<size_t>(nparams > 0 ? nparams : 1));
  int64_t t = 0;
  for (int32_t p = 0; p < nparams; ++p) {
    if (numels[p] < 0 || numels[p] > kInt32Max)
      return fail(numels[p] < 0 ? DELTA_E_INVALID : DELTA_E_RANGE,
                  "%s: numels[%d]=%lld outside [0, 2^31-1]", fn, p, (long long)numels[p]);
    table[p] = sbd::BlockedParam{numels[p], t};
    t += (numels[p] + sbd::kPosBlockElems - 1) / sbd::kPosBlockElems;
  }
  *nblocks = t;
  if (in_bytes >= 0 && 4 * t > in_bytes)
    return fail(DELTA_E_INVALID, "%s: %lld bytes hold less than the %lld block bases of the list",
                fn, (long long)in_bytes, (long long)t);
  const sbd::WsLayout L = sbd::ws_layout(sbd::max_tiles_for(0, nparams), nparams);
  if (ws == nullptr || ws_bytes < L.total)
    return fail(DELTA_E_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn, ws_bytes, L.total);
  if (!ws_aligned(ws)) return fail(DELTA_E_WORKSPACE, "%s: workspace not 256-byte aligned", fn);
  *d_table = reinterpret_cast<sbd::BlockedParam*>(static_cast<char*>(ws) + L.table);
  if (nparams == 0) return DELTA_OK;
  const hipError_t e = hipMemcpyAsync(*d_table, table.data(),
                                      sizeof(sbd::BlockedParam) * size_t(nparams),
                                      hipMemcpyHostToDevice, s);
  return e == hipSuccess ? DELTA_OK : hip_status(e, fn);
}

}  // namespace

extern "C" {

int64_t delta_wire_blocked_size(int32_t nparams, const int64_t* numels, int64_t entries) {
  if (nparams < 0 || entries < 0 || (nparams > 0 && numels == nullptr)) return -1;
  int64_t blocks = 0;
  for (int32_t p = 0; p < nparams; ++p) {
    if (numels[p] < 0 || numels[p] > kInt32Max) return -1;
    blocks += (numels[p] + sbd::kPosBlockElems - 1) / sbd::kPosBlockElems;
  }
  if (entries > (INT64_MAX - 4 * blocks) / 2) return -1;  // the size would not fit int64
  return 4 * blocks + 2 * entries;
}

delta_status delta_wire_encode_blocked(int32_t nparams, const int64_t* numels, const int32_t* idx,
                                       const int64_t* offsets, int64_t max_entries, uint8_t* out,
                                       int64_t out_capacity, void* ws, size_t ws_bytes,
                                       void* stream) {
  if (max_entries < 0 || out_capacity < 0)
    return fail(DELTA_E_INVALID, "delta_wire_encode_blocked: negative size");
  if (max_entries > kMaxCount || out_capacity > kMaxCount)
    return fail(DELTA_E_RANGE, "delta_wire_encode_blocked: size above 2^62");
  if (offsets == nullptr) return fail(DELTA_E_INVALID, "delta_wire_encode_blocked: null offsets");
  if (max_entries > 0 && idx == nullptr)
    return fail(DELTA_E_INVALID, "delta_wire_encode_blocked: null idx");
  if (out_capacity > 0 && out == nullptr)
    return fail(DELTA_E_INVALID, "delta_wire_encode_blocked: null output");
  if ((reinterpret_cast<uintptr_t>(out) & 3u) != 0)
    return fail(DELTA_E_INVALID, "delta_wire_encode_blocked: output not 4-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  sbd::BlockedParam* d_table = nullptr;
  int64_t nblocks = 0;
  const delta_status st = upload_blocked("delta_wire_encode_blocked", nparams, numels, ws,
                                         ws_bytes, s, &d_table, &nblocks);
  if (st != DELTA_OK) return st;
  g_error.clear();
  return hip_status(sbd::launch_wire_encode_blocked(nparams, d_table, nblocks, idx, offsets,
                                                    max_entries, out, out_capacity, s),
                    "delta_wire_encode_blocked launch");
}

delta_status delta_wire_decode_blocked(int32_t nparams, const int64_t* numels, const uint8_t* in,
                                       int64_t in_bytes, const int64_t* offsets,
                                       int64_t max_entries, int32_t* idx, int64_t* violations,
                                       void* ws, size_t ws_bytes, void* stream) {
  if (max_entries < 0 || in_bytes < 0)
    return fail(DELTA_E_INVALID, "delta_wire_decode_blocked: negative size");
  if (max_entries > kMaxCount || in_bytes > kMaxCount)
    return fail(DELTA_E_RANGE, "delta_wire_decode_blocked: size above 2^62");
  if (offsets == nullptr) return fail(DELTA_E_INVALID, "delta_wire_decode_blocked: null offsets");
  if (max_entries > 0 && idx == nullptr)
    return fail(DELTA_E_INVALID, "delta_wire_decode_blocked: null idx");
  if (in_bytes > 0 && in == nullptr)
    return fail(DELTA_E_INVALID, "delta_wire_decode_blocked: null input");
  if ((reinterpret_cast<uintptr_t>(in) & 3u) != 0)
    return fail(DELTA_E_INVALID, "delta_wire_decode_blocked: input not 4-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  sbd::BlockedParam* d_table = nullptr;
  int64_t nblocks = 0;
  const delta_status st = upload_blocked("delta_wire_decode_blocked", nparams, numels, ws,
                                         ws_bytes, s, &d_table, &nblocks, in_bytes);
  if (st != DELTA_OK) return st;
  g_error.clear();
  return hip_status(sbd::launch_wire_decode_blocked(nparams, d_table, nblocks, in, in_bytes,
                                                    offsets, max_entries, idx, violations, s),
                    "delta_wire_decode_blocked launch");
}

delta_status xor_mask(const uint16_t* old_bits, const uint16_t* new_bits, uint16_t* mask,
                      int64_t n, void* stream) {
  if (n < 0) return fail(DELTA_E_INVALID, "xor_mask: n=%lld < 0", (long long)n);
  if (n > kMaxCount) return fail(DELTA_E_RANGE, "xor_mask: n=%lld above 2^62", (long long)n);
  if (n > 0 && (old_bits == nullptr || new_bits == nullptr || mask == nullptr))
    return fail(DELTA_E_INVALID, "xor_mask: null pointer with n=%lld", (long long)n);
  g_error.clear();
  return hip_status(sbd::launch_xor_mask(old_bits, new_bits, mask, n,
                                         static_cast<hipStream_t>(stream)),
                    "xor_mask launch");
}

delta_status xor_apply(uint16_t* snapshot, const uint16_t* mask, int64_t n, void* stream) {
  if (n < 0) return fail(DELTA_E_INVALID, "xor_apply: n=%lld < 0", (long long)n);
  if (n > kMaxCount) return fail(DELTA_E_RANGE, "xor_apply: n=%lld above 2^62", (long long)n);
  if (n > 0 && (snapshot == nullptr || mask == nullptr))
    return fail(DELTA_E_INVALID, "xor_apply: null pointer with n=%lld", (long long)n);
  g_error.clear();
  return hip_status(sbd::launch_xor_apply(snapshot, mask, n, static_cast<hipStream_t>(stream)),
                    "xor_apply launch");
}

}  // extern "C"
