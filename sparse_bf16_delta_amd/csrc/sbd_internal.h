// Internal declarations shared by the HIP translation units of libsbd.
// Not installed; the public contract is include/sbd.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <string>

#include "sbd.h"

namespace sbd {

// A pointer loaded from memory (or built from an integer) is generic to the
// compiler, which then emits flat loads and stores.  The tensors here live in
// device memory, so this cast lets it emit global ones instead.
template <typename T>
__device__ __forceinline__ __attribute__((address_space(1))) T* global_ptr(T* p) {
  return (__attribute__((address_space(1))) T*)(p);
}

// 16-byte vector as the compiler's native type (loads and stores through
// address-space-qualified pointers work on it in both compilation passes).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load16(const void* p) {
  const u32x4 v = *global_ptr(static_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// The same, with the nontemporal hint: for data read exactly once.
__device__ __forceinline__ uint4 load16_stream(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(global_ptr(static_cast<const u32x4*>(p)));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void store16(void* p, const uint4& x) {
  u32x4 v;
  v.x = x.x;
  v.y = x.y;
  v.z = x.z;
  v.w = x.w;
  *global_ptr(static_cast<u32x4*>(p)) = v;
}

// ---------------------------------------------------------------------------
// Diff / compaction tiling.  One workgroup of 512 lanes (eight wave64s) owns a
// tile of kDiffIters * 512 * 8 = 32768 elements: every lane issues kDiffIters
// 16-byte loads per input, one wave covering 1 KB contiguous per load.  Tiles
// never straddle parameters.
// ---------------------------------------------------------------------------
constexpr int kDiffBlock = 512;
constexpr int kDiffWaves = kDiffBlock / 64;
constexpr int kVec = 8;  // bf16 per 16-byte load
constexpr int kDiffIters = 8;
constexpr int64_t kDiffTile = int64_t(kDiffBlock) * kVec * kDiffIters;  // 32768
// One workgroup per tile: the grid (tiles x 512 lanes) must stay below 2^32
// work-items.  2^23 tiles are 2.7e11 elements, more than HBM holds twice.
constexpr int64_t kMaxTiles = int64_t(1) << 23;

// Parameter descriptor as stored in the workspace (40 bytes).
struct DiffParam {
  const uint16_t* old_bits;
  const uint16_t* new_bits;
  int64_t numel;
  int64_t first_tile;
  int64_t flat_offset;  // added to every index in the sharded form (else 0)
};

// Per-tile descriptor written by the prepare kernel (32 bytes).
struct TileDesc {
  const uint16_t* old_bits;  // first element of the tile
  const uint16_t* new_bits;
  int32_t e0;                // parameter-local index of that element
  int32_t valid;             // elements of the tile inside the parameter
  int64_t flat_offset;       // the parameter's flat offset (sharded form)
};

// A tile with at most kStageCap changes is staged in LDS (4 bytes per entry)
// and then copied out: into its own compact 2 KB slot when it has at most
// kCompactCap changes, else into the staging arena shared by all tiles
// (filled in whole 16-byte quads from a counter; the worst case reserves
// kWideWords words per tile).  A denser tile stores its change mask (one byte
// per 16-byte chunk, 4 KB) in the arena; a tile that finds the arena full
// stores nothing and is recomputed from both inputs by the dense kernel.
constexpr int kStageCap = 8192;
constexpr int kCompactCap = 512;
constexpr int64_t kCompactWords = kCompactCap;  // uint32 per compact slot
constexpr int64_t kWideWords = kStageCap;       // arena uint32 reserved per tile (worst case)
// Tile counts are scanned in chunks of kScanChunk tiles, four per lane.
constexpr int kScanBlock = 1024;
constexpr int64_t kScanChunk = int64_t(kScanBlock) * 4;
// Consecutive tiles whose staged entries one placing workgroup copies.
constexpr int kPlaceTiles = 16;

struct SnapParam {
  uint16_t* snap;
  int64_t numel;
};

// Called by the 64 lanes of wave 0 only: the largest p in [0, nparams) with
// offsets[p] <= j -- the non-empty parameter holding entry j of a
// concatenated delta -- by a 64-way search (each step probes 64 evenly
// spaced offsets at once; two steps for up to 4096 parameters).
__device__ __forceinline__ int32_t find_param_wave0(const int64_t* __restrict__ offsets,
                                                    int32_t nparams, int64_t j) {
  const int lane = threadIdx.x & 63;
  int32_t lo = 0, hi = nparams;  // offsets[lo] <= j holds throughout
  while (hi - lo > 1) {
    const int32_t step = (hi - lo + 63) / 64;
    const int32_t probe = lo + lane * step;
    const uint64_t ok = __ballot(probe < hi && offsets[probe] <= j);
    lo += (63 - __builtin_clzll(ok)) * step;
    hi = lo + step < hi ? lo + step : hi;
  }
  return lo;
}

// Workspace layout (all offsets 256-byte aligned): a 256-byte header (the
// dense-tile count and the arena fill counter), then per tile a count, an
// in-chunk prefix, a dense-list entry, a descriptor, an arena position and a
// 2 KB compact slot, per chunk a total and a base, the parameter table, and
// last the staging arena: whatever the caller's workspace holds past
// `wide`, up to the worst case of 32 KB per tile at `total`.
struct WsLayout {
  size_t ndense;      // uint32: number of dense tiles
  size_t arena_next;  // uint64: arena quads handed out so far
  size_t counts;      // uint32 per tile: changed elements
  size_t inpfx;       // uint32 per tile: exclusive prefix inside its chunk
  size_t chunk_tot;   // uint32 per chunk
  size_t chunk_base;  // uint64 per chunk, then the total
  size_t dense_list;  // int32 per tile
  size_t tile_desc;   // TileDesc per tile
  size_t table;       // DiffParam / SnapParam per parameter
  size_t compact;     // kCompactWords uint32 per tile
  size_t wide;        // the staging arena: kWideWords uint32 per tile
  size_t tile_pos;    // uint64 per tile: its first arena quad
  size_t total;
};

WsLayout ws_layout(int64_t max_tiles, int32_t nparams);
int64_t max_tiles_for(int64_t total_elems, int32_t nparams);

// The calling thread's last-error text (abi.hip): fail_with formats it and
// returns `s`; clear_last_error empties it.
delta_status fail_with(delta_status s, const char* fmt, ...);
void clear_last_error();

// The runtime keeps one error per thread, set by any failed call, and a
// launch check reads it.  Every launcher clears it before launching, so a
// failure left by some earlier, unrelated call is not reported as its own.
inline void clear_stale_error() { (void)hipGetLastError(); }

// Launchers return hipSuccess or the launch error.
// idx is int32_t[capacity] (parameter-local indices) or, with global_idx,
// int64_t[capacity] holding flat_offset + local index (parameter lists only).
// arena_quads: 16-byte quads of staging arena at L.wide (any number, from 0
// to the worst case (L.total - L.wide) / 16); a tile that does not fit is
// handled as a dense tile.
hipError_t launch_diff(const DiffParam* d_table, const DiffParam& single, int32_t nparams,
                       int64_t total_tiles, void* idx, bool global_idx, uint16_t* val,
                       int64_t capacity, int64_t* nnz, int64_t* offsets, void* ws,
                       const WsLayout& L, uint64_t arena_quads, hipStream_t stream);
// The arena a workspace of ws_bytes leaves after the fixed regions.
uint64_t arena_quads_for(const WsLayout& L, size_t ws_bytes);

// total_elems: the elements of all snapshots of the launch (the kernel is
// chosen by the delta's size and its density bound max_nnz / total_elems).
hipError_t launch_apply(const SnapParam* d_table, const SnapParam& single, int32_t nparams,
                        const int64_t* offsets, const int32_t* idx, const uint16_t* val,
                        int64_t max_nnz, int64_t total_elems, int64_t* violations,
                        hipStream_t stream);

// The streamed receiver (stream.hip); on failure `err` receives the message.
size_t streamed_staging_size(int32_t nparams, int32_t nchunks, int32_t max_chunk_params,
                             int64_t max_chunk_nnz);
size_t xor_streamed_staging_size(int64_t chunk_elems);
delta_status apply_streamed_impl(int32_t nparams, uint16_t* const* snap_ptrs,
                                 const int64_t* numels, int32_t nchunks,
                                 const delta_host_chunk* chunks, void* staging,
                                 size_t staging_bytes, void* copy_stream, void* apply_stream,
                                 std::string& err);
// The host-direct receiver (stream.hip): the apply kernel reads the pinned
// host delta itself.
size_t host_apply_workspace_size(int32_t nparams);
delta_status apply_host_impl(int32_t nparams, uint16_t* const* snap_ptrs, const int64_t* numels,
                             const int32_t* idx_host, const uint16_t* val_host,
                             const int64_t* offsets_host, int64_t max_nnz, int64_t* violations,
                             void* ws, size_t ws_bytes, void* stream, std::string& err);
delta_status xor_apply_streamed_impl(uint16_t* snapshot, const uint16_t* mask_host, int64_t n,
                                     int64_t chunk_elems, void* staging, size_t staging_bytes,
                                     void* copy_stream, void* apply_stream, std::string& err);

// Wire encoding (wire.hip): widths are per parameter, in device memory.
hipError_t launch_wire_encode(int32_t nparams, const int32_t* widths, const int32_t* idx,
                              const int64_t* offsets, int64_t max_entries, uint8_t* positions,
                              int64_t positions_capacity, int64_t* pos_offsets,
                              hipStream_t stream);
hipError_t launch_wire_decode(int32_t nparams, const int32_t* widths, const uint8_t* positions,
                              int64_t positions_bytes, const int64_t* pos_offsets,
                              const int64_t* offsets, int64_t max_entries, int32_t* idx,
                              int64_t* violations, hipStream_t stream);
hipError_t launch_wire_hash(const uint8_t* positions, int64_t npos, const uint16_t* values,
                            int64_t nval, uint64_t* hashes, hipStream_t stream);
// hash, then checksum[0..1] = the 65-bit hash(positions) ^ (hash(values) << 1)
hipError_t launch_wire_checksum(const uint8_t* positions, int64_t npos, const uint16_t* values,
                                int64_t nval, uint64_t* checksum, hipStream_t stream);

// Blocked positions: blocks of kPosBlockElems elements per parameter; the
// device table gives each parameter's size and its first block in the flush.
constexpr int64_t kPosBlockElems = 65536;
struct BlockedParam {
  int64_t numel;
  int64_t tbase;
};
hipError_t launch_wire_encode_blocked(int32_t nparams, const BlockedParam* bp, int64_t nblocks,
                                      const int32_t* idx, const int64_t* offsets,
                                      int64_t max_entries, uint8_t* out, int64_t out_capacity,
                                      hipStream_t stream);
hipError_t launch_wire_decode_blocked(int32_t nparams, const BlockedParam* bp, int64_t nblocks,
                                      const uint8_t* in, int64_t in_bytes, const int64_t* offsets,
                                      int64_t max_entries, int32_t* idx, int64_t* violations,
                                      hipStream_t stream);

hipError_t launch_xor_mask(const uint16_t* a, const uint16_t* b, uint16_t* out, int64_t n,
                           hipStream_t stream);
hipError_t launch_xor_apply(uint16_t* snap, const uint16_t* mask, int64_t n,
                            hipStream_t stream);

}  // namespace sbd
