// Internal declarations shared by the HIP translation units of libsbd.
// Not installed; the public contract is include/sbd.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

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

__device__ __forceinline__ void store16(void* p, const uint4& x) {
  u32x4 v;
  v.x = x.x;
  v.y = x.y;
  v.z = x.z;
  v.w = x.w;
  *global_ptr(static_cast<u32x4*>(p)) = v;
}

// ---------------------------------------------------------------------------
// Diff / compaction tiling.  One workgroup of 256 lanes (four wave64s) owns a
// tile of kDiffIters * 256 * 8 elements: every lane issues kDiffIters 16-byte
// loads per input, one wave covering 1 KB contiguous per load.  Tiles never
// straddle parameters.
// ---------------------------------------------------------------------------
constexpr int kDiffBlock = 512;
constexpr int kDiffWaves = kDiffBlock / 64;
constexpr int kVec = 8;  // bf16 per 16-byte load
constexpr int kDiffIters = 8;
constexpr int64_t kDiffTile = int64_t(kDiffBlock) * kVec * kDiffIters;  // 16384
// One workgroup per tile: the grid (tiles x 256 lanes) must stay below 2^32
// work-items.  2^24 tiles are 2.7e11 elements, more than HBM holds twice.
constexpr int64_t kMaxTiles = int64_t(1) << 24;

// Parameter descriptor as stored in the workspace (32 bytes).
struct DiffParam {
  const uint16_t* old_bits;
  const uint16_t* new_bits;
  int64_t numel;
  int64_t first_tile;
};

// Per-tile descriptor written by the prepare kernel (32 bytes).
struct TileDesc {
  const uint16_t* old_bits;  // first element of the tile
  const uint16_t* new_bits;
  int32_t e0;                // parameter-local index of that element
  int32_t valid;             // elements of the tile inside the parameter
  int64_t pad;
};

// A tile's compacted entries are staged in LDS (4 bytes each) when at most
// this many elements changed; denser tiles are written directly.
constexpr int kStageCap = 4096;
// Tiles with at most this many changes are finished by wave 0 alone (the
// other waves leave early and free their registers for new workgroups).
constexpr int kSoloCap = 1024;

struct SnapParam {
  uint16_t* snap;
  int64_t numel;
};

// Workspace layout: [header 256 B | tile state 8 B/tile | tile descriptor
// 32 B/tile | parameter table 32 B/param].  All offsets are 256-byte aligned.
struct WsLayout {
  size_t flag;        // uint32 look-back timeout flag
  size_t state;       // uint64 per tile: status (2 bits) | count (62 bits)
  size_t tile_desc;   // TileDesc per tile
  size_t table;       // DiffParam / SnapParam per parameter
  size_t total;
};

WsLayout ws_layout(int64_t max_tiles, int32_t nparams);
int64_t max_tiles_for(int64_t total_elems, int32_t nparams);

// Launchers return hipSuccess or the launch error.
hipError_t launch_diff(const DiffParam* d_table, const DiffParam& single, int32_t nparams,
                       int64_t total_tiles, int32_t* idx, uint16_t* val, int64_t capacity,
                       int64_t* nnz, int64_t* offsets, void* ws, const WsLayout& L,
                       hipStream_t stream);

hipError_t launch_apply(const SnapParam* d_table, const SnapParam& single, int32_t nparams,
                        const int64_t* offsets, const int32_t* idx, const uint16_t* val,
                        int64_t max_nnz, int64_t* violations, hipStream_t stream);

hipError_t launch_xor_mask(const uint16_t* a, const uint16_t* b, uint16_t* out, int64_t n,
                           hipStream_t stream);
hipError_t launch_xor_apply(uint16_t* snap, const uint16_t* mask, int64_t n,
                            hipStream_t stream);

}  // namespace sbd
