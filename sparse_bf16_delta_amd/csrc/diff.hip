// diff.hip -- bitwise bf16 change detection fused with stream compaction.
//
// What is computed (verl PR #6974 review, code-snippet section,
// `shard_delta_indices`; TRL delta-sync article, sections 4.1-4.2): for every
// element i of a parameter, a change is `old_bits[i] != new_bits[i]` as 16-bit
// integers; the output lists the changed positions in ascending order (int32,
// parameter-local) with the new bits at those positions.  The batched form
// concatenates the parameters' outputs in list order with per-parameter
// counts (same review, `gather_v_batched_to_rank0`).
//
// How, on gfx950: three phases in six short launches (the tile table or a
// counter reset, count and stage, two scans, place, dense tiles), and no
// workgroup ever waits for another one.
//  1. Count and stage.  One workgroup of 512 lanes (eight wave64s) per tile
//     of 32768 elements; a tile never straddles a parameter.  A lane loads
//     eight 16-byte chunks of `old` and eight of `new`, in two halves of four
//     one after the other, so that four such workgroups share a CU (all
//     sixteen at once held the registers of only three: 2-4 % slower on the
//     7B-shaped list at 1.2 % and 11.6 % density).  Per 16-byte chunk the
//     lane forms an 8-bit change mask; its popcount is prefix-summed across
//     the wave with four ballots over its bits plus mbcnt, and each half's 32
//     (iteration, wave) group totals are scanned in LDS, giving every change
//     its slot inside the tile in ascending element order.  A tile with at
//     most 8192 changes (25 %) is compacted in LDS as (tile-local index << 16
//     | new bits) and copied with 16-byte nontemporal stores: a tile with up
//     to 512 changes into a
//     2 KB workspace slot of its own, a tile with more into a staging arena
//     shared by all tiles, at a position it takes with one atomic add on a
//     workspace counter (so the arena fills as one dense, ascending write
//     stream; fixed 16 KB slots, a few KB written in each, cost 1.3 ms more
//     on the 7B-shaped list at 8 % density, while for sparse tiles the
//     atomic's latency costs more than the slot saves).  A denser tile
//     stores its 4 KB change mask in the arena instead.  The arena is what
//     the caller's workspace holds past the fixed regions: a tile that finds
//     it full keeps nothing there and is treated as a dense tile whose mask
//     the dense kernel recomputes, so any arena size gives the same result,
//     and one sized from the caller's capacity never runs out while the
//     delta fits that capacity.  The tile count goes to a per-tile array and
//     the workgroup ends.
//  2. Scan.  One workgroup per 4096 tiles scans their counts (prefix inside
//     the chunk, chunk total) and lists the dense tiles; one workgroup scans
//     the chunk totals and writes the per-parameter counts and offsets.
//  3. Place.  One workgroup per 16 consecutive tiles copies their staged
//     entries to the final position: consecutive tiles have consecutive
//     outputs, so this is one contiguous run of coalesced idx and val
//     stores.  Dense tiles are re-read (`new` only, steered by the stored
//     mask) and written directly by a second, small grid.
// Why not a single pass with a look-back, in which a tile that learns the
// count of all tiles before it writes its entries in place: the tiles'
// states live in memory that workgroups on all eight XCDs read, so every
// read is a device-scope round trip, and a workgroup that waits holds its
// registers and LDS, which keeps the next tile's loads from being issued.
// Measured on the 7B-shaped list at 1.2 % (diff, ms): three phases 4.73; a
// bounded look-back where every tile placed itself after 1-3 reads of its
// 512 predecessors' states 6.85; a single read with staging as the fallback
// (7-15 % of the tiles placed) 5.07.  At 8 % and 11.6 % density the same
// look-backs cost 10-20 %, more than the 8 bytes per changed element that
// the staging round trip adds.
// Traffic: the 4n-byte read happens once; a staged tile adds 4 bytes written
// and 4 read per changed element, a dense tile re-reads `new` (2 bytes per
// element; both inputs if its mask found no room), and the tile count,
// prefix, position and descriptor add about 60 bytes per tile.
#include <atomic>

#include "sbd_internal.h"

namespace sbd {
namespace {

constexpr int kGroups = kDiffIters * kDiffWaves;
static_assert(kGroups <= 64, "one (iteration, wave) group per lane of a wave");
static_assert(kDiffIters <= 8, "a lane's change mask is at most 8 bytes");
static_assert(kDiffTile <= 65536, "tile-local indices are staged in 16 bits");
static_assert(kStageCap % 4 == 0, "staged entries are copied four at a time");
static_assert(kWideWords * 4 >= kDiffBlock * 8, "a tile's change mask fits its arena share");
constexpr uint64_t kMaskQuads = kDiffBlock * 8 / 16;  // arena quads of a dense tile's mask
static_assert(kCompactCap % 4 == 0 && kCompactCap <= kStageCap, "slot tiers");
static_assert(kScanChunk == kScanBlock * 4, "a scan lane takes four tiles");
static_assert(kMaxTiles / kScanChunk <= kScanBlock * 4, "the chunk totals fit one workgroup");

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// A tile whose entries did not fit the staging arena is handled as a dense
// tile: its count carries this flag (for the scan's dense list) and its
// arena position is kNoArena (for the placing kernel).
constexpr uint32_t kDenseFlag = 0x80000000u;
constexpr uint64_t kNoArena = ~0ull;

__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
}

// One bit per bf16 half of a 32-bit word: bit0 = low half differs.
__device__ __forceinline__ uint32_t word_mask(uint32_t a, uint32_t b) {
  const uint32_t x = a ^ b;
  return ((x & 0xFFFFu) != 0u ? 1u : 0u) | ((x >> 16) != 0u ? 2u : 0u);
}

__device__ __forceinline__ uint32_t change_mask8(const uint4& a, const uint4& b) {
  return word_mask(a.x, b.x) | (word_mask(a.y, b.y) << 2) | (word_mask(a.z, b.z) << 4) |
         (word_mask(a.w, b.w) << 6);
}

template <int S>
__device__ __forceinline__ uint16_t half_of(const uint4& v) {
  static_assert(S >= 0 && S < 8, "slot");
  const uint32_t w = (S >> 1) == 0 ? v.x : (S >> 1) == 1 ? v.y : (S >> 1) == 2 ? v.z : v.w;
  return static_cast<uint16_t>((S & 1) ? (w >> 16) : (w & 0xFFFFu));
}

// Exclusive prefix of c (0..8) over the lanes of the wave, and the wave total.
__device__ __forceinline__ uint32_t wave_prefix_c(uint32_t c, uint32_t& total) {
  const uint64_t b0 = __ballot(c & 1u);
  const uint64_t b1 = __ballot(c & 2u);
  const uint64_t b2 = __ballot(c & 4u);
  const uint64_t b3 = __ballot(c & 8u);
  total = __popcll(b0) + 2u * __popcll(b1) + 4u * __popcll(b2) + 8u * __popcll(b3);
  return lanes_below(b0) + 2u * lanes_below(b1) + 4u * lanes_below(b2) + 8u * lanes_below(b3);
}

// Inclusive prefix sum over the 64 lanes of a wave.
template <typename T>
__device__ __forceinline__ T wave_inclusive(T v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const T y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  return v;
}

template <int S>
__device__ __forceinline__ void stage_slot(uint32_t mm, uint32_t& pos, uint32_t local,
                                           const uint4& x, uint32_t* stage) {
  if (mm & (1u << S)) {
    stage[pos] = ((local + S) << 16) | half_of<S>(x);
    ++pos;
  }
}

// 16 bytes (8 elements) of a tile starting at tile-local element `local`;
// elements at or past `valid` read as zero.
__device__ __forceinline__ uint4 load_chunk(const uint16_t* __restrict__ base, int local,
                                            int valid, bool vec) {
  if (vec) return load16(base + local);
  const auto g = global_ptr(base);
  uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int s = 0; s < kVec; ++s)
    if (local + s < valid) w[s >> 1] |= uint32_t(g[local + s]) << (16 * (s & 1));
  return make_uint4(w[0], w[1], w[2], w[3]);
}

struct TileView {
  const uint16_t* ob;
  const uint16_t* nb;
  int32_t e0;           // parameter-local index of the tile's first element
  int32_t valid;        // elements of the tile inside the parameter
  int64_t flat_offset;  // the parameter's flat offset (sharded form)
};

template <bool kMany>
__device__ __forceinline__ TileView tile_view(const TileDesc* __restrict__ tdesc,
                                              const DiffParam& single, int64_t t) {
  TileView v;
  if constexpr (kMany) {
    const TileDesc td = tdesc[t];
    v.ob = td.old_bits;
    v.nb = td.new_bits;
    v.e0 = td.e0;
    v.valid = td.valid;
    v.flat_offset = td.flat_offset;
  } else {
    const int64_t first = t * kDiffTile;
    const int64_t left = single.numel - first;
    v.ob = single.old_bits + first;
    v.nb = single.new_bits + first;
    v.e0 = static_cast<int32_t>(first);
    v.valid = static_cast<int32_t>(left < kDiffTile ? left : kDiffTile);
    v.flat_offset = 0;
  }
  return v;
}

// From the lanes' change masks: each lane's offset inside its (iteration,
// wave) group (lp), each group's offset inside the tile in ascending element
// order -- iteration-major, then wave, then lane, then slot -- (goff), and the
// tile's count (agg), in every lane; gexcl is the offset of group `lane`.
// Contains one barrier; s_wtot must not be in use by other waves.
template <int N>
__device__ __forceinline__ void tile_offsets(const uint32_t (&m)[N], uint32_t (&lp)[N],
                                             uint32_t (&goff)[N], uint32_t& agg, uint32_t& gexcl,
                                             uint32_t* s_wtot, int lane, int wave) {
  static_assert(N * kDiffWaves <= 64, "one group per lane of a wave");
#pragma unroll
  for (int j = 0; j < N; ++j) {
    uint32_t tot;
    lp[j] = wave_prefix_c(static_cast<uint32_t>(__popc(m[j])), tot);
    if (lane == 0) s_wtot[j * kDiffWaves + wave] = tot;
  }
  __syncthreads();
  // every wave scans the 64 group totals itself: no second barrier
  const uint32_t own = lane < N * kDiffWaves ? s_wtot[lane] : 0u;
  const uint32_t inc = wave_inclusive(own, lane);
  const uint32_t excl = inc - own;
  gexcl = excl;
  agg = static_cast<uint32_t>(__shfl(static_cast<int>(inc), 63, 64));
#pragma unroll
  for (int j = 0; j < N; ++j)
    goff[j] = static_cast<uint32_t>(__shfl(static_cast<int>(excl), j * kDiffWaves + wave, 64));
}

// One half of a tile in the count kernel: iterations [H * kHalfIters,
// (H + 1) * kHalfIters), which hold the tile's elements [H * kDiffTile / 2,
// (H + 1) * kDiffTile / 2).  Loads both inputs, stores the lanes' change masks
// into m, and, if `stage` and the tile's entries so far fit, stages this
// half's entries in LDS after the `base` entries of the halves before it.
// Returns the half's count (uniform).  Contains one barrier; s_wtot must not
// be in use by other waves.
constexpr int kHalfIters = kDiffIters / 2;
static_assert(kHalfIters * 2 == kDiffIters, "a tile is two halves");
template <int H>
__device__ __forceinline__ uint32_t count_half(const TileView& tv, bool vec, int tid, int lane,
                                               int wave, uint32_t (&m)[kDiffIters], uint32_t base,
                                               bool stage, uint32_t* s_wtot, uint32_t* s_stage) {
  uint4 nv[kHalfIters];
  uint32_t mh[kHalfIters];
  if (vec) {
    const uint4* o4 = reinterpret_cast<const uint4*>(tv.ob) + H * kHalfIters * kDiffBlock + tid;
    const uint4* n4 = reinterpret_cast<const uint4*>(tv.nb) + H * kHalfIters * kDiffBlock + tid;
    uint4 ov[kHalfIters];
#pragma unroll
    for (int j = 0; j < kHalfIters; ++j) {
      ov[j] = load16_stream(o4 + j * kDiffBlock);
      nv[j] = load16_stream(n4 + j * kDiffBlock);
    }
#pragma unroll
    for (int j = 0; j < kHalfIters; ++j) mh[j] = change_mask8(ov[j], nv[j]);
  } else {
    // ragged last tile or unaligned parameter
#pragma unroll
    for (int j = 0; j < kHalfIters; ++j) {
      const int local = (H * kHalfIters + j) * kDiffBlock * kVec + tid * kVec;
      const uint4 o = load_chunk(tv.ob, local, tv.valid, false);
      nv[j] = load_chunk(tv.nb, local, tv.valid, false);
      mh[j] = change_mask8(o, nv[j]);
    }
  }
  uint32_t lp[kHalfIters], goff[kHalfIters], agg, gexcl;
  tile_offsets<kHalfIters>(mh, lp, goff, agg, gexcl, s_wtot, lane, wave);
  if (stage && base + agg <= static_cast<uint32_t>(kStageCap)) {
#pragma unroll
    for (int j = 0; j < kHalfIters; ++j) {
      const uint32_t mm = mh[j];
      if (mm != 0u) {
        uint32_t pos = base + goff[j] + lp[j];
        const uint32_t local =
            static_cast<uint32_t>((H * kHalfIters + j) * kDiffBlock * kVec + tid * kVec);
        const uint4 x = nv[j];
        stage_slot<0>(mm, pos, local, x, s_stage);
        stage_slot<1>(mm, pos, local, x, s_stage);
        stage_slot<2>(mm, pos, local, x, s_stage);
        stage_slot<3>(mm, pos, local, x, s_stage);
        stage_slot<4>(mm, pos, local, x, s_stage);
        stage_slot<5>(mm, pos, local, x, s_stage);
        stage_slot<6>(mm, pos, local, x, s_stage);
        stage_slot<7>(mm, pos, local, x, s_stage);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < kHalfIters; ++j) m[H * kHalfIters + j] = mh[j];
  return agg;
}

// For a parameter list: every tile's descriptor (base pointers, first index,
// length), so a workgroup needs one load, not a parameter search, before its
// data loads.
// Clears the staging arena's fill counter before the count kernel (the
// parameter-list form clears it in the prepare kernel instead).
__global__ __launch_bounds__(64) void zero_ctr_kernel(unsigned long long* ctr) {
  if (threadIdx.x == 0) *ctr = 0ull;
}

__global__ __launch_bounds__(256) void diff_prepare_kernel(const DiffParam* __restrict__ table,
                                                           int32_t nparams, int64_t total_tiles,
                                                           TileDesc* __restrict__ tdesc,
                                                           unsigned long long* __restrict__ ctr) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *ctr = 0ull;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; t < total_tiles; t += stride) {
    // largest p whose first tile is <= t (skips empty parameters)
    int32_t lo = 0, hi = nparams - 1;
    while (lo < hi) {
      const int32_t mid = (lo + hi + 1) >> 1;
      if (table[mid].first_tile <= t)
        lo = mid;
      else
        hi = mid - 1;
    }
    const DiffParam d = table[lo];
    const int64_t e0 = (t - d.first_tile) * kDiffTile;
    const int64_t left = d.numel - e0;
    TileDesc td;
    td.old_bits = d.old_bits + e0;
    td.new_bits = d.new_bits + e0;
    td.e0 = static_cast<int32_t>(e0);
    td.valid = static_cast<int32_t>(left < kDiffTile ? left : kDiffTile);
    td.flat_offset = d.flat_offset;
    tdesc[t] = td;
  }
}

// Phase 1: count the tile's changes; stage sparse tiles, record dense ones.
template <bool kMany>
__global__ __launch_bounds__(kDiffBlock) void diff_count_kernel(
    const TileDesc* __restrict__ tdesc, DiffParam single, uint32_t* __restrict__ counts,
    uint32_t* __restrict__ compact, uint32_t* __restrict__ wide, uint32_t* __restrict__ ndense,
    uint64_t* __restrict__ tile_pos, unsigned long long* __restrict__ ctr, uint64_t arena_quads) {
  __shared__ __attribute__((aligned(16))) uint32_t s_stage[kStageCap];
  __shared__ uint64_t s_pos;
  __shared__ uint32_t s_wtot[kHalfIters * kDiffWaves];
  __shared__ uint32_t s_wtot2[kHalfIters * kDiffWaves];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t tile = blockIdx.x;
  const TileView tv = tile_view<kMany>(tdesc, single, tile);
  const bool vec = tv.valid == kDiffTile &&
                   ((reinterpret_cast<uintptr_t>(tv.ob) | reinterpret_cast<uintptr_t>(tv.nb)) &
                    15u) == 0;

  // The tile in two halves, one after the other: half the tile's data is in
  // registers at a time, so more workgroups share a CU; the tile still takes
  // one count, one arena position and one copy-out.
  uint32_t m[kDiffIters];
  const uint32_t agg0 =
      count_half<0>(tv, vec, tid, lane, wave, m, 0u, true, s_wtot, s_stage);
  const uint32_t agg1 = count_half<1>(tv, vec, tid, lane, wave, m, agg0,
                                      agg0 <= static_cast<uint32_t>(kStageCap), s_wtot2, s_stage);
  const uint32_t agg = agg0 + agg1;
  const bool staged = agg <= static_cast<uint32_t>(kStageCap);
  const bool in_arena = staged && agg > static_cast<uint32_t>(kCompactCap);
  if (tid == 0) {
    uint32_t c = agg;
    if (!staged || in_arena) {
      // whole 16-byte quads of the arena, so every tile's run starts aligned:
      // a staged tile's entries, or a dense tile's change mask.  A tile that
      // finds the arena full keeps nothing there and is handled as a dense
      // tile whose mask is recomputed.
      const uint64_t q = staged ? (agg + 3u) / 4u : kMaskQuads;
      const uint64_t p = atomicAdd(ctr, static_cast<unsigned long long>(q));
      const bool fits = p + q <= arena_quads;
      s_pos = fits ? p : kNoArena;
      tile_pos[tile] = fits ? p : kNoArena;
      if (!fits && staged) c |= kDenseFlag;
    }
    counts[tile] = c;
    if (tile == 0) *ndense = 0u;  // the scan kernel, launched next, lists dense tiles
  }
  __syncthreads();
  const uint64_t at = (!staged || in_arena) ? s_pos : 0;
  if (staged && !(in_arena && at == kNoArena)) {
    // 16-byte copies with the nontemporal hint (the entries are read once,
    // by the placing kernel); the last one may carry up to three stale LDS
    // words past `agg`, which stay inside the slot or the tile's arena quads
    // and are never read.
    uint32_t* slot = in_arena ? wide + at * 4u : compact + tile * kCompactWords;
    for (uint32_t p = static_cast<uint32_t>(tid) * 4u; p < agg; p += kDiffBlock * 4u) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(&s_stage[p]);
      __builtin_nontemporal_store(w, global_ptr(reinterpret_cast<u32x4*>(slot + p)));
    }
  } else if (!staged && at != kNoArena) {
    // dense: the change mask in the arena, one byte per 16-byte chunk, 8 bytes per lane
    u32x2 w;
    w.x = 0u;
    w.y = 0u;
#pragma unroll
    for (int j = 0; j < kDiffIters; ++j) {
      if (j < 4)
        w.x |= m[j] << (8 * j);
      else
        w.y |= m[j] << (8 * (j - 4));
    }
    *global_ptr(reinterpret_cast<u32x2*>(wide + at * 4u) + tid) = w;
  }
}

// Phase 2a: per chunk of kScanChunk tiles, each tile's exclusive prefix
// inside the chunk and the chunk total; dense tiles are appended to a list
// (in no particular order).
__global__ __launch_bounds__(kScanBlock) void diff_scan_chunks_kernel(
    const uint32_t* __restrict__ counts, int64_t total_tiles, uint32_t* __restrict__ inpfx,
    uint32_t* __restrict__ chunk_tot, int32_t* __restrict__ dense_list,
    uint32_t* __restrict__ ndense) {
  __shared__ uint32_t s_w[kScanBlock / 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t t0 = int64_t(blockIdx.x) * kScanChunk + int64_t(tid) * 4;
  uint32_t v[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t t = t0 + q;
    const uint32_t raw = t < total_tiles ? counts[t] : 0u;
    v[q] = raw & ~kDenseFlag;
    if (v[q] > static_cast<uint32_t>(kStageCap) || (raw & kDenseFlag) != 0u)
      dense_list[atomicAdd(ndense, 1u)] = int32_t(t);
  }
  const uint32_t own = v[0] + v[1] + v[2] + v[3];
  const uint32_t inc = wave_inclusive(own, lane);
  if (lane == 63) s_w[wave] = inc;
  __syncthreads();
  uint32_t base = 0;
  for (int w = 0; w < wave; ++w) base += s_w[w];
  uint32_t run = base + inc - own;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (t0 + q < total_tiles) inpfx[t0 + q] = run;
    run += v[q];
  }
  if (tid == kScanBlock - 1) chunk_tot[blockIdx.x] = base + inc;
}

// Phase 2b: chunk bases (chunk_base[nchunks] = total) and the per-parameter
// counts and offsets.
template <bool kMany>
__global__ __launch_bounds__(kScanBlock) void diff_base_kernel(
    const DiffParam* __restrict__ table, int32_t nparams, int64_t total_tiles, int32_t nchunks,
    const uint32_t* __restrict__ inpfx, const uint32_t* __restrict__ chunk_tot,
    uint64_t* __restrict__ chunk_base, int64_t* __restrict__ nnz, int64_t* __restrict__ offsets) {
  __shared__ uint64_t s_base[kMaxTiles / kScanChunk + 1];
  __shared__ uint64_t s_w[kScanBlock / 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c0 = tid * 4;
  uint64_t v[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) v[q] = c0 + q < nchunks ? chunk_tot[c0 + q] : 0u;
  const uint64_t own = v[0] + v[1] + v[2] + v[3];
  const uint64_t inc = wave_inclusive(own, lane);
  if (lane == 63) s_w[wave] = inc;
  __syncthreads();
  uint64_t base = 0;
  for (int w = 0; w < wave; ++w) base += s_w[w];
  uint64_t run = base + inc - own;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (c0 + q < nchunks) {
      s_base[c0 + q] = run;
      chunk_base[c0 + q] = run;
    }
    run += v[q];
  }
  if (tid == kScanBlock - 1) {
    s_base[nchunks] = base + inc;
    chunk_base[nchunks] = base + inc;
  }
  __syncthreads();
  auto start = [&](int64_t ft) -> uint64_t {
    return ft < total_tiles ? s_base[ft / kScanChunk] + inpfx[ft] : s_base[nchunks];
  };
  for (int64_t p = tid; p <= nparams; p += kScanBlock) {
    const int64_t ft = p < nparams ? (kMany ? table[p].first_tile : 0) : total_tiles;
    const uint64_t off = start(ft);
    if (offsets) offsets[p] = static_cast<int64_t>(off);
    if (p < nparams) {
      const int64_t ft_next = (kMany && p + 1 < nparams) ? table[p + 1].first_tile : total_tiles;
      nnz[p] = static_cast<int64_t>(start(ft_next) - off);
    }
  }
}

// Phase 3a: copy the staged entries of `tiles_per_wg` consecutive tiles, from
// each tile's slot or arena position, to their final positions.  Consecutive
// tiles have consecutive outputs, so the staged tiles' entries are walked as
// one flat run (dense tiles, written by diff_dense_kernel, and empty ones are
// left out of it).
template <bool kMany, typename IdxT>
__global__ __launch_bounds__(kDiffBlock) void diff_place_kernel(
    const TileDesc* __restrict__ tdesc, int64_t total_tiles, int32_t nchunks, int32_t tiles_per_wg,
    const uint32_t* __restrict__ inpfx, const uint64_t* __restrict__ chunk_base,
    const uint32_t* __restrict__ compact, const uint32_t* __restrict__ wide,
    IdxT* __restrict__ idx, uint16_t* __restrict__ val, int64_t capacity,
    const uint64_t* __restrict__ tile_pos) {
  static_assert(sizeof(IdxT) == 8 ? kMany : true, "global indices need a parameter table");
  __shared__ uint64_t s_tpos[kPlaceTiles];
  constexpr int kUnroll = 4;
  __shared__ uint64_t s_off[kPlaceTiles + 1];  // output offset of each tile
  __shared__ IdxT s_first[kPlaceTiles];  // index written for the tile's first element
  __shared__ uint32_t s_run[kPlaceTiles + 1];  // start of the m-th staged tile in the flat run
  __shared__ int32_t s_tile[kPlaceTiles];      // which tile that is
  __shared__ int32_t s_nrun;
  const int tid = threadIdx.x;
  const int64_t t0 = int64_t(blockIdx.x) * tiles_per_wg;
  const int64_t left = total_tiles - t0;
  const int nt = static_cast<int>(left < tiles_per_wg ? left : tiles_per_wg);
  if (tid <= nt) {
    const int64_t t = t0 + tid;
    s_off[tid] = t < total_tiles ? chunk_base[t / kScanChunk] + inpfx[t] : chunk_base[nchunks];
    if (tid < nt) {
      s_tpos[tid] = tile_pos[t];
      if constexpr (kMany) {
        if constexpr (sizeof(IdxT) == 8)
          s_first[tid] = tdesc[t].flat_offset + tdesc[t].e0;
        else
          s_first[tid] = tdesc[t].e0;
      } else {
        s_first[tid] = static_cast<IdxT>(t * kDiffTile);
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t acc = 0;
    int r = 0;
    for (int k = 0; k < nt; ++k) {
      const uint64_t c = s_off[k + 1] - s_off[k];
      // staged: in its compact slot, or in the arena unless the arena was full
      if (c != 0 && c <= static_cast<uint64_t>(kStageCap) &&
          !(c > static_cast<uint64_t>(kCompactCap) && s_tpos[k] == kNoArena)) {
        s_tile[r] = k;
        s_run[r] = acc;
        acc += static_cast<uint32_t>(c);
        ++r;
      }
    }
    s_run[r] = acc;
    s_nrun = r;
  }
  __syncthreads();
  const uint32_t total = s_run[s_nrun];
  const uint64_t cap = static_cast<uint64_t>(capacity);
  int r = 0;  // staged tile of the current flat position; only moves forward
  for (uint32_t qb = static_cast<uint32_t>(tid); qb < total; qb += kUnroll * kDiffBlock) {
    uint32_t w[kUnroll];
    uint64_t jj[kUnroll];
    int kk[kUnroll];
    bool ok[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t q = qb + static_cast<uint32_t>(u * kDiffBlock);
      ok[u] = q < total;
      if (ok[u]) {
        while (s_run[r + 1] <= q) ++r;  // stops below s_nrun because q < total
        const int k = s_tile[r];
        const uint32_t p = q - s_run[r];
        jj[u] = s_off[k] + p;
        kk[u] = k;
        ok[u] = jj[u] < cap;
        const uint32_t* slot = s_off[k + 1] - s_off[k] <= static_cast<uint64_t>(kCompactCap)
                                   ? compact + (t0 + k) * kCompactWords
                                   : wide + s_tpos[k] * 4u;
        if (ok[u]) w[u] = *global_ptr(slot + p);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (ok[u]) {
        idx[jj[u]] = s_first[kk[u]] + static_cast<IdxT>(w[u] >> 16);
        val[jj[u]] = static_cast<uint16_t>(w[u] & 0xFFFFu);
      }
    }
  }
}

// Phase 3b: dense tiles, from their change masks and a second read of the
// changed 16-byte chunks of `new` -- or, for a tile that found no room in the
// arena, from a second read of both inputs.  Each of the tile's kDiffIters
// iterations (at most kDiffBlock * kVec entries) is staged in LDS and copied
// out with coalesced stores; the values are read a half tile at a time.
// (six waves per SIMD asked of the compiler: 80 registers, three workgroups
// per CU, without spilling to scratch; eight would spill)
template <bool kMany, typename IdxT>
__global__ __launch_bounds__(kDiffBlock) __attribute__((amdgpu_waves_per_eu(6))) void diff_dense_kernel(
    const TileDesc* __restrict__ tdesc, DiffParam single, const int32_t* __restrict__ dense_list,
    const uint32_t* __restrict__ ndense, const uint32_t* __restrict__ inpfx,
    const uint64_t* __restrict__ chunk_base, const uint32_t* __restrict__ wide,
    const uint64_t* __restrict__ tile_pos, IdxT* __restrict__ idx, uint16_t* __restrict__ val,
    int64_t capacity) {
  static_assert(sizeof(IdxT) == 8 ? kMany : true, "global indices need a parameter table");
  static_assert(kDiffBlock * kVec <= kStageCap, "one iteration of a tile fits the stage");
  __shared__ __attribute__((aligned(16))) uint32_t s_stage[kDiffBlock * kVec];
  __shared__ uint32_t s_wtot[kGroups];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const uint64_t cap = static_cast<uint64_t>(capacity);
  const uint32_t nd = *ndense;
  for (uint32_t i = blockIdx.x; i < nd; i += gridDim.x) {
    // opaque copy of the lane id: keeps the compiler from hoisting ~200
    // per-lane index constants out of this loop into registers
    int ltid = tid;
    asm volatile("" : "+v"(ltid));
    const int64_t t = dense_list[i];
    const TileView tv = tile_view<kMany>(tdesc, single, t);
    const bool vec = tv.valid == kDiffTile &&
                     ((reinterpret_cast<uintptr_t>(tv.ob) | reinterpret_cast<uintptr_t>(tv.nb)) &
                      15u) == 0;
    const uint64_t at = tile_pos[t];
    uint32_t m[kDiffIters];
    if (at != kNoArena) {  // the mask the count kernel stored
      const u32x2 mw = *global_ptr(reinterpret_cast<const u32x2*>(wide + at * 4u) + ltid);
#pragma unroll
      for (int j = 0; j < kDiffIters; ++j) m[j] = ((j < 4 ? mw.x : mw.y) >> (8 * (j & 3))) & 0xFFu;
    } else {
      // no room was left in the arena: compare the tile again, one chunk of
      // each input in flight at a time (a rare path; it must not raise the
      // kernel's register count), and read the changed values again below
#pragma unroll
      for (int j = 0; j < kDiffIters; ++j) {
        const int local = j * kDiffBlock * kVec + ltid * kVec;
        const uint4 o = load_chunk(tv.ob, local, tv.valid, vec);
        const uint4 n = load_chunk(tv.nb, local, tv.valid, vec);
        m[j] = change_mask8(o, n);
        asm volatile("" ::: "memory");  // keeps the next chunk's loads below this one
      }
    }
    uint32_t lp[kDiffIters], goff[kDiffIters], agg, gexcl;
    tile_offsets(m, lp, goff, agg, gexcl, s_wtot, lane, wave);
    const uint64_t tbase = chunk_base[t / kScanChunk] + inpfx[t];
    const IdxT first = sizeof(IdxT) == 8 ? static_cast<IdxT>(tv.flat_offset + tv.e0)
                                         : static_cast<IdxT>(tv.e0);
    // the changed chunks of `new`, a half of the tile at a time: with half
    // the values in registers, twice as many workgroups share a CU
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint4 x[kHalfIters];
#pragma unroll
      for (int k = 0; k < kHalfIters; ++k) {
        const int j = h * kHalfIters + k;
        x[k] = m[j] != 0u ? load_chunk(tv.nb, j * kDiffBlock * kVec + ltid * kVec, tv.valid, vec)
                          : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int k = 0; k < kHalfIters; ++k) {
        const int j = h * kHalfIters + k;
        // entries of iteration j occupy [jb, je) of the tile's output
        const uint32_t jb =
            static_cast<uint32_t>(__shfl(static_cast<int>(gexcl), j * kDiffWaves, 64));
        const uint32_t je =
            j + 1 < kDiffIters
                ? static_cast<uint32_t>(__shfl(static_cast<int>(gexcl), (j + 1) * kDiffWaves, 64))
                : agg;
        const uint32_t mm = m[j];
        if (mm != 0u) {
          uint32_t pos = goff[j] + lp[j] - jb;
          const uint32_t local = static_cast<uint32_t>(j * kDiffBlock * kVec + ltid * kVec);
          stage_slot<0>(mm, pos, local, x[k], s_stage);
          stage_slot<1>(mm, pos, local, x[k], s_stage);
          stage_slot<2>(mm, pos, local, x[k], s_stage);
          stage_slot<3>(mm, pos, local, x[k], s_stage);
          stage_slot<4>(mm, pos, local, x[k], s_stage);
          stage_slot<5>(mm, pos, local, x[k], s_stage);
          stage_slot<6>(mm, pos, local, x[k], s_stage);
          stage_slot<7>(mm, pos, local, x[k], s_stage);
        }
        __syncthreads();
        for (uint32_t p = static_cast<uint32_t>(tid); p < je - jb; p += kDiffBlock) {
          const uint64_t o = tbase + jb + p;
          if (o < cap) {
            const uint32_t w = s_stage[p];
            idx[o] = first + static_cast<IdxT>(w >> 16);
            val[o] = static_cast<uint16_t>(w & 0xFFFFu);
          }
        }
        __syncthreads();  // the stage is refilled by the next iteration
      }
    }
  }
}

// Workgroups of diff_dense_kernel<kMany> that are resident at once on the
// current device: its grid-stride loop hands each workgroup the same share of
// dense tiles, so a larger grid would leave a tail.  Queried once per device.
template <bool kMany, typename IdxT>
int64_t dense_grid_limit() {
  static std::atomic<int64_t> cached[64];  // zero-initialised; threads may race to fill it
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 256;
  }
  int64_t lim = cached[dev].load(std::memory_order_relaxed);
  if (lim == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, diff_dense_kernel<kMany, IdxT>,
                                                     kDiffBlock, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        per_cu < 1 || cus < 1) {
      (void)hipGetLastError();
      return 256;
    }
    lim = int64_t(per_cu) * cus;
    cached[dev].store(lim, std::memory_order_relaxed);
  }
  return lim;
}

}  // namespace

namespace {

// Phase 3: place the staged entries, then the dense tiles.
template <bool kMany, typename IdxT>
void launch_place(const TileDesc* tdesc, const DiffParam& single, int64_t total_tiles,
                  int32_t nchunks, const uint32_t* inpfx, const uint64_t* chunk_base,
                  const uint32_t* compact, const uint32_t* wide, const int32_t* dense_list,
                  const uint32_t* ndense, IdxT* idx, uint16_t* val, int64_t capacity,
                  const uint64_t* tile_pos, hipStream_t stream) {
  // about 8192 placing workgroups (up to kPlaceTiles tiles each): several
  // rounds of the GPU, so no long tail (on the Qwen3-0.6B-shaped list at 8 %,
  // the whole diff: 0.582 ms with 2048 workgroups of 8 tiles, 0.564 with
  // 8192 of 2; more entries in flight per lane was slower)
  int64_t per_wg = total_tiles / 8192;
  per_wg = per_wg < 1 ? 1 : (per_wg > kPlaceTiles ? kPlaceTiles : per_wg);
  const unsigned place_grid = static_cast<unsigned>((total_tiles + per_wg - 1) / per_wg);
  const int64_t dense_max = dense_grid_limit<kMany, IdxT>();
  const unsigned dense_grid =
      static_cast<unsigned>(total_tiles < dense_max ? total_tiles : dense_max);
  diff_place_kernel<kMany, IdxT><<<dim3(place_grid), dim3(kDiffBlock), 0, stream>>>(
      tdesc, total_tiles, nchunks, static_cast<int32_t>(per_wg), inpfx, chunk_base, compact, wide,
      idx, val, capacity, tile_pos);
  diff_dense_kernel<kMany, IdxT><<<dim3(dense_grid), dim3(kDiffBlock), 0, stream>>>(
      tdesc, single, dense_list, ndense, inpfx, chunk_base, wide, tile_pos, idx, val, capacity);
}

}  // namespace

hipError_t launch_diff(const DiffParam* d_table, const DiffParam& single, int32_t nparams,
                       int64_t total_tiles, void* idx, bool global_idx, uint16_t* val,
                       int64_t capacity, int64_t* nnz, int64_t* offsets, void* ws,
                       const WsLayout& L, uint64_t arena_quads, hipStream_t stream) {
  clear_stale_error();
  char* base = static_cast<char*>(ws);
  uint32_t* ndense = reinterpret_cast<uint32_t*>(base + L.ndense);
  uint32_t* counts = reinterpret_cast<uint32_t*>(base + L.counts);
  uint32_t* inpfx = reinterpret_cast<uint32_t*>(base + L.inpfx);
  uint32_t* chunk_tot = reinterpret_cast<uint32_t*>(base + L.chunk_tot);
  uint64_t* chunk_base = reinterpret_cast<uint64_t*>(base + L.chunk_base);
  int32_t* dense_list = reinterpret_cast<int32_t*>(base + L.dense_list);
  TileDesc* tdesc = reinterpret_cast<TileDesc*>(base + L.tile_desc);
  uint32_t* compact = reinterpret_cast<uint32_t*>(base + L.compact);
  uint32_t* wide = reinterpret_cast<uint32_t*>(base + L.wide);
  uint64_t* tile_pos = reinterpret_cast<uint64_t*>(base + L.tile_pos);
  unsigned long long* ctr = reinterpret_cast<unsigned long long*>(base + L.arena_next);
  // d_table == nullptr: one tensor (nparams == 1, `single`) or an empty list
  // (nparams == 0, no tiles).  Global indices come with a table only.
  const bool many = d_table != nullptr;
  if (global_idx && !many && total_tiles > 0) return hipErrorInvalidValue;
  const int32_t nchunks = static_cast<int32_t>((total_tiles + kScanChunk - 1) / kScanChunk);
  const unsigned grid = static_cast<unsigned>(total_tiles);  // total_tiles < kMaxTiles

  if (total_tiles > 0) {
    if (many) {
      int64_t prep_blocks = (total_tiles + 255) / 256;
      if (prep_blocks > 65536) prep_blocks = 65536;
      diff_prepare_kernel<<<dim3(unsigned(prep_blocks)), dim3(256), 0, stream>>>(
          d_table, nparams, total_tiles, tdesc, ctr);
      diff_count_kernel<true><<<dim3(grid), dim3(kDiffBlock), 0, stream>>>(
          tdesc, single, counts, compact, wide, ndense, tile_pos, ctr, arena_quads);
    } else {
      zero_ctr_kernel<<<dim3(1), dim3(64), 0, stream>>>(ctr);
      diff_count_kernel<false><<<dim3(grid), dim3(kDiffBlock), 0, stream>>>(
          nullptr, single, counts, compact, wide, ndense, tile_pos, ctr, arena_quads);
    }
    diff_scan_chunks_kernel<<<dim3(unsigned(nchunks)), dim3(kScanBlock), 0, stream>>>(
        counts, total_tiles, inpfx, chunk_tot, dense_list, ndense);
  }
  if (many)
    diff_base_kernel<true><<<dim3(1), dim3(kScanBlock), 0, stream>>>(
        d_table, nparams, total_tiles, nchunks, inpfx, chunk_tot, chunk_base, nnz, offsets);
  else
    diff_base_kernel<false><<<dim3(1), dim3(kScanBlock), 0, stream>>>(
        nullptr, nparams, total_tiles, nchunks, inpfx, chunk_tot, chunk_base, nnz, offsets);
  // checked here: the placing launcher's occupancy query clears the error state if it fails
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (total_tiles > 0) {
    if (many && global_idx)
      launch_place<true, int64_t>(tdesc, single, total_tiles, nchunks, inpfx, chunk_base, compact,
                                  wide, dense_list, ndense, static_cast<int64_t*>(idx), val,
                                  capacity, tile_pos, stream);
    else if (many)
      launch_place<true, int32_t>(tdesc, single, total_tiles, nchunks, inpfx, chunk_base, compact,
                                  wide, dense_list, ndense, static_cast<int32_t*>(idx), val,
                                  capacity, tile_pos, stream);
    else
      launch_place<false, int32_t>(tdesc, single, total_tiles, nchunks, inpfx, chunk_base, compact,
                                   wide, dense_list, ndense, static_cast<int32_t*>(idx), val,
                                   capacity, tile_pos, stream);
  }
  return hipGetLastError();
}

}  // namespace sbd
