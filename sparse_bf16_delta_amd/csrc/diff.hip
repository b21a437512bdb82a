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
// How, on gfx950:
//  * Each workgroup (256 lanes = 4 wave64s) owns one tile of 16384 elements
//    that never straddles a parameter.  A prepare kernel writes each tile's
//    descriptor (base pointers, first index, length), so a workgroup does one
//    uniform load before its data loads.  A lane issues eight 16-byte loads of
//    `old` and eight of `new` up front (all in flight together); one wave
//    covers 1 KB contiguous per load instruction.
//  * Per 16-byte chunk the lane forms an 8-bit change mask; its popcount
//    c in [0, 8] is prefix-summed across the wave with four ballots over the
//    bits of c plus mbcnt (no shuffles), giving each lane its output slot.
//  * Wave totals go through LDS; a 32-entry scan in wave 0 yields each
//    (iteration, wave) group's offset inside the tile, in ascending element
//    order (iteration-major, then wave, then lane, then slot), and the tile's
//    count, which is published at once.
//  * The compacted tile is staged in LDS as (tile-local index << 16 | bits),
//    4 bytes per entry, up to 4096 entries (16 KB); after the look-back the
//    workgroup copies it out with coalesced stores.  A denser tile skips the
//    staging and writes directly, re-reading its changed 16-byte chunks of
//    `new`, which it has just read and which are still cached.
//  * Tile offsets come from a single-pass decoupled look-back scan.  Tile t
//    is workgroup t: the dispatcher starts workgroups in increasing id order,
//    so every tile a workgroup waits for has already started.  (A global
//    atomic tile counter would guarantee that without relying on dispatch
//    order, but one serialized atomic per tile cost a third of the kernel's
//    time.)  Each tile publishes its count and then its inclusive prefix in
//    one 64-bit word (2-bit status | 62-bit count) with agent-scope atomics,
//    and wave 0 of a tile walks back 64 predecessors per step.  Only that
//    word carries information between workgroups, so relaxed atomics
//    suffice.
//  * Every wait is bounded: a tile that sees no progress for about 2^28
//    ticks of the constant-rate wall clock (about 2.7 s at 100 MHz) raises a
//    flag in the workspace and stops waiting; the finalize kernel then
//    reports -1 for every count instead of a wrong delta.
//  * Registers hold one tile's data only until it is staged, and LDS holds
//    16 KB per workgroup, so six workgroups share a CU.
//  * `old` and `new` are read exactly once: the 4n-byte read plus the 6-byte
//    write per changed element is the whole HBM traffic, apart from 40 bytes
//    of scan state and descriptor per tile.
#include "sbd_internal.h"

namespace sbd {
namespace {

constexpr uint64_t kFlagAgg = 1ull << 62;
constexpr uint64_t kFlagPfx = 2ull << 62;
constexpr uint64_t kCountMask = (1ull << 62) - 1;
// Longest wait for predecessor tiles, in wall-clock ticks.
constexpr long long kSpinTicks = 1ll << 28;

__device__ __forceinline__ uint64_t load_state(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_state(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

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

__device__ __forceinline__ uint64_t wave_sum64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <int S>
__device__ __forceinline__ void emit_slot(uint32_t mm, uint64_t& pos, int64_t ebase,
                                          const uint4& x, int32_t* __restrict__ idx,
                                          uint16_t* __restrict__ val, uint64_t cap) {
  if (mm & (1u << S)) {
    if (pos < cap) {
      idx[pos] = static_cast<int32_t>(ebase + S);
      val[pos] = half_of<S>(x);
    }
    ++pos;
  }
}

template <int S>
__device__ __forceinline__ void stage_slot(uint32_t mm, uint32_t& pos, uint32_t local,
                                           const uint4& x, uint32_t* stage) {
  if (mm & (1u << S)) {
    stage[pos] = ((local + S) << 16) | half_of<S>(x);
    ++pos;
  }
}

// Clears the scan state and the timeout flag; for a parameter list also
// writes every tile's descriptor (base pointers, first index, length), so the
// main kernel needs one load, not a parameter search, before its data loads.
template <bool kMany>
__global__ __launch_bounds__(256) void diff_prepare_kernel(const DiffParam* __restrict__ table,
                                                           int32_t nparams, int64_t total_tiles,
                                                           uint64_t* __restrict__ state,
                                                           TileDesc* __restrict__ tdesc,
                                                           uint32_t* __restrict__ flag) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; t < total_tiles; t += stride) {
    state[t] = 0;
    if constexpr (kMany) {
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
      td.pad = 0;
      tdesc[t] = td;
    }
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) *flag = 0u;
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

template <bool kMany>
__global__ __launch_bounds__(kDiffBlock) void diff_kernel(
    const TileDesc* __restrict__ tdesc, DiffParam single, int32_t* __restrict__ idx,
    uint16_t* __restrict__ val, int64_t capacity, uint64_t* __restrict__ state,
    uint32_t* __restrict__ flag) {
  constexpr int kGroups = kDiffIters * kDiffWaves;
  constexpr int kPerLane = (kGroups + 63) / 64;
  static_assert(kGroups <= 128, "groups must fit two per lane of one wave");
  static_assert(kDiffTile <= 65536, "tile-local indices are staged in 16 bits");
  __shared__ uint32_t s_stage[kStageCap];  // (tile-local index << 16) | new bits
  __shared__ uint32_t s_wtot[kGroups];
  __shared__ uint32_t s_woff[kGroups];
  __shared__ uint32_t s_agg;
  __shared__ uint64_t s_excl;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t tile = blockIdx.x;

  const uint16_t* ob;
  const uint16_t* nb;
  int32_t e0, valid;
  if constexpr (kMany) {
    const TileDesc td = tdesc[tile];
    ob = td.old_bits;
    nb = td.new_bits;
    e0 = td.e0;
    valid = td.valid;
  } else {
    const int64_t first = tile * kDiffTile;
    const int64_t left = single.numel - first;
    ob = single.old_bits + first;
    nb = single.new_bits + first;
    e0 = static_cast<int32_t>(first);
    valid = static_cast<int32_t>(left < kDiffTile ? left : kDiffTile);
  }
  const bool vec = valid == kDiffTile &&
                   ((reinterpret_cast<uintptr_t>(ob) | reinterpret_cast<uintptr_t>(nb)) & 15u) == 0;

  // ---- load, compare, count ------------------------------------------------
  uint4 nv[kDiffIters];
  uint32_t m[kDiffIters];
  if (vec) {
    const uint4* o4 = reinterpret_cast<const uint4*>(ob) + tid;
    const uint4* n4 = reinterpret_cast<const uint4*>(nb) + tid;
    uint4 ov[kDiffIters];
#pragma unroll
    for (int j = 0; j < kDiffIters; ++j) {
      ov[j] = load16(o4 + j * kDiffBlock);
      nv[j] = load16(n4 + j * kDiffBlock);
    }
#pragma unroll
    for (int j = 0; j < kDiffIters; ++j) m[j] = change_mask8(ov[j], nv[j]);
  } else {
    // ragged last tile or unaligned parameter
#pragma unroll
    for (int j = 0; j < kDiffIters; ++j) {
      const int local = j * kDiffBlock * kVec + tid * kVec;
      const uint4 o = load_chunk(ob, local, valid, false);
      nv[j] = load_chunk(nb, local, valid, false);
      m[j] = change_mask8(o, nv[j]);
    }
  }
  uint32_t lp[kDiffIters];
#pragma unroll
  for (int j = 0; j < kDiffIters; ++j) {
    uint32_t tot;
    lp[j] = wave_prefix_c(static_cast<uint32_t>(__popc(m[j])), tot);
    if (lane == 0) s_wtot[j * kDiffWaves + wave] = tot;
  }
  __syncthreads();

  // ---- wave 0: group offsets in element order; publish the tile count ------
  if (wave == 0) {
    // lane l owns groups [l * kPerLane, (l + 1) * kPerLane)
    uint32_t v[kPerLane];
    uint32_t own = 0;
#pragma unroll
    for (int q = 0; q < kPerLane; ++q) {
      const int g = lane * kPerLane + q;
      v[q] = g < kGroups ? s_wtot[g] : 0u;
      own += v[q];
    }
    uint32_t inc = own;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(inc, o, 64);
      if (lane >= o) inc += y;
    }
    uint32_t run = inc - own;
#pragma unroll
    for (int q = 0; q < kPerLane; ++q) {
      const int g = lane * kPerLane + q;
      if (g < kGroups) s_woff[g] = run;
      run += v[q];
    }
    const uint32_t agg = __shfl(inc, 63, 64);
    if (lane == 0) {
      s_agg = agg;
      store_state(&state[tile], (tile == 0 ? kFlagPfx : kFlagAgg) | agg);
    }
  }
  __syncthreads();

  // ---- stage the compacted tile in LDS (when it fits) ----------------------
  const uint32_t agg = s_agg;
  const bool staged = agg <= static_cast<uint32_t>(kStageCap);
  if (staged) {
#pragma unroll
    for (int j = 0; j < kDiffIters; ++j) {
      const uint32_t mm = m[j];
      if (mm != 0u) {
        uint32_t pos = s_woff[j * kDiffWaves + wave] + lp[j];
        const uint32_t local = static_cast<uint32_t>(j * kDiffBlock * kVec + tid * kVec);
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

  // ---- sparse tiles: waves 1-3 leave; wave 0 finishes alone ---------------
  const bool solo = agg <= static_cast<uint32_t>(kSoloCap);
  if (solo) {
    __syncthreads();  // staging complete
    if (wave != 0) return;
  }
  uint64_t excl = 0;
  // ---- wave 0: decoupled look-back over the preceding tiles ----------------
  if (wave == 0) {
    if (tile > 0) {
      int64_t hi = tile - 1;
      long long t_wait = -1;
      for (;;) {
        const int64_t t = hi - lane;
        const uint64_t f = t >= 0 ? load_state(&state[t]) : kFlagPfx;
        const uint64_t pfx = __ballot((f >> 62) == 2u);
        const uint64_t inv = __ballot((f >> 62) == 0u);
        // lanes up to and including the nearest published prefix
        const uint64_t upto = pfx ? (((pfx & (~pfx + 1ull)) << 1) - 1ull) : ~0ull;
        if (inv & upto) {
          const long long now = wall_clock64();
          if (t_wait < 0) {
            t_wait = now;
          } else if (now - t_wait > kSpinTicks ||
                     __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) {
            if (lane == 0)
              __hip_atomic_store(flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;  // give up: the counts are reported as failed
          }
          __builtin_amdgcn_s_sleep(1);
          continue;
        }
        t_wait = -1;
        excl += wave_sum64(((upto >> lane) & 1ull) ? (f & kCountMask) : 0ull);
        if (pfx) break;
        hi -= 64;
      }
      if (lane == 0) store_state(&state[tile], kFlagPfx | (excl + agg));
    }
    if (lane == 0) s_excl = excl;
  }
  if (!solo) {
    __syncthreads();
    excl = s_excl;
  }

  // ---- emit ----------------------------------------------------------------
  const uint64_t tbase = excl;
  const uint64_t cap = static_cast<uint64_t>(capacity);
  if (staged) {
    // coalesced copy of the staged entries
    const uint32_t step = solo ? 64u : uint32_t(kDiffBlock);
    for (uint32_t p = static_cast<uint32_t>(solo ? lane : tid); p < agg; p += step) {
      const uint64_t o = tbase + p;
      if (o < cap) {
        const uint32_t w = s_stage[p];
        idx[o] = e0 + static_cast<int32_t>(w >> 16);
        val[o] = static_cast<uint16_t>(w & 0xFFFFu);
      }
    }
  } else {
    // dense tile: re-read the changed chunks of `new` (just read, so cached)
#pragma unroll
    for (int j = 0; j < kDiffIters; ++j) {
      const uint32_t mm = m[j];
      if (mm != 0u) {
        uint64_t pos = tbase + s_woff[j * kDiffWaves + wave] + lp[j];
        const int local = j * kDiffBlock * kVec + tid * kVec;
        const uint4 x = load_chunk(nb, local, valid, vec);
        const int64_t ebase = int64_t(e0) + local;
        emit_slot<0>(mm, pos, ebase, x, idx, val, cap);
        emit_slot<1>(mm, pos, ebase, x, idx, val, cap);
        emit_slot<2>(mm, pos, ebase, x, idx, val, cap);
        emit_slot<3>(mm, pos, ebase, x, idx, val, cap);
        emit_slot<4>(mm, pos, ebase, x, idx, val, cap);
        emit_slot<5>(mm, pos, ebase, x, idx, val, cap);
        emit_slot<6>(mm, pos, ebase, x, idx, val, cap);
        emit_slot<7>(mm, pos, ebase, x, idx, val, cap);
      }
    }
  }
}

// Per-parameter counts and offsets from the tiles' inclusive prefixes.
template <bool kMany>
__global__ __launch_bounds__(256) void diff_finalize_kernel(const DiffParam* __restrict__ table,
                                                            int32_t nparams, int64_t total_tiles,
                                                            const uint64_t* __restrict__ state,
                                                            const uint32_t* __restrict__ flag,
                                                            int64_t* __restrict__ nnz,
                                                            int64_t* __restrict__ offsets) {
  const int64_t p = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (p > nparams) return;
  if (*flag != 0u) {  // a look-back wait timed out: no count is trustworthy
    if (offsets) offsets[p] = -1;
    if (p < nparams) nnz[p] = -1;
    return;
  }
  auto before = [&](int64_t ft) -> int64_t {
    return ft == 0 ? 0 : static_cast<int64_t>(state[ft - 1] & kCountMask);
  };
  int64_t ft = total_tiles;
  if (p < nparams) ft = kMany ? table[p].first_tile : 0;
  const int64_t off = before(ft);
  if (offsets) offsets[p] = off;
  if (p < nparams) {
    const int64_t ft_next = (kMany && p + 1 < nparams) ? table[p + 1].first_tile : total_tiles;
    nnz[p] = before(ft_next) - off;
  }
}

}  // namespace

hipError_t launch_diff(const DiffParam* d_table, const DiffParam& single, int32_t nparams,
                       int64_t total_tiles, int32_t* idx, uint16_t* val, int64_t capacity,
                       int64_t* nnz, int64_t* offsets, void* ws, const WsLayout& L,
                       hipStream_t stream) {
  char* base = static_cast<char*>(ws);
  uint32_t* flag = reinterpret_cast<uint32_t*>(base + L.flag);
  uint64_t* state = reinterpret_cast<uint64_t*>(base + L.state);
  TileDesc* tdesc = reinterpret_cast<TileDesc*>(base + L.tile_desc);
  // d_table == nullptr: one tensor (nparams == 1, `single`) or an empty list
  // (nparams == 0, no tiles).
  const bool many = d_table != nullptr;

  int64_t prep_blocks = (total_tiles + 255) / 256;
  if (prep_blocks < 1) prep_blocks = 1;
  if (prep_blocks > 65536) prep_blocks = 65536;
  if (many)
    diff_prepare_kernel<true><<<dim3(unsigned(prep_blocks)), dim3(256), 0, stream>>>(
        d_table, nparams, total_tiles, state, tdesc, flag);
  else
    diff_prepare_kernel<false><<<dim3(unsigned(prep_blocks)), dim3(256), 0, stream>>>(
        nullptr, nparams, total_tiles, state, tdesc, flag);

  if (total_tiles > 0) {
    // one workgroup per tile, in tile order (total_tiles <= kMaxTiles)
    if (many)
      diff_kernel<true><<<dim3(unsigned(total_tiles)), dim3(kDiffBlock), 0, stream>>>(
          tdesc, single, idx, val, capacity, state, flag);
    else
      diff_kernel<false><<<dim3(unsigned(total_tiles)), dim3(kDiffBlock), 0, stream>>>(
          nullptr, single, idx, val, capacity, state, flag);
  }

  const int64_t fin_blocks = (int64_t(nparams) + 1 + 255) / 256;
  if (many)
    diff_finalize_kernel<true><<<dim3(unsigned(fin_blocks)), dim3(256), 0, stream>>>(
        d_table, nparams, total_tiles, state, flag, nnz, offsets);
  else
    diff_finalize_kernel<false><<<dim3(unsigned(fin_blocks)), dim3(256), 0, stream>>>(
        nullptr, nparams, total_tiles, state, flag, nnz, offsets);
  return hipGetLastError();
}

}  // namespace sbd
