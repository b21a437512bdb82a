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
//    that never straddles a parameter.  A lane issues eight 16-byte loads of
//    `old` and eight of `new` up front (all in flight together), so one wave
//    covers 1 KB contiguous per load instruction.
//  * Per 16-byte chunk the lane forms an 8-bit change mask; its popcount
//    c in [0, 8] is prefix-summed across the wave with four ballots over the
//    bits of c plus mbcnt (no shuffles), giving each lane its output slot.
//  * Wave totals go through LDS; a 32-entry scan in wave 0 yields each
//    (iteration, wave) pair's offset inside the tile, in ascending element
//    order (iteration-major, then wave, then lane, then slot).
//  * Tile offsets come from a single-pass decoupled look-back scan: tiles are
//    taken in order from an atomic counter (so a tile only ever waits on
//    tiles already owned by running workgroups), each tile publishes its
//    count and then its inclusive prefix in one 64-bit word
//    (2-bit status | 62-bit count) with agent-scope atomics, and wave 0 of
//    the next tile walks back 64 predecessors per step.  Only that one word
//    carries information between workgroups, so relaxed atomics suffice.
//  * `old` and `new` are read exactly once: the 4n-byte read plus the 6-byte
//    write per changed element is the whole HBM traffic, apart from 8 bytes
//    of scan state and 4 bytes of tile->parameter map per tile.
#include "sbd_internal.h"

namespace sbd {
namespace {

constexpr uint64_t kFlagAgg = 1ull << 62;
constexpr uint64_t kFlagPfx = 2ull << 62;
constexpr uint64_t kCountMask = (1ull << 62) - 1;

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

// Clears the scan state and the tile counter; for a parameter list also
// records which parameter every tile belongs to.
template <bool kMany>
__global__ __launch_bounds__(256) void diff_prepare_kernel(const DiffParam* __restrict__ table,
                                                           int32_t nparams, int64_t total_tiles,
                                                           uint64_t* __restrict__ state,
                                                           int32_t* __restrict__ tile_param,
                                                           uint32_t* __restrict__ counter) {
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
      tile_param[t] = lo;
    }
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) *counter = 0u;
}

template <bool kMany>
__global__ __launch_bounds__(kDiffBlock) void diff_kernel(
    const DiffParam* __restrict__ table, DiffParam single, const int32_t* __restrict__ tile_param,
    int64_t total_tiles, int32_t* __restrict__ idx, uint16_t* __restrict__ val, int64_t capacity,
    uint64_t* __restrict__ state, uint32_t* __restrict__ counter) {
  __shared__ uint32_t s_tile;
  __shared__ uint32_t s_wtot[kDiffIters * kDiffWaves];
  __shared__ uint32_t s_woff[kDiffIters * kDiffWaves];
  __shared__ uint64_t s_excl;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const uint64_t cap = static_cast<uint64_t>(capacity);

  for (;;) {
    if (tid == 0) s_tile = atomicAdd(counter, 1u);
    __syncthreads();
    const int64_t tile = static_cast<int64_t>(
        static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(s_tile))));
    if (tile >= total_tiles) break;

    DiffParam d;
    if constexpr (kMany)
      d = table[tile_param[tile]];
    else
      d = single;
    const int64_t e0 = (tile - d.first_tile) * kDiffTile;
    const bool vec = (d.numel - e0 >= kDiffTile) &&
                     (((reinterpret_cast<uintptr_t>(d.old_bits) |
                        reinterpret_cast<uintptr_t>(d.new_bits)) & 15u) == 0);

    uint4 nv[kDiffIters];
    uint32_t m[kDiffIters];
    if (vec) {
      const uint4* o4 = reinterpret_cast<const uint4*>(d.old_bits + e0) + tid;
      const uint4* n4 = reinterpret_cast<const uint4*>(d.new_bits + e0) + tid;
      uint4 ov[kDiffIters];
#pragma unroll
      for (int j = 0; j < kDiffIters; ++j) {
        ov[j] = o4[j * kDiffBlock];
        nv[j] = n4[j * kDiffBlock];
      }
#pragma unroll
      for (int j = 0; j < kDiffIters; ++j) m[j] = change_mask8(ov[j], nv[j]);
    } else {
      // Ragged tail or unaligned parameter: guarded 2-byte loads, same order.
#pragma unroll
      for (int j = 0; j < kDiffIters; ++j) {
        const int64_t base = e0 + int64_t(j) * kDiffBlock * kVec + int64_t(tid) * kVec;
        uint32_t w[4] = {0u, 0u, 0u, 0u};
        uint32_t mm = 0u;
#pragma unroll
        for (int s = 0; s < kVec; ++s) {
          const int64_t i = base + s;
          uint32_t o = 0u, x = 0u;
          if (i < d.numel) {
            o = d.old_bits[i];
            x = d.new_bits[i];
          }
          mm |= (o != x ? 1u : 0u) << s;
          w[s >> 1] |= x << (16 * (s & 1));
        }
        nv[j] = make_uint4(w[0], w[1], w[2], w[3]);
        m[j] = mm;
      }
    }

    // Lane offsets within each (iteration, wave) group.
    uint32_t lp[kDiffIters];
#pragma unroll
    for (int j = 0; j < kDiffIters; ++j) {
      uint32_t tot;
      lp[j] = wave_prefix_c(static_cast<uint32_t>(__popc(m[j])), tot);
      if (lane == 0) s_wtot[j * kDiffWaves + wave] = tot;
    }
    __syncthreads();

    if (wave == 0) {
      // Exclusive scan of the 32 group totals in element order.
      constexpr int kGroups = kDiffIters * kDiffWaves;
      static_assert(kGroups <= 64, "groups must fit one wave");
      const uint32_t v = lane < kGroups ? s_wtot[lane] : 0u;
      uint32_t inc = v;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(inc, o, 64);
        if (lane >= o) inc += y;
      }
      if (lane < kGroups) s_woff[lane] = inc - v;
      const uint64_t agg = static_cast<uint64_t>(__shfl(inc, 63, 64));

      // Decoupled look-back over the tiles before this one.
      uint64_t excl = 0;
      if (tile == 0) {
        if (lane == 0) store_state(&state[0], kFlagPfx | agg);
      } else {
        if (lane == 0) store_state(&state[tile], kFlagAgg | agg);
        int64_t hi = tile - 1;
        for (;;) {
          const int64_t t = hi - lane;
          const uint64_t f = t >= 0 ? load_state(&state[t]) : kFlagPfx;
          const uint64_t pfx = __ballot((f >> 62) == 2u);
          const uint64_t inv = __ballot((f >> 62) == 0u);
          // lanes up to and including the nearest published prefix
          const uint64_t upto = pfx ? (((pfx & (~pfx + 1ull)) << 1) - 1ull) : ~0ull;
          if (inv & upto) {
            __builtin_amdgcn_s_sleep(1);
            continue;
          }
          excl += wave_sum64(((upto >> lane) & 1ull) ? (f & kCountMask) : 0ull);
          if (pfx) break;
          hi -= 64;
        }
        if (lane == 0) store_state(&state[tile], kFlagPfx | (excl + agg));
      }
      if (lane == 0) s_excl = excl;
    }
    __syncthreads();

    // Emit in ascending element order.
    const uint64_t tbase = s_excl;
#pragma unroll
    for (int j = 0; j < kDiffIters; ++j) {
      const uint32_t mm = m[j];
      if (mm != 0u) {
        uint64_t pos = tbase + s_woff[j * kDiffWaves + wave] + lp[j];
        const int64_t ebase = e0 + int64_t(j) * kDiffBlock * kVec + int64_t(tid) * kVec;
        const uint4 x = nv[j];
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
    __syncthreads();  // LDS is reused by the next tile
  }
}

// Per-parameter counts and offsets from the tiles' inclusive prefixes.
template <bool kMany>
__global__ __launch_bounds__(256) void diff_finalize_kernel(const DiffParam* __restrict__ table,
                                                            int32_t nparams, int64_t total_tiles,
                                                            const uint64_t* __restrict__ state,
                                                            int64_t* __restrict__ nnz,
                                                            int64_t* __restrict__ offsets) {
  const int64_t p = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (p > nparams) return;
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
  uint32_t* counter = reinterpret_cast<uint32_t*>(base + L.counter);
  uint64_t* state = reinterpret_cast<uint64_t*>(base + L.state);
  int32_t* tile_param = reinterpret_cast<int32_t*>(base + L.tile_param);
  // d_table == nullptr: one tensor (nparams == 1, `single`) or an empty list
  // (nparams == 0, no tiles).
  const bool many = d_table != nullptr;

  int64_t prep_blocks = (total_tiles + 255) / 256;
  if (prep_blocks < 1) prep_blocks = 1;
  if (prep_blocks > 65536) prep_blocks = 65536;
  if (many)
    diff_prepare_kernel<true><<<dim3(unsigned(prep_blocks)), dim3(256), 0, stream>>>(
        d_table, nparams, total_tiles, state, tile_param, counter);
  else
    diff_prepare_kernel<false><<<dim3(unsigned(prep_blocks)), dim3(256), 0, stream>>>(
        nullptr, nparams, total_tiles, state, tile_param, counter);

  if (total_tiles > 0) {
    // One workgroup per tile up to 2^20 workgroups; beyond that each
    // workgroup keeps taking tiles from the counter.
    const int64_t grid = total_tiles < (int64_t(1) << 20) ? total_tiles : (int64_t(1) << 20);
    if (many)
      diff_kernel<true><<<dim3(unsigned(grid)), dim3(kDiffBlock), 0, stream>>>(
          d_table, single, tile_param, total_tiles, idx, val, capacity, state, counter);
    else
      diff_kernel<false><<<dim3(unsigned(grid)), dim3(kDiffBlock), 0, stream>>>(
          nullptr, single, tile_param, total_tiles, idx, val, capacity, state, counter);
  }

  const int64_t fin_blocks = (int64_t(nparams) + 1 + 255) / 256;
  if (many)
    diff_finalize_kernel<true><<<dim3(unsigned(fin_blocks)), dim3(256), 0, stream>>>(
        d_table, nparams, total_tiles, state, nnz, offsets);
  else
    diff_finalize_kernel<false><<<dim3(unsigned(fin_blocks)), dim3(256), 0, stream>>>(
        nullptr, nparams, total_tiles, state, nnz, offsets);
  return hipGetLastError();
}

}  // namespace sbd
