// apply.hip -- scatter a sparse delta into resident bf16 snapshots, in place.
//
// What is computed (TRL delta-sync article, section 4.3: the receiver assigns
// the delta's values at its indices of the flattened bf16 snapshot; the vLLM
// sparse-transfer work it mentions does the same in place with index_copy_):
// snapshot[idx[j]] = val[j] for every entry j.  In the batched form, entry j
// belongs to the parameter p with offsets[p] <= j < offsets[p+1].
//
// How, on gfx950:
//  * The entries are taken in chunks of 2048 consecutive ones.  A workgroup
//    applies one chunk at a time, striding over the chunks of a bounded grid
//    (kApplyGridFactor below); a lane loads 8 entries as two 16-byte idx
//    loads and one 16-byte val load, so the delta is read once, coalesced.
//  * The memory system handles a 2-byte store to a line of HBM as a masked
//    write of its 32-byte sector; a sector written whole, or better a 64-byte
//    segment, costs it less.  So a chunk whose entries are well formed
//    (one parameter, all in range, strictly ascending) may rewrite the
//    segments strictly inside its span whole.  A "segment" is an aligned
//    64-byte unit of memory (32 bf16), whatever the snapshot's alignment.
//    How depends on the entries per element of span:
//      - sparse (more than kMergeSpread elements per entry, about 4 %
//        density or less), and only when the whole delta has at least
//        kSegMinTotal entries: the workgroup lists the segments its entries
//        touch (a scan in LDS); four lanes read, patch and write back each
//        listed segment, 16 bytes each, nontemporal.  A smaller delta keeps
//        2-byte stores: its touched segments fit in or near the 256 MB
//        memory-side cache, which absorbs masked stores (measured at
//        2^28-2^30 elements and 0.3-1 % density: 1-3x faster than the
//        rewrite); at the 79 million entries of a 7B-shaped step the rewrite
//        is 8 % faster;
//      - dense (kMergeMinSpread to kMergeSpread elements per entry, about
//        4 % to 33 %): nearly every segment is touched, so the workgroup
//        reads its whole span into LDS in 8192-element windows, patches it
//        from its entries (held in registers) and writes it back;
//      - denser still (runs that cover whole segments): 2-byte stores, which
//        already merge into full lines in L2 without reading the snapshot.
//    The first and the last touched segment, which a neighbouring chunk
//    (applied by another workgroup, possibly at the same time) may share,
//    are always written with 2-byte stores, as is every entry of a chunk
//    that breaks the precondition or spans parameters.
//  * Snapshot pointers come from the parameter table in memory; they are
//    cast to the global address space so the stores are global, not flat.
//  * The parameter of the chunk's first entry comes from one 64-way
//    search over the device offsets; each lane then walks forward.  The
//    offsets are read on the GPU, so no host round trip separates diff and
//    apply.
//  * An index outside [0, numel) is skipped, never written.  With unsorted
//    or repeated indices the values at those entries' positions are
//    unspecified; every other position keeps its value (a rewritten segment
//    is written back with the values read from it, and lies inside the
//    snapshot).
#include <atomic>

#include "sbd_internal.h"

namespace sbd {
namespace {

constexpr int kApplyBlock = 256;
constexpr int kApplyWaves = kApplyBlock / 64;
constexpr int kApplyPer = 8;
constexpr int kApplyChunk = kApplyBlock * kApplyPer;  // 2048 entries per chunk
// Elements of span per entry that choose between the ways of writing a
// well-formed workgroup's interior segments (see above).
constexpr int64_t kMergeSpread = 24;
constexpr int64_t kMergeMinSpread = 3;
constexpr int kSegElems = 32;                        // bf16 per 64-byte segment
constexpr int kSegLanes = kSegElems / kVec;          // 4 lanes x 16 bytes per segment
constexpr int kSegGroups = kApplyBlock / kSegLanes;  // segments per workgroup pass
constexpr int kSegUnroll = 4;                        // segments in flight per lane
// Fewest delta entries for which sparse workgroups rewrite whole segments.
constexpr int64_t kSegMinTotal = int64_t(1) << 25;
constexpr int kMergeWindow = 8192;  // snapshot elements patched in LDS at a time
static_assert(kMergeWindow % kSegElems == 0, "windows hold whole segments");

enum ApplyMode : int { kScatter = 0, kWindows = 1, kSegments = 2 };

// The touched-segment list of a sparse workgroup (16 KB, the window's size).
struct SegList {
  uint32_t pos[kApplyChunk];    // per entry: its index plus the segment shift
  uint16_t val[kApplyChunk];    // per entry: its value
  uint16_t first[kApplyChunk];  // the first entry of each listed segment
};

struct ApplyShared {
  int64_t total;
  int32_t p0;
  int32_t one_param;  // every entry of the chunk belongs to parameter p0
  uint32_t wmin[kApplyWaves];
  uint32_t wmax[kApplyWaves];
  uint32_t wcnt[kApplyWaves];
  int32_t wfirst[kApplyWaves];  // first and last entry of each wave, for the order check
  int32_t wlast[kApplyWaves];
  uint32_t wsegs[kApplyWaves];  // listed segments per wave
  uint32_t last_first;          // the first entry in the last touched segment
  union {
    __attribute__((aligned(16))) uint16_t win[kMergeWindow];  // snapshot window being patched
    __attribute__((aligned(16))) SegList sl;
  };
};

__global__ __launch_bounds__(64) void zero_i64_kernel(int64_t* p) {
  if (threadIdx.x == 0) *p = 0;
}

// Element `k` (0..7) of a 16-byte vector of bf16 set to `v`.
__device__ __forceinline__ void set_elem(u32x4& x, uint32_t k, uint32_t v) {
  const uint32_t s = (k & 1u) * 16u;
  const uint32_t keep = ~(0xFFFFu << s), put = v << s;
  const uint32_t q = k >> 1;
  x.x = q == 0u ? (x.x & keep) | put : x.x;
  x.y = q == 1u ? (x.y & keep) | put : x.y;
  x.z = q == 2u ? (x.z & keep) | put : x.z;
  x.w = q == 3u ? (x.w & keep) | put : x.w;
}

// Applies entries [j0, j0 + kApplyChunk) of the delta.  Every lane of the
// workgroup reaches the end (the violation count is a wave reduction).
// Returns true, uniformly over the workgroup, when j0 lies at or past the
// delta's total, and then does nothing.
// kSegOK: the segment rewrite is compiled in (the launch's capacity allows a
// delta of kSegMinTotal entries); without it the kernel needs fewer registers.
template <bool kMany, bool kSegOK>
__device__ __forceinline__ bool apply_chunk(
    int64_t j0, const SnapParam* __restrict__ table, const SnapParam& single, int32_t nparams,
    const int64_t* __restrict__ offsets, const int32_t* __restrict__ idx,
    const uint16_t* __restrict__ val, int64_t max_nnz, int64_t* __restrict__ violations,
    ApplyShared& sh) {
  if (threadIdx.x < 64) {
    int64_t total = max_nnz;
    if constexpr (kMany) {
      const int64_t t = offsets[nparams];
      total = t < max_nnz ? t : max_nnz;
      if (j0 < total) {
        const int lane = threadIdx.x;
        const int32_t lo = find_param_wave0(offsets, nparams, j0);
        if (lane == 0) {
          sh.p0 = lo;
          const int64_t end = j0 + kApplyChunk < total ? j0 + kApplyChunk : total;
          sh.one_param = offsets[lo + 1] >= end ? 1 : 0;
        }
      }
    } else {
      if (threadIdx.x == 0) sh.one_param = 1;
    }
    if (threadIdx.x == 0) sh.total = total;
  }
  __syncthreads();
  const int64_t total = sh.total;
  if (j0 >= total) return true;  // uniform over the workgroup
  const int n_entries = total - j0 < kApplyChunk ? int(total - j0) : kApplyChunk;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int e0 = int(threadIdx.x) * kApplyPer;  // the lane's first entry in the chunk
  const int64_t jt = j0 + e0;
  int64_t bad = 0;
  int32_t iv[kApplyPer];
  uint16_t vv[kApplyPer];
  if (jt < total) {
    const bool vec = (jt + kApplyPer <= total) &&
                     (((reinterpret_cast<uintptr_t>(idx) | reinterpret_cast<uintptr_t>(val)) &
                       15u) == 0);
    if (vec) {
      const int4 a = reinterpret_cast<const int4*>(idx + jt)[0];
      const int4 b = reinterpret_cast<const int4*>(idx + jt)[1];
      const uint4 v = reinterpret_cast<const uint4*>(val + jt)[0];
      iv[0] = a.x; iv[1] = a.y; iv[2] = a.z; iv[3] = a.w;
      iv[4] = b.x; iv[5] = b.y; iv[6] = b.z; iv[7] = b.w;
      vv[0] = uint16_t(v.x); vv[1] = uint16_t(v.x >> 16);
      vv[2] = uint16_t(v.y); vv[3] = uint16_t(v.y >> 16);
      vv[4] = uint16_t(v.z); vv[5] = uint16_t(v.z >> 16);
      vv[6] = uint16_t(v.w); vv[7] = uint16_t(v.w >> 16);
    } else {
#pragma unroll
      for (int r = 0; r < kApplyPer; ++r) {
        const int64_t j = jt + r;
        iv[r] = j < total ? idx[j] : 0;
        vv[r] = j < total ? val[j] : uint16_t(0);
      }
    }
  } else {
#pragma unroll
    for (int r = 0; r < kApplyPer; ++r) {
      iv[r] = 0;
      vv[r] = 0;
    }
  }

  // ---- choose how to write (uniform over the workgroup) --------------------
  // Segments are numbered from the 64-byte segment holding the snapshot's
  // element 0, which sits `shift` elements into it: element i is in segment
  // (i + shift) / 32.  For a well-formed chunk the segments strictly between
  // the first and the last touched one hold the elements [lo_end, hi_start).
  int mode = kScatter;
  uint32_t shift = 0, ufirst = 0, ulast = 0, lo_end = 0, hi_start = 0;
  SnapParam dm = single;
  if (sh.one_param) {
    if constexpr (kMany) dm = table[sh.p0];
    shift = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(dm.snap) & 63u) >> 1;
    if ((reinterpret_cast<uintptr_t>(dm.snap) & 1u) == 0) {
      uint32_t umin = 0xFFFFFFFFu, umax = 0u, cnt = 0u;
      bool sorted = true, any = false;
      int32_t first = 0, last = 0;
#pragma unroll
      for (int r = 0; r < kApplyPer; ++r) {
        if (e0 + r < n_entries) {
          const uint32_t i = static_cast<uint32_t>(iv[r]);
          if (static_cast<uint64_t>(i) < static_cast<uint64_t>(dm.numel)) {
            umin = i < umin ? i : umin;
            umax = i > umax ? i : umax;
            ++cnt;
          }
          if (any && !(iv[r] > last)) sorted = false;
          if (!any) first = iv[r];
          last = iv[r];
          any = true;
        }
      }
      // ascending across neighbouring lanes of the wave
      const int32_t prev_last = __shfl_up(last, 1, 64);
      const int prev_any = __shfl_up(any ? 1 : 0, 1, 64);
      if (lane > 0 && prev_any && any && !(first > prev_last)) sorted = false;
      const bool wave_sorted = __ballot(!sorted) == 0ull;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const uint32_t a = static_cast<uint32_t>(__shfl_xor(static_cast<int>(umin), o, 64));
        const uint32_t b = static_cast<uint32_t>(__shfl_xor(static_cast<int>(umax), o, 64));
        umin = a < umin ? a : umin;
        umax = b > umax ? b : umax;
        cnt += static_cast<uint32_t>(__shfl_xor(static_cast<int>(cnt), o, 64));
      }
      if (lane == 0) {
        sh.wmin[wave] = umin;
        sh.wmax[wave] = umax;
        sh.wcnt[wave] = wave_sorted ? cnt : 0xFFFFFFFFu;
        sh.wfirst[wave] = first;  // lane 0 holds the wave's first entry
      }
      const int next_any = __shfl_down(any ? 1 : 0, 1, 64);  // every lane takes part
      if (any && (lane == 63 || !next_any)) sh.wlast[wave] = last;  // the wave's last entry
      __syncthreads();
      uint32_t gmin = 0xFFFFFFFFu, gmax = 0u, gcnt = 0u;
      bool well_formed = true;
#pragma unroll
      for (int w = 0; w < kApplyWaves; ++w) {
        gmin = sh.wmin[w] < gmin ? sh.wmin[w] : gmin;
        gmax = sh.wmax[w] > gmax ? sh.wmax[w] : gmax;
        if (sh.wcnt[w] == 0xFFFFFFFFu) well_formed = false;
        gcnt += sh.wcnt[w];
        // ascending across the boundary between waves w - 1 and w
        if (w > 0 && w * 64 * kApplyPer < n_entries && !(sh.wfirst[w] > sh.wlast[w - 1]))
          well_formed = false;
      }
      well_formed = well_formed && gcnt == static_cast<uint32_t>(n_entries);  // all in range
      if (well_formed && gcnt > 0u) {
        // indices are below 2^31, so these stay within 32 bits
        ufirst = (gmin + shift) / kSegElems;
        ulast = (gmax + shift) / kSegElems;
        const int64_t span = int64_t(gmax - gmin) + 1;
        if (ulast >= ufirst + 2u) {
          if (span > kMergeSpread * int64_t(gcnt)) {
            if (kSegOK && total >= kSegMinTotal) mode = kSegments;
          } else if (span >= kMergeMinSpread * int64_t(gcnt)) {
            mode = kWindows;
          }
        }
        lo_end = (ufirst + 1u) * kSegElems - shift;
        hi_start = ulast * kSegElems - shift;
      }
    }
  }

  // ---- entry by entry: every entry, or only the edge segments' ------------
  if (jt < total) {
    int32_t p = 0;
    SnapParam d = single;
    int64_t seg_start = 0, seg_end = total;
    if constexpr (kMany) {
      p = sh.p0;
      seg_start = offsets[p];
      seg_end = offsets[p + 1];
      while (seg_end <= jt) {
        ++p;
        seg_start = seg_end;
        seg_end = offsets[p + 1];
      }
      d = table[p];
    }
    int32_t prev = 0;
    bool have_prev = false;
    if (violations != nullptr && jt > seg_start) {
      prev = idx[jt - 1];
      have_prev = true;
    }
#pragma unroll
    for (int r = 0; r < kApplyPer; ++r) {
      const int64_t j = jt + r;
      if (j < total) {
        if constexpr (kMany) {
          if (j >= seg_end) {
            do {
              ++p;
              seg_start = seg_end;
              seg_end = offsets[p + 1];
            } while (seg_end <= j);
            d = table[p];
            have_prev = false;
          }
        }
        const uint32_t i = static_cast<uint32_t>(iv[r]);
        const bool in_range = static_cast<uint64_t>(i) < static_cast<uint64_t>(d.numel);
        const bool interior = mode != kScatter && i >= lo_end && i < hi_start;
        if (in_range && !interior) *global_ptr(d.snap + i) = vv[r];
        if (violations != nullptr) {
          bad += (!in_range || (have_prev && iv[r] <= prev)) ? 1 : 0;
          prev = iv[r];
          have_prev = true;
        }
      }
    }
  }

  // ---- sparse: list the touched interior segments, then rewrite each -----
  if constexpr (kSegOK) {
    if (mode == kSegments) {
      // The 64-byte-aligned address of segment 0.
      const uintptr_t seg0 = reinterpret_cast<uintptr_t>(dm.snap) - 2u * shift;
      // The entry before the lane's first one: the previous lane's last, or
      // for a wave's lane 0 the previous wave's last (entry 0 needs none).
      int32_t before = __shfl_up(iv[kApplyPer - 1], 1, 64);
      if (lane == 0) before = wave > 0 ? sh.wlast[wave - 1] : 0;
      uint32_t pu = (static_cast<uint32_t>(before) + shift) / kSegElems;
      uint32_t leads = 0u, nlead = 0u;
#pragma unroll
      for (int r = 0; r < kApplyPer; ++r) {
        const int e = e0 + r;
        const uint32_t u = (static_cast<uint32_t>(iv[r]) + shift) / kSegElems;
        const bool lead = e < n_entries && (e == 0 || u != pu);
        pu = u;
        if (lead && u > ufirst && u < ulast) {
          leads |= 1u << r;
          ++nlead;
        }
        if (lead && u == ulast) sh.last_first = uint32_t(e);
      }
      // the lane's entries, as 16-byte LDS stores
#pragma unroll
      for (int h = 0; h < kApplyPer; h += 4) {
        u32x4 w;
        w.x = static_cast<uint32_t>(iv[h + 0]) + shift;
        w.y = static_cast<uint32_t>(iv[h + 1]) + shift;
        w.z = static_cast<uint32_t>(iv[h + 2]) + shift;
        w.w = static_cast<uint32_t>(iv[h + 3]) + shift;
        *reinterpret_cast<u32x4*>(&sh.sl.pos[e0 + h]) = w;
      }
      {
        u32x4 w;
        w.x = uint32_t(vv[0]) | (uint32_t(vv[1]) << 16);
        w.y = uint32_t(vv[2]) | (uint32_t(vv[3]) << 16);
        w.z = uint32_t(vv[4]) | (uint32_t(vv[5]) << 16);
        w.w = uint32_t(vv[6]) | (uint32_t(vv[7]) << 16);
        *reinterpret_cast<u32x4*>(&sh.sl.val[e0]) = w;
      }
      // slots in the list: a workgroup scan of the lanes' leader counts
      uint32_t incl = nlead;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = static_cast<uint32_t>(__shfl_up(static_cast<int>(incl), o, 64));
        if (lane >= o) incl += t;
      }
      if (lane == 63) sh.wsegs[wave] = incl;
      __syncthreads();
      uint32_t slot = incl - nlead, ns = 0u;
#pragma unroll
      for (int w = 0; w < kApplyWaves; ++w) {
        slot += w < wave ? sh.wsegs[w] : 0u;
        ns += sh.wsegs[w];
      }
#pragma unroll
      for (int r = 0; r < kApplyPer; ++r) {
        if ((leads >> r) & 1u) {
          sh.sl.first[slot] = static_cast<uint16_t>(e0 + r);
          ++slot;
        }
      }
      __syncthreads();
      // four lanes per listed segment: read it, patch it, write it back
      const uint32_t g = threadIdx.x / kSegLanes;
      const uint32_t sub = threadIdx.x % kSegLanes;
      const uint32_t last_first = sh.last_first;
      for (uint32_t s0 = 0; s0 < ns; s0 += kSegGroups * kSegUnroll) {
        u32x4 x[kSegUnroll];
#pragma unroll
        for (int k = 0; k < kSegUnroll; ++k) {
          const uint32_t s = s0 + k * kSegGroups + g;
          if (s < ns) {
            const uint32_t u = sh.sl.pos[sh.sl.first[s]] / kSegElems;
            const uintptr_t a = seg0 + uintptr_t(u) * 64u + sub * 16u;
            x[k] = __builtin_nontemporal_load(global_ptr(reinterpret_cast<const u32x4*>(a)));
          }
        }
#pragma unroll
        for (int k = 0; k < kSegUnroll; ++k) {
          const uint32_t s = s0 + k * kSegGroups + g;
          if (s < ns) {
            const uint32_t eb = sh.sl.first[s];
            const uint32_t ee = s + 1u < ns ? uint32_t(sh.sl.first[s + 1u]) : last_first;
            for (uint32_t e = eb; e < ee; ++e) {
              const uint32_t off = sh.sl.pos[e] % kSegElems;
              if (off / kVec == sub) set_elem(x[k], off % kVec, sh.sl.val[e]);
            }
            const uint32_t u = sh.sl.pos[eb] / kSegElems;
            const uintptr_t a = seg0 + uintptr_t(u) * 64u + sub * 16u;
            __builtin_nontemporal_store(x[k], global_ptr(reinterpret_cast<u32x4*>(a)));
          }
        }
      }
    }
  }

  // ---- dense: window by window, read whole segments into LDS, patch them
  // from the lanes' entries, write them back whole ---------------------------
  if (mode == kWindows) {
    for (uint32_t w0 = lo_end; w0 < hi_start; w0 += kMergeWindow) {
      const uint32_t w1 = hi_start - w0 < uint32_t(kMergeWindow) ? hi_start : w0 + kMergeWindow;
      for (uint32_t c = threadIdx.x; c < (w1 - w0) / kVec; c += kApplyBlock) {
        const u32x4 x = *global_ptr(reinterpret_cast<const u32x4*>(dm.snap + w0) + c);
        *reinterpret_cast<u32x4*>(&sh.win[c * kVec]) = x;
      }
      __syncthreads();
#pragma unroll
      for (int r = 0; r < kApplyPer; ++r) {
        const uint32_t i = static_cast<uint32_t>(iv[r]);
        if (e0 + r < n_entries && i >= w0 && i < w1) sh.win[i - w0] = vv[r];
      }
      __syncthreads();
      for (uint32_t c = threadIdx.x; c < (w1 - w0) / kVec; c += kApplyBlock) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(&sh.win[c * kVec]);
        *global_ptr(reinterpret_cast<u32x4*>(dm.snap + w0) + c) = x;
      }
      __syncthreads();  // the window is refilled next
    }
  }
  if (violations != nullptr) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) bad += __shfl_xor(bad, o, 64);
    if (lane == 0 && bad != 0)
      atomicAdd(reinterpret_cast<unsigned long long*>(violations),
                static_cast<unsigned long long>(bad));
  }
  return false;
}

template <bool kMany, bool kSegOK>
__global__ __launch_bounds__(kApplyBlock) void apply_kernel(
    const SnapParam* __restrict__ table, SnapParam single, int32_t nparams,
    const int64_t* __restrict__ offsets, const int32_t* __restrict__ idx,
    const uint16_t* __restrict__ val, int64_t max_nnz, int64_t* __restrict__ violations) {
  __shared__ ApplyShared sh;
  const int64_t nchunks = (max_nnz + kApplyChunk - 1) / kApplyChunk;
  for (int64_t chunk = blockIdx.x; chunk < nchunks; chunk += gridDim.x) {
    const bool past = apply_chunk<kMany, kSegOK>(chunk * kApplyChunk, table, single, nparams,
                                                 offsets, idx, val, max_nnz, violations, sh);
    __syncthreads();  // the shared state is rewritten by the next chunk
    if (past) break;  // this workgroup's later chunks lie past the total too
  }
}

// The grid is bounded by kApplyGridFactor times the workgroups the GPU holds
// at once, queried once per device; each workgroup then strides over chunks.
// A caller that passes its buffer's capacity as max_nnz (diff and apply in one
// stream, no host read of the count) would otherwise launch one workgroup per
// chunk of that capacity, most of which find no entries and exit: on the
// 7B-shaped list at 1.2 % with a capacity of an eighth of the elements, about
// 370,000 such workgroups took 0.1 ms.  Measured against one workgroup per
// chunk: equal or faster on every list and density tried (up to 7 % at 8-12 %
// density); a factor of 1 or 2 was 10-25 % slower (too little dynamic
// balancing between chunks of different cost).
constexpr int64_t kApplyGridFactor = 16;

template <bool kMany, bool kSegOK>
int64_t apply_grid_limit() {
  static std::atomic<int64_t> cached[64];  // zero-initialised; threads may race to fill it
  constexpr int64_t kFallback = 256 * 8 * kApplyGridFactor;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return kFallback;
  }
  int64_t lim = cached[dev].load(std::memory_order_relaxed);
  if (lim == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, apply_kernel<kMany, kSegOK>,
                                                     kApplyBlock, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        per_cu < 1 || cus < 1) {
      (void)hipGetLastError();
      return kFallback;
    }
    lim = int64_t(per_cu) * cus * kApplyGridFactor;
    cached[dev].store(lim, std::memory_order_relaxed);
  }
  return lim;
}

template <bool kMany, bool kSegOK>
void launch_apply_kernel(unsigned blocks, const SnapParam* d_table, const SnapParam& single,
                         int32_t nparams, const int64_t* offsets, const int32_t* idx,
                         const uint16_t* val, int64_t max_nnz, int64_t* violations,
                         hipStream_t stream) {
  const int64_t lim = apply_grid_limit<kMany, kSegOK>();
  if (int64_t(blocks) > lim) blocks = static_cast<unsigned>(lim);
  apply_kernel<kMany, kSegOK><<<dim3(blocks), dim3(kApplyBlock), 0, stream>>>(
      d_table, single, nparams, offsets, idx, val, max_nnz, violations);
}

}  // namespace

hipError_t launch_apply(const SnapParam* d_table, const SnapParam& single, int32_t nparams,
                        const int64_t* offsets, const int32_t* idx, const uint16_t* val,
                        int64_t max_nnz, int64_t* violations, hipStream_t stream) {
  clear_stale_error();
  if (violations != nullptr) zero_i64_kernel<<<dim3(1), dim3(64), 0, stream>>>(violations);
  if (max_nnz > 0) {
    int64_t blocks = (max_nnz + kApplyChunk - 1) / kApplyChunk;
    if (blocks > (int64_t(1) << 20)) blocks = int64_t(1) << 20;
    const unsigned b = unsigned(blocks);
    // the segment rewrite needs a delta of kSegMinTotal entries, which only a
    // capacity that large can hold
    const bool seg = max_nnz >= kSegMinTotal;
    if (d_table != nullptr) {
      if (seg)
        launch_apply_kernel<true, true>(b, d_table, single, nparams, offsets, idx, val, max_nnz,
                                        violations, stream);
      else
        launch_apply_kernel<true, false>(b, d_table, single, nparams, offsets, idx, val, max_nnz,
                                         violations, stream);
    } else {
      if (seg)
        launch_apply_kernel<false, true>(b, nullptr, single, 1, nullptr, idx, val, max_nnz,
                                         violations, stream);
      else
        launch_apply_kernel<false, false>(b, nullptr, single, 1, nullptr, idx, val, max_nnz,
                                          violations, stream);
    }
  }
  return hipGetLastError();
}

}  // namespace sbd
