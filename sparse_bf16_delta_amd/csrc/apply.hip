// apply.hip -- scatter a sparse delta into resident bf16 snapshots, in place.
//
// What is computed (TRL delta-sync article, section 4.3: the receiver assigns
// the delta's values at its indices of the flattened bf16 snapshot; the vLLM
// sparse-transfer work it mentions does the same in place with index_copy_):
// snapshot[idx[j]] = val[j] for every entry j.  In the batched form, entry j
// belongs to the parameter p with offsets[p] <= j < offsets[p+1].
//
// How, on gfx950.  The memory system handles a 2-byte store to HBM as a
// masked write of its 32-byte sector; a sector written whole, or better a
// 64-byte segment, costs it less.  So a chunk of entries that is well formed
// (one parameter, all in range, strictly ascending) may rewrite the segments
// strictly inside its span whole.  A "segment" is an aligned 64-byte unit of
// memory (32 bf16), whatever the snapshot's alignment.  The first and the
// last touched segment of a chunk, which a neighbouring chunk (applied by
// another workgroup, possibly at the same time) may share, are always written
// with 2-byte stores, as is every entry of a chunk that breaks the
// precondition or spans parameters.  How the interior is written depends on
// the elements of span per entry:
//   - sparse (more than kMergeSpread elements per entry, about 5 % density or
//     less): read, patch and write back each touched segment (the segment
//     rewrite), but only for deltas of at least kSegMinTotal entries.  A
//     smaller delta's touched segments fit in or near the 256 MB memory-side
//     cache, which absorbs masked stores (measured at 2^28-2^30 elements and
//     0.3-1 % density: 2-byte stores 1-3x faster than the rewrite);
//   - dense (kMergeMinSpread to kMergeSpread elements per entry, about 5 % to
//     33 %): nearly every segment is touched, so the workgroup reads its
//     whole span into LDS in 8192-element windows, patches it from its
//     entries (held in registers) and writes it back, with nontemporal
//     accesses and the next window's loads in flight meanwhile (on the
//     Qwen3-0.6B-shaped list at 8 %: 0.539 ms cached and one window at a
//     time, 0.488 nontemporal, 0.457 with the next window in flight;
//     4096- or 16384-element windows were slower);
//   - denser still (runs that cover whole segments): 2-byte stores, which
//     already merge into full lines in L2 without reading the snapshot.
//
// Two kernels share these rules:
//  * apply_kernel (deltas below kSegMinTotal entries, and larger ones above
//    about 2.8 % density): 256-lane workgroups with chunks of 2048 entries,
//    or for deltas of kSegMinTotal entries or more that average
//    kWidePerParam entries per parameter 512-lane ones with chunks of 4096
//    (8 entries per lane: two 16-byte idx loads and one 16-byte val load), a
//    grid bounded at kApplyGridFactor times the workgroups the GPU holds at
//    once, striding over the chunks; scatter, windows, and for deltas of
//    kSegMinTotal entries or more the segment rewrite in passes of one
//    segment per four lanes, four passes in flight.
//  * apply_big_kernel (deltas of kSegMinTotal entries or more at about 2.8 %
//    density or less): 1024-lane workgroups, chunks of 1024 entries (one per
//    lane), one chunk per workgroup in dispatch order.  The
//    segment rewrite's cost is set by how HBM sees the reads and writes, and
//    it is lowest when the workgroups in flight cover one narrow, advancing
//    band of the snapshot -- which the hardware dispatcher gives for free
//    when every workgroup takes the next small chunk and exits.  Measured on
//    the 7B-shaped delta's 66.4 million touched segments (read and rewrite
//    of a precomputed list, nontemporal): one pass per 1024-lane workgroup,
//    4 lanes per segment, 2.38 ms; the same in 256- or 512-lane workgroups
//    2.47-2.58 ms; workgroups that each walk a chunk of a few hundred
//    segments in several passes, or a persistent grid striding over chunks,
//    2.71-2.78 ms; 8 segments in flight per lane 3.2 ms; cached instead of
//    nontemporal accesses 3.0 ms; 32-byte units 4.0 ms, 128-byte lines 2.73.
//    In each touched segment four lanes read 16 bytes each, patch them from
//    the entries (staged in LDS) and write them back; a chunk's segments
//    (about 860 at 1.2 % density) take a few passes, three in flight per lane.
//  * Snapshot pointers come from the parameter table in memory; they are
//    cast to the global address space so the stores are global, not flat.
//  * The parameter of the chunk's first entry comes from one 64-way search
//    over the device offsets; the offsets are read on the GPU, so no host
//    round trip separates diff and apply.
//  * An index outside [0, numel) is skipped, never written.  With unsorted
//    or repeated indices the values at those entries' positions are
//    unspecified; every other position keeps its value (a rewritten segment
//    is written back with the values read from it, and lies inside the
//    snapshot).
#include <atomic>

#include "sbd_internal.h"

namespace sbd {
namespace {

// apply_kernel's workgroup width, 8 entries per lane: 256 lanes (2048-entry
// chunks), or 512 (4096-entry chunks) for the large deltas that
// launch_apply_kernel picks.
constexpr int kApplyNarrow = 256;
constexpr int kApplyWide = 512;
constexpr int kApplyPer = 8;
// Elements of span per entry that choose between the ways of writing a
// well-formed chunk's interior segments (see above).  Segments against
// windows on the 7B-shaped list, ms: at 4.7 % density 5.42 / 5.80, at 5.9 %
// 5.85 / 5.85, at 3.5 % 4.44 / 4.71, on the Qwen3-0.6B list at 8 % windows
// either way.
constexpr int64_t kMergeSpread = 20;
constexpr int64_t kMergeMinSpread = 3;
constexpr int kSegElems = 32;                // bf16 per 64-byte segment
constexpr int kSegLanes = kSegElems / kVec;  // 4 lanes x 16 bytes per segment
constexpr int kSegUnroll = 4;                        // segments in flight per lane
// Fewest delta entries for which sparse chunks rewrite whole segments.
constexpr int64_t kSegMinTotal = int64_t(1) << 25;
// Fewest elements per delta entry for the large-delta kernel (about 2.8 %
// density or less; see launch_apply_kernels).
constexpr int64_t kBigSpread = 36;
constexpr int kMergeWindow = 8192;  // snapshot elements patched in LDS at a time
static_assert(kMergeWindow % kSegElems == 0, "windows hold whole segments");

// Large deltas: one entry per lane of a 1024-lane workgroup.
constexpr int kBigBlock = 1024;
constexpr int kBigWaves = kBigBlock / 64;
constexpr int kBigChunk = kBigBlock;
constexpr int kBigSegPass = kBigBlock / kSegLanes;  // segments rewritten per pass
// Segments in flight per four lanes: the loads of three passes are issued
// before the first pass is patched and written.  On the 7B-shaped delta, one
// pass at a time 2.69 ms, two 2.60 ms, four 2.78 ms (the floor of the bare
// read and rewrite of its touched segments, one pass per workgroup, 2.48 ms
// on that machine); on another, two 2.61, three 2.54, four 2.78 ms, and at
// 2.4 % density 3.72 / 3.62 / 5.10 ms (at 3.5 %, two and three alike).
constexpr int kBigSegDepth = 3;
// At most this many workgroups per launch; each strides over chunks beyond
// it (2^17 chunks of 1024 entries: a delta of 134 million entries takes one
// pass).  A launch whose max_nnz (a buffer's capacity) far exceeds the true
// total therefore starts at most this many workgroups that find no work.
constexpr int64_t kBigGridCap = int64_t(1) << 17;

enum ApplyMode : int { kScatter = 0, kWindows = 1, kSegments = 2 };

// The touched-segment list of a sparse workgroup (8 bytes per entry of its
// chunk: 16 KB, the window's size, for 256 lanes).
template <int kChunk>
struct SegList {
  uint32_t pos[kChunk];    // per entry: its index plus the segment shift
  uint16_t val[kChunk];    // per entry: its value
  uint16_t first[kChunk];  // the first entry of each listed segment
};

template <int kB>
struct ApplyShared {
  static constexpr int kApplyWaves = kB / 64;
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
    __attribute__((aligned(16))) SegList<kB * kApplyPer> sl;
  };
};

// The touched-segment list of a sparse chunk of the large-delta kernel.
struct BigSegList {
  uint32_t pos[kBigChunk];    // per entry: its index plus the segment shift
  uint16_t val[kBigChunk];    // per entry: its value
  uint16_t first[kBigChunk];  // the first entry of each listed segment
};

struct BigShared {
  int64_t total;
  int32_t p0;
  int32_t one_param;
  uint32_t wmin[kBigWaves];
  uint32_t wmax[kBigWaves];
  uint32_t wcnt[kBigWaves];
  int32_t wfirst[kBigWaves];
  int32_t wlast[kBigWaves];
  uint32_t wsegs[kBigWaves];  // listed segments per wave
  uint32_t last_first;        // the first entry in the last touched segment
  union {
    __attribute__((aligned(16))) uint16_t win[kMergeWindow];
    __attribute__((aligned(16))) BigSegList sl;
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

// Wave 0 of a workgroup: the delta's applicable total, the parameter of
// entry j0 and whether the chunk [j0, j0 + chunk) stays in it, into LDS.
template <bool kMany, typename Shared>
__device__ __forceinline__ void chunk_head(int64_t j0, int chunk, int32_t nparams,
                                          const int64_t* __restrict__ offsets, int64_t max_nnz,
                                          Shared& sh) {
  if (threadIdx.x < 64) {
    int64_t total = max_nnz;
    if constexpr (kMany) {
      const int64_t t = offsets[nparams];
      total = t < max_nnz ? t : max_nnz;
      if (j0 < total) {
        const int32_t lo = find_param_wave0(offsets, nparams, j0);
        if (threadIdx.x == 0) {
          sh.p0 = lo;
          const int64_t end = j0 + chunk < total ? j0 + chunk : total;
          sh.one_param = offsets[lo + 1] >= end ? 1 : 0;
        }
      }
    } else {
      if (threadIdx.x == 0) {
        sh.p0 = 0;
        sh.one_param = 1;
      }
    }
    if (threadIdx.x == 0) sh.total = total;
  }
}

// Applies entries [j0, j0 + kApplyChunk) of the delta.  Every lane of the
// workgroup reaches the end (the violation count is a wave reduction).
// Returns true, uniformly over the workgroup, when j0 lies at or past the
// delta's total, and then does nothing.
// kSegOK: the segment rewrite is compiled in (the launch's capacity allows a
// delta of kSegMinTotal entries); without it the kernel needs fewer registers.
template <bool kMany, bool kSegOK, int kB>
__device__ __forceinline__ bool apply_chunk(
    int64_t j0, const SnapParam* __restrict__ table, const SnapParam& single, int32_t nparams,
    const int64_t* __restrict__ offsets, const int32_t* __restrict__ idx,
    const uint16_t* __restrict__ val, int64_t max_nnz, int64_t* __restrict__ violations,
    ApplyShared<kB>& sh) {
  constexpr int kApplyBlock = kB;
  constexpr int kApplyWaves = kB / 64;
  constexpr int kApplyChunk = kB * kApplyPer;
  constexpr int kSegGroups = kB / kSegLanes;  // segments per pass
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
  // from the lanes' entries, write them back whole.  The next window's loads
  // are issued into registers before this one is patched and written, so
  // they are in flight meanwhile ------------------------------------------
  if (mode == kWindows) {
    constexpr int kWinPer = kMergeWindow / kVec / kApplyBlock;  // 16-byte loads per lane
    constexpr uint32_t kWinQuads = kMergeWindow / kVec;
    static_assert(kWinPer * kApplyBlock * kVec == kMergeWindow, "a window is whole rounds");
    // lo_end and hi_start bound whole 64-byte segments, so the interior is
    // 16-byte aligned and a whole number of 16-byte quads
    const u32x4* src = reinterpret_cast<const u32x4*>(dm.snap + lo_end);
    const uint32_t nq = (hi_start - lo_end) / kVec;
    u32x4 r[kWinPer];
#pragma unroll
    for (int t = 0; t < kWinPer; ++t) {
      const uint32_t c = uint32_t(t * kApplyBlock) + threadIdx.x;
      if (c < nq) r[t] = __builtin_nontemporal_load(global_ptr(src + c));
    }
    for (uint32_t q0 = 0; q0 < nq; q0 += kWinQuads) {
#pragma unroll
      for (int t = 0; t < kWinPer; ++t) {
        const uint32_t k = uint32_t(t * kApplyBlock) + threadIdx.x;
        if (q0 + k < nq) *reinterpret_cast<u32x4*>(&sh.win[k * kVec]) = r[t];
      }
      __syncthreads();
      if (q0 + kWinQuads < nq) {
#pragma unroll
        for (int t = 0; t < kWinPer; ++t) {
          const uint32_t c = q0 + kWinQuads + uint32_t(t * kApplyBlock) + threadIdx.x;
          if (c < nq) r[t] = __builtin_nontemporal_load(global_ptr(src + c));
        }
      }
      const uint32_t w0 = lo_end + q0 * kVec;
      const uint32_t w1 = nq - q0 < kWinQuads ? hi_start : w0 + kMergeWindow;
#pragma unroll
      for (int e = 0; e < kApplyPer; ++e) {
        const uint32_t i = static_cast<uint32_t>(iv[e]);
        if (e0 + e < n_entries && i >= w0 && i < w1) sh.win[i - w0] = vv[e];
      }
      __syncthreads();
#pragma unroll
      for (int t = 0; t < kWinPer; ++t) {
        const uint32_t k = uint32_t(t * kApplyBlock) + threadIdx.x;
        if (q0 + k < nq) {
          const u32x4 x = *reinterpret_cast<const u32x4*>(&sh.win[k * kVec]);
          __builtin_nontemporal_store(x, global_ptr(const_cast<u32x4*>(src) + q0 + k));
        }
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

template <bool kMany, bool kSegOK, int kB>
__global__ __launch_bounds__(kB) void apply_kernel(
    const SnapParam* __restrict__ table, SnapParam single, int32_t nparams,
    const int64_t* __restrict__ offsets, const int32_t* __restrict__ idx,
    const uint16_t* __restrict__ val, int64_t max_nnz, int64_t* __restrict__ violations) {
  constexpr int kApplyChunk = kB * kApplyPer;
  __shared__ ApplyShared<kB> sh;
  const int64_t nchunks = (max_nnz + kApplyChunk - 1) / kApplyChunk;
  for (int64_t chunk = blockIdx.x; chunk < nchunks; chunk += gridDim.x) {
    const bool past = apply_chunk<kMany, kSegOK, kB>(chunk * kApplyChunk, table, single, nparams,
                                                     offsets, idx, val, max_nnz, violations, sh);
    __syncthreads();  // the shared state is rewritten by the next chunk
    if (past) break;  // this workgroup's later chunks lie past the total too
  }
}

// Applies entries [j0, j0 + kBigChunk) of a delta of at least kSegMinTotal
// entries, one per lane; the same contract as apply_chunk.
template <bool kMany>
__device__ __forceinline__ bool apply_big_chunk(
    int64_t j0, const SnapParam* __restrict__ table, const SnapParam& single, int32_t nparams,
    const int64_t* __restrict__ offsets, const int32_t* __restrict__ idx,
    const uint16_t* __restrict__ val, int64_t max_nnz, int64_t* __restrict__ violations,
    BigShared& sh) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t j = j0 + tid;
  int32_t iv = 0;
  uint16_t vv = 0;
  if (j < max_nnz) {
    iv = idx[j];
    vv = val[j];
  }
  chunk_head<kMany>(j0, kBigChunk, nparams, offsets, max_nnz, sh);
  __syncthreads();
  const int64_t total = sh.total;
  if (j0 >= total) return true;
  const int n_entries = total - j0 < kBigChunk ? int(total - j0) : kBigChunk;
  const bool have = tid < n_entries;
  int mode = kScatter;
  uint32_t shift = 0, ufirst = 0, ulast = 0, lo_end = 0, hi_start = 0;
  SnapParam dm = single;
  if (sh.one_param) {
    if constexpr (kMany) dm = table[sh.p0];
    shift = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(dm.snap) & 63u) >> 1;
    if ((reinterpret_cast<uintptr_t>(dm.snap) & 1u) == 0) {
      const uint32_t i = static_cast<uint32_t>(iv);
      const bool in = have && static_cast<uint64_t>(i) < static_cast<uint64_t>(dm.numel);
      uint32_t umin = in ? i : 0xFFFFFFFFu, umax = in ? i : 0u, cnt = in ? 1u : 0u;
      const int32_t prev = __shfl_up(iv, 1, 64);
      const bool sorted = !(have && lane > 0 && !(iv > prev));
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
        sh.wfirst[wave] = iv;
      }
      const bool next_have = __shfl_down(have ? 1 : 0, 1, 64) != 0;
      if (have && (lane == 63 || !next_have)) sh.wlast[wave] = iv;
      __syncthreads();
      uint32_t gmin = 0xFFFFFFFFu, gmax = 0u, gcnt = 0u;
      bool ok = true;
      if (lane < kBigWaves) {
        gmin = sh.wmin[lane];
        gmax = sh.wmax[lane];
        gcnt = sh.wcnt[lane];
        ok = gcnt != 0xFFFFFFFFu &&
             (lane == 0 || lane * 64 >= n_entries || sh.wfirst[lane] > sh.wlast[lane - 1]);
        if (!ok) gcnt = 0u;
      }
#pragma unroll
      for (int o = kBigWaves / 2; o > 0; o >>= 1) {
        const uint32_t a = static_cast<uint32_t>(__shfl_xor(static_cast<int>(gmin), o, 64));
        const uint32_t b = static_cast<uint32_t>(__shfl_xor(static_cast<int>(gmax), o, 64));
        gmin = a < gmin ? a : gmin;
        gmax = b > gmax ? b : gmax;
        gcnt += static_cast<uint32_t>(__shfl_xor(static_cast<int>(gcnt), o, 64));
      }
      gmin = static_cast<uint32_t>(__shfl(static_cast<int>(gmin), 0, 64));
      gmax = static_cast<uint32_t>(__shfl(static_cast<int>(gmax), 0, 64));
      gcnt = static_cast<uint32_t>(__shfl(static_cast<int>(gcnt), 0, 64));
      const bool well_formed =
          __ballot(!ok) == 0ull && gcnt == static_cast<uint32_t>(n_entries);
      if (well_formed && gcnt > 0u) {
        ufirst = (gmin + shift) / kSegElems;
        ulast = (gmax + shift) / kSegElems;
        const int64_t span = int64_t(gmax - gmin) + 1;
        if (ulast >= ufirst + 2u) {
          if (span > kMergeSpread * int64_t(gcnt))
            mode = total >= kSegMinTotal ? kSegments : kScatter;
          else if (span >= kMergeMinSpread * int64_t(gcnt))
            mode = kWindows;
        }
        lo_end = (ufirst + 1u) * kSegElems - shift;
        hi_start = ulast * kSegElems - shift;
      }
    }
  }
  int64_t bad = 0;
  if (have) {
    int32_t p = 0;
    SnapParam d = single;
    int64_t seg_start = 0;
    if constexpr (kMany) {
      p = sh.p0;
      if (!sh.one_param) {
        int64_t seg_end = offsets[p + 1];
        while (seg_end <= j) seg_end = offsets[++p + 1];
      }
      seg_start = offsets[p];
      d = table[p];
    }
    const uint32_t i = static_cast<uint32_t>(iv);
    const bool in_range = static_cast<uint64_t>(i) < static_cast<uint64_t>(d.numel);
    const bool interior = mode != kScatter && i >= lo_end && i < hi_start;
    if (in_range && !interior) *global_ptr(d.snap + i) = vv;
    if (violations != nullptr) {
      int32_t prev = __shfl_up(iv, 1, 64);
      if (lane == 0 && j > seg_start) prev = idx[j - 1];
      bad = (!in_range || (j > seg_start && iv <= prev)) ? 1 : 0;
    }
  }
  if (mode == kSegments) {
    const uintptr_t seg0 = reinterpret_cast<uintptr_t>(dm.snap) - 2u * shift;
    int32_t before = __shfl_up(iv, 1, 64);
    if (lane == 0) before = wave > 0 ? sh.wlast[wave - 1] : 0;
    const uint32_t u = (static_cast<uint32_t>(iv) + shift) / kSegElems;
    const uint32_t pu = (static_cast<uint32_t>(before) + shift) / kSegElems;
    const bool lead = have && (tid == 0 || u != pu);
    const bool listed = lead && u > ufirst && u < ulast;
    if (lead && u == ulast) sh.last_first = uint32_t(tid);
    sh.sl.pos[tid] = static_cast<uint32_t>(iv) + shift;
    sh.sl.val[tid] = vv;
    const uint64_t lb = __ballot(listed);
    if (lane == 0) sh.wsegs[wave] = static_cast<uint32_t>(__popcll(lb));
    __syncthreads();
    uint32_t before_w = 0u, ns = lane < kBigWaves ? sh.wsegs[lane] : 0u;
    before_w = lane < wave ? ns : 0u;
#pragma unroll
    for (int o = kBigWaves / 2; o > 0; o >>= 1) {
      before_w += static_cast<uint32_t>(__shfl_xor(static_cast<int>(before_w), o, 64));
      ns += static_cast<uint32_t>(__shfl_xor(static_cast<int>(ns), o, 64));
    }
    before_w = static_cast<uint32_t>(__shfl(static_cast<int>(before_w), 0, 64));
    ns = static_cast<uint32_t>(__shfl(static_cast<int>(ns), 0, 64));
    const uint32_t slot = before_w + static_cast<uint32_t>(__popcll(lb & ((1ull << lane) - 1ull)));
    if (listed) sh.sl.first[slot] = static_cast<uint16_t>(tid);
    __syncthreads();
    const uint32_t g = static_cast<uint32_t>(tid) / kSegLanes;
    const uint32_t sub = static_cast<uint32_t>(tid) % kSegLanes;
    const uint32_t last_first = sh.last_first;
    for (uint32_t s0 = g; s0 < ns; s0 += kBigSegDepth * kBigSegPass) {
      u32x4 x[kBigSegDepth];
      uintptr_t aa[kBigSegDepth];
#pragma unroll
      for (int k = 0; k < kBigSegDepth; ++k) {
        const uint32_t s = s0 + k * kBigSegPass;
        if (s < ns) {
          const uint32_t eb = sh.sl.first[s];
          aa[k] = seg0 + uintptr_t(sh.sl.pos[eb] / kSegElems) * 64u + sub * 16u;
          x[k] = __builtin_nontemporal_load(global_ptr(reinterpret_cast<const u32x4*>(aa[k])));
        }
      }
#pragma unroll
      for (int k = 0; k < kBigSegDepth; ++k) {
        const uint32_t s = s0 + k * kBigSegPass;
        if (s < ns) {
          const uint32_t eb = sh.sl.first[s];
          const uint32_t ee = s + 1u < ns ? uint32_t(sh.sl.first[s + 1u]) : last_first;
          for (uint32_t e = eb; e < ee; ++e) {
            const uint32_t off = sh.sl.pos[e] % kSegElems;
            if (off / kVec == sub) set_elem(x[k], off % kVec, sh.sl.val[e]);
          }
          __builtin_nontemporal_store(x[k], global_ptr(reinterpret_cast<u32x4*>(aa[k])));
        }
      }
    }
  }
  if (mode == kWindows) {
    const uint32_t i = static_cast<uint32_t>(iv);
    for (uint32_t w0 = lo_end; w0 < hi_start; w0 += kMergeWindow) {
      const uint32_t w1 = hi_start - w0 < uint32_t(kMergeWindow) ? hi_start : w0 + kMergeWindow;
      for (uint32_t c = threadIdx.x; c < (w1 - w0) / kVec; c += kBigBlock) {
        const u32x4 x =
            __builtin_nontemporal_load(global_ptr(reinterpret_cast<const u32x4*>(dm.snap + w0) + c));
        *reinterpret_cast<u32x4*>(&sh.win[c * kVec]) = x;
      }
      __syncthreads();
      if (have && i >= w0 && i < w1) sh.win[i - w0] = vv;
      __syncthreads();
      for (uint32_t c = threadIdx.x; c < (w1 - w0) / kVec; c += kBigBlock) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(&sh.win[c * kVec]);
        __builtin_nontemporal_store(x, global_ptr(reinterpret_cast<u32x4*>(dm.snap + w0) + c));
      }
      __syncthreads();
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

template <bool kMany>
__global__ __launch_bounds__(kBigBlock) void apply_big_kernel(
    const SnapParam* __restrict__ table, SnapParam single, int32_t nparams,
    const int64_t* __restrict__ offsets, const int32_t* __restrict__ idx,
    const uint16_t* __restrict__ val, int64_t max_nnz, int64_t* __restrict__ violations) {
  __shared__ BigShared sh;
  const int64_t nchunks = (max_nnz + kBigChunk - 1) / kBigChunk;
  for (int64_t chunk = blockIdx.x; chunk < nchunks; chunk += gridDim.x) {
    const bool past = apply_big_chunk<kMany>(chunk * kBigChunk, table, single, nparams, offsets,
                                             idx, val, max_nnz, violations, sh);
    __syncthreads();  // the shared state is rewritten by the next chunk
    if (past) break;
  }
}

// The grid of apply_kernel is bounded by kApplyGridFactor times the
// workgroups the GPU holds at once, queried once per device; each workgroup
// then strides over chunks.  A caller that passes its buffer's capacity as
// max_nnz (diff and apply in one stream, no host read of the count) would
// otherwise launch one workgroup per chunk of that capacity, most of which
// find no entries and exit: on the 7B-shaped list at 1.2 % with a capacity of
// an eighth of the elements, about 370,000 such workgroups took 0.1 ms.
// Measured against one workgroup per chunk: equal or faster on every list and
// density tried (up to 7 % at 8-12 % density); a factor of 1 or 2 was 10-25 %
// slower (too little dynamic balancing between chunks of different cost).
constexpr int64_t kApplyGridFactor = 16;

template <bool kMany, bool kSegOK, int kB>
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
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, apply_kernel<kMany, kSegOK, kB>,
                                                     kB, 0) != hipSuccess ||
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

template <bool kMany, bool kSegOK, int kB>
void launch_apply_kernel(const SnapParam* d_table, const SnapParam& single, int32_t nparams,
                         const int64_t* offsets, const int32_t* idx, const uint16_t* val,
                         int64_t max_nnz, int64_t* violations, hipStream_t stream) {
  constexpr int64_t kApplyChunk = int64_t(kB) * kApplyPer;
  int64_t blocks = (max_nnz + kApplyChunk - 1) / kApplyChunk;
  const int64_t lim = apply_grid_limit<kMany, kSegOK, kB>();
  if (blocks > lim) blocks = lim;
  apply_kernel<kMany, kSegOK, kB><<<dim3(unsigned(blocks)), dim3(kB), 0, stream>>>(
      d_table, single, nparams, offsets, idx, val, max_nnz, violations);
}

// Entries per parameter (max_nnz over nparams) from which a delta of at
// least kSegMinTotal entries runs in 512-lane workgroups.  A chunk that
// straddles parameters writes every entry with 2-byte stores, so longer
// chunks pay off only where parameters hold many chunks each.  Measured (ms,
// 256 / 512 lanes): one 405B-shaped layer at 8 % 2.84 / 2.72; 7B-shaped list
// fp32-master 8 % 6.04 / 5.84, bf16 3.5 % 4.45 / 4.35, 11.6 % 5.34 / 5.29,
// its first 48 million entries alone 0.727 / 0.723; the Qwen3-0.6B-shaped
// list at 8 % (155,000 entries per parameter) 0.465 / 0.490.
constexpr int64_t kWidePerParam = int64_t(1) << 20;

// Which kernel: apply_big_kernel when the delta is large enough for the
// segment rewrite and sparse enough (max_nnz entries over total_elems
// elements leave at least kBigSpread elements per entry); else apply_kernel,
// which also rewrites the segments of sparse chunks when max_nnz allows
// kSegMinTotal entries (a capacity far above the true count, or a denser
// delta).  Where both rewrite segments, one chunk per 1024-lane workgroup
// wins while the touched segments are few and far apart, and apply_kernel's
// 256-lane passes win once most segments are touched; on the 7B-shaped list
// (ms, large-delta / general): 1.2 % 2.53 / 2.89, 1.8 % 3.26 / 3.72, 2.4 %
// 3.60 / 3.78, 2.9 % 4.22 / 4.16, 3.5 % 4.86 / 4.44.  The windows of mid-density chunks run better in 256-lane
// workgroups issuing several loads per lane: a dense in-place read and
// rewrite measured 6.1 TB/s in that shape against 4.0 TB/s in 1024-lane
// workgroups with one load per lane (the Qwen3-0.6B-shaped list at 8 %:
// 0.51 ms against 0.77 ms).
template <bool kMany>
void launch_apply_kernels(const SnapParam* d_table, const SnapParam& single, int32_t nparams,
                          const int64_t* offsets, const int32_t* idx, const uint16_t* val,
                          int64_t max_nnz, int64_t total_elems, int64_t* violations,
                          hipStream_t stream) {
  if (max_nnz >= kSegMinTotal && max_nnz <= total_elems / kBigSpread) {
    int64_t blocks = (max_nnz + kBigChunk - 1) / kBigChunk;
    if (blocks > kBigGridCap) blocks = kBigGridCap;
    apply_big_kernel<kMany><<<dim3(unsigned(blocks)), dim3(kBigBlock), 0, stream>>>(
        d_table, single, nparams, offsets, idx, val, max_nnz, violations);
  } else if (max_nnz >= kSegMinTotal && max_nnz / nparams >= kWidePerParam) {
    launch_apply_kernel<kMany, true, kApplyWide>(d_table, single, nparams, offsets, idx, val,
                                                 max_nnz, violations, stream);
  } else if (max_nnz >= kSegMinTotal) {
    launch_apply_kernel<kMany, true, kApplyNarrow>(d_table, single, nparams, offsets, idx, val,
                                                   max_nnz, violations, stream);
  } else {
    launch_apply_kernel<kMany, false, kApplyNarrow>(d_table, single, nparams, offsets, idx, val,
                                                    max_nnz, violations, stream);
  }
}

}  // namespace

hipError_t launch_apply(const SnapParam* d_table, const SnapParam& single, int32_t nparams,
                        const int64_t* offsets, const int32_t* idx, const uint16_t* val,
                        int64_t max_nnz, int64_t total_elems, int64_t* violations,
                        hipStream_t stream) {
  clear_stale_error();
  if (violations != nullptr) zero_i64_kernel<<<dim3(1), dim3(64), 0, stream>>>(violations);
  if (max_nnz > 0) {
    if (d_table != nullptr)
      launch_apply_kernels<true>(d_table, single, nparams, offsets, idx, val, max_nnz,
                                 total_elems, violations, stream);
    else
      launch_apply_kernels<false>(nullptr, single, 1, nullptr, idx, val, max_nnz, total_elems,
                                  violations, stream);
  }
  return hipGetLastError();
}

}  // namespace sbd
