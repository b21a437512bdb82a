// apply.hip -- scatter a sparse delta into resident bf16 snapshots, in place.
//
// What is computed (TRL delta-sync article, section 4.3: the receiver assigns
// the delta's values at its indices of the flattened bf16 snapshot; the vLLM
// sparse-transfer work it mentions does the same in place with index_copy_):
// snapshot[idx[j]] = val[j] for every entry j.  In the batched form, entry j
// belongs to the parameter p with offsets[p] <= j < offsets[p+1].
//
// How, on gfx950:
//  * Each workgroup owns 2048 consecutive entries; a lane loads 8 of them as
//    two 16-byte idx loads and one 16-byte val load, so the delta is read
//    once, coalesced.
//  * Sparse entries (the usual case, about 1 % of a tensor) are scattered
//    with 2-byte stores.  Indices within a parameter ascend, so stores to
//    the same 128-byte line come close together and merge in L2; HBM then
//    sees masked partial writes of the touched sectors and no reads of the
//    snapshot.  (Reading and rewriting whole 64-byte segments instead moved
//    three times the bytes and measured no faster at 1 % density.)
//  * Dense entries: when a workgroup's entries lie in one parameter and span
//    at most kMergeSpread elements per entry (about 4 % density or more,
//    where nearly every line is touched and masked writes dominate), the
//    workgroup instead reads the lines strictly inside that span into LDS,
//    8192 elements at a time, patches them from its entries (held in
//    registers) and writes them back whole.  The two edge lines, which a
//    neighbouring workgroup may share, are still written entry by entry.
//  * Snapshot pointers come from the parameter table in memory; they are
//    cast to the global address space so the stores are global, not flat.
//  * The parameter of the workgroup's first entry comes from one 64-way
//    search over the device offsets; each lane then walks forward.  The
//    offsets are read on the GPU, so no host round trip separates diff and
//    apply.
//  * An index outside [0, numel) is skipped, never written.  With unsorted
//    or repeated indices the values at those entries' positions are
//    unspecified; every other position keeps its value.
#include "sbd_internal.h"

namespace sbd {
namespace {

constexpr int kApplyBlock = 256;
constexpr int kApplyWaves = kApplyBlock / 64;
constexpr int kApplyPer = 8;
constexpr int64_t kApplyChunk = int64_t(kApplyBlock) * kApplyPer;
// A workgroup merges whole lines when its in-range entries span between
// kMergeMinSpread and kMergeSpread elements per entry (about 4 % to 33 %
// density): then most lines are touched but few are covered whole.  Denser
// entries cover whole lines, which the scatter's stores already merge into
// full writes in L2 without reading the snapshot.
constexpr int64_t kMergeSpread = 24;
constexpr int64_t kMergeMinSpread = 3;
constexpr int kLineElems = 64;       // bf16 per 128-byte line
constexpr int kMergeWindow = 8192;   // snapshot elements patched in LDS at a time
static_assert(kMergeWindow % kLineElems == 0, "windows hold whole lines");

struct ApplyShared {
  int64_t total;
  int32_t p0;
  int32_t one_param;  // every entry of the chunk belongs to parameter p0
  uint32_t wmin[kApplyWaves];
  uint32_t wmax[kApplyWaves];
  uint32_t wcnt[kApplyWaves];
  int32_t wfirst[kApplyWaves];  // first and last entry of each wave, for the order check
  int32_t wlast[kApplyWaves];
  __attribute__((aligned(16))) uint16_t win[kMergeWindow];  // snapshot window being patched
};

__global__ __launch_bounds__(64) void zero_i64_kernel(int64_t* p) {
  if (threadIdx.x == 0) *p = 0;
}

// Applies entries [j0, j0 + kApplyChunk) of the delta.  Every lane of the
// workgroup reaches the end (the violation count is a wave reduction).
template <bool kMany>
__device__ __forceinline__ void apply_chunk(
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
  if (j0 >= total) return;  // uniform over the workgroup
  const int64_t n_entries = total - j0 < kApplyChunk ? total - j0 : kApplyChunk;

  const int64_t jt = j0 + int64_t(threadIdx.x) * kApplyPer;
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

  // ---- merge or scatter (uniform over the workgroup) ------------------------
  // Merge when the chunk lies in one 16-byte-aligned snapshot, all its
  // entries are in range and strictly ascending, and they are dense; then the
  // lines strictly between the first and the last touched line,
  // [lo_end, hi_start), are rewritten whole.  A chunk that breaks the
  // precondition always takes the entry-by-entry path.
  bool merge = false;
  uint32_t lo_end = 0, hi_start = 0;
  SnapParam dm = single;
  if (sh.one_param) {
    if constexpr (kMany) dm = table[sh.p0];
    if ((reinterpret_cast<uintptr_t>(dm.snap) & 15u) == 0) {
      uint32_t umin = 0xFFFFFFFFu, umax = 0u, cnt = 0u;
      bool sorted = true, any = false;
      int32_t first = 0, last = 0;
#pragma unroll
      for (int r = 0; r < kApplyPer; ++r) {
        const int64_t e = int64_t(threadIdx.x) * kApplyPer + r;
        if (e < n_entries) {
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
      const int lane = threadIdx.x & 63;
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
      const int wave = threadIdx.x >> 6;
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
        const int64_t e = int64_t(w) * 64 * kApplyPer;
        if (w > 0 && e < n_entries && !(sh.wfirst[w] > sh.wlast[w - 1])) well_formed = false;
      }
      well_formed = well_formed && gcnt == static_cast<uint32_t>(n_entries);  // all in range
      if (well_formed && gcnt > 0u) {
        const uint32_t first_line = gmin / kLineElems, last_line = gmax / kLineElems;
        const int64_t span = int64_t(gmax - gmin) + 1;
        merge = last_line >= first_line + 2u && span <= kMergeSpread * int64_t(gcnt) &&
                span >= kMergeMinSpread * int64_t(gcnt);
        lo_end = (first_line + 1u) * kLineElems;
        hi_start = last_line * kLineElems;
      }
    }
  }

  // ---- entry by entry: every entry, or only the edge lines' when merging ---
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
        const bool merged = merge && i >= lo_end && i < hi_start;
        if (in_range && !merged) *global_ptr(d.snap + i) = vv[r];
        if (violations != nullptr) {
          bad += (!in_range || (have_prev && iv[r] <= prev)) ? 1 : 0;
          prev = iv[r];
          have_prev = true;
        }
      }
    }
  }

  // ---- line merge: window by window, read whole lines into LDS, patch them
  // from the lanes' entries, write them back whole ---------------------------
  if (merge) {
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
        if (int64_t(threadIdx.x) * kApplyPer + r < n_entries && i >= w0 && i < w1)
          sh.win[i - w0] = vv[r];
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
    if ((threadIdx.x & 63) == 0 && bad != 0)
      atomicAdd(reinterpret_cast<unsigned long long*>(violations),
                static_cast<unsigned long long>(bad));
  }
}

template <bool kMany>
__global__ __launch_bounds__(kApplyBlock) void apply_kernel(
    const SnapParam* __restrict__ table, SnapParam single, int32_t nparams,
    const int64_t* __restrict__ offsets, const int32_t* __restrict__ idx,
    const uint16_t* __restrict__ val, int64_t max_nnz, int64_t* __restrict__ violations) {
  __shared__ ApplyShared sh;
  const int64_t nchunks = (max_nnz + kApplyChunk - 1) / kApplyChunk;
  for (int64_t chunk = blockIdx.x; chunk < nchunks; chunk += gridDim.x) {
    apply_chunk<kMany>(chunk * kApplyChunk, table, single, nparams, offsets, idx, val, max_nnz,
                       violations, sh);
    __syncthreads();  // the shared state is rewritten by the next chunk
  }
}

}  // namespace

hipError_t launch_apply(const SnapParam* d_table, const SnapParam& single, int32_t nparams,
                        const int64_t* offsets, const int32_t* idx, const uint16_t* val,
                        int64_t max_nnz, int64_t* violations, hipStream_t stream) {
  if (violations != nullptr) zero_i64_kernel<<<dim3(1), dim3(64), 0, stream>>>(violations);
  if (max_nnz > 0) {
    int64_t blocks = (max_nnz + kApplyChunk - 1) / kApplyChunk;
    if (blocks > (int64_t(1) << 20)) blocks = int64_t(1) << 20;
    if (d_table != nullptr)
      apply_kernel<true><<<dim3(unsigned(blocks)), dim3(kApplyBlock), 0, stream>>>(
          d_table, single, nparams, offsets, idx, val, max_nnz, violations);
    else
      apply_kernel<false><<<dim3(unsigned(blocks)), dim3(kApplyBlock), 0, stream>>>(
          nullptr, single, 1, nullptr, idx, val, max_nnz, violations);
  }
  return hipGetLastError();
}

}  // namespace sbd
