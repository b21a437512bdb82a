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
//  * Indices within a parameter ascend, so the lanes of a wave write
//    ascending addresses: stores to the same 128-byte snapshot line come
//    from neighbouring lanes and merge in L2 before the line goes to HBM.
//    HBM then sees masked partial writes of the touched 32-byte sectors and
//    no reads of the snapshot.  (Reading and rewriting whole 64-byte
//    segments instead moves three times the bytes and measured no faster at
//    1 % density, and far slower on dense deltas.)
//  * Snapshot pointers come from the parameter table in memory; they are
//    cast to the global address space so the stores are global, not flat.
//  * The parameter of the workgroup's first entry comes from one binary
//    search over the device offsets; each lane then walks forward.  The
//    offsets are read on the GPU, so no host round trip separates diff and
//    apply.
//  * An index outside [0, numel) is skipped, never written.
#include "sbd_internal.h"

namespace sbd {
namespace {

constexpr int kApplyBlock = 256;
constexpr int kApplyPer = 8;
constexpr int64_t kApplyChunk = int64_t(kApplyBlock) * kApplyPer;

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
    int32_t& s_p0, int64_t& s_total) {
  if (threadIdx.x < 64) {
    int64_t total = max_nnz;
    if constexpr (kMany) {
      const int64_t t = offsets[nparams];
      total = t < max_nnz ? t : max_nnz;
      if (j0 < total) {
        // Largest p with offsets[p] <= j0 -- the non-empty parameter holding
        // j0 -- by a 64-way search in wave 0: each step probes 64 evenly
        // spaced offsets at once (two steps for up to 4096 parameters).
        const int lane = threadIdx.x;
        int32_t lo = 0, hi = nparams;  // offsets[lo] <= j0 holds throughout
        while (hi - lo > 1) {
          const int32_t step = (hi - lo + 63) / 64;
          const int32_t probe = lo + lane * step;
          const uint64_t ok = __ballot(probe < hi && offsets[probe] <= j0);
          lo += (63 - __builtin_clzll(ok)) * step;
          hi = lo + step < hi ? lo + step : hi;
        }
        if (lane == 0) s_p0 = lo;
      }
    }
    if (threadIdx.x == 0) s_total = total;
  }
  __syncthreads();
  const int64_t total = s_total;
  if (j0 >= total) return;  // uniform over the workgroup

  const int64_t jt = j0 + int64_t(threadIdx.x) * kApplyPer;
  int64_t bad = 0;
  if (jt < total) {
    int32_t iv[kApplyPer];
    uint16_t vv[kApplyPer];
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

    int32_t p = 0;
    SnapParam d = single;
    int64_t seg_start = 0, seg_end = total;
    if constexpr (kMany) {
      p = s_p0;
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
        if (in_range) *global_ptr(d.snap + i) = vv[r];
        if (violations != nullptr) {
          bad += (!in_range || (have_prev && iv[r] <= prev)) ? 1 : 0;
          prev = iv[r];
          have_prev = true;
        }
      }
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
  __shared__ int32_t s_p0;
  __shared__ int64_t s_total;
  const int64_t nchunks = (max_nnz + kApplyChunk - 1) / kApplyChunk;
  for (int64_t chunk = blockIdx.x; chunk < nchunks; chunk += gridDim.x) {
    apply_chunk<kMany>(chunk * kApplyChunk, table, single, nparams, offsets, idx, val, max_nnz,
                       violations, s_p0, s_total);
    __syncthreads();  // s_p0 / s_total are rewritten by the next chunk
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
