// ceiling.hip -- reference kernels that measure what the memory system
// sustains, for the benchmark's ceilings (not part of the delta library and
// not linked into it).  Each does the plainest thing at one pass per
// workgroup in dispatch order, with 16-byte nontemporal accesses:
//   sbd_ceiling_copy        dst = src (one read stream, one write stream)
//   sbd_ceiling_read2       read two arrays (the diff's input pattern)
//   sbd_ceiling_rewrite     a[i] = a[i] in place (read and write the same lines)
//   sbd_ceiling_segments    read and rewrite a listed set of 64-byte segments
//                           of one buffer, four lanes per segment: the memory
//                           work of a sparse apply without finding the
//                           segments or patching them
// Launch shapes were swept on 13.5 GB operands (256-1024 lanes, 1-4 accesses
// per lane, grid-stride against one pass); these are the fastest found.
// The rewriting kernels XOR a run-time word (always 0) into all four words
// they write back: a store of the value just loaded from the same address is
// otherwise removed by the compiler, load and all, and a store with only some
// words changed is narrowed to those words.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 ld(const u32x4* p) {
  return __builtin_nontemporal_load((const __attribute__((address_space(1))) u32x4*)p);
}
__device__ __forceinline__ void st(u32x4* p, u32x4 v) {
  __builtin_nontemporal_store(v, (__attribute__((address_space(1))) u32x4*)p);
}

constexpr int kCopyBlock = 1024;  // one 16-byte access per lane
constexpr int kRewriteBlock = 256, kRewritePer = 4;
constexpr int kReadBlock = 512, kReadPer = 2;
constexpr int kSegBlock = 1024;   // 256 segments per workgroup

__global__ __launch_bounds__(kCopyBlock) void copy_kernel(const u32x4* __restrict__ src,
                                                          u32x4* __restrict__ dst, int64_t n16) {
  const int64_t i = int64_t(blockIdx.x) * kCopyBlock + threadIdx.x;
  if (i < n16) st(dst + i, ld(src + i));
}

__global__ __launch_bounds__(kReadBlock) void read2_kernel(const u32x4* __restrict__ a,
                                                           const u32x4* __restrict__ b,
                                                           int64_t n16, uint32_t* __restrict__ sink) {
  const int64_t i0 = int64_t(blockIdx.x) * kReadBlock * kReadPer + threadIdx.x;
  u32x4 x[kReadPer], y[kReadPer];
#pragma unroll
  for (int p = 0; p < kReadPer; ++p) {
    const int64_t i = i0 + int64_t(p) * kReadBlock;
    if (i < n16) {
      x[p] = ld(a + i);
      y[p] = ld(b + i);
    }
  }
  uint32_t acc = 0;
#pragma unroll
  for (int p = 0; p < kReadPer; ++p)
    if (i0 + int64_t(p) * kReadBlock < n16)
      acc ^= x[p].x ^ x[p].y ^ x[p].z ^ x[p].w ^ y[p].x ^ y[p].y ^ y[p].z ^ y[p].w;
  // keeps the loads; written only if the XOR of the lane's words is this value
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

__global__ __launch_bounds__(kRewriteBlock) void rewrite_kernel(u32x4* __restrict__ a, int64_t n16,
                                                                 uint32_t zero) {
  const int64_t i0 = int64_t(blockIdx.x) * kRewriteBlock * kRewritePer + threadIdx.x;
  u32x4 x[kRewritePer];
#pragma unroll
  for (int p = 0; p < kRewritePer; ++p) {
    const int64_t i = i0 + int64_t(p) * kRewriteBlock;
    if (i < n16) x[p] = ld(a + i);
  }
#pragma unroll
  for (int p = 0; p < kRewritePer; ++p) {
    const int64_t i = i0 + int64_t(p) * kRewriteBlock;
    if (i < n16) {
      x[p] ^= zero;
      st(a + i, x[p]);
    }
  }
}

__global__ __launch_bounds__(kSegBlock) void segments_kernel(u32x4* __restrict__ base,
                                                             const int64_t* __restrict__ segs,
                                                             int64_t nsegs, uint32_t zero) {
  const int64_t s = int64_t(blockIdx.x) * (kSegBlock / 4) + threadIdx.x / 4;
  if (s < nsegs) {
    u32x4* p = base + segs[s] * 4 + threadIdx.x % 4;
    u32x4 x = ld(p);
    x ^= zero;
    st(p, x);
  }
}

unsigned grid_for(int64_t work, int64_t per_block) {
  return static_cast<unsigned>((work + per_block - 1) / per_block);
}

}  // namespace

extern "C" {

// Each returns 0, or a HIP error code; sizes in bytes must be multiples of 16
// and pointers 16-byte aligned (checked: -1 otherwise).
int sbd_ceiling_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (bytes < 0 || bytes % 16 || (reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16)
    return -1;
  if (bytes == 0) return 0;
  copy_kernel<<<grid_for(bytes / 16, kCopyBlock), kCopyBlock, 0, (hipStream_t)stream>>>(
      (const u32x4*)src, (u32x4*)dst, bytes / 16);
  return (int)hipGetLastError();
}

int sbd_ceiling_read2(const void* a, const void* b, int64_t bytes, void* sink4, void* stream) {
  if (bytes < 0 || bytes % 16 || (reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b)) % 16 ||
      sink4 == nullptr)
    return -1;
  if (bytes == 0) return 0;
  read2_kernel<<<grid_for(bytes / 16, kReadBlock * kReadPer), kReadBlock, 0, (hipStream_t)stream>>>(
      (const u32x4*)a, (const u32x4*)b, bytes / 16, (uint32_t*)sink4);
  return (int)hipGetLastError();
}

int sbd_ceiling_rewrite(void* a, int64_t bytes, void* stream) {
  if (bytes < 0 || bytes % 16 || reinterpret_cast<uintptr_t>(a) % 16) return -1;
  if (bytes == 0) return 0;
  rewrite_kernel<<<grid_for(bytes / 16, kRewriteBlock * kRewritePer), kRewriteBlock, 0,
                   (hipStream_t)stream>>>((u32x4*)a, bytes / 16, 0u);
  return (int)hipGetLastError();
}

// segs: nsegs ascending 64-byte segment numbers relative to base (64-byte
// aligned), each below bytes / 64 -- the caller guarantees the bound.
int sbd_ceiling_segments(void* base, int64_t bytes, const int64_t* segs, int64_t nsegs,
                         void* stream) {
  if (bytes < 0 || nsegs < 0 || reinterpret_cast<uintptr_t>(base) % 64 || (nsegs > 0 && !segs))
    return -1;
  if (nsegs == 0) return 0;
  segments_kernel<<<grid_for(nsegs, kSegBlock / 4), kSegBlock, 0, (hipStream_t)stream>>>(
      (u32x4*)base, segs, nsegs, 0u);
  return (int)hipGetLastError();
}

}  // extern "C"
