// xor.hip -- the XOR-mask mode: mask = old ^ new and snapshot ^= mask.
//
// What is computed (humans& weight-sync summary, first paragraph): the
// trainer XORs old and new weights bit by bit into a mask the size of the
// model; the receiver XORs that mask into its old weights to obtain the new
// ones, with no floating-point arithmetic.  Applying the same mask twice
// restores the original.
//
// How, on gfx950: xor_mask is a pure stream.  Each workgroup of 1024 lanes moves one
// 16-byte vector per lane per operand (16 KB per operand per workgroup), all
// loads in flight before the stores.  Measured on 13.5 GB operands, spreading
// the 16 KB over 1024 lanes with one load each streams better (about 77 % of
// peak) than 256 lanes with four loads each (73 %) or any deeper per-lane
// queue.  A grid-stride loop bounds the grid.  Loads and stores carry the
// nontemporal hint: every byte is touched once, so keeping it in the caches
// only evicts other data (measured: about 5 % more bandwidth).  The mask may
// alias an input (and the snapshot is both input and output), so no pointer
// is declared restrict.  Unaligned operands fall back to 2-byte accesses.
// xor_apply reads the whole mask but touches only the snapshot lines where it
// is nonzero (below).
#include "sbd_internal.h"

namespace sbd {
namespace {

constexpr int kXorBlock = 1024;
constexpr int kXorIters = 1;
constexpr int64_t kXorChunkVec = int64_t(kXorBlock) * kXorIters;  // uint4 per workgroup step

__global__ __launch_bounds__(kXorBlock) void xor_vec_kernel(const uint4* a, const uint4* b,
                                                            uint4* out, int64_t nvec,
                                                            const uint16_t* a_tail,
                                                            const uint16_t* b_tail,
                                                            uint16_t* out_tail, int tail) {
  const int64_t stride = int64_t(gridDim.x) * kXorChunkVec;
  for (int64_t base = int64_t(blockIdx.x) * kXorChunkVec; base < nvec; base += stride) {
    uint4 x[kXorIters], y[kXorIters];
#pragma unroll
    for (int k = 0; k < kXorIters; ++k) {
      const int64_t v = base + int64_t(k) * kXorBlock + threadIdx.x;
      if (v < nvec) {
        const u32x4 p = __builtin_nontemporal_load(global_ptr(reinterpret_cast<const u32x4*>(a + v)));
        const u32x4 q = __builtin_nontemporal_load(global_ptr(reinterpret_cast<const u32x4*>(b + v)));
        x[k] = make_uint4(p.x, p.y, p.z, p.w);
        y[k] = make_uint4(q.x, q.y, q.z, q.w);
      }
    }
#pragma unroll
    for (int k = 0; k < kXorIters; ++k) {
      const int64_t v = base + int64_t(k) * kXorBlock + threadIdx.x;
      if (v < nvec) {
        u32x4 r;
        r.x = x[k].x ^ y[k].x;
        r.y = x[k].y ^ y[k].y;
        r.z = x[k].z ^ y[k].z;
        r.w = x[k].w ^ y[k].w;
        __builtin_nontemporal_store(r, global_ptr(reinterpret_cast<u32x4*>(out + v)));
      }
    }
  }
  // the last n % 8 elements
  if (blockIdx.x == 0 && int(threadIdx.x) < tail)
    out_tail[threadIdx.x] = uint16_t(a_tail[threadIdx.x] ^ b_tail[threadIdx.x]);
}

// snapshot ^= mask, reading and rewriting only the snapshot units (kSkipLanes
// consecutive 16-byte chunks) whose mask is nonzero: where the mask is zero
// the XOR changes nothing, so the snapshot is not touched there at all.  A
// touched unit is written whole, so HBM never sees a masked partial write.
// Measured on the 7B-shaped list at 1.2 % density (xor_apply, ms): 16-byte
// units 5.69, 32 B 5.62, 64 B 4.75, 128 B 4.57, 256 B 5.70; no skipping 6.50.
constexpr int kSkipLanes = 8;  // 128 bytes: one L2 line
static_assert(kSkipLanes >= 1 && kSkipLanes <= 64 && (kSkipLanes & (kSkipLanes - 1)) == 0,
              "a unit is a power-of-two number of lanes of one wave");

__global__ __launch_bounds__(kXorBlock) void xor_apply_vec_kernel(uint4* snap, const uint4* mask,
                                                                  int64_t nvec, uint16_t* snap_tail,
                                                                  const uint16_t* mask_tail,
                                                                  int tail) {
  static_assert(kXorIters == 1, "one chunk per lane per step");
  const int64_t stride = int64_t(gridDim.x) * kXorBlock;
  // `base` is uniform over the workgroup, so every lane reaches the shuffles
  for (int64_t base = int64_t(blockIdx.x) * kXorBlock; base < nvec; base += stride) {
    const int64_t v = base + threadIdx.x;
    u32x4 mk = {0u, 0u, 0u, 0u};
    if (v < nvec) mk = __builtin_nontemporal_load(global_ptr(reinterpret_cast<const u32x4*>(mask + v)));
    int nz = (mk.x | mk.y | mk.z | mk.w) != 0u ? 1 : 0;
#pragma unroll
    for (int o = 1; o < kSkipLanes; o <<= 1) nz |= __shfl_xor(nz, o, 64);
    if (nz && v < nvec) {
      u32x4 sv = __builtin_nontemporal_load(global_ptr(reinterpret_cast<const u32x4*>(snap + v)));
      sv ^= mk;
      __builtin_nontemporal_store(sv, global_ptr(reinterpret_cast<u32x4*>(snap + v)));
    }
  }
  // the last n % 8 elements
  if (blockIdx.x == 0 && int(threadIdx.x) < tail) {
    const uint16_t m = mask_tail[threadIdx.x];
    if (m != 0u) snap_tail[threadIdx.x] = uint16_t(snap_tail[threadIdx.x] ^ m);
  }
}

__global__ __launch_bounds__(kXorBlock) void xor_apply_scalar_kernel(uint16_t* snap,
                                                                     const uint16_t* mask,
                                                                     int64_t n) {
  const int64_t stride = int64_t(gridDim.x) * kXorBlock;
  for (int64_t i = int64_t(blockIdx.x) * kXorBlock + threadIdx.x; i < n; i += stride) {
    const uint16_t m = mask[i];
    if (m != 0u) snap[i] = uint16_t(snap[i] ^ m);
  }
}

__global__ __launch_bounds__(kXorBlock) void xor_scalar_kernel(const uint16_t* a,
                                                               const uint16_t* b, uint16_t* out,
                                                               int64_t n) {
  const int64_t stride = int64_t(gridDim.x) * kXorBlock;
  for (int64_t i = int64_t(blockIdx.x) * kXorBlock + threadIdx.x; i < n; i += stride)
    out[i] = uint16_t(a[i] ^ b[i]);
}

hipError_t launch_xor3(const uint16_t* a, const uint16_t* b, uint16_t* out, int64_t n,
                       hipStream_t stream) {
  clear_stale_error();
  if (n <= 0) return hipSuccess;
  const bool aligned = ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b) |
                         reinterpret_cast<uintptr_t>(out)) & 15u) == 0;
  if (aligned) {
    const int64_t nvec = n / kVec;
    const int tail = int(n - nvec * kVec);
    int64_t blocks = (nvec + kXorChunkVec - 1) / kXorChunkVec;
    if (blocks < 1) blocks = 1;
    if (blocks > (int64_t(1) << 20)) blocks = int64_t(1) << 20;
    xor_vec_kernel<<<dim3(unsigned(blocks)), dim3(kXorBlock), 0, stream>>>(
        reinterpret_cast<const uint4*>(a), reinterpret_cast<const uint4*>(b),
        reinterpret_cast<uint4*>(out), nvec, a + nvec * kVec, b + nvec * kVec,
        out + nvec * kVec, tail);
  } else {
    int64_t blocks = (n + kXorBlock - 1) / kXorBlock;
    if (blocks > (int64_t(1) << 20)) blocks = int64_t(1) << 20;
    xor_scalar_kernel<<<dim3(unsigned(blocks)), dim3(kXorBlock), 0, stream>>>(a, b, out, n);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_xor_mask(const uint16_t* a, const uint16_t* b, uint16_t* out, int64_t n,
                           hipStream_t stream) {
  return launch_xor3(a, b, out, n, stream);
}

hipError_t launch_xor_apply(uint16_t* snap, const uint16_t* mask, int64_t n,
                            hipStream_t stream) {
  clear_stale_error();
  if (n <= 0) return hipSuccess;
  const bool aligned =
      ((reinterpret_cast<uintptr_t>(snap) | reinterpret_cast<uintptr_t>(mask)) & 15u) == 0;
  if (aligned) {
    const int64_t nvec = n / kVec;
    const int tail = int(n - nvec * kVec);
    int64_t blocks = (nvec + kXorBlock - 1) / kXorBlock;
    if (blocks < 1) blocks = 1;
    if (blocks > (int64_t(1) << 20)) blocks = int64_t(1) << 20;
    xor_apply_vec_kernel<<<dim3(unsigned(blocks)), dim3(kXorBlock), 0, stream>>>(
        reinterpret_cast<uint4*>(snap), reinterpret_cast<const uint4*>(mask), nvec,
        snap + nvec * kVec, mask + nvec * kVec, tail);
  } else {
    int64_t blocks = (n + kXorBlock - 1) / kXorBlock;
    if (blocks > (int64_t(1) << 20)) blocks = int64_t(1) << 20;
    xor_apply_scalar_kernel<<<dim3(unsigned(blocks)), dim3(kXorBlock), 0, stream>>>(snap, mask, n);
  }
  return hipGetLastError();
}

}  // namespace sbd
