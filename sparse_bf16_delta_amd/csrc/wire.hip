// wire.hip -- the wire encoding of a batched delta and its checksum.
//
// What is computed (verl PR #6974 review, encode.py: `DeltaParam`,
// `DeltaFlush`, `checksum`): the positions of a flush are one byte block,
// parameter after parameter, each position written little-endian with the
// parameter's width of 2 or 4 bytes (2 when the parameter has at most 65536
// elements, so that every local index fits); each parameter records where its
// positions start and end in the block.  The checksum mixes two hashes --
// torch.hash_tensor's XOR of the elements widened to 64 bits -- of the byte
// block (bytes zero-extended) and of the values (bf16 widened to IEEE double,
// taken as bits): hash(positions) ^ (hash(values) << 1).
//
// How, on gfx950: a one-workgroup scan gives every parameter's byte offset
// (count times width); encode and decode give each workgroup 2048 consecutive
// entries, find the parameter of the first with a 64-way search in wave 0 and
// walk forward per lane, consecutive lanes taking consecutive entries.
// Positions are written and read as 2-byte halves, which every offset is
// aligned to (all widths are even).  The hash is an XOR reduction: 16-byte
// words per lane, then the wave with shuffles, the workgroup in LDS, and one
// 64-bit atomic XOR per workgroup over a bounded grid (atomics on one address
// serialise: one per wave over 8192 workgroups took 0.8 ms on a 7B delta).
#include "sbd_internal.h"

namespace sbd {
namespace {

constexpr int kWireBlock = 256;
constexpr int kWirePer = 16;
constexpr int64_t kWireChunk = int64_t(kWireBlock) * kWirePer;
constexpr int kScanThreads = 1024;

// pos_offsets[p] = sum over q < p of (offsets[q+1] - offsets[q]) * widths[q].
__global__ __launch_bounds__(kScanThreads) void wire_offsets_kernel(
    int32_t nparams, const int32_t* __restrict__ widths, const int64_t* __restrict__ offsets,
    int64_t* __restrict__ pos_offsets) {
  __shared__ int64_t s_w[kScanThreads / 64];
  __shared__ int64_t s_carry;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) s_carry = 0;
  __syncthreads();
  for (int32_t base = 0; base < nparams; base += kScanThreads) {
    const int32_t p = base + tid;
    const int64_t own = p < nparams ? (offsets[p + 1] - offsets[p]) * widths[p] : 0;
    int64_t inc = own;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int64_t y = __shfl_up(inc, o, 64);
      if (lane >= o) inc += y;
    }
    if (lane == 63) s_w[wave] = inc;
    __syncthreads();
    int64_t before = s_carry;
    for (int w = 0; w < wave; ++w) before += s_w[w];
    if (p < nparams) pos_offsets[p] = before + inc - own;
    __syncthreads();  // everyone has read s_carry and s_w
    if (tid == kScanThreads - 1) s_carry = before + inc;
    __syncthreads();
  }
  if (tid == 0) pos_offsets[nparams] = s_carry;
}

template <bool kDecode>
__global__ __launch_bounds__(kWireBlock) void wire_code_kernel(
    int32_t nparams, const int32_t* __restrict__ widths, const int64_t* __restrict__ offsets,
    const int64_t* __restrict__ pos_offsets, int64_t max_entries, int32_t* __restrict__ idx,
    uint8_t* __restrict__ positions, int64_t positions_capacity) {
  __shared__ int32_t s_p0;
  __shared__ int64_t s_total;
  const int64_t nchunks = (max_entries + kWireChunk - 1) / kWireChunk;
  for (int64_t chunk = blockIdx.x; chunk < nchunks; chunk += gridDim.x) {
    const int64_t j0 = chunk * kWireChunk;
    if (threadIdx.x < 64) {
      const int64_t t = offsets[nparams];
      const int64_t total = t < max_entries ? t : max_entries;
      if (j0 < total) {
        const int32_t p0 = find_param_wave0(offsets, nparams, j0);
        if (threadIdx.x == 0) s_p0 = p0;
      }
      if (threadIdx.x == 0) s_total = total;
    }
    __syncthreads();
    const int64_t total = s_total;
    if (j0 < total) {  // uniform over the workgroup
      // consecutive lanes take consecutive entries (coalesced); each lane's
      // parameter cursor only moves forward
      int32_t p = s_p0;
      int64_t seg_end = offsets[p + 1];
      int w = widths[p];
      int64_t base = pos_offsets[p] - offsets[p] * w;  // byte of entry j is base + j * w
#pragma unroll
      for (int r = 0; r < kWirePer; ++r) {
        const int64_t j = j0 + int64_t(r) * kWireBlock + threadIdx.x;
        if (j < total) {
          if (seg_end <= j) {
            do {
              seg_end = offsets[++p + 1];
            } while (seg_end <= j);
            w = widths[p];
            base = pos_offsets[p] - offsets[p] * w;
          }
          const int64_t at = base + j * w;
          auto half = reinterpret_cast<uint16_t*>(positions + at);
          if constexpr (kDecode) {
            uint32_t v = *global_ptr(half);
            if (w == 4) v |= uint32_t(*global_ptr(half + 1)) << 16;
            idx[j] = static_cast<int32_t>(v);
          } else {
            if (at + w <= positions_capacity) {
              const uint32_t v = static_cast<uint32_t>(idx[j]);
              *global_ptr(half) = static_cast<uint16_t>(v & 0xFFFFu);
              if (w == 4) *global_ptr(half + 1) = static_cast<uint16_t>(v >> 16);
            }
          }
        }
      }
    }
    __syncthreads();  // s_p0 / s_total are rewritten by the next chunk
  }
}

// IEEE widening of a bf16 pattern to double, as bits; a NaN keeps its payload
// and becomes quiet (what converting through float and double does).
__device__ __forceinline__ uint64_t bf16_to_f64_bits(uint32_t b) {
  const uint64_t sign = uint64_t(b >> 15) << 63;
  const uint32_t e = (b >> 7) & 0xFFu;
  const uint64_t m = b & 0x7Fu;
  if (e == 0xFFu) return sign | (uint64_t(0x7FF) << 52) | (m << 45) | (m ? (1ull << 51) : 0ull);
  if (e != 0u) return sign | (uint64_t(e - 127 + 1023) << 52) | (m << 45);
  if (m == 0u) return sign;
  const int k = 31 - __builtin_clz(static_cast<uint32_t>(m));  // leading one, 0..6
  return sign | (uint64_t(k - 133 + 1023) << 52) | ((m << (52 - k)) & ((1ull << 52) - 1));
}

__global__ __launch_bounds__(64) void wire_hash_zero_kernel(uint64_t* hashes) {
  if (threadIdx.x < 2) hashes[threadIdx.x] = 0;
}

__global__ __launch_bounds__(kWireBlock) void wire_hash_kernel(const uint8_t* __restrict__ pos,
                                                               int64_t npos,
                                                               const uint16_t* __restrict__ val,
                                                               int64_t nval,
                                                               uint64_t* __restrict__ hashes) {
  constexpr int kUnroll = 4;
  __shared__ uint64_t s_h[2][kWireBlock / 64];
  const int64_t stride = int64_t(gridDim.x) * kWireBlock;
  const int64_t t0 = int64_t(blockIdx.x) * kWireBlock + threadIdx.x;
  // bytes: the XOR of 16-byte words, folded to one byte at the end (whole
  // words only when the block is 16-byte aligned)
  uint32_t hb = 0;
  const int64_t nvec = (reinterpret_cast<uintptr_t>(pos) & 15u) == 0 ? npos / 16 : 0;
  const auto pw = global_ptr(reinterpret_cast<const u32x4*>(pos));
  for (int64_t v = t0; v < nvec; v += kUnroll * stride) {
    u32x4 w[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t vu = v + u * stride;
      w[u] = vu < nvec ? pw[vu] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) hb ^= w[u].x ^ w[u].y ^ w[u].z ^ w[u].w;
  }
  for (int64_t i = nvec * 16 + t0; i < npos; i += stride) hb ^= pos[i];
  uint64_t hp = (hb ^ (hb >> 8) ^ (hb >> 16) ^ (hb >> 24)) & 0xFFu;
  // values: 8 per 16-byte word when aligned
  uint64_t hv = 0;
  const int64_t nval8 = (reinterpret_cast<uintptr_t>(val) & 15u) == 0 ? nval / 8 : 0;
  const auto vw = global_ptr(reinterpret_cast<const u32x4*>(val));
  for (int64_t v = t0; v < nval8; v += kUnroll * stride) {
    u32x4 w[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t vu = v + u * stride;
      w[u] = vu < nval8 ? vw[vu] : u32x4{0u, 0u, 0u, 0u};  // +0.0 widens to 0: XOR-neutral
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        hv ^= bf16_to_f64_bits(w[u][q] & 0xFFFFu) ^ bf16_to_f64_bits(w[u][q] >> 16);
  }
  for (int64_t i = nval8 * 8 + t0; i < nval; i += stride) hv ^= bf16_to_f64_bits(val[i]);
  // wave, then workgroup, then one atomic XOR per workgroup and hash
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    hp ^= __shfl_xor(hp, o, 64);
    hv ^= __shfl_xor(hv, o, 64);
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    s_h[0][wave] = hp;
    s_h[1][wave] = hv;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t a = 0, b = 0;
#pragma unroll
    for (int w = 0; w < kWireBlock / 64; ++w) {
      a ^= s_h[0][w];
      b ^= s_h[1][w];
    }
    if (a) atomicXor(reinterpret_cast<unsigned long long*>(&hashes[0]), a);
    if (b) atomicXor(reinterpret_cast<unsigned long long*>(&hashes[1]), b);
  }
}

unsigned code_grid(int64_t max_entries) {
  int64_t blocks = (max_entries + kWireChunk - 1) / kWireChunk;
  if (blocks < 1) blocks = 1;
  if (blocks > (int64_t(1) << 20)) blocks = int64_t(1) << 20;
  return static_cast<unsigned>(blocks);
}

}  // namespace

hipError_t launch_wire_encode(int32_t nparams, const int32_t* widths, const int32_t* idx,
                              const int64_t* offsets, int64_t max_entries, uint8_t* positions,
                              int64_t positions_capacity, int64_t* pos_offsets,
                              hipStream_t stream) {
  clear_stale_error();
  wire_offsets_kernel<<<dim3(1), dim3(kScanThreads), 0, stream>>>(nparams, widths, offsets,
                                                                   pos_offsets);
  if (nparams > 0 && max_entries > 0)
    wire_code_kernel<false><<<dim3(code_grid(max_entries)), dim3(kWireBlock), 0, stream>>>(
        nparams, widths, offsets, pos_offsets, max_entries, const_cast<int32_t*>(idx), positions,
        positions_capacity);
  return hipGetLastError();
}

hipError_t launch_wire_decode(int32_t nparams, const int32_t* widths, const uint8_t* positions,
                              const int64_t* pos_offsets, const int64_t* offsets,
                              int64_t max_entries, int32_t* idx, hipStream_t stream) {
  clear_stale_error();
  if (nparams > 0 && max_entries > 0)
    wire_code_kernel<true><<<dim3(code_grid(max_entries)), dim3(kWireBlock), 0, stream>>>(
        nparams, widths, offsets, pos_offsets, max_entries, idx,
        const_cast<uint8_t*>(positions), 0);
  return hipGetLastError();
}

hipError_t launch_wire_hash(const uint8_t* positions, int64_t npos, const uint16_t* values,
                            int64_t nval, uint64_t* hashes, hipStream_t stream) {
  clear_stale_error();
  wire_hash_zero_kernel<<<dim3(1), dim3(64), 0, stream>>>(hashes);
  // a bounded grid: every workgroup ends in one atomic per hash on the same
  // two addresses, which serialise
  const int64_t work = (npos / 16 > nval / 8 ? npos / 16 : nval / 8);
  int64_t blocks = (work + kWireBlock * 16 - 1) / (kWireBlock * 16);
  if (blocks < 1) blocks = 1;
  if (blocks > 2048) blocks = 2048;
  wire_hash_kernel<<<dim3(unsigned(blocks)), dim3(kWireBlock), 0, stream>>>(positions, npos,
                                                                           values, nval, hashes);
  return hipGetLastError();
}

}  // namespace sbd
