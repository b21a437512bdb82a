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

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWireBlock = 256;
constexpr int kWirePer = 16;
static_assert(kWirePer % 4 == 0, "the blocked decode takes four entries per lane");
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

// Encode writes a position only if all its bytes fit `positions_capacity`.
// Decode reads one only if its bytes lie inside the block
// (`positions_capacity` is then the block's size) and inside its parameter's
// span [pos_offsets[p], pos_offsets[p+1]); otherwise it writes -1 (never a
// valid index) and counts the entry in `violations` (if not null).
template <bool kDecode>
__global__ __launch_bounds__(kWireBlock) void wire_code_kernel(
    int32_t nparams, const int32_t* __restrict__ widths, const int64_t* __restrict__ offsets,
    const int64_t* __restrict__ pos_offsets, int64_t max_entries, int32_t* __restrict__ idx,
    uint8_t* __restrict__ positions, int64_t positions_capacity,
    unsigned long long* __restrict__ violations) {
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
      int64_t span_lo = kDecode ? pos_offsets[p] : 0;
      int64_t span_end = kDecode ? pos_offsets[p + 1] : 0;
      int64_t bad = 0;
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
            if constexpr (kDecode) {
              span_lo = pos_offsets[p];
              span_end = pos_offsets[p + 1];
            }
          }
          const int64_t at = base + j * w;
          auto half = reinterpret_cast<uint16_t*>(positions + at);
          if constexpr (kDecode) {
            if (at >= span_lo && at >= 0 && at + w <= span_end && at + w <= positions_capacity &&
                (at & 1) == 0) {
              uint32_t v = *global_ptr(half);
              if (w == 4) v |= uint32_t(*global_ptr(half + 1)) << 16;
              idx[j] = static_cast<int32_t>(v);
            } else {
              idx[j] = -1;
              ++bad;
            }
          } else {
            if (at + w <= positions_capacity) {
              const uint32_t v = static_cast<uint32_t>(idx[j]);
              *global_ptr(half) = static_cast<uint16_t>(v & 0xFFFFu);
              if (w == 4) *global_ptr(half + 1) = static_cast<uint16_t>(v >> 16);
            }
          }
        }
      }
      if (kDecode && violations != nullptr) {
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) bad += __shfl_xor(bad, o, 64);
        if ((threadIdx.x & 63) == 0 && bad != 0)
          atomicAdd(violations, static_cast<unsigned long long>(bad));
      }
    }
    __syncthreads();  // s_p0 / s_total are rewritten by the next chunk
  }
}

// Decode's per-parameter check: the span pos_offsets[p+1] - pos_offsets[p]
// must be the parameter's count times its width; each parameter that is not
// adds one to `violations` (its entries are then checked one by one above).
__global__ __launch_bounds__(256) void wire_spans_kernel(int32_t nparams,
                                                         const int32_t* __restrict__ widths,
                                                         const int64_t* __restrict__ offsets,
                                                         const int64_t* __restrict__ pos_offsets,
                                                         unsigned long long* __restrict__ violations) {
  const int32_t p = int32_t(blockIdx.x) * 256 + int32_t(threadIdx.x);
  if (p < nparams) {
    const int64_t count = offsets[p + 1] - offsets[p];
    if (count < 0 || pos_offsets[p + 1] - pos_offsets[p] != count * widths[p])
      atomicAdd(violations, 1ull);
  }
}

__global__ __launch_bounds__(64) void wire_zero_kernel(unsigned long long* v) {
  if (threadIdx.x == 0) *v = 0ull;
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

// The flush checksum from the two hashes, in place: checksum = hash(positions)
// ^ (hash(values) << 1), 65 bits as two words (low 64, then bit 64).
__global__ __launch_bounds__(64) void wire_checksum_kernel(uint64_t* hashes) {
  if (threadIdx.x == 0) {
    const uint64_t hp = hashes[0], hv = hashes[1];
    hashes[0] = hp ^ (hv << 1);
    hashes[1] = hv >> 63;
  }
}

// ---------------------------------------------------------------------------
// Blocked positions (2 bytes per position for any parameter size): the
// parameter's index range is cut into blocks of kPosBlockElems elements; each
// block stores the count of the parameter's entries before it (uint32, the
// block's base in its entry list) and each entry its offset inside its block
// (uint16).  Layout: the block tables of all parameters, then the offsets of
// all entries in entry order.
// ---------------------------------------------------------------------------
// Largest p with bp[p].tbase <= t: the parameter holding global block t (a
// parameter with no blocks shares its tbase with the next and is skipped).
__device__ __forceinline__ int32_t block_param(const BlockedParam* __restrict__ bp,
                                               int32_t nparams, int64_t t) {
  int32_t lo = 0, hi = nparams - 1;
  while (lo < hi) {
    const int32_t mid = (lo + hi + 1) >> 1;
    if (bp[mid].tbase <= t)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// One thread per block: its base, the first entry of its parameter at or
// above the block's first element (a binary search over the ascending
// indices), as a 4-byte word at out[4t] when it fits.
__global__ __launch_bounds__(256) void wire_blocked_table_kernel(
    int32_t nparams, const BlockedParam* __restrict__ bp, int64_t nblocks,
    const int32_t* __restrict__ idx, const int64_t* __restrict__ offsets, int64_t max_entries,
    uint8_t* __restrict__ out, int64_t out_capacity) {
  const int64_t t0 = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t stride = int64_t(gridDim.x) * 256;
  const int64_t tot = offsets[nparams] < max_entries ? offsets[nparams] : max_entries;
  for (int64_t t = t0; t < nblocks; t += stride) {
    const int32_t p = block_param(bp, nparams, t);
    const int64_t b = t - bp[p].tbase;
    const int64_t first = offsets[p];
    int64_t lo = first, hi = offsets[p + 1] < tot ? offsets[p + 1] : tot;
    if (hi < lo) hi = lo;
    const int64_t target = b * kPosBlockElems;
    while (lo < hi) {  // first entry with idx >= target
      const int64_t mid = lo + ((hi - lo) >> 1);
      if (int64_t(idx[mid]) < target)
        lo = mid + 1;
      else
        hi = mid;
    }
    if (4 * t + 4 <= out_capacity)
      *global_ptr(reinterpret_cast<uint32_t*>(out + 4 * t)) = static_cast<uint32_t>(lo - first);
  }
}

// Every entry's offset inside its block, 2 bytes at out[lows + 2j]: the low
// 16 bits of its parameter-local index, since blocks start at multiples of
// 65536.  Four entries per lane: one 16-byte load of their indices and one
// 8-byte store (two 4-byte ones where the offsets start only 4-byte aligned;
// `out` is 4-byte aligned and `lows` a multiple of 4), entry by entry at the
// capacity's edge or for an unaligned idx.
__global__ __launch_bounds__(256) void wire_blocked_lows_kernel(
    int32_t nparams, const int32_t* __restrict__ idx, const int64_t* __restrict__ offsets,
    int64_t max_entries, uint8_t* __restrict__ out, int64_t lows, int64_t out_capacity) {
  const int64_t tot = offsets[nparams] < max_entries ? offsets[nparams] : max_entries;
  const bool in16 = (reinterpret_cast<uintptr_t>(idx) & 15u) == 0;
  const bool out8 = ((reinterpret_cast<uintptr_t>(out) + uintptr_t(lows)) & 7u) == 0;
  const int64_t stride = int64_t(gridDim.x) * 256 * 4;
  for (int64_t j = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 4; j < tot; j += stride) {
    uint8_t* dst = out + lows + 2 * j;
    if (in16 && j + 4 <= tot && lows + 2 * j + 8 <= out_capacity) {
      const u32x4 v = *global_ptr(reinterpret_cast<const u32x4*>(idx + j));
      const uint32_t w0 = (v.x & 0xFFFFu) | (v.y << 16);
      const uint32_t w1 = (v.z & 0xFFFFu) | (v.w << 16);
      if (out8) {
        u32x2 w;
        w.x = w0;
        w.y = w1;
        *global_ptr(reinterpret_cast<u32x2*>(dst)) = w;
      } else {
        *global_ptr(reinterpret_cast<uint32_t*>(dst)) = w0;
        *global_ptr(reinterpret_cast<uint32_t*>(dst + 4)) = w1;
      }
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (j + k < tot && lows + 2 * (j + k) + 2 <= out_capacity)
          *global_ptr(reinterpret_cast<uint16_t*>(dst + 2 * k)) =
              static_cast<uint16_t>(static_cast<uint32_t>(idx[j + k]) & 0xFFFFu);
    }
  }
}

// Decode: workgroups of kWireChunk consecutive entries as wire_code_kernel;
// each lane keeps a (parameter, block) cursor that only moves forward, found
// by a binary search over the parameter's bases when the parameter changes.
// An entry whose offset lies past `in_bytes`, or whose position falls outside
// its parameter, becomes -1 and is counted in `violations` (if not null).
__global__ __launch_bounds__(kWireBlock) void wire_blocked_decode_kernel(
    int32_t nparams, const BlockedParam* __restrict__ bp, int64_t nblocks,
    const uint8_t* __restrict__ in, int64_t in_bytes, const int64_t* __restrict__ offsets,
    int64_t max_entries, int32_t* __restrict__ idx, unsigned long long* __restrict__ violations) {
  __shared__ int32_t s_p0;
  __shared__ int64_t s_b0;  // the block of the chunk's first entry in parameter s_p0
  __shared__ int64_t s_total;
  const auto words = global_ptr(reinterpret_cast<const uint32_t*>(in));
  const int64_t lows = 4 * nblocks;
  const int64_t nchunks = (max_entries + kWireChunk - 1) / kWireChunk;
  for (int64_t chunk = blockIdx.x; chunk < nchunks; chunk += gridDim.x) {
    const int64_t j0 = chunk * kWireChunk;
    if (threadIdx.x < 64) {
      const int64_t t = offsets[nparams];
      const int64_t total = t < max_entries ? t : max_entries;
      if (j0 < total) {
        const int32_t p0 = find_param_wave0(offsets, nparams, j0);
        // the last block whose base is <= the first entry's place in its
        // parameter, by a 64-way search over the parameter's bases (each step
        // probes 64 evenly spaced bases at once; three steps for 2^18 blocks)
        const int64_t local = j0 - offsets[p0];
        const int64_t tb = bp[p0].tbase;
        int64_t lo = 0, hi = (bp[p0].numel + kPosBlockElems - 1) / kPosBlockElems;
        while (hi - lo > 1) {
          const int64_t step = (hi - lo + 63) / 64;
          const int64_t probe = lo + int64_t(threadIdx.x) * step;
          const uint64_t ok = __ballot(probe < hi && int64_t(words[tb + probe]) <= local);
          if (ok == 0u) break;  // a malformed table (its first base above the entry); checked apart
          lo += int64_t(63 - __builtin_clzll(ok)) * step;
          hi = lo + step < hi ? lo + step : hi;
        }
        if (threadIdx.x == 0) {
          s_p0 = p0;
          s_b0 = lo;
        }
      }
      if (threadIdx.x == 0) s_total = total;
    }
    __syncthreads();
    const int64_t total = s_total;
    if (j0 < total) {
      int32_t p = s_p0;
      int64_t seg_end = offsets[p + 1];
      int64_t first = offsets[p];
      // the chunk's entries in s_p0 start from its first entry's block and walk forward
      int64_t numel = bp[p].numel, tb = bp[p].tbase, b = s_b0;
      int64_t nb = (numel + kPosBlockElems - 1) / kPosBlockElems;
      // the base of the cursor's next block, kept in a register: the table
      // is read again only when an entry passes it
      constexpr int64_t kNone = INT64_MAX;
      int64_t nxt = b + 1 < nb ? int64_t(words[tb + b + 1]) : kNone;
      int64_t bad = 0;
      // four consecutive entries per lane: one 8-byte (or two 4-byte) load of
      // their offsets and one 16-byte store of their positions, where the
      // buffers' alignment allows (uniform over the launch; `in` is 4-byte
      // aligned, checked on the host, and so is every group of four offsets)
      const bool off8 = ((reinterpret_cast<uintptr_t>(in) + uintptr_t(lows)) & 7u) == 0;
      const bool out16 = (reinterpret_cast<uintptr_t>(idx) & 15u) == 0;
#pragma unroll 2
      for (int r = 0; r < kWirePer / 4; ++r) {
        const int64_t jb = j0 + int64_t(r) * kWireBlock * 4 + int64_t(threadIdx.x) * 4;
        if (jb < total) {
          const int64_t at = lows + 2 * jb;
          const bool whole = jb + 4 <= total && at + 8 <= in_bytes;
          uint32_t o16[4];
          if (whole && off8) {
            const u32x2 w = *global_ptr(reinterpret_cast<const u32x2*>(in + at));
            o16[0] = w.x & 0xFFFFu;
            o16[1] = w.x >> 16;
            o16[2] = w.y & 0xFFFFu;
            o16[3] = w.y >> 16;
          } else if (whole) {
            const uint32_t w0 = *global_ptr(reinterpret_cast<const uint32_t*>(in + at));
            const uint32_t w1 = *global_ptr(reinterpret_cast<const uint32_t*>(in + at + 4));
            o16[0] = w0 & 0xFFFFu;
            o16[1] = w0 >> 16;
            o16[2] = w1 & 0xFFFFu;
            o16[3] = w1 >> 16;
          } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
              o16[k] = jb + k < total && at + 2 * k + 2 <= in_bytes
                           ? uint32_t(*global_ptr(reinterpret_cast<const uint16_t*>(in + at + 2 * k)))
                           : 0xFFFFFFFFu;  // missing: decoded as -1
          }
          int32_t out[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int64_t j = jb + k;
            out[k] = -1;
            if (j < total) {
              if (seg_end <= j) {
                do {
                  seg_end = offsets[++p + 1];
                } while (seg_end <= j);
                first = offsets[p];
                numel = bp[p].numel;
                nb = (numel + kPosBlockElems - 1) / kPosBlockElems;
                tb = bp[p].tbase;
                b = -1;
              }
              const int64_t local = j - first;
              if (b < 0 || local >= nxt) {
                // the last block whose base is <= local lies past the cursor:
                // one step forward covers dense data, a search the rest
                int64_t lo = b < 0 ? 0 : b + 1;
                if (b < 0 || (lo + 1 < nb && int64_t(words[tb + lo + 1]) <= local)) {
                  int64_t hi = nb - 1;
                  while (lo < hi) {
                    const int64_t mid = (lo + hi + 1) >> 1;
                    if (int64_t(words[tb + mid]) <= local)
                      lo = mid;
                    else
                      hi = mid - 1;
                  }
                }
                b = lo;
                nxt = b + 1 < nb ? int64_t(words[tb + b + 1]) : kNone;
              }
              int64_t v = -1;
              if (nb > 0 && o16[k] <= 0xFFFFu) {
                v = b * kPosBlockElems + int64_t(o16[k]);
                if (v >= numel) v = -1;
              }
              out[k] = static_cast<int32_t>(v);
              bad += v < 0 ? 1 : 0;
            }
          }
          if (jb + 4 <= total && out16) {
            u32x4 w;
            w.x = uint32_t(out[0]);
            w.y = uint32_t(out[1]);
            w.z = uint32_t(out[2]);
            w.w = uint32_t(out[3]);
            *global_ptr(reinterpret_cast<u32x4*>(idx + jb)) = w;
          } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
              if (jb + k < total) idx[jb + k] = out[k];
          }
        }
      }
      if (violations != nullptr) {
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) bad += __shfl_xor(bad, o, 64);
        if ((threadIdx.x & 63) == 0 && bad != 0)
          atomicAdd(violations, static_cast<unsigned long long>(bad));
      }
    }
    __syncthreads();
  }
}

// Table check for decode: per block, the first base is 0 and bases do not
// decrease or exceed the parameter's count; each block that breaks this adds
// one to `violations`.
__global__ __launch_bounds__(256) void wire_blocked_check_kernel(
    int32_t nparams, const BlockedParam* __restrict__ bp, int64_t nblocks,
    const uint8_t* __restrict__ in, const int64_t* __restrict__ offsets,
    unsigned long long* __restrict__ violations) {
  const auto words = global_ptr(reinterpret_cast<const uint32_t*>(in));
  const int64_t stride = int64_t(gridDim.x) * 256;
  for (int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x; t < nblocks; t += stride) {
    const int32_t p = block_param(bp, nparams, t);
    const int64_t b = t - bp[p].tbase;
    const int64_t nb = (bp[p].numel + kPosBlockElems - 1) / kPosBlockElems;
    const int64_t count = offsets[p + 1] - offsets[p];
    const int64_t base = words[t];
    const int64_t next = b + 1 < nb ? int64_t(words[t + 1]) : count;
    if ((b == 0 && base != 0) || base > next || next > count) atomicAdd(violations, 1ull);
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
        positions_capacity, nullptr);
  return hipGetLastError();
}

hipError_t launch_wire_decode(int32_t nparams, const int32_t* widths, const uint8_t* positions,
                              int64_t positions_bytes, const int64_t* pos_offsets,
                              const int64_t* offsets, int64_t max_entries, int32_t* idx,
                              int64_t* violations, hipStream_t stream) {
  clear_stale_error();
  auto v = reinterpret_cast<unsigned long long*>(violations);
  if (v != nullptr) {
    wire_zero_kernel<<<dim3(1), dim3(64), 0, stream>>>(v);
    if (nparams > 0)
      wire_spans_kernel<<<dim3(unsigned((nparams + 255) / 256)), dim3(256), 0, stream>>>(
          nparams, widths, offsets, pos_offsets, v);
  }
  if (nparams > 0 && max_entries > 0)
    wire_code_kernel<true><<<dim3(code_grid(max_entries)), dim3(kWireBlock), 0, stream>>>(
        nparams, widths, offsets, pos_offsets, max_entries, idx,
        const_cast<uint8_t*>(positions), positions_bytes, v);
  return hipGetLastError();
}

hipError_t launch_wire_checksum(const uint8_t* positions, int64_t npos, const uint16_t* values,
                                int64_t nval, uint64_t* checksum, hipStream_t stream) {
  const hipError_t e = launch_wire_hash(positions, npos, values, nval, checksum, stream);
  if (e != hipSuccess) return e;
  wire_checksum_kernel<<<dim3(1), dim3(64), 0, stream>>>(checksum);
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

namespace sbd {

hipError_t launch_wire_encode_blocked(int32_t nparams, const BlockedParam* bp, int64_t nblocks,
                                      const int32_t* idx, const int64_t* offsets,
                                      int64_t max_entries, uint8_t* out, int64_t out_capacity,
                                      hipStream_t stream) {
  clear_stale_error();
  if (nparams <= 0) return hipSuccess;
  if (nblocks > 0) {
    int64_t g = (nblocks + 255) / 256;
    if (g > 4096) g = 4096;
    wire_blocked_table_kernel<<<dim3(unsigned(g)), dim3(256), 0, stream>>>(
        nparams, bp, nblocks, idx, offsets, max_entries, out, out_capacity);
  }
  if (max_entries > 0) {
    int64_t g = (max_entries + 1023) / 1024;
    if (g > 65536) g = 65536;
    wire_blocked_lows_kernel<<<dim3(unsigned(g)), dim3(256), 0, stream>>>(
        nparams, idx, offsets, max_entries, out, 4 * nblocks, out_capacity);
  }
  return hipGetLastError();
}

hipError_t launch_wire_decode_blocked(int32_t nparams, const BlockedParam* bp, int64_t nblocks,
                                      const uint8_t* in, int64_t in_bytes, const int64_t* offsets,
                                      int64_t max_entries, int32_t* idx, int64_t* violations,
                                      hipStream_t stream) {
  clear_stale_error();
  auto v = reinterpret_cast<unsigned long long*>(violations);
  if (v != nullptr) {
    wire_zero_kernel<<<dim3(1), dim3(64), 0, stream>>>(v);
    if (nparams > 0 && nblocks > 0) {
      int64_t g = (nblocks + 255) / 256;
      if (g > 4096) g = 4096;
      wire_blocked_check_kernel<<<dim3(unsigned(g)), dim3(256), 0, stream>>>(nparams, bp, nblocks,
                                                                            in, offsets, v);
    }
  }
  if (nparams > 0 && max_entries > 0)
    wire_blocked_decode_kernel<<<dim3(code_grid(max_entries)), dim3(kWireBlock), 0, stream>>>(
        nparams, bp, nblocks, in, in_bytes, offsets, max_entries, idx, v);
  return hipGetLastError();
}

}  // namespace sbd
