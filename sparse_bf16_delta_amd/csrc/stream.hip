// stream.hip -- the receiver's streaming step: a delta (or XOR mask) that sits
// in pinned host memory is copied to the GPU chunk by chunk and applied to the
// resident snapshots, the copy of one chunk overlapping the apply of the one
// before.
//
// What is computed is exactly delta_apply_many (or xor_apply) over the whole
// delta; only the order of copies and kernels differs.  The TRL delta-sync
// article (section 4.3, vLLM side) applies deltas into the resident bf16
// snapshot; the XOR summary (third paragraph) overlaps mask decompression
// with the apply on the receiver.  Here the overlap is HBM-side apply against
// the host-to-device DMA.
//
// How: two staging slots in one caller-provided device buffer.  Chunk c uses
// slot c % 2.  On the copy stream, chunk c waits until the apply of chunk c-2
// (the slot's previous tenant) is done, then its idx and val are copied in
// (two async copies from pinned memory) and an event marks them present.  On
// the apply stream, the apply of chunk c waits for that event.  The snapshot
// table of the whole list and every chunk's offsets are copied once, up
// front: each copy on a stream costs tens of microseconds beyond its bytes,
// which on a 7B-shaped delta in 32 chunks with a third copy per chunk ate the
// whole overlap.  Both calls return after the last apply completes, so every
// host buffer and event they use is free again on return.
//
// The host-direct receiver (apply_host_impl) needs no staging at all: the
// apply kernel itself reads idx and val from the pinned host buffers, which
// the runtime maps into the GPU's address space, so the transfer and the
// apply proceed together at the host link's rate with no copy engine, no
// chunking and no events (the 7B-shaped delta: 8.54 ms against 8.28 ms for a
// bare copy and 9.88 ms streamed).  A dense XOR mask does not gain from it
// (245 ms against 239 streamed): the copy engine moves it better.
#include <cstdio>
#include <string>
#include <vector>

#include "sbd.h"
#include "sbd_internal.h"

namespace {

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// The most entries (or XOR elements) a staging slot is sized for: beyond it
// the slot's byte size would not fit size_t.
constexpr int64_t kMaxStagedEntries = INT64_MAX / 16;

// Staging layout: [table: SnapParam x nparams][offsets: int64 x nchunks x
// (max_params + 1)][slot 0][slot 1], each slot [idx: int32 x max_nnz][val:
// uint16 x max_nnz].
struct StagingLayout {
  size_t table, offsets;
  size_t slot[2];
  size_t idx, val;  // offsets of the parts inside a slot
  size_t total;
};

// total == SIZE_MAX: the layout would not fit size_t (no buffer can hold it).
StagingLayout staging_layout(int32_t nparams, int32_t nchunks, int32_t max_chunk_params,
                             int64_t max_chunk_nnz) {
  StagingLayout L{};
  const uint64_t noffsets =
      uint64_t(nchunks > 0 ? nchunks : 1) * (uint64_t(max_chunk_params > 0 ? max_chunk_params : 0) + 1);
  if (noffsets > SIZE_MAX / 64 || max_chunk_nnz > kMaxStagedEntries) {
    L.total = SIZE_MAX;
    return L;
  }
  L.table = 0;
  L.offsets = align256(sizeof(sbd::SnapParam) * size_t(nparams > 0 ? nparams : 1));
  const size_t off_bytes =
      align256(sizeof(int64_t) * size_t(nchunks > 0 ? nchunks : 1) * (size_t(max_chunk_params) + 1));
  const size_t nnz = size_t(max_chunk_nnz > 0 ? max_chunk_nnz : 1);
  L.idx = 0;
  L.val = align256(sizeof(int32_t) * nnz);
  const size_t slot_bytes = L.val + align256(sizeof(uint16_t) * nnz);
  L.slot[0] = L.offsets + off_bytes;
  L.slot[1] = L.slot[0] + slot_bytes;
  L.total = L.slot[1] + slot_bytes;
  return L;
}

// Events for the two slots; destroyed when the call ends (after the final
// synchronisation, so none is still pending).
struct SlotEvents {
  hipEvent_t copied[2] = {nullptr, nullptr};
  hipEvent_t applied[2] = {nullptr, nullptr};
  hipError_t create() {
    for (int s = 0; s < 2; ++s) {
      hipError_t e = hipEventCreateWithFlags(&copied[s], hipEventDisableTiming);
      if (e != hipSuccess) return e;
      e = hipEventCreateWithFlags(&applied[s], hipEventDisableTiming);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  ~SlotEvents() {
    for (int s = 0; s < 2; ++s) {
      if (copied[s]) (void)hipEventDestroy(copied[s]);
      if (applied[s]) (void)hipEventDestroy(applied[s]);
    }
  }
};

}  // namespace

namespace sbd {

size_t streamed_staging_size(int32_t nparams, int32_t nchunks, int32_t max_chunk_params,
                             int64_t max_chunk_nnz) {
  const size_t t = staging_layout(nparams, nchunks, max_chunk_params, max_chunk_nnz).total;
  return t == SIZE_MAX ? 0 : t;
}

size_t xor_streamed_staging_size(int64_t chunk_elems) {
  if (chunk_elems > kMaxStagedEntries) return 0;
  return 2 * align256(sizeof(uint16_t) * size_t(chunk_elems));
}

delta_status apply_streamed_impl(int32_t nparams, uint16_t* const* snap_ptrs,
                                 const int64_t* numels, int32_t nchunks,
                                 const delta_host_chunk* chunks, void* staging,
                                 size_t staging_bytes, void* copy_stream, void* apply_stream,
                                 std::string& err) {
  char buf[256];
  auto fail = [&](delta_status s, const char* m) {
    err = m;
    return s;
  };
  if (nparams < 0 || nchunks < 0) return fail(DELTA_E_INVALID, "delta_apply_streamed: negative count");
  if ((nchunks > 0 && chunks == nullptr) ||
      (nparams > 0 && (snap_ptrs == nullptr || numels == nullptr)))
    return fail(DELTA_E_INVALID, "delta_apply_streamed: null argument");
  std::vector<SnapParam> table(static_cast<size_t>(nparams));
  for (int32_t p = 0; p < nparams; ++p) {
    if (numels[p] < 0 || numels[p] > 2147483647LL) {
      snprintf(buf, sizeof buf, "delta_apply_streamed: numels[%d]=%lld outside [0, 2^31-1]", p,
               (long long)numels[p]);
      return fail(numels[p] < 0 ? DELTA_E_INVALID : DELTA_E_RANGE, buf);
    }
    if (numels[p] > 0 && snap_ptrs[p] == nullptr) {
      snprintf(buf, sizeof buf, "delta_apply_streamed: null snapshot for parameter %d", p);
      return fail(DELTA_E_INVALID, buf);
    }
    table[p] = SnapParam{snap_ptrs[p], numels[p]};
  }
  int32_t max_params = 0;
  int64_t max_nnz = 0;
  for (int32_t c = 0; c < nchunks; ++c) {
    const delta_host_chunk& ch = chunks[c];
    if (ch.nparams < 0 || ch.first_param < 0 || int64_t(ch.first_param) + ch.nparams > nparams) {
      snprintf(buf, sizeof buf, "delta_apply_streamed: chunk %d covers parameters outside the list",
               c);
      return fail(DELTA_E_INVALID, buf);
    }
    if (ch.nparams == 0) continue;
    if (ch.offsets == nullptr || ch.offsets[0] != 0) {
      snprintf(buf, sizeof buf, "delta_apply_streamed: chunk %d offsets missing or not from 0", c);
      return fail(DELTA_E_INVALID, buf);
    }
    for (int32_t p = 0; p < ch.nparams; ++p)
      if (ch.offsets[p + 1] < ch.offsets[p]) {
        snprintf(buf, sizeof buf, "delta_apply_streamed: chunk %d offsets decrease", c);
        return fail(DELTA_E_INVALID, buf);
      }
    const int64_t nnz = ch.offsets[ch.nparams];
    if (nnz > kMaxStagedEntries) {
      snprintf(buf, sizeof buf, "delta_apply_streamed: chunk %d holds %lld entries, more than "
               "a staging buffer can address", c, (long long)nnz);
      return fail(DELTA_E_RANGE, buf);
    }
    if (nnz > 0 && (ch.idx == nullptr || ch.val == nullptr)) {
      snprintf(buf, sizeof buf, "delta_apply_streamed: chunk %d has entries but null idx/val", c);
      return fail(DELTA_E_INVALID, buf);
    }
    max_params = ch.nparams > max_params ? ch.nparams : max_params;
    max_nnz = nnz > max_nnz ? nnz : max_nnz;
  }
  const StagingLayout L = staging_layout(nparams, nchunks, max_params, max_nnz);
  if (L.total == SIZE_MAX)
    return fail(DELTA_E_RANGE, "delta_apply_streamed: the staging layout does not fit size_t");
  if (staging == nullptr || staging_bytes < L.total) {
    snprintf(buf, sizeof buf, "delta_apply_streamed: staging %zu bytes, need %zu", staging_bytes,
             L.total);
    return fail(DELTA_E_WORKSPACE, buf);
  }
  hipStream_t cs = static_cast<hipStream_t>(copy_stream);
  hipStream_t as = static_cast<hipStream_t>(apply_stream);
  char* base = static_cast<char*>(staging);
  SnapParam* d_table = reinterpret_cast<SnapParam*>(base + L.table);
  int64_t* d_offsets = reinterpret_cast<int64_t*>(base + L.offsets);
  // every chunk's offsets, at stride max_params + 1
  const size_t ostride = size_t(max_params) + 1;
  std::vector<int64_t> all_offsets(size_t(nchunks > 0 ? nchunks : 1) * ostride, 0);
  for (int32_t c = 0; c < nchunks; ++c)
    for (int32_t p = 0; p <= chunks[c].nparams && chunks[c].nparams > 0; ++p)
      all_offsets[size_t(c) * ostride + size_t(p)] = chunks[c].offsets[p];
  SlotEvents ev;
  hipError_t e = ev.create();
  // pageable sources: HIP has staged them when each call returns
  if (e == hipSuccess && nparams > 0)
    e = hipMemcpyAsync(d_table, table.data(), sizeof(SnapParam) * table.size(),
                       hipMemcpyHostToDevice, cs);
  if (e == hipSuccess && nchunks > 0)
    e = hipMemcpyAsync(d_offsets, all_offsets.data(), sizeof(int64_t) * all_offsets.size(),
                       hipMemcpyHostToDevice, cs);
  if (e != hipSuccess) return fail(DELTA_E_HIP, hipGetErrorString(e));
  for (int32_t c = 0; c < nchunks && e == hipSuccess; ++c) {
    const delta_host_chunk& ch = chunks[c];
    if (ch.nparams == 0) continue;
    const int s = c & 1;
    char* slot = base + L.slot[s];
    const int64_t nnz = ch.offsets[ch.nparams];
    if (c >= 2) e = hipStreamWaitEvent(cs, ev.applied[s], 0);  // slot's previous chunk is done
    if (e == hipSuccess && nnz > 0)
      e = hipMemcpyAsync(slot + L.idx, ch.idx, sizeof(int32_t) * size_t(nnz),
                         hipMemcpyHostToDevice, cs);
    if (e == hipSuccess && nnz > 0)
      e = hipMemcpyAsync(slot + L.val, ch.val, sizeof(uint16_t) * size_t(nnz),
                         hipMemcpyHostToDevice, cs);
    if (e == hipSuccess) e = hipEventRecord(ev.copied[s], cs);
    if (e == hipSuccess) e = hipStreamWaitEvent(as, ev.copied[s], 0);
    int64_t chunk_elems = 0;
    for (int32_t q = 0; q < ch.nparams; ++q) chunk_elems += numels[ch.first_param + q];
    if (e == hipSuccess)
      e = launch_apply(d_table + ch.first_param, SnapParam{nullptr, 0}, ch.nparams,
                       d_offsets + size_t(c) * ostride,
                       reinterpret_cast<const int32_t*>(slot + L.idx),
                       reinterpret_cast<const uint16_t*>(slot + L.val), nnz, chunk_elems,
                       nullptr, as);
    if (e == hipSuccess) e = hipEventRecord(ev.applied[s], as);
  }
  // every copy waits on an apply, so the apply stream finishing means all done
  const hipError_t e2 = hipStreamSynchronize(as);
  const hipError_t e3 = hipStreamSynchronize(cs);
  if (e == hipSuccess) e = e2 != hipSuccess ? e2 : e3;
  if (e != hipSuccess) return fail(DELTA_E_HIP, hipGetErrorString(e));
  return DELTA_OK;
}

delta_status xor_apply_streamed_impl(uint16_t* snapshot, const uint16_t* mask_host, int64_t n,
                                     int64_t chunk_elems, void* staging, size_t staging_bytes,
                                     void* copy_stream, void* apply_stream, std::string& err) {
  char buf[256];
  auto fail = [&](delta_status s, const char* m) {
    err = m;
    return s;
  };
  if (n < 0 || chunk_elems <= 0) return fail(DELTA_E_INVALID, "xor_apply_streamed: n < 0 or chunk_elems <= 0");
  if (chunk_elems > kMaxStagedEntries)
    return fail(DELTA_E_RANGE, "xor_apply_streamed: chunk_elems too large for a staging slot");
  if (n > 0 && (snapshot == nullptr || mask_host == nullptr))
    return fail(DELTA_E_INVALID, "xor_apply_streamed: null pointer");
  // two slots of chunk_elems bf16, each 256-byte aligned
  const size_t slot_bytes = align256(sizeof(uint16_t) * size_t(chunk_elems));
  if (staging == nullptr || staging_bytes < 2 * slot_bytes) {
    snprintf(buf, sizeof buf, "xor_apply_streamed: staging %zu bytes, need %zu", staging_bytes,
             2 * slot_bytes);
    return fail(DELTA_E_WORKSPACE, buf);
  }
  hipStream_t cs = static_cast<hipStream_t>(copy_stream);
  hipStream_t as = static_cast<hipStream_t>(apply_stream);
  char* base = static_cast<char*>(staging);
  SlotEvents ev;
  hipError_t e = ev.create();
  int64_t c = 0;
  for (int64_t first = 0; first < n && e == hipSuccess; first += chunk_elems, ++c) {
    const int s = int(c & 1);
    const int64_t len = n - first < chunk_elems ? n - first : chunk_elems;
    uint16_t* slot = reinterpret_cast<uint16_t*>(base + s * slot_bytes);
    if (c >= 2) e = hipStreamWaitEvent(cs, ev.applied[s], 0);
    if (e == hipSuccess)
      e = hipMemcpyAsync(slot, mask_host + first, sizeof(uint16_t) * size_t(len),
                         hipMemcpyHostToDevice, cs);
    if (e == hipSuccess) e = hipEventRecord(ev.copied[s], cs);
    if (e == hipSuccess) e = hipStreamWaitEvent(as, ev.copied[s], 0);
    if (e == hipSuccess) e = launch_xor_apply(snapshot + first, slot, len, as);
    if (e == hipSuccess) e = hipEventRecord(ev.applied[s], as);
  }
  const hipError_t e2 = hipStreamSynchronize(as);
  const hipError_t e3 = hipStreamSynchronize(cs);
  if (e == hipSuccess) e = e2 != hipSuccess ? e2 : e3;
  if (e != hipSuccess) return fail(DELTA_E_HIP, hipGetErrorString(e));
  return DELTA_OK;
}

size_t host_apply_workspace_size(int32_t nparams) {
  const size_t k = size_t(nparams > 0 ? nparams : 0);
  return align256(sizeof(SnapParam) * (k > 0 ? k : 1)) + align256(sizeof(int64_t) * (k + 1));
}

namespace {

// The device address of `count` elements of `size` bytes at host address p,
// or nullptr unless all of them lie inside one pinned host allocation that
// the runtime has mapped for the GPU (nothing reaches a kernel unchecked: a
// range that ran into unmapped memory would fault the GPU).  A failed query
// leaves the runtime's per-thread error set, which the next launch check
// would report as its own, so it is cleared here.
const void* mapped(const void* p, int64_t count, size_t size) {
  if (count < 0 || uint64_t(count) > UINT64_MAX / size) return nullptr;  // no byte count wraps
  uint64_t start = 0, range = 0;
  void* d = nullptr;
  const uint64_t a = reinterpret_cast<uintptr_t>(p);
  const uint64_t bytes = uint64_t(count) * size;
  const bool ok =
      hipPointerGetAttribute(&start, HIP_POINTER_ATTRIBUTE_RANGE_START_ADDR,
                             reinterpret_cast<hipDeviceptr_t>(const_cast<void*>(p))) == hipSuccess &&
      hipPointerGetAttribute(&range, HIP_POINTER_ATTRIBUTE_RANGE_SIZE,
                             reinterpret_cast<hipDeviceptr_t>(const_cast<void*>(p))) == hipSuccess &&
      a >= start && bytes <= range && a - start <= range - bytes &&
      hipHostGetDevicePointer(&d, const_cast<void*>(p), 0) == hipSuccess && d != nullptr;
  if (!ok) {
    (void)hipGetLastError();
    return nullptr;
  }
  return d;
}

}  // namespace

delta_status apply_host_impl(int32_t nparams, uint16_t* const* snap_ptrs, const int64_t* numels,
                             const int32_t* idx_host, const uint16_t* val_host,
                             const int64_t* offsets_host, int64_t max_nnz, int64_t* violations,
                             void* ws, size_t ws_bytes, void* stream, std::string& err) {
  char buf[256];
  auto fail = [&](delta_status st, const char* m) {
    err = m;
    return st;
  };
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (nparams < 0 || max_nnz < 0)
    return fail(DELTA_E_INVALID, "delta_apply_many_host: nparams < 0 or max_nnz < 0");
  if (nparams > 0 && (snap_ptrs == nullptr || numels == nullptr || offsets_host == nullptr))
    return fail(DELTA_E_INVALID, "delta_apply_many_host: null argument");
  // the snapshot table and the offsets travel together in one copy
  const size_t table_bytes = align256(sizeof(SnapParam) * size_t(nparams > 0 ? nparams : 1));
  std::vector<char> host(host_apply_workspace_size(nparams), 0);
  SnapParam* table = reinterpret_cast<SnapParam*>(host.data());
  int64_t* offs = reinterpret_cast<int64_t*>(host.data() + table_bytes);
  int64_t total_elems = 0;
  for (int32_t p = 0; p < nparams; ++p) {
    if (numels[p] < 0 || numels[p] > 2147483647LL) {
      snprintf(buf, sizeof buf, "delta_apply_many_host: numels[%d]=%lld outside [0, 2^31-1]", p,
               (long long)numels[p]);
      return fail(numels[p] < 0 ? DELTA_E_INVALID : DELTA_E_RANGE, buf);
    }
    if (numels[p] > 0 && snap_ptrs[p] == nullptr) {
      snprintf(buf, sizeof buf, "delta_apply_many_host: null snapshot for parameter %d", p);
      return fail(DELTA_E_INVALID, buf);
    }
    table[p] = SnapParam{snap_ptrs[p], numels[p]};
    total_elems += numels[p];
  }
  int64_t total = 0;
  if (nparams > 0) {
    if (offsets_host[0] != 0)
      return fail(DELTA_E_INVALID, "delta_apply_many_host: offsets[0] != 0");
    for (int32_t p = 0; p < nparams; ++p) {
      if (offsets_host[p + 1] < offsets_host[p]) {
        snprintf(buf, sizeof buf, "delta_apply_many_host: offsets decrease at parameter %d", p);
        return fail(DELTA_E_INVALID, buf);
      }
    }
    for (int32_t p = 0; p <= nparams; ++p) offs[p] = offsets_host[p];
    total = offsets_host[nparams] < max_nnz ? offsets_host[nparams] : max_nnz;
  }
  const int32_t* d_idx = nullptr;
  const uint16_t* d_val = nullptr;
  if (total > 0) {
    d_idx = static_cast<const int32_t*>(mapped(idx_host, total, sizeof(int32_t)));
    d_val = static_cast<const uint16_t*>(mapped(val_host, total, sizeof(uint16_t)));
    if (d_idx == nullptr || d_val == nullptr) {
      snprintf(buf, sizeof buf,
               "delta_apply_many_host: idx and val must be pinned host memory (hipHostMalloc, "
               "torch pin_memory) holding %lld entries",
               (long long)total);
      return fail(DELTA_E_INVALID, buf);
    }
  }
  if (ws == nullptr || ws_bytes < host.size()) {
    snprintf(buf, sizeof buf, "delta_apply_many_host: workspace %zu bytes, need %zu", ws_bytes,
             host.size());
    return fail(DELTA_E_WORKSPACE, buf);
  }
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return fail(DELTA_E_WORKSPACE, "delta_apply_many_host: workspace not 256-byte aligned");
  hipError_t e = hipSuccess;
  if (total > 0)
    e = hipMemcpyAsync(ws, host.data(), host.size(), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) {
    const SnapParam* d_table = static_cast<const SnapParam*>(ws);
    const int64_t* d_offs =
        reinterpret_cast<const int64_t*>(static_cast<const char*>(ws) + table_bytes);
    e = launch_apply(total > 0 ? d_table : nullptr, SnapParam{nullptr, 0}, nparams, d_offs,
                     d_idx, d_val, total, total_elems, violations, s);
  }
  if (e != hipSuccess) return fail(DELTA_E_HIP, hipGetErrorString(e));
  return DELTA_OK;
}

}  // namespace sbd
