// abi_smoke.cpp -- the C ABI of include/sbd.h used from native code, with no
// Python in the process: device buffers from hipMalloc, the calls on a HIP
// stream, and the results checked by the properties that define them.
//
//   * delta_diff: the count equals the number of positions whose 16-bit
//     patterns differ, the indices ascend strictly, and each value is new's
//     pattern at its index (TRL delta-sync article, sections 4.1-4.2);
//   * delta_apply of that delta turns old into new bit for bit (section 4.3);
//   * xor_mask / xor_apply: old ^ mask == new, and again gives old back
//     (humans& XOR summary, first paragraph);
//   * delta_diff_many / delta_apply_many over a split of the same elements
//     give the same entries with per-parameter local indices.
//
// Exit status 0 when every check holds; a message names the first failure.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "sbd.h"

namespace {

int fail(const char* what) {
  std::fprintf(stderr, "abi_smoke: %s (%s)\n", what, delta_last_error());
  return 1;
}

#define HIP_OK(x)                                                                   \
  do {                                                                              \
    if ((x) != hipSuccess) {                                                        \
      std::fprintf(stderr, "abi_smoke: %s failed: %s\n", #x, hipGetErrorString(x)); \
      return 1;                                                                     \
    }                                                                               \
  } while (0)

// xorshift64*, seeded: the test's own inputs
uint64_t next(uint64_t& s) {
  s ^= s >> 12;
  s ^= s << 25;
  s ^= s >> 27;
  return s * 2685821657736338717ull;
}

}  // namespace

int main() {
  const int64_t n = 3 * 32768 + 1234;  // several tiles and a ragged tail
  std::vector<uint16_t> old_h(n), new_h(n);
  uint64_t s = 0x9E3779B97F4A7C15ull;
  int64_t want = 0;
  for (int64_t i = 0; i < n; ++i) {
    old_h[i] = static_cast<uint16_t>(next(s));
    new_h[i] = old_h[i];
    if (next(s) % 100 < 3) {  // about 3 % changed
      new_h[i] = static_cast<uint16_t>(old_h[i] ^ (1u + next(s) % 0xFFFFu));
      ++want;
    }
  }
  hipStream_t st;
  HIP_OK(hipStreamCreate(&st));
  uint16_t *d_old, *d_new, *d_snap, *d_mask, *d_val;
  int32_t* d_idx;
  int64_t *d_nnz, *d_offsets, *d_nnz_many;
  HIP_OK(hipMalloc(&d_old, n * 2));
  HIP_OK(hipMalloc(&d_new, n * 2));
  HIP_OK(hipMalloc(&d_snap, n * 2));
  HIP_OK(hipMalloc(&d_mask, n * 2));
  HIP_OK(hipMalloc(&d_val, n * 2));
  HIP_OK(hipMalloc(&d_idx, n * 4));
  HIP_OK(hipMalloc(&d_nnz, 8));
  HIP_OK(hipMalloc(&d_nnz_many, 3 * 8));
  HIP_OK(hipMalloc(&d_offsets, 4 * 8));
  const size_t ws_bytes = delta_workspace_size(n, 3);
  void* d_ws;
  HIP_OK(hipMalloc(&d_ws, ws_bytes));
  HIP_OK(hipMemcpy(d_old, old_h.data(), n * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_new, new_h.data(), n * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_snap, old_h.data(), n * 2, hipMemcpyHostToDevice));

  // ---- delta_diff, then delta_apply into a copy of old
  if (delta_diff(d_old, d_new, n, d_idx, d_val, n, d_nnz, d_ws, ws_bytes, st) != DELTA_OK)
    return fail("delta_diff");
  int64_t nnz = -1;
  HIP_OK(hipMemcpyAsync(&nnz, d_nnz, 8, hipMemcpyDeviceToHost, st));
  HIP_OK(hipStreamSynchronize(st));
  if (nnz != want) return fail("delta_diff count differs from the differing positions");
  std::vector<int32_t> idx(nnz);
  std::vector<uint16_t> val(nnz);
  HIP_OK(hipMemcpy(idx.data(), d_idx, nnz * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(val.data(), d_val, nnz * 2, hipMemcpyDeviceToHost));
  for (int64_t j = 0; j < nnz; ++j) {
    if (j > 0 && idx[j] <= idx[j - 1]) return fail("delta_diff indices not strictly ascending");
    if (idx[j] < 0 || idx[j] >= n || old_h[idx[j]] == new_h[idx[j]])
      return fail("delta_diff index names an unchanged position");
    if (val[j] != new_h[idx[j]]) return fail("delta_diff value is not new's pattern");
  }
  if (delta_apply(d_snap, n, d_idx, d_val, nnz, st) != DELTA_OK)
    return fail("delta_apply");
  std::vector<uint16_t> got(n);
  HIP_OK(hipMemcpyAsync(got.data(), d_snap, n * 2, hipMemcpyDeviceToHost, st));
  HIP_OK(hipStreamSynchronize(st));
  if (std::memcmp(got.data(), new_h.data(), n * 2) != 0) return fail("apply(old, diff) != new");

  // ---- XOR mode: the mask takes the snapshot (now new) back to old, then again to new
  if (xor_mask(d_old, d_new, d_mask, n, st) != DELTA_OK) return fail("xor_mask");
  if (xor_apply(d_snap, d_mask, n, st) != DELTA_OK) return fail("xor_apply");
  HIP_OK(hipMemcpyAsync(got.data(), d_snap, n * 2, hipMemcpyDeviceToHost, st));
  HIP_OK(hipStreamSynchronize(st));
  if (std::memcmp(got.data(), old_h.data(), n * 2) != 0) return fail("new ^ mask != old");

  // ---- the batched pair over three parameters cut from the same elements
  const int64_t cut[4] = {0, 777, 40000, n};
  const uint16_t* optrs[3];
  const uint16_t* nptrs[3];
  uint16_t* sptrs[3];
  int64_t numels[3];
  for (int p = 0; p < 3; ++p) {
    optrs[p] = d_old + cut[p];
    nptrs[p] = d_new + cut[p];
    sptrs[p] = d_snap + cut[p];
    numels[p] = cut[p + 1] - cut[p];
  }
  if (delta_diff_many(3, optrs, nptrs, numels, d_idx, d_val, n, d_nnz_many, d_offsets, d_ws,
                      ws_bytes, st) != DELTA_OK)
    return fail("delta_diff_many");
  int64_t offsets[4];
  HIP_OK(hipMemcpyAsync(offsets, d_offsets, sizeof offsets, hipMemcpyDeviceToHost, st));
  HIP_OK(hipStreamSynchronize(st));
  std::vector<int32_t> idx_many(offsets[3]);
  HIP_OK(hipMemcpy(idx_many.data(), d_idx, offsets[3] * 4, hipMemcpyDeviceToHost));
  if (offsets[0] != 0 || offsets[3] != nnz) return fail("delta_diff_many total");
  for (int p = 0; p < 3; ++p)
    for (int64_t j = offsets[p]; j < offsets[p + 1]; ++j)
      if (idx_many[j] + cut[p] != idx[j]) return fail("delta_diff_many entry differs");
  // snapshot is old again: apply the batched delta and expect new
  if (delta_apply_many(3, sptrs, numels, d_idx, d_val, d_offsets, n, nullptr, d_ws, ws_bytes,
                       st) != DELTA_OK)
    return fail("delta_apply_many");
  HIP_OK(hipMemcpyAsync(got.data(), d_snap, n * 2, hipMemcpyDeviceToHost, st));
  HIP_OK(hipStreamSynchronize(st));
  if (std::memcmp(got.data(), new_h.data(), n * 2) != 0) return fail("apply_many != new");

  // ---- an argument error comes back as a status with a message, nothing launched
  if (delta_diff(d_old, d_new, -1, d_idx, d_val, n, d_nnz, d_ws, ws_bytes, st) != DELTA_E_INVALID)
    return fail("negative n not rejected");

  for (void* p : {(void*)d_old, (void*)d_new, (void*)d_snap, (void*)d_mask, (void*)d_val,
                  (void*)d_idx, (void*)d_nnz, (void*)d_nnz_many, (void*)d_offsets, d_ws})
    HIP_OK(hipFree(p));
  HIP_OK(hipStreamDestroy(st));
  std::printf("abi_smoke ok: %lld elements, %lld changed, diff/apply/xor and the batched pair "
              "checked\n", (long long)n, (long long)nnz);
  return 0;
}
