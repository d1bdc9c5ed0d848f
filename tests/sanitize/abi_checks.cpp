// Host-only driver of the C ABI's host-side logic (argument checks, size queries, plans, page-table
// and shared-prefix checks) for a build with AddressSanitizer and UndefinedBehaviorSanitizer.  The
// launch functions of the kernels' translation units are stubs here: nothing reaches a GPU, and
// every call below either fails its checks or needs no device at all.  Exit status 0 when every
// expectation holds (the sanitizers abort on their own findings).
#include <climits>
#include <cstdint>
#include <cstdio>
#include <vector>

#include "oscar.h"
#include "oscar_internal.h"

namespace oscar {
hipError_t launch_bf16_decode(const Bf16DecodeArgs&, const Bf16Plan&, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_bf16_store(const Bf16StoreArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_demote(const DemoteArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_probe_read(const void*, size_t, uint32_t*, int, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_probe_gather(const void*, const int32_t*, int, int, int, int, int, int,
                               uint32_t*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t scratch_on_current_device(void**) { return hipErrorNotSupported; }
hipError_t launch_prep(const AppendArgs*, const QueryArgs*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_decode(const DecodeArgs&, const Plan&, uint32_t, hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace oscar

namespace {
int failures = 0;
#define EXPECT(cond)                                                           \
  do {                                                                         \
    if (!(cond)) {                                                             \
      std::fprintf(stderr, "line %d: expected %s\n", __LINE__, #cond);          \
      ++failures;                                                              \
    }                                                                          \
  } while (0)

oscar_layout layout(int hq = 32, int hkv = 8, int group = 128, int pages = 64, int seqs = 4,
                    int per_seq = 16, int kind = 0) {
  return oscar_layout{128, group, hq, hkv, 64, 64, 256, pages, seqs, per_seq, kind};
}

// a pointer the checks accept (aligned, not NULL); never dereferenced on these paths
void* fake(uintptr_t at = 1 << 20) { return reinterpret_cast<void*>(at); }
}  // namespace

int main() {
  // ---- layouts and size queries, including extreme values
  const oscar_layout good = layout();
  EXPECT(oscar_abi_version() == OSCAR_ABI_VERSION);
  EXPECT(oscar_pool_bytes(&good) > 0);
  const int extremes[] = {INT_MIN, -1, 0, 1, 3, 64, 65535, 1 << 20, INT_MAX};
  for (int v : extremes) {
    oscar_layout l = good;
    for (int field = 0; field < 11; ++field) {
      l = good;
      reinterpret_cast<int32_t*>(&l)[field] = v;
      (void)oscar_pool_bytes(&l);
      (void)oscar_sink_bytes(&l);
      (void)oscar_recent_bytes(&l);
      (void)oscar_page_block_bytes(&l);
      (void)oscar_decode_workspace_bytes(&l, 4, 100000);
      (void)oscar_bf16_pool_bytes(&l);
    }
    for (int w : extremes) {
      (void)oscar_decode_workspace_bytes(&good, v, w);
      (void)oscar_decode_workspace_bytes_prefix(&good, v, w, 511);
      (void)oscar_decode_workspace_bytes_prefix(&good, 4, w, v);
      (void)oscar_bf16_decode_workspace_bytes(&good, v, w);
      int32_t pps = 0;
      (void)oscar_decode_splits(&good, v, w, &pps);
      (void)oscar_decode_step_launches(&good, v, w);
    }
  }
  EXPECT(oscar_decode_workspace_bytes(nullptr, 1, 1000) == 0);
  EXPECT(oscar_decode_splits(&good, -1, 1000, nullptr) == -1);
  EXPECT(oscar_decode_step_launches(&good, 1, 100000) == 2);

  // ---- page-table checks on exactly sized host arrays
  {
    const oscar_layout l = layout(32, 8, 128, 64, 4, 16);
    std::vector<int32_t> table(4 * 16), lens(4);
    for (int b = 0; b < 4; ++b)
      for (int j = 0; j < 16; ++j) table[b * 16 + j] = b * 16 + j;
    for (int b = 0; b < 4; ++b) lens[b] = 320 + 64 * (3 + b);
    EXPECT(oscar_check_page_table(&l, table.data(), lens.data(), 4, 0) == OSCAR_OK);
    EXPECT(oscar_check_page_table(&l, table.data(), lens.data(), 4, 64) == OSCAR_OK);
    lens[3] = 320 + 64 * 16 + 1;   // one page past the row
    EXPECT(oscar_check_page_table(&l, table.data(), lens.data(), 4, 0) != OSCAR_OK);
    lens[3] = 320;
    table[1] = 64;                  // an id past the pool, in a page sequence 0 uses
    EXPECT(oscar_check_page_table(&l, table.data(), lens.data(), 4, 0) != OSCAR_OK);
    table[1] = 1;
    table[16 + 1] = 1;              // sequence 1 aliases sequence 0's page 1 past its page 0
    EXPECT(oscar_check_page_table(&l, table.data(), lens.data(), 4, 0) != OSCAR_OK);
    table[16 + 0] = 0;              // now a common prefix of two pages: allowed to read
    EXPECT(oscar_check_page_table(&l, table.data(), lens.data(), 4, 0) == OSCAR_OK);
    lens[1] = 320 + 64;             // ... but not to demote into (copy-on-write rule)
    EXPECT(oscar_check_page_table(&l, table.data(), lens.data(), 4, 8) != OSCAR_OK);
    for (int v : extremes) {
      lens[2] = v;
      (void)oscar_check_page_table(&l, table.data(), lens.data(), 4, 3);
      (void)oscar_check_page_table(&l, table.data(), lens.data(), 4, v);
    }
    EXPECT(oscar_check_page_table(&l, nullptr, lens.data(), 4, 0) == OSCAR_ERR_NULL);

    // shared-prefix description
    std::vector<int32_t> ids = {0, 1}, shared = {2, 2, 0, 0};
    EXPECT(oscar_check_shared_prefix(&l, table.data(), 4, ids.data(), shared.data(), 2) ==
           OSCAR_OK);
    shared[2] = 3;                  // more shared pages than the prefix has
    EXPECT(oscar_check_shared_prefix(&l, table.data(), 4, ids.data(), shared.data(), 2) !=
           OSCAR_OK);
    shared[2] = 1;                  // sequence 2's page 0 is not the prefix's
    EXPECT(oscar_check_shared_prefix(&l, table.data(), 4, ids.data(), shared.data(), 2) !=
           OSCAR_OK);
  }

  // ---- entry points: every check fails before a launch
  {
    const oscar_layout l = layout(32, 8, 128, 64, 4, 1600);
    void* p = fake();
    const int32_t* ip = static_cast<const int32_t*>(p);
    const float* fp = static_cast<const float*>(p);
    EXPECT(oscar_decode_step(&l, p, ip, p, p, p, p, fp, fp, fp, fp, nullptr, nullptr, p, p, ip, ip,
                             nullptr, 0.f, static_cast<float*>(p), nullptr, p, 1 << 30, 1, 100000,
                             nullptr) == OSCAR_ERR_NULL);
    for (uint32_t stages : {0u, 16u, 2u, 4u, 13u})
      EXPECT(oscar_decode_step_stages(&l, p, ip, p, p, p, p, fp, fp, fp, fp, nullptr, nullptr, p,
                                      p, ip, ip, p, 0.f, static_cast<float*>(p), nullptr, p,
                                      1 << 30, 1, 100000, stages, nullptr) == OSCAR_ERR_RANGE);
    EXPECT(oscar_decode_attn(&l, p, ip, p, p, p, p, ip, ip, p, fp, fp, 0.f,
                             static_cast<float*>(p), nullptr, p, 16, 1, 100000, nullptr) ==
           OSCAR_ERR_WORKSPACE);
    for (int v : extremes) {
      (void)oscar_decode_attn(&l, p, ip, p, p, p, p, ip, ip, p, fp, fp, 0.f,
                              static_cast<float*>(p), nullptr, p, 1 << 30, v, v, nullptr);
      (void)oscar_decode_step_noalloc(&l, p, ip, p, p, p, p, fp, fp, fp, fp, nullptr, nullptr, p,
                                      p, ip, ip, nullptr, 0.f, static_cast<float*>(p), nullptr,
                                      v, v, nullptr);
    }
    EXPECT(oscar_last_error()[0] != '\0');
  }

  if (failures) std::fprintf(stderr, "%d expectation(s) failed\n", failures);
  else std::printf("host ABI checks under the sanitizers: all expectations hold\n");
  return failures ? 1 : 0;
}
