// CPU check of the library's host code (workspace sizing, carving and argument checks) at the
// extremes of every entry point, built with AddressSanitizer and UndefinedBehaviorSanitizer and
// linked with host stand-ins for the HIP runtime and the kernel launchers (stubs.cpp), which
// verify that every region a call carves lies inside the workspace it was given.
//
// Device pointers are fake addresses that nothing dereferences; the workspaces are address
// ranges of the sizes the library asks for, so sizes far beyond host memory are covered.
// Prints a summary and exits nonzero on any violation or unexpected return code.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "vap.h"

extern uintptr_t check_ws_begin, check_ws_end;
extern long check_violations, check_launches;

namespace {

long failures = 0, calls = 0;
const uintptr_t kWs = 0x100000000000ull;      // fake workspace base (256-byte aligned)
void* fake(uintptr_t a) { return reinterpret_cast<void*>(a); }
void* const D1 = fake(0x7e0000000000ull);     // fake 16-byte aligned device data
void* const D2 = fake(0x7e4000000000ull);
void* const D3 = fake(0x7e8000000000ull);
void* const D4 = fake(0x7ec000000000ull);
void* const D5 = fake(0x7f0000000000ull);
void* const D6 = fake(0x7f4000000000ull);
void* const D7 = fake(0x7f8000000000ull);
void* const D8 = fake(0x7fc000000000ull);

void* workspace(size_t bytes) {
  check_ws_begin = kWs;
  check_ws_end = kWs + bytes;
  return fake(kWs);
}

// rc must equal `want`; a call that returns VAP_OK must have launched something
void expect(int rc, int want, long launches_before, const char* what) {
  ++calls;
  const bool launched = check_launches > launches_before;
  if (rc != want || (rc == VAP_OK && !launched) || (rc != VAP_OK && launched)) {
    ++failures;
    std::fprintf(stderr, "FAIL %s: rc %d (want %d), launched %d: %s\n", what, rc, want, (int)launched,
                 vap_last_error_message());
  }
}

vap_attn_shape shape(int B, int Hq, int Hkv, int D, int BS, int NB, int MB, int T) {
  vap_attn_shape s{};
  s.num_seqs = B;
  s.num_q_heads = Hq;
  s.num_kv_heads = Hkv;
  s.head_dim = D;
  s.block_size = BS;
  s.num_blocks = NB;
  s.max_blocks_per_seq = MB;
  s.total_q = T;
  s.scale = 0.f;
  return s;
}

void attention_case(const vap_attn_shape& s) {
  const size_t hi = vap_attn_workspace_bytes(&s), lo = vap_attn_workspace_min_bytes(&s);
  if (hi == 0 || lo == 0 || lo > hi) {
    ++failures;
    std::fprintf(stderr, "FAIL sizes B=%d T=%d: min %zu default %zu\n", s.num_seqs, s.total_q, lo, hi);
    return;
  }
  const size_t mid = (lo + (hi - lo) / 3) / 256 * 256;
  for (size_t bytes : {hi, lo, mid > lo ? mid : lo, hi + 4096}) {
    long l0 = check_launches;
    expect(paged_attn_step(D1, D2, (const int32_t*)D3, (const int32_t*)D4, (const int32_t*)D5, (float*)D6, &s,
                           workspace(bytes), bytes, nullptr),
           VAP_OK, l0, "paged_attn_step");
    l0 = check_launches;
    expect(paged_attn_step_u8(D1, D2, (const float*)D7, (const int32_t*)D3, (const int32_t*)D4, (const int32_t*)D5,
                              (float*)D6, &s, workspace(bytes), bytes, nullptr),
           VAP_OK, l0, "paged_attn_step_u8");
    l0 = check_launches;
    expect(paged_attn_step_fp8(D1, D2, (const float*)D7, (const int32_t*)D3, (const int32_t*)D4, (const int32_t*)D5,
                               (float*)D6, &s, workspace(bytes), bytes, nullptr),
           VAP_OK, l0, "paged_attn_step_fp8");
    l0 = check_launches;
    expect(paged_attn_step_tree(D1, D2, nullptr, (const int32_t*)D3, (const int32_t*)D4, (const int32_t*)D5,
                                (const uint64_t*)D8, (float*)D6, &s, workspace(bytes), bytes, nullptr),
           VAP_OK, l0, "paged_attn_step_tree");
    l0 = check_launches;
    expect(kv_append(D1, D2, D3, nullptr, (const int32_t*)D4, (const int32_t*)D5, (const int32_t*)D6, &s,
                     workspace(bytes), bytes, nullptr),
           VAP_OK, l0, "kv_append");
    l0 = check_launches;
    expect(kv_commit(D3, (float*)D7, (const int32_t*)D4, (const int32_t*)D5, (const int32_t*)D6, (const int32_t*)D8,
                     64, (const int32_t*)D1, (int32_t*)D5, &s, workspace(bytes), bytes, nullptr),
           VAP_OK, l0, "kv_commit");
  }
  const long l0 = check_launches;
  expect(paged_attn_step(D1, D2, (const int32_t*)D3, (const int32_t*)D4, (const int32_t*)D5, (float*)D6, &s,
                         workspace(lo - 256), lo - 256, nullptr),
         VAP_ENOSPC, l0, "paged_attn_step below the minimum workspace");
}

void verify_case(int B, int k, int V) {
  const size_t n = vap_verify_workspace_bytes(B, k, V);
  long l0 = check_launches;
  expect(spec_verify((const float*)D1, k ? (const float*)D2 : nullptr, k ? (const int32_t*)D3 : nullptr,
                     (const float*)D4, (int32_t*)D5, (int32_t*)D6, B, k, V, workspace(n), n, nullptr),
         VAP_OK, l0, "spec_verify");
  l0 = check_launches;
  expect(spec_verify((const float*)D1, (const float*)D2, (const int32_t*)D3, (const float*)D4, (int32_t*)D5,
                     (int32_t*)D6, B, k, V, workspace(n - 8), n - 8, nullptr),
         VAP_ENOSPC, l0, "spec_verify below its workspace");
  const size_t nl = vap_verify_logits_workspace_bytes(B, k, V);
  const long long rows = (long long)B * (2 * k + 1) * ((V + 2047) / 2048);
  l0 = check_launches;
  expect(spec_verify_logits((const float*)D1, k ? (const float*)D2 : nullptr, k ? (const int32_t*)D3 : nullptr,
                            (const float*)D4, (const float*)D7, (int32_t*)D5, (int32_t*)D6, B, k, V, workspace(nl), nl,
                            nullptr),
         rows + 8192 < (1LL << 31) ? VAP_OK : VAP_EINVAL, l0, "spec_verify_logits");
}

void tree_case(int B, int N, int V) {
  const size_t n = vap_tree_verify_workspace_bytes(B);
  long l0 = check_launches;
  expect(spec_verify_tree((const float*)D1, (const float*)D2, (const int32_t*)D3, (const int32_t*)D4,
                          (const float*)D5, (int32_t*)D6, (int32_t*)D7, (int32_t*)D8, B, N, V, workspace(n), n, nullptr),
         VAP_OK, l0, "spec_verify_tree");
  l0 = check_launches;
  expect(spec_verify_tree((const float*)D1, (const float*)D2, (const int32_t*)D3, (const int32_t*)D4,
                          (const float*)D5, (int32_t*)D6, (int32_t*)D7, (int32_t*)D8, B, N, V, workspace(n - 8), n - 8,
                          nullptr),
         VAP_ENOSPC, l0, "spec_verify_tree below its workspace");
}

}  // namespace

int main() {
  // attention: decode, verify, prefill-like and tree-like batches at the sequence limits, both
  // head sizes and block sizes, the LDS plan and the plan-kernel paths (above 2048 sequences)
  for (int B : {1, 7, 2048, 2049, 8192})
    for (int D : {64, 128})
      for (int BS : {16, 32})
        for (int q : {1, 5, 64}) {
          const int MB = 32768 / BS;
          attention_case(shape(B, 64, 8, D, BS, B * 4 + 1, MB, B * q));
          attention_case(shape(B, 8, 8, D, BS, B + 1, 8, B * q));
        }
  // verification at its extremes: batch up to 2^22, k up to 64, vocabulary up to 2^20
  for (int B : {1, 16, 1024, 8192, 1 << 22})
    for (int k : {0, 4, 64})
      for (int V : {1, 3, 1000, 128256, 262144, 262145, 300001, 1 << 20}) verify_case(B, k, V);
  for (int B : {1, 64, 8192, 1 << 22})
    for (int N : {1, 16, 64})
      for (int V : {1, 3001, 128256, 262145, 1 << 20}) tree_case(B, N, V);

  // argument errors are reported, nothing launched
  vap_attn_shape bad = shape(4, 8, 3, 128, 16, 10, 4, 4);
  long l0 = check_launches;
  expect(paged_attn_step(D1, D2, (const int32_t*)D3, (const int32_t*)D4, (const int32_t*)D5, (float*)D6, &bad,
                         workspace(1 << 20), 1 << 20, nullptr),
         VAP_EINVAL, l0, "Hq not a multiple of Hkv");
  l0 = check_launches;
  expect(spec_verify(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 4, 65, 10, nullptr, 0, nullptr), VAP_EINVAL,
         l0, "k above 64");
  l0 = check_launches;
  expect(spec_verify_tree((const float*)D1, (const float*)D2, (const int32_t*)D3, (const int32_t*)D4, (const float*)D5,
                          (int32_t*)D6, (int32_t*)D7, (int32_t*)D8, 4, 65, 10, workspace(1 << 20), 1 << 20, nullptr),
         VAP_EINVAL, l0, "tree above 64 nodes");

  // the error word of a real buffer: read, cleared through the fill launcher
  std::vector<int32_t> word(64, 0x10);
  check_ws_begin = reinterpret_cast<uintptr_t>(word.data());
  check_ws_end = check_ws_begin + word.size() * 4;
  int32_t err = 0;
  ++calls;
  if (vap_get_device_error(word.data(), nullptr, &err, 1) != VAP_OK || err != 0x10) {
    ++failures;
    std::fprintf(stderr, "FAIL vap_get_device_error: %d\n", err);
  }

  std::printf("%ld calls, %ld launches checked, %ld carving violations, %ld failures\n", calls, check_launches,
              check_violations, failures);
  return (failures == 0 && check_violations == 0) ? 0 : 1;
}
