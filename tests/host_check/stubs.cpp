// Host-only stand-ins for the HIP runtime and the library's kernel launchers, linked with the
// library's host code (api.cpp) for a CPU run under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// The runtime stand-ins model one gfx950 device with 256 CUs.  Every launcher checks that each
// device region the host code carved for the launch lies inside the workspace the harness
// declared (check_ws_begin .. check_ws_end) and is aligned as the kernels need; a violation is
// counted and printed.  Nothing here touches the carved addresses: the harness passes address
// ranges that are not backed by memory, so the checks cover sizes far beyond host RAM.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <cstring>

#include "vap_internal.h"

uintptr_t check_ws_begin = 0, check_ws_end = 0;
long check_violations = 0, check_launches = 0;

namespace {

void need(bool ok, const char* what, const void* p, long long bytes) {
  if (!ok) {
    ++check_violations;
    std::fprintf(stderr, "VIOLATION %s: %p + %lld outside [%#llx, %#llx)\n", what, p, bytes,
                 (unsigned long long)check_ws_begin, (unsigned long long)check_ws_end);
  }
}

// [p, p + bytes) inside the workspace, p aligned to `align`
void region(const void* p, long long bytes, const char* what, int align = 4) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  need(bytes >= 0 && a >= check_ws_begin && a + (uintptr_t)bytes <= check_ws_end, what, p, bytes);
  need(a % (uintptr_t)align == 0, what, p, bytes);
}

}  // namespace

// ---- HIP runtime ---------------------------------------------------------------------------
extern "C" {
hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_tR0600* prop, int) {
  std::memset(prop, 0, sizeof(*prop));
  prop->multiProcessorCount = 256;
  std::strcpy(prop->gcnArchName, "gfx950:sramecc+:xnack-");
  return hipSuccess;
}
hipError_t hipOccupancyMaxActiveBlocksPerMultiprocessor(int* n, const void*, int, size_t) {
  *n = 2;
  return hipSuccess;
}
hipError_t hipEventCreate(hipEvent_t* e) {
  static int token;
  *e = reinterpret_cast<hipEvent_t>(&token);
  return hipSuccess;
}
hipError_t hipEventElapsedTime(float* ms, hipEvent_t, hipEvent_t) {
  *ms = 0.f;
  return hipSuccess;
}
hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipMemcpy(void* dst, const void* src, size_t n, hipMemcpyKind) {
  std::memcpy(dst, src, n);   // only the error word of a real (small) buffer is ever copied
  return hipSuccess;
}
const char* hipGetErrorString(hipError_t) { return "stub"; }
}

// ---- launchers -----------------------------------------------------------------------------
namespace vap {

static void attn_regions(const AttnParams& p, int D, bool plan_in_ws) {
  region(p.hdr, sizeof(AttnHeader), "attention header", 256);
  region(p.desc, (long long)p.NH * 32, "descriptors", 16);
  region(p.part_ml, (long long)p.NH * 2 * p.RG * 8, "partial (m, l)", 8);
  region(p.part_acc, (long long)p.NH * 2 * p.RG * D * 4, "partial rows", 16);
  if (plan_in_ws) {
    region(p.g_L, (long long)p.B * 4, "plan lengths");
    region(p.g_Q, (long long)p.B * 4, "plan q_lens");
    region(p.q_off, (long long)p.B * 4, "plan q offsets");
    region(p.seq_off, (long long)(p.B + 1) * 4, "plan work offsets");
    region(p.wave_seq, (long long)p.W * 4, "plan wave sequences");
  }
  need(p.W >= 1 && p.NH >= p.W && p.NH <= p.W + p.pool_max, "holder count", p.desc, p.NH);
}

hipError_t launch_attn_plan(const AttnParams& p, hipStream_t) {
  ++check_launches;
  attn_regions(p, 64, true);
  return hipSuccess;
}
hipError_t launch_attn_main(const AttnParams& p, int D, int, int NRT, int kv, int num_wg, int wg_waves, hipStream_t,
                            KTimer) {
  need(kv >= 0 && kv <= 2 && (kv == 0) == (p.kcodes == nullptr), "cache format", p.desc, kv);
  ++check_launches;
  attn_regions(p, D, p.B > kLdsPlanMaxSeqs);
  need(p.RG == 16 * NRT, "rows per unit", p.desc, p.RG);
  need((long long)num_wg * wg_waves == p.W, "worker waves", p.desc, p.W);
  return hipSuccess;
}
hipError_t launch_attn_combine(const AttnParams& p, int D, int, bool, hipStream_t) {
  ++check_launches;
  attn_regions(p, D, p.B > kLdsPlanMaxSeqs);
  return hipSuccess;
}
const void* attn_main_kernel_ptr(int, int, int, bool, bool) {
  static int token;
  return &token;
}
size_t attn_main_lds_bytes(int B) { return size_t(4 * B + 1) * sizeof(int); }

hipError_t launch_spec_verify(const VerifyParams& p, bool, hipStream_t, KTimer) {
  ++check_launches;
  region(p.err, 4, "verify error word");
  region(p.rec.base, (long long)p.B * p.rec.stride, "verify records", 16);
  need(p.C >= 1 && p.C <= kMaxChunks && (long long)p.C * p.CS >= p.V && p.CS % 4 == 0 && p.CS <= 4096,
       "verify chunks", p.rec.base, p.C);
  // no empty chunk, and chunks a wave sums in one piece wherever the vocabulary allows
  need((long long)(p.C - 1) * p.CS < p.V, "verify chunks: an empty chunk", p.rec.base, p.C);
  need((long long)p.V > (long long)kMaxChunks * kDrawPiece || p.CS <= kDrawPiece, "verify chunks: longer than a piece",
       p.rec.base, p.CS);
  need(p.WPS >= 1 && p.WPS <= p.C && (long long)((p.C + p.WPS - 1) / p.WPS) * (p.WPS - 1) < p.C, "verify workgroups",
       p.rec.base, p.WPS);
  return hipSuccess;
}
hipError_t launch_spec_verify_logits(const VerifyParams& p, bool v, hipStream_t s, KTimer t) {
  region(p.part, (long long)p.B * (2 * p.k + 1) * p.C1 * (long long)sizeof(LogitRowStat), "logit partials", 16);
  return launch_spec_verify(p, v, s, t);
}
hipError_t launch_logit_stats(const LogitStatsParams& p, bool, int num_wg, hipStream_t, KTimer) {
  ++check_launches;
  region(p.err, 4, "statistics error word");
  region(p.part, (long long)p.B * (2 * p.k + 1) * p.C * (long long)sizeof(LogitRowStat), "logit partials", 16);
  region(p.rec.base, (long long)p.B * p.rec.stride, "logit records", 16);
  need(p.VC >= 1 && p.VC <= kMaxChunks && num_wg >= 1, "statistics grid", p.part, p.VC);
  return hipSuccess;
}
hipError_t launch_tree_verify(const TreeVerifyParams& p, hipStream_t, KTimer) {
  ++check_launches;
  region(p.err, 4, "tree error word");
  region(p.rec.base, (long long)p.B * p.rec.stride, "tree records", 16);
  return hipSuccess;
}
hipError_t launch_tree_draw(const TreeDrawParams& p, bool, hipStream_t, KTimer) {
  ++check_launches;
  region(p.rec.base, (long long)p.B * p.rec.stride, "tree draw records", 16);
  need(p.C >= 1 && p.C <= kMaxChunks && (long long)p.C * p.CS >= p.V && p.WPS >= 1 && p.WPS <= p.C, "draw chunks",
       p.rec.base, p.C);
  need((long long)(p.C - 1) * p.CS < p.V && p.CS % 4 == 0 && p.CS <= 4096, "draw chunks: empty or too long",
       p.rec.base, p.CS);
  need((long long)p.V > (long long)kMaxChunks * kDrawPiece || p.CS <= kDrawPiece, "draw chunks: longer than a piece",
       p.rec.base, p.CS);
  return hipSuccess;
}
hipError_t launch_kv_append(const KVAppendParams& p, int, bool, int, hipStream_t, KTimer) {
  ++check_launches;
  region(p.err, 4, "append error word");
  return hipSuccess;
}
hipError_t launch_kv_commit(const KVCommitParams& p, bool, hipStream_t, KTimer) {
  ++check_launches;
  region(p.err, 4, "commit error word");
  return hipSuccess;
}
hipError_t launch_fill_zero(void* dst, size_t bytes, hipStream_t) {
  ++check_launches;
  region(dst, (long long)bytes, "fill");
  return hipSuccess;
}
hipError_t launch_stream_copy(void*, const void*, size_t, hipStream_t) { return hipSuccess; }
hipError_t launch_stream_read(const void*, size_t, void*, hipStream_t) { return hipSuccess; }

}  // namespace vap
