// spec_verify_static: spec_verify for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid allocation).  Its scratch -- the
// per-sequence records of spec_verify's kernel (arrival ticket, published chunk sums) and a
// header -- lives in a static device array of this file instead of a caller's workspace.
//
// The array exists once per device the library runs on and holds kStaticVerifySeqs records.  In
// host code its name is only a host-side stand-in, so at the first call on each device (with
// that device current) its device address is looked up with hipGetSymbolAddress and kept; every
// launch gets that address.  The same first call zero-fills the array on the caller's stream;
// from then on every completed call leaves its tickets and slots at zero again (the kernel's
// own protocol), so no later call clears anything.  All calls on one device share the array:
// calls that overlap in time on one device race, so they must be ordered (one stream, or
// synchronised), like calls that share a workspace.
#include <mutex>

#include "vap_internal.h"

namespace vap {
namespace {

constexpr int kStaticVerifySeqs = 4096;
constexpr size_t kStaticHeader = 256;
constexpr size_t kStaticBytes = kStaticHeader + (size_t)kStaticVerifySeqs * kVerifyRec;   // 8,454,400 bytes

static __device__ __align__(256) unsigned char scratch[kStaticBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
char* g_scratch[kMaxDevices];   // device address of `scratch` on each device (null until looked up)

// This device's scratch address; looked up (and the array zero-filled on `stream`) at the first
// call on the device.  Returns a VAP_* code.
int device_scratch(hipStream_t stream, char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return host_error(VAP_ENODEV, "no current device");
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return host_error(VAP_EHIP, "hipGetSymbolAddress of the static scratch failed");
    e = launch_fill_zero(ptr, kStaticBytes, stream);
    if (e != hipSuccess) return host_error(VAP_EHIP, "zero-filling the static scratch failed");
    g_scratch[dev] = static_cast<char*>(ptr);
  }
  *out = g_scratch[dev];
  return VAP_OK;
}

}  // namespace
}  // namespace vap

extern "C" int spec_verify_static(const float* p, const float* q, const int32_t* draft_ids, const float* uniforms,
                                  int32_t* out_ids, int32_t* n_accepted, int32_t num_seqs, int32_t k, int32_t vocab,
                                  int32_t* device_error, void* stream_) {
  using namespace vap;
  if (num_seqs > kStaticVerifySeqs) {
    return host_error(VAP_EINVAL, "spec_verify_static: num_seqs above the static scratch's 4096 sequences "
                                  "(use spec_verify with a workspace)");
  }
  if (num_seqs <= 0) return verify_dispatch(p, q, draft_ids, uniforms, out_ids, n_accepted, num_seqs, k, vocab,
                                            nullptr, nullptr, static_cast<hipStream_t>(stream_));
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  char* base = nullptr;
  const int rc = device_scratch(stream, &base);
  if (rc != VAP_OK) return rc;
  // error bits go to the caller's word when given, else to the scratch header (not read back)
  int32_t* err = device_error != nullptr ? device_error : reinterpret_cast<int32_t*>(base);
  return verify_dispatch(p, q, draft_ids, uniforms, out_ids, n_accepted, num_seqs, k, vocab, base + kStaticHeader,
                         err, stream);
}
