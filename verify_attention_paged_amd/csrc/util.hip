// Small utility kernels: workspace zero fill and a plain streaming copy (bandwidth ceiling and
// hardware byte-counter calibration).
#include "vap_internal.h"

namespace vap {
namespace {

__global__ __launch_bounds__(256) void fill_zero_kernel(uint4* dst16, size_t n16, unsigned char* tail, size_t ntail) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
    dst16[i] = make_uint4(0, 0, 0, 0);
  }
  if (blockIdx.x == 0 && threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

__global__ __launch_bounds__(256) void stream_copy_kernel(uint4* __restrict__ dst, const uint4* __restrict__ src, size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  // four independent 16-byte loads in flight per thread
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    dst[i] = a;
    dst[i + stride] = b;
    dst[i + 2 * stride] = c;
    dst[i + 3 * stride] = d;
  }
  for (; i < n16; i += stride) dst[i] = src[i];
}

__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ src, size_t n16, uint4* sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint4 acc = make_uint4(0, 0, 0, 0);
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    acc.x ^= a.x ^ b.x ^ c.x ^ d.x;
    acc.y ^= a.y ^ b.y ^ c.y ^ d.y;
    acc.z ^= a.z ^ b.z ^ c.z ^ d.z;
    acc.w ^= a.w ^ b.w ^ c.w ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = src[i];
    acc.x ^= a.x; acc.y ^= a.y; acc.z ^= a.z; acc.w ^= a.w;
  }
  if (acc.x == 0x9e3779b9u && acc.y == 0x7f4a7c15u && acc.z == 0xf39cc060u && acc.w == 0x5ced1c1du)
    sink[blockIdx.x] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* src, size_t bytes, void* sink, hipStream_t stream) {
  const size_t n16 = bytes / 16;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  size_t grid = (size_t)cus * 8;
  const size_t need = (n16 + 255) / 256;
  if (grid > need) grid = need ? need : 1;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                     reinterpret_cast<const uint4*>(src), n16, reinterpret_cast<uint4*>(sink));
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* dst, size_t bytes, hipStream_t stream) {
  // the workspace start is 256-byte aligned by contract; the tail below 16 bytes is done bytewise
  const size_t n16 = bytes / 16;
  const size_t ntail = bytes - n16 * 16;
  const size_t blocks = n16 ? (n16 + 255) / 256 : 1;
  const unsigned grid = (unsigned)(blocks < 8192 ? blocks : 8192);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(grid), dim3(256), 0, stream,
                     reinterpret_cast<uint4*>(dst), n16, reinterpret_cast<unsigned char*>(dst) + n16 * 16, ntail);
  return hipGetLastError();
}

hipError_t launch_stream_copy(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  const size_t n16 = bytes / 16;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  size_t grid = (size_t)cus * 8;
  const size_t need = (n16 + 255) / 256;
  if (grid > need) grid = need ? need : 1;
  hipLaunchKernelGGL(stream_copy_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                     reinterpret_cast<uint4*>(dst), reinterpret_cast<const uint4*>(src), n16);
  return hipGetLastError();
}

}  // namespace vap
