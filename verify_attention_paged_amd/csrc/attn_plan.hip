// Plan kernel of paged_attn_step for batches above 2048 sequences (smaller batches build the
// same tables inside every attention workgroup, in LDS).
//
// One workgroup of 1024 threads
//   * validates each sequence's lengths (1 <= q_len <= ctx_len <= table capacity, packed rows
//     inside total_q) and flags the rest in the sticky error word; invalid sequences get no
//     work,
//   * computes each sequence's first packed query row (exclusive scan of q_lens: ragged rows
//     without padding -- tempatgunting.com article, section "Implementation Details That Affect
//     Tail Latency"),
//   * counts each sequence's work: UH + ceil(ctx_len / block_size) work blocks for every (KV
//     head, row group) unit, where a row group is RG of the G * q_len query rows sharing a KV
//     head and UH stands for the fixed cost of starting a unit,
//   * records the sequence holding the first work block of each worker wave, the waves
//     splitting the total work TB evenly: wave w owns [w*TB/W', (w+1)*TB/W'), W' = min(W, TB).
#include "attn_internal.h"

namespace vap {
namespace {

template <typename T>
__device__ __forceinline__ T wave_inclusive_scan(T x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const T y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  return x;
}

// Exclusive scan over the 1024-thread workgroup; `total` receives the workgroup sum.
template <typename T>
__device__ __forceinline__ T block_exclusive_scan(T x, T* s_tmp, T& total) {
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const T incl = wave_inclusive_scan(x);
  if (lane == 63) s_tmp[wv] = incl;
  __syncthreads();
  if (wv == 0) {
    const T t = lane < kPlanThreads / 64 ? s_tmp[lane] : T(0);
    const T ti = wave_inclusive_scan(t);
    if (lane < kPlanThreads / 64) s_tmp[lane] = ti - t;
    if (lane == kPlanThreads / 64 - 1) s_tmp[kPlanThreads / 64] = ti;
  }
  __syncthreads();
  const T excl = s_tmp[wv] + incl - x;
  total = s_tmp[kPlanThreads / 64];
  __syncthreads();
  return excl;
}

__global__ __launch_bounds__(kPlanThreads) void attn_plan_kernel(const AttnParams P) {
  __shared__ int32_t s_off[kMaxSeqs + 1];
  __shared__ long long s_tmp64[kPlanThreads / 64 + 1];
  __shared__ int32_t s_tmp32[kPlanThreads / 64 + 1];

  const int tid = threadIdx.x;
  const long long cap = (long long)P.MB * P.BS;
  long long carry_q = 0;
  int32_t carry_w = 0;
  int32_t errbits = 0;

  for (int base = 0; base < P.B; base += kPlanThreads) {
    const int s = base + tid;
    int32_t Q = 0, L = 0;
    if (s < P.B) {
      Q = P.q_lens[s];
      L = P.ctx_lens[s];
    }
    const long long qc = (s < P.B && Q > 0) ? (long long)Q : 0;
    long long qtot;
    const long long qoff = block_exclusive_scan<long long>(qc, s_tmp64, qtot) + carry_q;
    bool valid = false;
    if (s < P.B) {
      if (Q < 1 || L < Q || (long long)L > cap) errbits |= VAP_DERR_LENS;
      else if (qoff + Q > P.total_q) errbits |= VAP_DERR_TOTAL_Q;
      else valid = true;
    }
    const int32_t work = valid ? (P.UH + (L + P.BS - 1) / P.BS) * ((P.G * Q + P.RG - 1) / P.RG) * P.Hkv : 0;
    int32_t wtot;
    const int32_t woff = block_exclusive_scan<int32_t>(work, s_tmp32, wtot) + carry_w;
    if (s < P.B) {
      P.g_L[s] = valid ? L : 0;
      P.g_Q[s] = valid ? Q : 1;
      P.q_off[s] = valid ? (int32_t)qoff : 0;
      P.seq_off[s] = woff;
      s_off[s] = woff;
    }
    carry_q += qtot;
    carry_w += wtot;
  }
  if (tid == 0) {
    s_off[P.B] = carry_w;
    P.seq_off[P.B] = carry_w;
    P.hdr->total_work = carry_w;
    if (carry_q != (long long)P.total_q) errbits |= VAP_DERR_TOTAL_Q;
  }
  __syncthreads();

  const int32_t TB = s_off[P.B];
  const int W = min(P.W, TB);
  for (int w = tid; w < W; w += kPlanThreads) {
    const long long b0 = (long long)w * TB / W;
    int lo = 0, hi = P.B;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_off[mid] <= b0) lo = mid; else hi = mid - 1;
    }
    P.wave_seq[w] = lo;
  }
  if (errbits) atomicOr(&P.hdr->err, errbits);
}

}  // namespace

hipError_t launch_attn_plan(const AttnParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(attn_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace vap
