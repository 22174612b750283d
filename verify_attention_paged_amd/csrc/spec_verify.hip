// Speculative-decoding verification kernel (gfx950).
//
// What is computed, per sequence b (neuralmasteryai.com "Continuous Batching & Speculative
// Decoding", section "The Modified Rejection Sampling Algorithm"; syslabs.in "Continuous
// Batching and Speculative Decoding: How Modern LLM Serving Engines Actually Work", section
// "The core idea"):
//   1. accept test: draft x_i passes when p_i(x_i) > 0 and r_i * q_i(x_i) <= p_i(x_i) (the exact
//      form of r_i <= min(1, p/q), evaluated in fp64 where the product of two fp32 values is
//      exact); n = index of the first failure, or k;
//   2. the row to draw from: w = max(0, p_n - q_n) when n < k, else the bonus row w = p_k;
//   3. Z = sum(w) and running sums C_x in fp64;
//   4. t = u_k * Z and the emitted token is the smallest x with C_x > t;
//   5. out_ids = accepted drafts, the emitted token, then -1; n_accepted = n.
//
// How: one launch, one workgroup per (sequence, vocabulary chunk).  Every workgroup redoes the k gathers of
// step 1 (2k scattered loads, cheaper than a second launch), streams its chunk of the row it
// needs with 16-byte loads, and publishes the chunk's fp64 sum.  An arrival counter per
// sequence elects the last workgroup, which scans the C chunk sums, finds the chunk that
// holds t and rescans only that chunk to pick the token.  The counter returns to 0, so the
// workspace is ready for the next call.  All bytes of the vocabulary are read once, in
// parallel over about 2 x (number of CUs) workgroups.
#include "vap_internal.h"

namespace vap {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ double residual_or_p(float p, float q, bool residual) {
  const double d = residual ? (double)p - (double)q : (double)p;
  return residual ? fmax(0.0, d) : d;
}

__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d);
  return x;
}

// Fixed-order workgroup sum (same tree every time).
__device__ __forceinline__ double block_sum(double x, double* s_red) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  x = wave_sum(x);
  if (lane == 0) s_red[wv] = x;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) t += s_red[i];
  __syncthreads();
  return t;
}

// Exclusive workgroup scan of one double per thread; `total` gets the sum.
__device__ __forceinline__ double block_exclusive_scan(double x, double* s_red, double& total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  double incl = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const double y = __shfl_up(incl, d);
    if (lane >= d) incl += y;
  }
  if (lane == 63) s_red[wv] = incl;
  __syncthreads();
  double before = 0.0;
  total = 0.0;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) {
    if (i < wv) before += s_red[i];
    total += s_red[i];
  }
  __syncthreads();
  return before + incl - x;
}

__device__ __forceinline__ int block_min(int x, int* s_int) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x = min(x, __shfl_xor(x, d));
  if (lane == 0) s_int[wv] = x;
  __syncthreads();
  int t = s_int[0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) t = min(t, s_int[i]);
  __syncthreads();
  return t;
}

__device__ __forceinline__ int block_max(int x, int* s_int) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x = max(x, __shfl_xor(x, d));
  if (lane == 0) s_int[wv] = x;
  __syncthreads();
  int t = s_int[0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) t = max(t, s_int[i]);
  __syncthreads();
  return t;
}

// Sum of w over [x0, x1) (at most kMaxChunkLen elements).  Thread-strided 16-byte loads, all
// issued before the first is used (one memory round trip for the whole chunk); loads past
// the chunk read a clamped in-bounds address and are discarded.
constexpr int kMaxChunkLen = 4096;

template <bool VEC4>
__device__ __forceinline__ double chunk_partial(const float* prow, const float* qrow, bool residual,
                                                int x0, int x1) {
  double acc = 0.0;
  if (VEC4) {
    constexpr int kIt = kMaxChunkLen / (4 * kThreads);
    float4 pv[kIt], qv[kIt];
#pragma unroll
    for (int i = 0; i < kIt; ++i) {
      const int x = min(x0 + 4 * ((int)threadIdx.x + i * kThreads), x1 - 4);
      pv[i] = *reinterpret_cast<const float4*>(prow + x);
      qv[i] = residual ? *reinterpret_cast<const float4*>(qrow + x) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int i = 0; i < kIt; ++i) {
      if (x0 + 4 * ((int)threadIdx.x + i * kThreads) < x1)
        acc += residual_or_p(pv[i].x, qv[i].x, residual) + residual_or_p(pv[i].y, qv[i].y, residual) +
               residual_or_p(pv[i].z, qv[i].z, residual) + residual_or_p(pv[i].w, qv[i].w, residual);
    }
  } else {
    constexpr int kIt = kMaxChunkLen / kThreads;
    float pv[kIt], qv[kIt];
#pragma unroll
    for (int i = 0; i < kIt; ++i) {
      const int x = min(x0 + (int)threadIdx.x + i * kThreads, x1 - 1);
      pv[i] = prow[x];
      qv[i] = residual ? qrow[x] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < kIt; ++i)
      if (x0 + (int)threadIdx.x + i * kThreads < x1) acc += residual_or_p(pv[i], qv[i], residual);
  }
  return acc;
}

// Smallest x in chunk [x0, x1) whose running sum base + C exceeds t (INT_MAX if none), with
// the running sum taken in ascending token id; also the largest x with w_x > 0 (-1 if none).
// Each thread takes a contiguous slice of at most kSlice elements held in registers (chunks
// are at most kThreads * kSlice long), so the scan never goes back to memory.
constexpr int kSlice = 16;

template <bool VEC4>
__device__ __forceinline__ void chunk_select(const float* prow, const float* qrow, bool residual,
                                             int x0, int x1, double base, double t,
                                             double* s_red, int* s_int, int& first_above,
                                             int& last_positive) {
  const int len = x1 - x0;
  const int per = ((len + kThreads - 1) / kThreads + 3) & ~3;   // multiple of 4, <= kSlice
  const int a = x0 + min(len, (int)threadIdx.x * per);
  const int b = x0 + min(len, (int)threadIdx.x * per + per);
  // every load is issued up front at a clamped in-bounds address; elements past the slice
  // are masked below (a + j < b)
  float pv[kSlice], qv[kSlice];
#pragma unroll
  for (int j = 0; j < kSlice; j += 4) {
    if (VEC4) {   // chunk and slice lengths are multiples of 4
      const int x = min(a + j, x1 - 4);
      const float4 u = *reinterpret_cast<const float4*>(prow + x);
      const float4 y = residual ? *reinterpret_cast<const float4*>(qrow + x) : make_float4(0.f, 0.f, 0.f, 0.f);
      pv[j] = u.x; pv[j + 1] = u.y; pv[j + 2] = u.z; pv[j + 3] = u.w;
      qv[j] = y.x; qv[j + 1] = y.y; qv[j + 2] = y.z; qv[j + 3] = y.w;
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int x = min(a + j + u, x1 - 1);
        pv[j + u] = prow[x];
        qv[j + u] = residual ? qrow[x] : 0.f;
      }
    }
  }
  double mine = 0.0;
  int lastpos = -1;
#pragma unroll
  for (int j = 0; j < kSlice; ++j) {
    const double wx = (a + j < b) ? residual_or_p(pv[j], residual ? qv[j] : 0.f, residual) : 0.0;
    mine += wx;
    if (wx > 0.0) lastpos = a + j;
  }
  double total;
  const double before = block_exclusive_scan(mine, s_red, total);
  double run = base + before;
  int found = INT_MAX;
#pragma unroll
  for (int j = 0; j < kSlice; ++j) {
    const double wx = (a + j < b) ? residual_or_p(pv[j], residual ? qv[j] : 0.f, residual) : 0.0;
    run += wx;
    if (found == INT_MAX && a + j < b && run > t) found = a + j;
  }
  first_above = block_min(found, s_int);
  last_positive = block_max(lastpos, s_int);
}

template <bool VEC4>
__global__ __launch_bounds__(kThreads) void spec_verify_kernel(const VerifyParams P) {
  __shared__ int s_n;
  __shared__ int s_last;
  __shared__ int s_ids[64];          // draft ids (accepted ones are copied to the output)
  __shared__ float s_uk;             // u_k, the uniform of the final draw
  __shared__ double s_loc[2];        // base (sum before the chosen chunk), t
  __shared__ int s_cstar;
  __shared__ double s_red[kThreads / 64];
  __shared__ int s_int[kThreads / 64];

  const int C = P.C;
  const int b = blockIdx.x / C;
  const int cidx = blockIdx.x - b * C;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int k = P.k, V = P.V;

  // 1. accept tests (first wave; k <= 64); the second wave fetches u_k meanwhile
  if (tid == 64) s_uk = P.uniforms[(long long)b * (k + 1) + k];
  if (tid < 64) {
    bool reject = false;
    if (lane < k) {
      const int x = P.draft_ids[(long long)b * k + lane];
      const bool inside = x >= 0 && x < V;
      float pv = 0.f, qv = 0.f;
      if (inside) {
        pv = P.p[((long long)b * (k + 1) + lane) * V + x];
        qv = P.q[((long long)b * k + lane) * V + x];
      } else if (cidx == 0) {
        atomicOr(P.err, VAP_DERR_DRAFT_ID);
      }
      const double r = (double)P.uniforms[(long long)b * (k + 1) + lane];
      reject = !(pv > 0.f && r * (double)qv <= (double)pv);
      s_ids[lane] = x;
    }

    const unsigned long long m = __ballot(reject);
    if (lane == 0) s_n = m ? (__ffsll((long long)m) - 1) : k;
  }
  __syncthreads();
  const int n = s_n;
  const bool residual = n < k;
  const float* prow = P.p + ((long long)b * (k + 1) + n) * V;
  const float* qrow = residual ? P.q + ((long long)b * k + n) * V : prow;

  // 2-3. this chunk's sum of w
  const int x0 = cidx * P.CS;
  const int x1 = min(V, x0 + P.CS);
  double part = block_sum(chunk_partial<VEC4>(prow, qrow, residual, x0, x1), s_red);
  if (tid == 0) {
    // publish the chunk sum with an agent-coherent (write-through) store, wait until it has
    // completed, then arrive; the L2-wide writeback/invalidate of an agent-scope fence is not
    // needed because every cross-workgroup value goes through agent-scope accesses
    __hip_atomic_store(reinterpret_cast<unsigned long long*>(P.chunk_sums) + (long long)b * C + cidx,
                       (unsigned long long)__double_as_longlong(part), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    const int ticket = __hip_atomic_fetch_add(P.tickets_end - (b + 1), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (ticket == C - 1);
  }
  __syncthreads();
  if (!s_last) return;

  // 4. last workgroup of sequence b: locate t among the chunk sums (one wave, each lane holds
  // up to four consecutive chunks; C <= 256), then inside one chunk
  if (tid == 0) __hip_atomic_store(P.tickets_end - (b + 1), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  bool use_res = residual;
  const float* srow_q = qrow;
  double Z = 0.0;
  if (tid < 64) {
    double cs[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ci = 4 * lane + j;
      cs[j] = ci < C ? __longlong_as_double((long long)__hip_atomic_load(
                           reinterpret_cast<unsigned long long*>(P.chunk_sums) + (long long)b * C + ci,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
                     : 0.0;
    }
    const double mine = (cs[0] + cs[1]) + (cs[2] + cs[3]);
    double incl = mine;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const double y = __shfl_up(incl, d);
      if (lane >= d) incl += y;
    }
    Z = __shfl(incl, 63);
    if (Z > 0.0) {
      const double t = (double)s_uk * Z;
      // first chunk whose inclusive running sum exceeds t; else (rounding left t at or above
      // the total) the last chunk with a positive sum
      double run = incl - mine;
      int first = INT_MAX, lastnz = -1;
      double base_first = 0.0, base_last = 0.0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ci = 4 * lane + j;
        if (ci < C && first == INT_MAX && run + cs[j] > t) { first = ci; base_first = run; }
        if (ci < C && cs[j] > 0.0) { lastnz = ci; base_last = run; }
        run += cs[j];
      }
      const unsigned long long mf = __ballot(first != INT_MAX);
      const unsigned long long ml = __ballot(lastnz >= 0);
      if (mf) {
        const int src = __ffsll((long long)mf) - 1;
        if (lane == src) { s_cstar = first; s_loc[0] = base_first; s_loc[1] = t; }
      } else {
        const int src = 63 - __clzll((long long)ml);
        if (lane == src) { s_cstar = lastnz; s_loc[0] = base_last; s_loc[1] = t; }
      }
    } else if (lane == 0) {
      s_cstar = -1;
    }
  }
  __syncthreads();
  int token = 0;
  int cstar = s_cstar;
  double base = s_loc[0], t = s_loc[1];
  if (cstar < 0) {
    // empty residual: draw from p_n itself (its chunk sums are computed here)
    use_res = false;
    srow_q = prow;
    double cs = 0.0;
    for (int j = 0; j < C; ++j) {
      const int a = j * P.CS, e = min(V, a + P.CS);
      const double sj = block_sum(chunk_partial<VEC4>(prow, prow, false, a, e), s_red);
      if (tid == j) cs = sj;
    }
    double before = block_exclusive_scan(cs, s_red, Z);
    if (Z > 0.0) {
      t = (double)s_uk * Z;
      const int cand = (tid < C && before + cs > t) ? tid : INT_MAX;
      cstar = block_min(cand, s_int);
      const int lastnz = block_max((tid < C && cs > 0.0) ? tid : -1, s_int);
      if (cstar == INT_MAX) cstar = lastnz;
      if (tid == cstar) s_loc[0] = before;
      __syncthreads();
      base = s_loc[0];
      __syncthreads();
    } else if (tid == 0) {
      atomicOr(P.err, VAP_DERR_EMPTY_ROW);
    }
  }
  if (cstar >= 0) {
    const int a = cstar * P.CS, e = min(V, a + P.CS);
    int first_above, last_positive;
    chunk_select<VEC4>(prow, srow_q, use_res, a, e, base, t, s_red, s_int, first_above, last_positive);
    token = (first_above != INT_MAX) ? first_above : (last_positive >= 0 ? last_positive : 0);
  }

  // 5. outputs
  if (tid <= k) {
    int v;
    if (tid < n) v = s_ids[tid];
    else if (tid == n) v = token;
    else v = -1;
    P.out_ids[(long long)b * (k + 1) + tid] = v;
  }
  if (tid == 0) P.n_accepted[b] = n;
}

}  // namespace

hipError_t launch_spec_verify(const VerifyParams& p, bool vec4, hipStream_t stream, KTimer t) {
  const dim3 grid((unsigned)((long long)p.C * p.B));
  if (vec4) {
    hipExtLaunchKernelGGL(spec_verify_kernel<true>, grid, dim3(kThreads), 0, stream, t.start, t.stop, 0, p);
  } else {
    hipExtLaunchKernelGGL(spec_verify_kernel<false>, grid, dim3(kThreads), 0, stream, t.start, t.stop, 0, p);
  }
  return hipGetLastError();
}

}  // namespace vap
