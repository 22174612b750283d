// Verification of a draft token tree (gfx950).
//
// What is computed, per sequence: the chain rule of modified rejection sampling
// (neuralmasteryai.com "Continuous Batching & Speculative Decoding", section "The Modified
// Rejection Sampling Algorithm") walked over a draft token tree (same page, section "4. Tree
// Attention & Medusa Heads"):
//   * start at the root (node 0) with the current target distribution p_cur = p[0];
//   * test the current node u's children in index order: child c with token x passes when
//     p_cur(x) > 0 and r_c * q[u](x) <= p_cur(x) (fp64); after each rejection p_cur becomes
//     max(0, p_cur - q[u]) / Z (unchanged when Z = 0);
//   * the first child that passes is accepted (its token emitted) and the walk continues under
//     it with p_cur = p[child];
//   * when no child is left, one token is drawn from p_cur: t = u_0 * sum(p_cur), the smallest x
//     whose running sum exceeds t.
//
// How: S workgroups of 1024 threads per sequence walk it in lockstep (the walk is sequential,
// every rejection needs a vocabulary-wide fp64 sum).  Each takes 1/S of the vocabulary in a
// residual pass; the S partial sums are exchanged through the workspace (write-through stores,
// an arrival counter, a bounded wait) and added in part order, so every part holds the same sum
// and takes the same decisions.  S is chosen on the host so that all B*S workgroups fit on the
// GPU at once (at most one per CU).  p_cur is never stored.  After j rejections at node u (all
// against the same draft row q = q[u]) the residual has the closed form
//     p_cur(x) = max(0, p(x) - c_j q(x)) / D_j,   c_0 = 0, D_0 = 1,
//     c_{j+1} = c_j + D_j,   D_{j+1} = sum_x max(0, p(x) - c_{j+1} q(x))
// (induction on max(0, max(0, p - c q) / D - q) = max(0, p - (c + D) q) / D), and a zero sum keeps
// (c, D).  So the accept test evaluates p_cur at one token on one thread and each rejection costs
// one streaming fp64 pass over the two rows.  The walk ends by recording (node, c, n); the final
// draw over the unnormalised weights max(0, p - c q) (the inverse CDF is scale-invariant) is a
// second kernel, tree_draw_kernel in spec_verify.hip, spread over about two workgroups per CU
// like spec_verify's draw.  Values differ from the oracle's step-by-step residuals only by
// rounding.
#include "vap_internal.h"

namespace vap {
namespace {

constexpr int kThreads = 1024;
constexpr int kMaxNodes = 64;
constexpr int kIt = 8;     // float4 pairs per thread in flight per round of a residual pass
static_assert(4 * kIt * kThreads == kTreeRoundTokens, "the host sizes walk parts by this round");

__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d);
  return x;
}

// Fixed-order workgroup sum of one double per thread.
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

// unnormalised residual weight max(0, p - c q) of one token (c = 0: p itself)
__device__ __forceinline__ double weight(float p, float q, double c) {
  return fmax(0.0, fma(-c, (double)q, (double)p));
}

// Wait bound of the exchange between the parts of a sequence: about a quarter of a second.  The
// parts are all resident (the host sizes the grid for that), so the bound is only reached if
// something else holds the CUs; the sum is then incomplete, VAP_DERR_SYNC is set and the part
// stops waiting for the rest of its walk (so such a call still ends quickly).
constexpr int kSpinMax = 1 << 18;

// Sum of the S parts' partial sums of pass r of sequence b (every part calls this with its own
// partial).  Slots alternate between two banks by pass parity: a part can be at most one pass
// ahead of another, so a bank is never rewritten before every part has read it.
__device__ __forceinline__ double exchange_sum(const TreeVerifyParams& P, int b, int part, int r, double partial,
                                               double* s_val, int* s_timeout) {
  const int S = P.S;
  unsigned long long* slots = reinterpret_cast<unsigned long long*>(P.xch) + (long long)b * P.xch_stride + (r & 1) * S;
  int32_t* cnt = P.tickets_end - (b + 1);   // the sequence's ticket, zero at the start of the call
  if (threadIdx.x == 0) {
    __hip_atomic_store(slots + part, (unsigned long long)__double_as_longlong(partial), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);        // the slot is written before this part arrives
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int target = S * (r + 1);
    int it = 0;
    if (!*s_timeout) {
      while (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target && ++it < kSpinMax)
        __builtin_amdgcn_s_sleep(2);
    }
    if (it >= kSpinMax) {
      atomicOr(P.err, VAP_DERR_SYNC);
      *s_timeout = 1;
    }
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const double v = lane < S ? __longlong_as_double((long long)__hip_atomic_load(slots + lane, __ATOMIC_RELAXED,
                                                                                    __HIP_MEMORY_SCOPE_AGENT))
                              : 0.0;
    double t = 0.0;
    for (int j = 0; j < S; ++j) t += __shfl(v, j);   // part order, the same in every part
    if (lane == 0) *s_val = t;
  }
  __syncthreads();
  return *s_val;
}

__global__ __launch_bounds__(kThreads) void tree_verify_kernel(const TreeVerifyParams P) {
  __shared__ int s_par[kMaxNodes];
  __shared__ int s_tok[kMaxNodes];
  __shared__ float s_u[kMaxNodes];
  __shared__ double s_cd[2];           // (c, D) of the current node
  __shared__ double s_red[kThreads / 64];
  __shared__ int s_next;
  __shared__ int s_accept;
  __shared__ int s_ids[kMaxNodes];
  __shared__ int s_path[kMaxNodes];
  __shared__ double s_sum;
  __shared__ int s_timeout;

  const int S = P.S;
  const int b = blockIdx.x / S;
  const int part = blockIdx.x - b * S;  // this workgroup's share of every residual pass
  const int tid = threadIdx.x;
  int r = 0;                            // residual passes taken so far (the same in every part)
  const int N = P.N, V = P.V;
  const long long row0 = (long long)b * N;
  if (tid < N) {
    int par = P.parents[row0 + tid];
    const bool ok = (tid == 0) ? (par == -1) : (par >= 0 && par < tid);
    if (!ok) {
      atomicOr(P.err, VAP_DERR_TREE);
      par = (tid == 0) ? -1 : -2;          // an invalid node is never anyone's child
    }
    s_par[tid] = par;
    s_tok[tid] = P.tokens[row0 + tid];
    s_u[tid] = P.uniforms[row0 + tid];
  }
  __syncthreads();

  if (tid == 0) {
    s_cd[0] = 0.0;
    s_cd[1] = 1.0;
    s_timeout = 0;
  }
  __syncthreads();
  int u = 0, n = 0, last = 0;
  double c_end = -1.0, c_end_prev = 0.0;   // set when the walk ends in a rejection
  while (true) {
    // next untested child of u (children have larger indices than their parent)
    if (tid < 64) {
      const bool is_kid = tid < N && tid > last && s_par[tid] == u;
      const unsigned long long m = __ballot(is_kid);
      if (tid == 0) s_next = m ? (__ffsll((long long)m) - 1) : -1;
    }
    __syncthreads();
    const int c = s_next;
    if (c < 0) {
      c_end = s_cd[0];
      c_end_prev = s_cd[0];
      break;
    }
    const float* prow = P.p + (row0 + u) * (long long)V;
    const float* qrow = P.q + (row0 + u) * (long long)V;
    if (tid == 0) {
      const int x = s_tok[c];
      const bool inside = x >= 0 && x < V;
      if (!inside) atomicOr(P.err, VAP_DERR_DRAFT_ID);
      const float qf = inside ? qrow[x] : 0.f;
      const double qx = qf;
      const double px = inside ? weight(prow[x], qf, s_cd[0]) / s_cd[1] : 0.0;
      s_accept = (px > 0.0 && (double)s_u[c] * qx <= px) ? 1 : 0;
    }
    __syncthreads();
    if (s_accept) {
      if (tid == 0) {
        s_ids[n] = s_tok[c];
        s_path[n] = c;
      }
      if (tid == 0) {
        s_cd[0] = 0.0;
        s_cd[1] = 1.0;
      }
      ++n;
      u = c;
      last = c;
      __syncthreads();
      continue;
    }
    // rejection: the next residual, c' = c + D and D' = sum_x max(0, p - c' q).  When u has no
    // child left to test, D' is not needed: the walk ends here and the draw kernel takes the
    // weights max(0, p - c' q), falling back to max(0, p - c q) if they are all zero (the zero
    // sum that keeps (c, D) in the walk).
    const double cn = s_cd[0] + s_cd[1];
    if (tid < 64) {
      const unsigned long long more = __ballot(tid < N && tid > c && s_par[tid] == u);
      if (tid == 0) s_next = more ? 1 : 0;
    }
    __syncthreads();
    if (!s_next) {
      c_end = cn;
      c_end_prev = s_cd[0];
      break;
    }
    double acc = 0.0;
    const bool vec4 = P.vec4;
    if (vec4) {
      const int V4 = V >> 2;
      const int e0 = (int)((long long)V4 * part / S), e1 = (int)((long long)V4 * (part + 1) / S);
      for (int base = e0; base < e1; base += kIt * kThreads) {
        float4 pv[kIt], qv[kIt];
#pragma unroll
        for (int i = 0; i < kIt; ++i) {
          const int e = min(base + i * kThreads + tid, V4 - 1);
          pv[i] = reinterpret_cast<const float4*>(prow)[e];
          qv[i] = reinterpret_cast<const float4*>(qrow)[e];
        }
#pragma unroll
        for (int i = 0; i < kIt; ++i) {
          if (base + i * kThreads + tid < e1) {
            acc += (weight(pv[i].x, qv[i].x, cn) + weight(pv[i].y, qv[i].y, cn)) +
                   (weight(pv[i].z, qv[i].z, cn) + weight(pv[i].w, qv[i].w, cn));
          }
        }
      }
    } else {
      const int x0 = (int)((long long)V * part / S), x1 = (int)((long long)V * (part + 1) / S);
      for (int x = x0 + tid; x < x1; x += kThreads) acc += weight(prow[x], qrow[x], cn);
    }
    double D = block_sum(acc, s_red);
    if (S > 1) D = exchange_sum(P, b, part, r, D, &s_sum, &s_timeout);
    ++r;
    if (tid == 0 && D > 0.0) {
      s_cd[0] = cn;
      s_cd[1] = D;
    }
    last = c;
    __syncthreads();
  }
  // the walk ends at node u after n acceptances: the final draw (tree_draw_kernel, spread over
  // the GPU) takes max(0, p - c q) of u with this c, and writes its token at out_ids[n]
  if (part != 0) return;
  if (tid < N) {
    P.out_ids[row0 + tid] = tid < n ? s_ids[tid] : -1;
    P.out_path[row0 + tid] = tid < n ? s_path[tid] : -1;
  }
  if (tid == 0) {
    // the draw kernel's chunks arrive on the same ticket after the parts' S * r arrivals
    P.draws[b] = TreeDraw{c_end, c_end_prev, u, n, S > 1 ? S * r : 0, 0};
    P.n_accepted[b] = n;
  }
}

}  // namespace

hipError_t launch_tree_verify(const TreeVerifyParams& p, hipStream_t stream, KTimer t) {
  hipExtLaunchKernelGGL(tree_verify_kernel, dim3((unsigned)(p.B * p.S)), dim3(kThreads), 0, stream, t.start, t.stop, 0,
                        p);
  return hipGetLastError();
}

}  // namespace vap
