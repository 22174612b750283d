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
// How: one workgroup of 1024 threads walks each sequence (the walk is sequential, and every
// rejection with children left to test needs a vocabulary-wide fp64 sum, which the workgroup
// streams itself: no workgroup ever waits for another).  p_cur is never stored.  After j
// rejections at node u (all against the same draft row q = q[u]) the residual has the closed
// form
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

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
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
      for (int base = 0; base < V4; base += kIt * kThreads) {
        float4 pv[kIt], qv[kIt];
#pragma unroll
        for (int i = 0; i < kIt; ++i) {
          const int e = min(base + i * kThreads + tid, V4 - 1);
          pv[i] = reinterpret_cast<const float4*>(prow)[e];
          qv[i] = reinterpret_cast<const float4*>(qrow)[e];
        }
#pragma unroll
        for (int i = 0; i < kIt; ++i) {
          if (base + i * kThreads + tid < V4) {
            acc += (weight(pv[i].x, qv[i].x, cn) + weight(pv[i].y, qv[i].y, cn)) +
                   (weight(pv[i].z, qv[i].z, cn) + weight(pv[i].w, qv[i].w, cn));
          }
        }
      }
    } else {
      for (int x = tid; x < V; x += kThreads) acc += weight(prow[x], qrow[x], cn);
    }
    const double D = block_sum(acc, s_red);
    if (tid == 0 && D > 0.0) {
      s_cd[0] = cn;
      s_cd[1] = D;
    }
    last = c;
    __syncthreads();
  }
  // the walk ends at node u after n acceptances: the final draw (tree_draw_kernel, spread over
  // the GPU) takes max(0, p - c q) of u with this c, and writes its token at out_ids[n]
  if (tid < N) {
    P.out_ids[row0 + tid] = tid < n ? s_ids[tid] : -1;
    P.out_path[row0 + tid] = tid < n ? s_path[tid] : -1;
  }
  if (tid == 0) {
    *P.rec.at<TreeDraw>(b, kTreeRecDraw) = TreeDraw{c_end, c_end_prev, u, n};
    P.n_accepted[b] = n;
  }
}

}  // namespace

hipError_t launch_tree_verify(const TreeVerifyParams& p, hipStream_t stream, KTimer t) {
  hipExtLaunchKernelGGL(tree_verify_kernel, dim3((unsigned)p.B), dim3(kThreads), 0, stream, t.start, t.stop, 0, p);
  return hipGetLastError();
}

}  // namespace vap
