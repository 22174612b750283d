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
// How: one workgroup of 1024 threads per sequence (the walk is sequential, every rejection needs
// a vocabulary-wide fp64 sum).  p_cur is never stored.  After j rejections at node u (all
// against the same draft row q = q[u]) the residual has the closed form
//     p_cur(x) = max(0, p(x) - c_j q(x)) / D_j,   c_0 = 0, D_0 = 1,
//     c_{j+1} = c_j + D_j,   D_{j+1} = sum_x max(0, p(x) - c_{j+1} q(x))
// (induction on max(0, max(0, p - c q) / D - q) = max(0, p - (c + D) q) / D), and a zero sum keeps
// (c, D).  So the accept test evaluates p_cur at one token on one thread, each rejection costs
// one streaming fp64 pass over the two rows, and the final draw scans the unnormalised weights
// max(0, p - c q) (the inverse CDF is scale-invariant).  Values differ from the oracle's
// step-by-step residuals only by rounding.
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

// Exclusive workgroup scan of one double per thread; `total` receives the sum.
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
  __shared__ int s_found;
  __shared__ int s_slice;
  __shared__ double s_base;
  __shared__ double s_chunk[kThreads];

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
  int u = 0, n = 0, last = 0;
  while (true) {
    // next untested child of u (children have larger indices than their parent)
    if (tid < 64) {
      const bool is_kid = tid < N && tid > last && s_par[tid] == u;
      const unsigned long long m = __ballot(is_kid);
      if (tid == 0) s_next = m ? (__ffsll((long long)m) - 1) : -1;
    }
    __syncthreads();
    const int c = s_next;
    if (c < 0) break;
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
    // rejection: the next residual, c' = c + D and D' = sum_x max(0, p - c' q)
    const double cn = s_cd[0] + s_cd[1];
    double part = 0.0;
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
            part += (weight(pv[i].x, qv[i].x, cn) + weight(pv[i].y, qv[i].y, cn)) +
                    (weight(pv[i].z, qv[i].z, cn) + weight(pv[i].w, qv[i].w, cn));
          }
        }
      }
    } else {
      for (int x = tid; x < V; x += kThreads) part += weight(prow[x], qrow[x], cn);
    }
    const double S = block_sum(part, s_red);
    if (tid == 0 && S > 0.0) {
      s_cd[0] = cn;
      s_cd[1] = S;
    }
    last = c;
    __syncthreads();
  }
  const double cf = s_cd[0];

  // final draw from the weights max(0, p - cf q) of node u, in ascending token id.
  // Level 1: the vocabulary is cut into chunks of CH = 1024 m tokens (at most 1024 chunks); a
  // wave sums a chunk with coalesced 16-byte loads (two chunks in flight), a block scan places
  // the chunks.  Level 2: one wave walks the chunk holding t, 256 tokens (a float4 per lane)
  // at a time in ascending order, with a running carry.
  const float* prow = P.p + (row0 + u) * (long long)V;
  const float* qrow = P.q + (row0 + u) * (long long)V;
  const int m = (V + kThreads * kThreads - 1) / (kThreads * kThreads);
  const int CH = kThreads * m;
  const int nch = (V + CH - 1) / CH;
  const int lane = tid & 63, wv = tid >> 6;
  // weights of the 4 tokens at x .. x+3 (0 past the end); scalar loads when rows are not
  // 16-byte aligned or V is not a multiple of 4
  auto weights4 = [&](int x, double (&w)[4]) {
    if (P.vec4 && x + 3 < V) {
      const float4 pv = *reinterpret_cast<const float4*>(prow + x);
      const float4 qv = *reinterpret_cast<const float4*>(qrow + x);
      w[0] = weight(pv.x, qv.x, cf); w[1] = weight(pv.y, qv.y, cf);
      w[2] = weight(pv.z, qv.z, cf); w[3] = weight(pv.w, qv.w, cf);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int xe = min(x + e, V - 1);
        const float pe = prow[xe], qe = qrow[xe];
        w[e] = (x + e < V) ? weight(pe, qe, cf) : 0.0;
      }
    }
  };
  double lastw_pos = -1.0;
  for (int k0 = wv; k0 < nch; k0 += 2 * (kThreads / 64)) {
    double acc[2] = {0.0, 0.0};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = k0 + h * (kThreads / 64);
      if (k < nch) {
        for (int i = 0; i < CH / 256; ++i) {
          const int x = k * CH + 256 * i + 4 * lane;
          if (x < V) {
            double w[4];
            weights4(x, w);
            acc[h] += (w[0] + w[1]) + (w[2] + w[3]);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (w[e] > 0.0) lastw_pos = fmax(lastw_pos, (double)(x + e));
          }
        }
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = k0 + h * (kThreads / 64);
      const double cs = wave_sum(acc[h]);
      if (k < nch && lane == 0) s_chunk[k] = cs;
    }
  }
  __syncthreads();
  const double cs = tid < nch ? s_chunk[tid] : 0.0;
  double Zf;
  const double before = block_exclusive_scan(cs, s_red, Zf);
  if (tid == 0) {
    s_found = INT_MAX;
    s_slice = INT_MAX;
  }
  __syncthreads();
  int token = 0;
  if (Zf > 0.0) {
    const double t = (double)s_u[0] * Zf;
    // the chunk holding t (rounding can let two neighbours claim it: the first one wins)
    if (tid < nch && before <= t && before + cs > t) atomicMin(&s_slice, tid);
    __syncthreads();
    if (tid == s_slice) s_base = before;
    __syncthreads();
    const int T = s_slice == INT_MAX ? -1 : s_slice;
    if (T >= 0 && tid < 64) {
      double carry = s_base;
      for (int i = 0; i < CH / 256; ++i) {
        const int x = T * CH + 256 * i + 4 * lane;
        double w[4] = {0.0, 0.0, 0.0, 0.0};
        if (x < V) weights4(x, w);
        const double l0 = w[0], l1 = l0 + w[1], l2 = l1 + w[2], l3 = l2 + w[3];
        double incl = l3;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const double y = __shfl_up(incl, d);
          if (lane >= d) incl += y;
        }
        const double pre = carry + incl - l3;        // running sum before this lane's 4 tokens
        int hit = INT_MAX;
        if (pre + l0 > t) hit = x;
        else if (pre + l1 > t) hit = x + 1;
        else if (pre + l2 > t) hit = x + 2;
        else if (pre + l3 > t) hit = x + 3;
        if (hit >= V) hit = INT_MAX;
        const unsigned long long mk = __ballot(hit != INT_MAX);
        if (mk) {
          const int src = __ffsll((long long)mk) - 1;
          const int h = __shfl(hit, src);
          if (lane == 0) s_found = h;
          break;
        }
        carry += __shfl(incl, 63);
      }
    }
    __syncthreads();
    token = s_found;
    if (token == INT_MAX) {                 // rounding left t at or past the total
      if (tid == 0) s_found = -1;
      __syncthreads();
      if (lastw_pos >= 0.0) atomicMax(&s_found, (int)lastw_pos);
      __syncthreads();
      token = max(s_found, 0);
    }
  } else if (tid == 0) {
    atomicOr(P.err, VAP_DERR_EMPTY_ROW);
  }

  if (tid < N) {
    int id = -1, node = -1;
    if (tid < n) {
      id = s_ids[tid];
      node = s_path[tid];
    } else if (tid == n) {
      id = token;
    }
    P.out_ids[row0 + tid] = id;
    P.out_path[row0 + tid] = node;
  }
  if (tid == 0) P.n_accepted[b] = n;
}

}  // namespace

hipError_t launch_tree_verify(const TreeVerifyParams& p, hipStream_t stream, KTimer t) {
  hipExtLaunchKernelGGL(tree_verify_kernel, dim3((unsigned)p.B), dim3(kThreads), 0, stream, t.start, t.stop, 0, p);
  return hipGetLastError();
}

}  // namespace vap
