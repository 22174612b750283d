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
// How.  p_cur is never stored.  After j rejections at node u (all against the same draft row
// q = q[u]) the residual has the closed form
//     p_cur(x) = max(0, p(x) - c_j q(x)) / D_j,   c_0 = 0, D_0 = 1,
//     c_{j+1} = c_j + D_j,   D_{j+1} = sum_x max(0, p(x) - c_{j+1} q(x))
// (induction on max(0, max(0, p - c q) / D - q) = max(0, p - (c + D) q) / D), and a zero sum keeps
// (c, D).  So an accept test needs p(x) and q(x) at the child's own token only: the walker loads
// those two values for every child at the start, and its tests touch no memory.  What remains
// sequential is one vocabulary-wide fp64 sum per rejection that leaves children to test.
//
// S workgroups of 1024 threads walk each sequence together (S = 1 for large batches).  Every
// one of them walks the whole tree from the same preloaded values, so all take the same
// decisions and reach each residual sum at about the same moment; there, each computes its own
// share of the sum's chunks (chunk j goes to workgroup j mod S; chunks are whole float4s, see
// walk_chunks), publishes them in slots of the sequence's record, and reads the others'.  A
// workgroup waits for the others' chunk sums only while they keep arriving (a short, bounded
// wait) and then computes every missing chunk itself, so none depends on another being
// resident.  All compute a chunk with the same code, in the same order, so a sum -- and with it
// the walk -- does not depend on who computed its chunks or on timing.  Workgroup 0 writes the
// results.  The final draw over the unnormalised weights max(0, p - c q) (the inverse CDF is
// scale-invariant) is a second kernel, tree_draw_kernel in spec_verify.hip, which also clears
// the walk's slots.  Values differ from the oracle's step-by-step residuals only by rounding.
#include "vap_internal.h"

namespace vap {
namespace {

constexpr int kThreads = 1024;
constexpr int kMaxNodes = 64;
constexpr int kRound = 2;    // float4 pairs (or 4x that many floats) per chunk and thread in flight
constexpr int kBatch = 4;    // chunks computed together

// Fixed-order workgroup sums of NB doubles per thread: thread k < NB returns the sum of the
// threads' x[k] (other threads return 0).
template <int NB>
__device__ __forceinline__ double block_sums(const double (&x)[NB], double (*s_red)[kThreads / 64]) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    const double v = wave_incl_scan(x[k]);   // lane 63 holds the wave's sum
    if (lane == 63) s_red[k][wv] = v;
  }
  __syncthreads();
  double t = 0.0;
  if (threadIdx.x < NB) {
    for (int i = 0; i < kThreads / 64; ++i) t += s_red[threadIdx.x][i];
  }
  __syncthreads();
  return t;
}

// unnormalised residual weight max(0, p - c q) of one token (c = 0: p itself)
__device__ __forceinline__ double weight(float p, float q, double c) {
  return fmax(0.0, fma(-c, (double)q, (double)p));
}

// This thread's partial sums of max(0, p - c q) over chunks js[0 .. n-1] (n <= NB) of the row
// pair: thread t takes the chunk's float4s t, t + 1024, ... (VEC4) or its elements t, t + 1024,
// ..., and adds them in that order.  Every load of a round is issued before any is used.
template <bool VEC4, int NB>
__device__ void chunk_partials(const float* prow, const float* qrow, double c, const int (&js)[kBatch], int n,
                               WalkChunks wc, int V, double (&acc)[NB]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int k = 0; k < NB; ++k) acc[k] = 0.0;
  if constexpr (VEC4) {
    const int per = wc.CS / 4, V4 = V / 4;
    for (int r = 0; r < per; r += kRound * kThreads) {
      float4 pv[NB][kRound], qv[NB][kRound];
#pragma unroll
      for (int k = 0; k < NB; ++k) {
#pragma unroll
        for (int i = 0; i < kRound; ++i) {
          const int e = min(((k < n) ? js[k] : js[0]) * per + r + i * kThreads + tid, V4 - 1);
          pv[k][i] = reinterpret_cast<const float4*>(prow)[e];
          qv[k][i] = reinterpret_cast<const float4*>(qrow)[e];
        }
      }
#pragma unroll
      for (int k = 0; k < NB; ++k) {
#pragma unroll
        for (int i = 0; i < kRound; ++i) {
          const int off = r + i * kThreads + tid;
          if (k < n && off < per && js[k] * per + off < V4)
            acc[k] += (weight(pv[k][i].x, qv[k][i].x, c) + weight(pv[k][i].y, qv[k][i].y, c)) +
                      (weight(pv[k][i].z, qv[k][i].z, c) + weight(pv[k][i].w, qv[k][i].w, c));
        }
      }
    }
  } else {
    constexpr int kR = 4 * kRound;
    const int per = wc.CS;
    for (int r = 0; r < per; r += kR * kThreads) {
      float pv[NB][kR], qv[NB][kR];
#pragma unroll
      for (int k = 0; k < NB; ++k) {
#pragma unroll
        for (int i = 0; i < kR; ++i) {
          const int e = min(((k < n) ? js[k] : js[0]) * per + r + i * kThreads + tid, V - 1);
          pv[k][i] = prow[e];
          qv[k][i] = qrow[e];
        }
      }
#pragma unroll
      for (int k = 0; k < NB; ++k) {
#pragma unroll
        for (int i = 0; i < kR; ++i) {
          const int off = r + i * kThreads + tid;
          if (k < n && off < per && js[k] * per + off < V) acc[k] += weight(pv[k][i], qv[k][i], c);
        }
      }
    }
  }
}

// Chunk sums of chunks js[0 .. n-1]: thread k < n returns the sum of chunk js[k].  One chunk, or
// two with 16-byte loads (S workgroups sharing 16 chunks: one each at S = 16, two at S = 8), load
// and reduce only their own data; the kBatch form would issue the loads of kBatch chunks and
// kBatch reductions.
template <bool VEC4, int NB>
__device__ __forceinline__ double chunk_sums_n(const float* prow, const float* qrow, double c, const int (&js)[kBatch],
                                               int n, WalkChunks wc, int V, double (*s_red)[kThreads / 64]) {
  double part[NB];
  chunk_partials<VEC4, NB>(prow, qrow, c, js, n, wc, V, part);
  return block_sums<NB>(part, s_red);
}

template <bool VEC4>
__device__ __forceinline__ double chunk_sums(const float* prow, const float* qrow, double c, const int (&js)[kBatch],
                                             int n, WalkChunks wc, int V, double (*s_red)[kThreads / 64]) {
  if (n == 1) return chunk_sums_n<VEC4, 1>(prow, qrow, c, js, n, wc, V, s_red);
  if (VEC4 && n == 2) return chunk_sums_n<VEC4, 2>(prow, qrow, c, js, n, wc, V, s_red);   // (scalar loads: spills)
  return chunk_sums_n<VEC4, kBatch>(prow, qrow, c, js, n, wc, V, s_red);
}

__device__ __forceinline__ unsigned long long* walk_sum(const TreeVerifyParams& P, int b, int pass, int j) {
  return P.rec.at<unsigned long long>(b, kTreeRecWalk) + pass * kWalkChunks + j;
}

__device__ __forceinline__ unsigned long long now_ticks() { return __builtin_amdgcn_s_memrealtime(); }

template <bool VEC4>
__global__ __launch_bounds__(kThreads) void tree_verify_kernel(const TreeVerifyParams P) {
  __shared__ int s_par[kMaxNodes];
  __shared__ int s_tok[kMaxNodes];
  __shared__ float s_u[kMaxNodes];
  __shared__ float s_px[kMaxNodes];    // p[parent](token) of each child
  __shared__ float s_qx[kMaxNodes];    // q[parent](token) of each child
  __shared__ double s_red[kBatch][kThreads / 64];
  __shared__ double s_cs[kWalkChunks];
  __shared__ unsigned s_have;
  __shared__ int s_flag;
  __shared__ int s_ids[kMaxNodes];     // accepted tokens and nodes
  __shared__ int s_path[kMaxNodes];

  const int S = P.S;
  const int L = seq_major_index();       // a sequence's S workgroups on one XCD
  const int b = L / S;
  const int role = L - b * S;            // 0 writes the results
  const int tid = threadIdx.x;
  const int N = P.N, V = P.V;
  const long long row0 = (long long)b * N;
  const WalkChunks wc = walk_chunks(V);
  if (tid < N) {
    int par = P.parents[row0 + tid];
    const bool ok = (tid == 0) ? (par == -1) : (par >= 0 && par < tid);
    if (!ok) {
      if (role == 0) atomicOr(P.err, VAP_DERR_TREE);
      par = (tid == 0) ? -1 : -2;          // an invalid node is never anyone's child
    }
    s_par[tid] = par;
    s_tok[tid] = P.tokens[row0 + tid];
    s_u[tid] = P.uniforms[row0 + tid];
  }
  __syncthreads();
  // every child's p and q at its own token (the accept tests need nothing else)
  if (tid > 0 && tid < N) {
    const int par = s_par[tid], x = s_tok[tid];
    float px = 0.f, qx = 0.f;
    if (par >= 0 && x >= 0 && x < V) {
      px = P.p[(row0 + par) * (long long)V + x];
      qx = P.q[(row0 + par) * (long long)V + x];
    }
    s_px[tid] = px;
    s_qx[tid] = qx;
  }
  __syncthreads();

  // D = sum_x max(0, p - cn q) of node u.  The first kWalkPasses sums of a walk are shared:
  // this workgroup computes and publishes chunks j = role, role + S, ..., then gathers the
  // others' while they keep arriving; every chunk still missing it computes itself.
  int npass = 0;
  auto residual_sum = [&](int u, double cn) -> double {
    const float* prow = P.p + (row0 + u) * (long long)V;
    const float* qrow = P.q + (row0 + u) * (long long)V;
    const unsigned full = (wc.C >= 32) ? ~0u : ((1u << wc.C) - 1u);
    const int pass = (S > 1 && npass < kWalkPasses) ? npass++ : -1;
    unsigned mine = 0u;
    if (pass >= 0)
      for (int j = role; j < wc.C; j += S) mine |= 1u << j;
    // chunks of `todo`, kBatch at a time; published when shared
    auto compute = [&](unsigned todo, bool publish) {
      while (todo != 0u) {               // (uniform: every thread holds the same mask)
        int js[kBatch];
        int n = 0;
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
          js[k] = todo ? __ffs((int)todo) - 1 : js[0];
          n += todo ? 1 : 0;
          todo &= todo - 1u;
        }
        const double v = chunk_sums<VEC4>(prow, qrow, cn, js, n, wc, V, s_red);
        if (tid < n) {
          int jj = js[0];
#pragma unroll
          for (int k = 1; k < kBatch; ++k) jj = (tid == k) ? js[k] : jj;
          s_cs[jj] = v;
          if (publish) publish_slot(walk_sum(P, b, pass, jj), v);
        }
      }
    };
    compute(mine, true);
    if (tid == 0) s_have = mine;
    __syncthreads();
    if (pass >= 0 && (s_have != full)) {
      unsigned long long t_last = now_ticks();
      unsigned have_prev = mine;
      while (true) {
        if (tid < wc.C && !((s_have >> tid) & 1u)) {
          const unsigned long long x =
              __hip_atomic_load(walk_sum(P, b, pass, tid), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (x != 0ull) {
            s_cs[tid] = __longlong_as_double((long long)~x);
            atomicOr(&s_have, 1u << tid);
          }
        }
        __syncthreads();
        if (tid == 0) {
          const unsigned have = s_have;
          const unsigned long long t = now_ticks();
          if (have != have_prev) t_last = t;
          have_prev = have;
          s_flag = (have == full || t - t_last > (unsigned long long)P.wait_ticks) ? 1 : 0;
        }
        __syncthreads();
        if (s_flag) break;
        __builtin_amdgcn_s_sleep(2);
      }
    }
    compute(full & ~s_have, false);
    __syncthreads();
    double D = 0.0;
    for (int j = 0; j < wc.C; ++j) D += s_cs[j];
    __syncthreads();
    return D;
  };

  double cc = 0.0, DD = 1.0;     // (c, D) of the current node
  int u = 0, n = 0, last = 0;
  double c_end = -1.0, c_end_prev = 0.0;
  while (true) {
    // next untested child of u (children have larger indices than their parent)
    if (tid < 64) {
      const unsigned long long m = __ballot(tid < N && tid > last && s_par[tid] == u);
      if (tid == 0) s_flag = m ? (__ffsll((long long)m) - 1) : -1;
    }
    __syncthreads();
    const int c = s_flag;
    __syncthreads();
    if (c < 0) {
      c_end = cc;
      c_end_prev = cc;
      break;
    }
    const int x = s_tok[c];
    const bool inside = x >= 0 && x < V;
    if (!inside && tid == 0 && role == 0) atomicOr(P.err, VAP_DERR_DRAFT_ID);
    const double qx = inside ? (double)s_qx[c] : 0.0;
    const double px = inside ? weight(s_px[c], s_qx[c], cc) / DD : 0.0;
    if (px > 0.0 && (double)s_u[c] * qx <= px) {    // accepted (every thread takes the same decision)
      if (tid == 0) {
        s_ids[n] = x;
        s_path[n] = c;
      }
      ++n;
      u = c;
      last = c;
      cc = 0.0;
      DD = 1.0;
      continue;
    }
    // rejection: the next residual, c' = c + D and D' = sum_x max(0, p - c' q).  When u has no
    // child left to test, D' is not needed: the walk ends here and the draw kernel takes the
    // weights max(0, p - c' q), falling back to max(0, p - c q) if they are all zero (the zero
    // sum that keeps (c, D) in the walk).
    const double cn = cc + DD;
    if (tid < 64) {
      const unsigned long long more = __ballot(tid < N && tid > c && s_par[tid] == u);
      if (tid == 0) s_flag = more ? 1 : 0;
    }
    __syncthreads();
    const bool more = s_flag != 0;
    __syncthreads();
    if (!more) {
      c_end = cn;
      c_end_prev = cc;
      break;
    }
    const double D = residual_sum(u, cn);
    if (D > 0.0) {
      cc = cn;
      DD = D;
    }
    last = c;
  }
  if (role != 0) return;
  // the walk ends at node u after n acceptances: the final draw (tree_draw_kernel, spread over
  // the GPU) takes max(0, p - c q) of u with this c, and writes its token at out_ids[n]
  __syncthreads();
  if (tid < N) {
    P.out_ids[row0 + tid] = tid < n ? s_ids[tid] : -1;
    P.out_path[row0 + tid] = tid < n ? s_path[tid] : -1;
  }
  if (tid == 0) {
    *P.rec.at<TreeDraw>(b, kTreeRecDraw) = TreeDraw{c_end, c_end_prev, u, n, S > 1 ? npass : 0, 0};
    P.n_accepted[b] = n;
  }
}

}  // namespace

hipError_t launch_tree_verify(const TreeVerifyParams& p, hipStream_t stream, KTimer t) {
  const dim3 grid((unsigned)((long long)p.B * p.S));
  if (p.vec4)
    hipExtLaunchKernelGGL(tree_verify_kernel<true>, grid, dim3(kThreads), 0, stream, t.start, t.stop, 0, p);
  else
    hipExtLaunchKernelGGL(tree_verify_kernel<false>, grid, dim3(kThreads), 0, stream, t.start, t.stop, 0, p);
  return hipGetLastError();
}

}  // namespace vap
