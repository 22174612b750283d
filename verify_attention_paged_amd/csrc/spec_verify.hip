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
// How: one launch.  The vocabulary is cut into C chunks of at most 1024 tokens where the
// vocabulary allows (up to 4096 above 256 * 1024 tokens; about eight chunks per CU over the
// batch), and each sequence gets WPS workgroups that take consecutive chunks, one wave per chunk
// (four chunks per workgroup for small batches; for large batches a wave streams many chunks, so
// the accept tests are not paid per chunk).  Every workgroup redoes the k gathers of step 1 (2k
// scattered loads, cheaper than a second launch); each wave streams its chunks of the row it
// needs with 16-byte loads and publishes each chunk's fp64 sum.  An arrival counter per sequence
// elects the last workgroup, which scans the C chunk sums, finds the chunk that holds t and
// rescans only that chunk to pick the token.  The counter and the published sums return to 0, so
// the workspace is ready for the next call.  All bytes of the vocabulary are read once.
//
// Verification from logits (tempatgunting.com article, section "Speculative Decoding: Turning
// Verification Parallelism into Latency Wins": the verify pass yields logits and tokens are
// sampled from logits): p_i = softmax(z_p,i / T), q_i = softmax(z_q,i / T) for a temperature
// T > 0, then the same rule; at T = 0 (same page, section "Frequently Asked Questions": exact
// token matching) a draft passes when it is its target row's first argmax and the emitted token
// is the argmax of row n.  A statistics kernel of persistent waves reduces every 2048-token
// chunk of every logit row to (max, first argmax, S = sum 2^((z - max) log2(e) / T)), loading
// its next chunk while it computes the current one; each verification workgroup then merges
// the chunks of its own sequence's rows in LDS (M = max m_c, S = sum S_c 2^((m_c - M) log2(e) / T),
// in chunk order, so every workgroup of a sequence gets the same values) and evaluates
// p(x) = 2^((z_x - M) log2(e) / T) / S wherever the rule needs a probability.  No probability
// row is written.  The exponentials are taken in fp64 (exp2_f64, exp2_64th), which keeps every
// decision within rounding of the fp64 oracle.
#include <cfloat>
#include <type_traits>
#include <utility>

#include "vap_internal.h"

namespace vap {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ double residual_or_p(float p, float q, bool residual) {
  const double d = residual ? (double)p - (double)q : (double)p;
  return residual ? fmax(0.0, d) : d;
}

// 2^(b / 64) in fp64 for b <= 0 (arguments below -69120 = 64 * -1080, and NaN, give 0):
// b = n + r with n = rint(b) and |r| <= 1/2; 2^(n/64) = 2^(n >> 6) * 2^((n & 63)/64), the second
// factor from a 64-entry table (tab, filled by fill_exp2_table), and 2^(r/64) = e^(r ln 2 / 64)
// from its Taylor series through r^3 (coefficients (ln 2 / 64)^i / i!, truncation below 4e-11
// relative).  A caller that scales its argument by a per-row factor folds the 64 into that
// factor: scaling by a power of two is exact, so the result is that of exp2_f64.
__device__ __forceinline__ void fill_exp2_table(double* tab) {
  if (threadIdx.x < 64) tab[threadIdx.x] = exp2((double)threadIdx.x / 64.0);
}

__device__ __forceinline__ double exp2_64th(double b, const double* tab) {
  b = fmax(b, -69120.0);
  const double n = rint(b);
  const double r = b - n;                          // exact
  const int ni = (int)n;
  double p = 0.055504108664821576 / 262144.0;      // (ln 2)^3 / 3! / 64^3
  p = fma(p, r, 0.2402265069591007 / 4096.0);      // (ln 2)^2 / 2! / 64^2
  p = fma(p, r, 0.6931471805599453 / 64.0);        // ln 2 / 64
  p = fma(p, r, 1.0);
  return ldexp(p * tab[ni & 63], ni >> 6);
}

// 2^a for a <= 0 (below -1080, and NaN, give 0)
__device__ __forceinline__ double exp2_f64(double a, const double* tab) { return exp2_64th(a * 64.0, tab); }

// Weight of a token in the row that is sampled, from the two values loaded for it (the target
// and draft entries; the draft entry is 0 and unused when !residual).
struct ProbWeight {
  bool residual;
  __device__ __forceinline__ double operator()(float p, float q) const { return residual_or_p(p, q, residual); }
};

struct LogitWeight {
  bool residual;
  double nmp, nmq, c64, inv_sp, inv_sq;  // -(row max) * c64, 64 log2(e) / T, reciprocals of the row sums
  const double* tab;                     // 2^(j/64) table in LDS
  __device__ __forceinline__ double operator()(float zp, float zq) const {
    // p and q are each rounded before the difference: fusing q's product into the
    // subtraction would leave p's rounding error behind where p = q (an empty residual)
#pragma clang fp contract(off)
    const double p = exp2_64th(fma((double)zp, c64, nmp), tab) * inv_sp;
    return residual ? fmax(0.0, p - exp2_64th(fma((double)zq, c64, nmq), tab) * inv_sq) : p;
  }
};

// Final draw of a draft-tree walk: max(0, p - c q) with the closed-form residual's c (the tree
// walk's weight; c = 0 is p itself).
struct TreeDrawWeight {
  bool residual;
  double c;
  __device__ __forceinline__ double operator()(float p, float q) const {
    return residual ? fmax(0.0, fma(-c, (double)q, (double)p)) : (double)p;
  }
};

// Fixed-order workgroup sum (same order every time).
__device__ __forceinline__ double block_sum(double x, double* s_red) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  x = wave_incl_scan(x);
  if (lane == 63) s_red[wv] = x;
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
  const double incl = wave_incl_scan(x);
  const double excl = dpp_f64<kDppWaveShr1>(incl);   // lane - 1's inclusive sum; 0 on lane 0
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
  return before + excl;
}

// The value of the first thread (in thread order) with `has`: one ballot per wave, then the
// waves in order; INT_MAX if none.
__device__ __forceinline__ int block_first(bool has, int x, int* s_int) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const unsigned long long m = __ballot(has);
  if (lane == 0) s_int[wv] = m ? __builtin_amdgcn_readlane(x, __ffsll((long long)m) - 1) : INT_MAX;
  __syncthreads();
  int t = INT_MAX;
#pragma unroll
  for (int i = kThreads / 64 - 1; i >= 0; --i) t = s_int[i] != INT_MAX ? s_int[i] : t;
  __syncthreads();
  return t;
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

typedef float f32x4 __attribute__((ext_vector_type(4)));

// 16-byte load, non-temporal for NT: bytes that no other load of the call reads again, streamed by
// workgroups that read many chunks, run closer to the HBM peak that way
template <bool NT>
__device__ __forceinline__ float4 ld_f4(const float* p) {
  f32x4 v;
  if constexpr (NT) v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  else v = *reinterpret_cast<const f32x4*>(p);
  return make_float4(v[0], v[1], v[2], v[3]);
}

// A thread's share of one chunk in registers: loaded (every load issued at once), then summed
// (chunk_partial does both; the fallback of finish_draw sums whole chunks with it).
template <bool VEC4>
struct ChunkRegs {
  static constexpr int kIt = VEC4 ? kMaxChunkLen / (4 * kThreads) : kMaxChunkLen / kThreads;
  float4 pv[VEC4 ? kIt : 1], qv[VEC4 ? kIt : 1];
  float ps[VEC4 ? 1 : kIt], qs[VEC4 ? 1 : kIt];
};

template <bool VEC4, bool NT>
__device__ __forceinline__ void chunk_load(ChunkRegs<VEC4>& r, const float* prow, const float* qrow, bool residual,
                                           int x0, int x1) {
  constexpr int kIt = ChunkRegs<VEC4>::kIt;
#pragma unroll
  for (int i = 0; i < kIt; ++i) {
    if constexpr (VEC4) {
      const int x = min(x0 + 4 * ((int)threadIdx.x + i * kThreads), x1 - 4);
      r.pv[i] = ld_f4<NT>(prow + x);
      r.qv[i] = residual ? ld_f4<NT>(qrow + x) : make_float4(0.f, 0.f, 0.f, 0.f);
    } else {
      const int x = min(x0 + (int)threadIdx.x + i * kThreads, x1 - 1);
      r.ps[i] = prow[x];
      r.qs[i] = residual ? qrow[x] : 0.f;
    }
  }
}

template <bool VEC4, class W>
__device__ __forceinline__ double chunk_sum(const ChunkRegs<VEC4>& r, const W& w, int x0, int x1) {
  constexpr int kIt = ChunkRegs<VEC4>::kIt;
  double acc = 0.0;
#pragma unroll
  for (int i = 0; i < kIt; ++i) {
    if constexpr (VEC4) {
      if (x0 + 4 * ((int)threadIdx.x + i * kThreads) < x1)
        acc += w(r.pv[i].x, r.qv[i].x) + w(r.pv[i].y, r.qv[i].y) + w(r.pv[i].z, r.qv[i].z) + w(r.pv[i].w, r.qv[i].w);
    } else {
      if (x0 + (int)threadIdx.x + i * kThreads < x1) acc += w(r.ps[i], r.qs[i]);
    }
  }
  return acc;
}

template <bool VEC4, class W, bool NT = false>
__device__ __forceinline__ double chunk_partial(const float* prow, const float* qrow, const W& w, int x0, int x1) {
  ChunkRegs<VEC4> r;
  chunk_load<VEC4, NT>(r, prow, qrow, w.residual, x0, x1);
  return chunk_sum<VEC4>(r, w, x0, x1);
}

// Smallest x in chunk [x0, x1) whose running sum base + C exceeds t (INT_MAX if none), with
// the running sum taken in ascending token id; also the largest x with w_x > 0 (-1 if none).
// Each thread takes a contiguous slice of at most kSlice elements held in registers (chunks
// are at most kThreads * kSlice long), so the scan never goes back to memory: kSlice = 4 for
// chunks of up to kDrawPiece tokens, 16 for the longer chunks of vocabularies above 256 kDrawPiece.
template <bool VEC4, int kSlice, class W>
__device__ __forceinline__ void chunk_select(const float* prow, const float* qrow, const W& w,
                                             int x0, int x1, double base, double t,
                                             double* s_red, int* s_int, int& first_above,
                                             int& last_positive) {
  const bool residual = w.residual;
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
  double wv[kSlice];   // each weight is evaluated once and kept for the second pass
  double mine = 0.0;
  int lastpos = -1;
#pragma unroll
  for (int j = 0; j < kSlice; ++j) {
    wv[j] = (a + j < b) ? w(pv[j], qv[j]) : 0.0;
    mine += wv[j];
    if (wv[j] > 0.0) lastpos = a + j;
  }
  double total;
  const double before = block_exclusive_scan(mine, s_red, total);
  double run = base + before;
  int found = INT_MAX;
#pragma unroll
  for (int j = 0; j < kSlice; ++j) {
    const double wx = wv[j];
    run += wx;
    if (found == INT_MAX && a + j < b && run > t) found = a + j;
  }
  // slices are in token order, so the first thread that found one holds the smallest x
  first_above = block_first(found != INT_MAX, found, s_int);
  // needed only when rounding left t at or past the chunk's total (uniform branch)
  last_positive = first_above == INT_MAX ? block_max(lastpos, s_int) : -1;
}

__device__ __forceinline__ void argmax_merge(float& m, int& i, float om, int oi) {
  // selects, not a branch: inside the DPP steps a branch costs an exec-mask round per step
  const bool take = (om > m) | ((om == m) & (oi < i));
  m = take ? om : m;
  i = take ? oi : i;
}

// One DPP step of the wave's (max, first argmax): lanes without a source take (-inf, INT_MAX).
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ void argmax_dpp_step(float& m, int& i) {
  const float om = __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(-INFINITY), __float_as_int(m), CTRL,
                                                              ROW_MASK, 0xf, false));
  const int oi = __builtin_amdgcn_update_dpp(INT_MAX, i, CTRL, ROW_MASK, 0xf, false);
  argmax_merge(m, i, om, oi);
}

// The wave's max and the smallest index holding it, on every lane: the steps of wave_incl_scan
// with argmax_merge (associative and commutative), then lane 63's result.  The wave must be
// fully active.
__device__ __forceinline__ void wave_argmax(float& m, int& i) {
  argmax_dpp_step<kDppRowShr + 1>(m, i);
  argmax_dpp_step<kDppRowShr + 2>(m, i);
  argmax_dpp_step<kDppRowShr + 4>(m, i);
  argmax_dpp_step<kDppRowShr + 8>(m, i);
  argmax_dpp_step<kDppRowBcast15, 0xa>(m, i);
  argmax_dpp_step<kDppRowBcast31, 0xc>(m, i);
  m = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 63));
  i = __builtin_amdgcn_readlane(i, 63);
}


// Merge the chunk partials of `rows` consecutive logit rows (part: [rows][C1]) into s_st: per
// row M = max m_c with its first argmax, and (unless greedy) S = sum_c S_c 2^((m_c - M) cT), in a
// fixed order.  Partials are staged through LDS in groups of rows; wave w merges rows w, w+4, ...
constexpr int kMergeStage = 2048;   // 16-byte partials staged per pass (32 KB)
constexpr int kMergePre = 4;        // partials per thread loaded ahead (one pass of up to 1024)
static_assert(kMergePre == 4, "the verification kernel holds four prefetched partials per thread");

// rows [r0, r0 + nr) from the staged partials (their first row at s_stage[0]); ends with a barrier
__device__ void merge_staged_rows(const uint4* s_stage, int C1, int r0, int nr, bool greedy, double cT,
                                  LogitRowStat* s_st, const double* tab) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int rr = wv; rr < nr; rr += kThreads / 64) {
    const LogitRowStat* st = reinterpret_cast<const LogitRowStat*>(s_stage) + rr * C1;
    float M = -INFINITY;
    int I = INT_MAX;
    for (int c = lane; c < C1; c += 64) argmax_merge(M, I, st[c].m, st[c].argmax);
    wave_argmax(M, I);
    double S = 0.0;
    if (!greedy) {
      for (int c = lane; c < C1; c += 64) S += st[c].S * exp2_f64(((double)st[c].m - (double)M) * cT, tab);
      S = wave_total(S);
    }
    if (lane == 0) s_st[r0 + rr] = LogitRowStat{S, M, I};
  }
  __syncthreads();
}

__device__ void merge_row_stats(const LogitRowStat* part, int C1, int rows, bool greedy, double cT,
                                LogitRowStat* s_st, uint4* s_stage, const double* tab) {
  const int tid = threadIdx.x;
  const int per = max(1, kMergeStage / C1);
  for (int r0 = 0; r0 < rows; r0 += per) {
    const int nr = min(per, rows - r0);
    const uint4* src = reinterpret_cast<const uint4*>(part + (long long)r0 * C1);
    for (int e = tid; e < nr * C1; e += kThreads) s_stage[e] = src[e];
    __syncthreads();
    merge_staged_rows(s_stage, C1, r0, nr, greedy, cT, s_st, tab);
  }
}

// A workgroup that has published the sums of its chunks arrives on the sequence's ticket (thread
// 0 only).  The workgroup that takes the last ticket (value `last`) resets the ticket for the next
// call and returns true; it then reads every chunk's slot, waiting for any not yet visible
// (read_slot), and clears them.
__device__ __forceinline__ bool arrive(int32_t* ticket, int last) {
  const int t = __hip_atomic_fetch_add(ticket, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (t != last) return false;
  __hip_atomic_store(ticket, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// Sums of w over this workgroup's chunks [c0, c1) of the row(s) at prow / qrow, each published to
// its slot: wave v sums chunks c0 + v, c0 + v + 4, ..., each in pieces of up to kDrawPiece tokens
// (lane-strided 16-byte loads, the next piece's loads in flight while one is summed), and its
// lane 0 publishes the chunk's sum.  Launches whose workgroups take kNtChunks chunks or more
// (large batches, where the draw streams at bandwidth) load them non-temporally (NT): bytes that
// no other load of the call reads again run closer to the HBM peak that way, while small
// batches, bound by their round trips, measured slightly slower.
template <bool VEC4>
struct PieceRegs {
  static constexpr int kIt = VEC4 ? kDrawPiece / 256 : kDrawPiece / 64;   // per lane
  float4 pv[VEC4 ? kIt : 1], qv[VEC4 ? kIt : 1];
  float ps[VEC4 ? 1 : kIt], qs[VEC4 ? 1 : kIt];
};

template <bool VEC4, bool NT, class W>
__device__ __forceinline__ void publish_chunk_sums(const float* prow, const float* qrow, const W& w, int c0, int c1,
                                                   int CS, int V, unsigned long long* slots) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  constexpr int kIt = PieceRegs<VEC4>::kIt;
  const int np = (CS + kDrawPiece - 1) / kDrawPiece;            // pieces per chunk
  const int nc = c1 - c0 > wv ? (c1 - c0 - wv + 3) / 4 : 0;    // this wave's chunks
  const int n = nc * np;                                        // this wave's pieces
  // piece f: chunk c0 + wv + 4 (f / np), tokens [x0, x1)
  auto range = [&](int f, int& x0, int& x1) {
    const int c = c0 + wv + 4 * (f / np);
    const int e = min(V, c * CS + CS);
    x0 = c * CS + (f % np) * kDrawPiece;
    x1 = min(e, x0 + kDrawPiece);
  };
  auto load = [&](PieceRegs<VEC4>& r, int f) {
    int x0, x1;
    range(f, x0, x1);
#pragma unroll
    for (int i = 0; i < kIt; ++i) {
      if constexpr (VEC4) {
        const int x = min(x0 + 4 * (lane + 64 * i), x1 - 4);
        r.pv[i] = ld_f4<NT>(prow + x);
        r.qv[i] = w.residual ? ld_f4<NT>(qrow + x) : make_float4(0.f, 0.f, 0.f, 0.f);
      } else {
        const int x = min(x0 + lane + 64 * i, x1 - 1);
        r.ps[i] = prow[x];
        r.qs[i] = w.residual ? qrow[x] : 0.f;
      }
    }
  };
  double acc = 0.0;
  auto finish = [&](const PieceRegs<VEC4>& r, int f) {
    int x0, x1;
    range(f, x0, x1);
#pragma unroll
    for (int i = 0; i < kIt; ++i) {
      if constexpr (VEC4) {
        if (x0 + 4 * (lane + 64 * i) < x1)
          acc += w(r.pv[i].x, r.qv[i].x) + w(r.pv[i].y, r.qv[i].y) + w(r.pv[i].z, r.qv[i].z) + w(r.pv[i].w, r.qv[i].w);
      } else {
        if (x0 + lane + 64 * i < x1) acc += w(r.ps[i], r.qs[i]);
      }
    }
    if (f % np == np - 1) {   // the chunk's last piece
      const double part = wave_total(acc);
      if (lane == 0) publish_slot(slots + c0 + wv + 4 * (f / np), part);
      acc = 0.0;
    }
  };
  PieceRegs<VEC4> ra, rb;
  if (n > 0) load(ra, 0);
  for (int f = 0; f < n; f += 2) {
    if (f + 1 < n) load(rb, f + 1);
    finish(ra, f);
    if (f + 1 >= n) break;
    if (f + 2 < n) load(ra, f + 2);
    finish(rb, f + 1);
  }
}

// Step 4 of a draw by the last workgroup of a sequence: with every chunk's sum of w published
// (slots[0 .. C), read and cleared here), find the chunk holding t = u Z (one wave; each lane
// holds up to four consecutive chunks, C <= 256), then the token inside it.  If Z = 0 the weights `fallback`
// are drawn from instead (their chunk sums computed here); if those are all zero too,
// VAP_DERR_EMPTY_ROW and token 0.  If rounding leaves t at or past the total, the last token
// with positive weight.
template <bool VEC4, class W>
__device__ int finish_draw(unsigned long long* slots, int C, int CS, int V, float uk, const float* prow,
                           const float* qrow, const W& w, const W& fallback, int32_t* err, double* s_loc,
                           int& s_cstar, double* s_red, int* s_int) {
  const int tid = threadIdx.x, lane = tid & 63;
  W wsel = w;
  const float* srow_q = qrow;
  double Z = 0.0;
  if (tid < 64) {
    double cs[4];
    bool late = false;
    // the lane's four slots in one round trip (lanes past C read chunk C - 1 and ignore it); a
    // slot not yet visible is waited for
    unsigned long long x[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      x[j] = __hip_atomic_load(slots + min(4 * lane + j, C - 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ci = 4 * lane + j;
      cs[j] = ci >= C ? 0.0 : (x[j] != 0ull ? __longlong_as_double((long long)~x[j]) : read_slot(slots + ci, &late));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (4 * lane + j < C) clear_slot(slots + 4 * lane + j);
    if (late) atomicOr(err, VAP_DERR_SYNC);
    const double mine = (cs[0] + cs[1]) + (cs[2] + cs[3]);
    const double incl = wave_incl_scan(mine);
    Z = lane_value(incl, 63);
    if (Z > 0.0) {
      const double t = (double)uk * Z;
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
    // empty weights: draw from the fallback weights (their chunk sums are computed here)
    wsel = fallback;
    srow_q = fallback.residual ? qrow : prow;
    double cs = 0.0;
    for (int j = 0; j < C; ++j) {
      const int a = j * CS, e = min(V, a + CS);
      const double sj = block_sum(chunk_partial<VEC4>(prow, srow_q, wsel, a, e), s_red);
      if (tid == j) cs = sj;
    }
    double before = block_exclusive_scan(cs, s_red, Z);
    if (Z > 0.0) {
      t = (double)uk * Z;
      const int cand = (tid < C && before + cs > t) ? tid : INT_MAX;
      cstar = block_min(cand, s_int);
      const int lastnz = block_max((tid < C && cs > 0.0) ? tid : -1, s_int);
      if (cstar == INT_MAX) cstar = lastnz;
      if (tid == cstar) s_loc[0] = before;
      __syncthreads();
      base = s_loc[0];
      __syncthreads();
    } else if (tid == 0) {
      atomicOr(err, VAP_DERR_EMPTY_ROW);
    }
  }
  if (cstar >= 0) {
    const int a = cstar * CS, e = min(V, a + CS);
    int first_above, last_positive;
    if (CS <= kDrawPiece)
      chunk_select<VEC4, kDrawPiece / kThreads>(prow, srow_q, wsel, a, e, base, t, s_red, s_int, first_above, last_positive);
    else
      chunk_select<VEC4, kMaxChunkLen / kThreads>(prow, srow_q, wsel, a, e, base, t, s_red, s_int, first_above,
                                                  last_positive);
    token = (first_above != INT_MAX) ? first_above : (last_positive >= 0 ? last_positive : 0);
  }
  return token;
}

// Temperature of sequence b in verification from logits: T > 0 samples; T = 0, and any value
// that is negative or not finite (reported), is greedy.
__device__ __forceinline__ bool greedy_temperature(float T) { return !(T > 0.f && T <= FLT_MAX); }

template <bool VEC4, bool LOGITS, bool NT>
__global__ __launch_bounds__(kThreads) void spec_verify_kernel(const VerifyParams P) {
  using W = std::conditional_t<LOGITS, LogitWeight, ProbWeight>;
  __shared__ int s_n;
  __shared__ int s_last;
  __shared__ int s_ids[64];          // draft ids (accepted ones are copied to the output)
  __shared__ float s_uk;             // u_k, the uniform of the final draw
  __shared__ double s_loc[2];        // base (sum before the chosen chunk), t
  __shared__ int s_cstar;
  __shared__ double s_red[kThreads / 64];
  __shared__ int s_int[kThreads / 64];
  __shared__ LogitRowStat s_st[LOGITS ? 2 * 64 + 1 : 1];        // merged row statistics
  __shared__ uint4 s_stage[LOGITS ? kMergeStage : 1];           // staged chunk partials
  __shared__ double s_tab[LOGITS ? 64 : 1];                     // 2^(j/64)

  const int C = P.C, WPS = P.WPS;
  const int L = seq_major_index();
  const int b = L / WPS;
  const int wg = L - b * WPS;                     // this workgroup's chunks: [c0, c1)
  const int G = (C + WPS - 1) / WPS;
  const int c0 = wg * G, c1 = min(C, c0 + G);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int k = P.k, V = P.V;
  const long long srow = (long long)b * (2 * k + 1);   // first statistics row of sequence b
  bool greedy = false;
  double cT = 0.0;
  // the first wave's draft token, its uniform and (both paths) the two entries at that token:
  // loaded before the merge of the row statistics, which they do not depend on
  // (a token outside [0, V) reads entry 0 and is rejected; the loads take no branch, so that no
  // wait for them is placed before the merge's own loads)
  int x = 0;
  float r = 0.f, px = 0.f, qx = 0.f;
  if (tid == 64) s_uk = P.uniforms[(long long)b * (k + 1) + k];
  if (tid < k) {
    x = P.draft_ids[(long long)b * k + lane];
    r = P.uniforms[(long long)b * (k + 1) + lane];
    const int xc = (x >= 0 && x < V) ? x : 0;
    px = P.p[((long long)b * (k + 1) + lane) * V + xc];
    qx = P.q[((long long)b * k + lane) * V + xc];
  }
  const bool inside = x >= 0 && x < V;
  if constexpr (LOGITS) {
    // the partials of all 2k + 1 rows (a greedy sequence's draft rows are merged but unused), in
    // one pass when they fit kMergePre per thread, loaded before the temperature is known
    const int C1 = P.C1, rows = 2 * k + 1, n_el = rows * C1;
    const uint4* src = reinterpret_cast<const uint4*>(P.part + srow * C1);
    const bool one_pass = n_el <= kMergePre * kThreads && n_el <= kMergeStage;
    // (four named registers: an array here is kept in scratch memory)
    uint4 pre0, pre1, pre2, pre3;
    if (one_pass) {
      pre0 = src[min(tid, n_el - 1)];
      pre1 = src[min(tid + kThreads, n_el - 1)];
      pre2 = src[min(tid + 2 * kThreads, n_el - 1)];
      pre3 = src[min(tid + 3 * kThreads, n_el - 1)];
    }
    const float T = P.temps[b];
    greedy = greedy_temperature(T);
    if (!(T >= 0.f && T <= FLT_MAX) && wg == 0 && tid == 0) atomicOr(P.err, VAP_DERR_TEMP);
    cT = greedy ? 0.0 : 1.4426950408889634 / (double)T;
    fill_exp2_table(s_tab);   // visible after the merge's first barrier
    if (one_pass) {
      if (tid < n_el) s_stage[tid] = pre0;
      if (tid + kThreads < n_el) s_stage[tid + kThreads] = pre1;
      if (tid + 2 * kThreads < n_el) s_stage[tid + 2 * kThreads] = pre2;
      if (tid + 3 * kThreads < n_el) s_stage[tid + 3 * kThreads] = pre3;
      __syncthreads();
      merge_staged_rows(s_stage, C1, 0, greedy ? k + 1 : rows, greedy, cT, s_st, s_tab);
    } else {
      merge_row_stats(P.part + srow * C1, C1, greedy ? k + 1 : rows, greedy, cT, s_st, s_stage, s_tab);
    }
    // the gathered values are first used here: without this the compiler converts them where
    // they are loaded, which waits for those loads before the partials' loads are issued
    asm volatile("" : "+v"(px), "+v"(qx), "+v"(r));
  }

  // 1. accept tests (first wave; k <= 64)
  if (tid < 64) {
    bool reject = false;
    if (lane < k) {
      if (!inside && wg == 0) atomicOr(P.err, VAP_DERR_DRAFT_ID);
      if constexpr (!LOGITS) {
        reject = !(inside && px > 0.f && (double)r * (double)qx <= (double)px);
      } else {
        if (!inside) {
          reject = true;
        } else if (greedy) {
          reject = x != s_st[lane].argmax;
        } else {
          const LogitRowStat sp = s_st[lane], sq = s_st[k + 1 + lane];
          const double pv = exp2_f64(((double)px - sp.m) * cT, s_tab) / sp.S;
          const double qv = exp2_f64(((double)qx - sq.m) * cT, s_tab) / sq.S;
          reject = !(pv > 0.0 && (double)r * qv <= pv);
        }
      }
      s_ids[lane] = x;
    }

    const unsigned long long m = __ballot(reject);
    if (lane == 0) s_n = m ? (__ffsll((long long)m) - 1) : k;
  }
  __syncthreads();
  const int n = s_n;
  if constexpr (LOGITS) {
    if (greedy) {   // exact matching: the emitted token is the argmax of target row n
      if (wg == 0) {
        if (tid <= k)
          P.out_ids[(long long)b * (k + 1) + tid] = tid < n ? s_ids[tid] : (tid == n ? s_st[n].argmax : -1);
        if (tid == 0) P.n_accepted[b] = n;
      }
      return;
    }
  }
  const bool residual = n < k;
  const float* prow = P.p + ((long long)b * (k + 1) + n) * V;
  const float* qrow = residual ? P.q + ((long long)b * k + n) * V : prow;
  W w;
  if constexpr (LOGITS) {
    const LogitRowStat sp = s_st[n];
    const LogitRowStat sq = residual ? s_st[k + 1 + n] : sp;
    w = LogitWeight{residual, -(double)sp.m * (64.0 * cT), -(double)sq.m * (64.0 * cT), 64.0 * cT, 1.0 / sp.S,
                    1.0 / sq.S, s_tab};
  } else {
    w = ProbWeight{residual};
  }

  // 2-3. the sums of w over this workgroup's chunks
  unsigned long long* sums = P.rec.at<unsigned long long>(b, kVerifyRecSums);
  publish_chunk_sums<VEC4, NT>(prow, qrow, w, c0, c1, P.CS, V, sums);
  __syncthreads();   // every wave has published before the workgroup arrives
  if (tid == 0) s_last = arrive(P.rec.ticket(b), WPS - 1);
  __syncthreads();
  if (!s_last) return;

  // 4. last workgroup of sequence b: the chunk holding t, then the token inside it
  W p_only = w;   // an empty residual falls back to the row p_n itself
  p_only.residual = false;
  const int token = finish_draw<VEC4>(sums, C, P.CS, V, s_uk, prow, qrow, w, p_only,
                                      P.err, s_loc, s_cstar, s_red, s_int);

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

// f(0), f(1), ... with compile-time arguments, stopping at the first that returns true
template <typename F, int... I>
__device__ __forceinline__ bool each_until(F& f, std::integer_sequence<int, I...>) {
  return (f(std::integral_constant<int, I>{}) || ...);
}

constexpr int kStatTempsLds = 4096;   // 16 KB
#ifndef VAP_STAT_STAGES
#define VAP_STAT_STAGES 2
#endif
constexpr int kStatStages = VAP_STAT_STAGES;   // statistics items per wave in flight or in reduction

// Row statistics of the logits (see LogitRowStat), per chunk of kStatChunk tokens: persistent
// waves take (row, chunk) items with a grid stride and keep the next kStatStages - 1 items'
// loads in flight while they reduce the current one (each lane holds 32 tokens; max and first
// argmax by compares per lane and DPP steps, then the fp64 sum of exponentials).  Each item
// writes its partial with a plain store; the verification kernel merges them.  Draft rows of
// greedy sequences are skipped.
//
// Every item issues the same loads on every path: an item with nothing to read (past the last
// one, or a skipped draft row) reads the first 16 bytes of the target logits in every lane.
// With loads that depend on the path, the compiler's wait counts must assume the shortest
// queue, and the reduce of one item then waits for the loads of the next.
//
// TLDS: the batch's temperatures are staged in LDS (batches of up to kStatTempsLds sequences);
// a global load of the temperature would make the next item's loads wait for the current one's.
template <bool VEC4, bool TLDS>
__global__ __launch_bounds__(kThreads) void logit_stats_kernel(const LogitStatsParams P) {
  constexpr int kEl = kStatChunk / 64;
  __shared__ double s_tab[64];
  __shared__ float s_temps[TLDS ? kStatTempsLds : 1];
  const int lane = threadIdx.x & 63;
  const int k = P.k, C = P.C, V = P.V;
  const int rows_per_seq = 2 * k + 1;
  const int items = P.B * rows_per_seq * C;             // < 2^31 (checked on the host)
  const int stride = gridDim.x * (kThreads / 64);
  fill_exp2_table(s_tab);
  if (TLDS)
    for (int i = threadIdx.x; i < P.B; i += kThreads) s_temps[i] = P.temps[i];

  struct Item {
    const float* z;
    int x0, x1;
    bool need, greedy;
    double c64;   // 64 log2(e) / T
  };
  auto item_of = [&](int it) __attribute__((always_inline)) {
    Item d;
    d.need = false;
    d.greedy = true;
    d.c64 = 0.0;
    d.z = P.zp;
    d.x0 = 0;
    d.x1 = VEC4 ? 4 : 1;
    if (it < items) {
      const int row = it / C;
      const int c = it - row * C;
      const int b = row / rows_per_seq, r = row - b * rows_per_seq;
      const float T = TLDS ? s_temps[b] : P.temps[b];
      d.greedy = greedy_temperature(T);
      if (!(d.greedy && r > k)) {
        d.need = true;
        d.c64 = d.greedy ? 0.0 : 64.0 * (1.4426950408889634 / (double)T);
        d.z = r <= k ? P.zp + ((long long)b * (k + 1) + r) * V : P.zq + ((long long)b * k + (r - k - 1)) * V;
        d.x0 = c * kStatChunk;
        d.x1 = min(V, d.x0 + kStatChunk);
      }
    }
    return d;
  };
  // lane's element j: VEC4 -> x0 + 4 (lane + 64 (j / 4)) + j % 4, else x0 + lane + 64 j (both
  // increase with j); loads past the chunk read a clamped address and are masked
  auto index = [&](const Item& d, int j) __attribute__((always_inline)) {
    return VEC4 ? d.x0 + 4 * (lane + 64 * (j >> 2)) + (j & 3) : d.x0 + lane + 64 * j;
  };
  auto load = [&](const Item& d, float (&v)[kEl]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kEl; j += 4) {
      if (VEC4) {
        const float4 u = *reinterpret_cast<const float4*>(d.z + min(index(d, j), d.x1 - 4));
        v[j] = u.x; v[j + 1] = u.y; v[j + 2] = u.z; v[j + 3] = u.w;
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) v[j + u] = d.z[min(index(d, j + u), d.x1 - 1)];
      }
    }
  };
  auto reduce = [&](const Item& d, int it, float (&v)[kEl]) __attribute__((always_inline)) {
    if (!d.need) return;
    // the last chunk of a row: elements past its end become -inf, which are never the max and
    // whose exponential is exactly 0, so one reduction serves every chunk
    if (d.x1 - d.x0 != kStatChunk) {
#pragma unroll
      for (int j = 0; j < kEl; ++j) v[j] = index(d, j) < d.x1 ? v[j] : -INFINITY;
    }
    float m = -INFINITY;
    int mi = INT_MAX;
#pragma unroll
    for (int j = 0; j < kEl; ++j) {
      const bool take = v[j] > m;
      m = take ? v[j] : m;
      mi = take ? index(d, j) : mi;
    }
    wave_argmax(m, mi);
    double S = 0.0;
    if (!d.greedy) {
      // 64 (z - m) log2(e) / T as one fma with the rounded product m c64: an argument error of
      // ulp(m c64), a relative error near 1e-14 in the term, far below the polynomial's 4e-11
      const double mc64 = -(double)m * d.c64;
#pragma unroll
      for (int j = 0; j < kEl; ++j) S += exp2_64th(fma((double)v[j], d.c64, mc64), s_tab);
      S = wave_total(S);
    }
    if (lane == 0) P.part[it] = LogitRowStat{S, m, mi};
  };

  // this call's verification tickets and chunk-sum slots start at zero whatever an earlier call
  // of another shape left there (the verification kernel runs after this one, in stream order)
  const long long words = (long long)P.B * (P.VC + 1);
  for (long long e = (long long)blockIdx.x * kThreads + threadIdx.x; e < words; e += (long long)gridDim.x * kThreads) {
    const long long b = e / (P.VC + 1);
    const int j = (int)(e - b * (P.VC + 1));
    if (j == 0) *P.rec.ticket(b) = 0;
    else P.rec.at<unsigned long long>(b, kVerifyRecSums)[j - 1] = 0ull;
  }
  __syncthreads();
  int it = __builtin_amdgcn_readfirstlane((int)blockIdx.x * (kThreads / 64) + (int)(threadIdx.x >> 6));
  if (it >= items) return;
  // kStatStages buffers in rotation: the loads of the next kStatStages - 1 items are in flight
  // while one is reduced (the rotation is unrolled, so every buffer stays in registers)
  float v[kStatStages][kEl];
  Item d[kStatStages];
#pragma unroll
  for (int s = 0; s + 1 < kStatStages; ++s) {
    d[s] = item_of(it + s * stride);
    load(d[s], v[s]);
  }
  // one step per buffer s (a compile-time index): refill the buffer reduced last, reduce s;
  // true once the wave's last item is reduced
  auto step = [&](auto sc) __attribute__((always_inline)) {
    constexpr int s = decltype(sc)::value;
    constexpr int n = (s + kStatStages - 1) % kStatStages;
    d[n] = item_of(it + (kStatStages - 1) * stride);
    load(d[n], v[n]);
    reduce(d[s], it, v[s]);
    if (it + stride >= items) return true;
    it += stride;
    return false;
  };
  while (!each_until(step, std::make_integer_sequence<int, kStatStages>{})) {
  }
}

// Final draw of spec_verify_tree (the walk itself is tree_verify_kernel in spec_verify_tree.hip):
// one workgroup per (sequence, vocabulary chunk) sums its chunk of the weights max(0, p - c q)
// of the node where the sequence's walk ended and publishes the sum; the last workgroup of the
// sequence finds the token t = u_0 Z falls on, in ascending token id, as in spec_verify.
template <bool VEC4, bool NT>
__global__ __launch_bounds__(kThreads) void tree_draw_kernel(const TreeDrawParams P) {
  __shared__ int s_last;
  __shared__ double s_loc[2];
  __shared__ int s_cstar;
  __shared__ double s_red[kThreads / 64];
  __shared__ int s_int[kThreads / 64];
  const int C = P.C, WPS = P.WPS;
  const int L = seq_major_index();
  const int b = L / WPS;
  const int wg = L - b * WPS;                     // this workgroup's chunks: [c0, c1)
  const int G = (C + WPS - 1) / WPS;
  const int c0 = wg * G, c1 = min(C, c0 + G);
  const int tid = threadIdx.x;
  const TreeDraw d = *P.rec.at<const TreeDraw>(b, kTreeRecDraw);
  if (wg == 0 && d.passes > 0) {
    // the walk's shared chunk sums are consumed (the walk kernel has finished): zero them for
    // the next call
    unsigned long long* wslots = P.rec.at<unsigned long long>(b, kTreeRecWalk);
    for (int i = tid; i < d.passes * kWalkChunks; i += kThreads) clear_slot(wslots + i);
  }
  const long long row = (long long)b * P.N + d.node;
  const float* prow = P.p + row * P.V;
  const float* qrow = P.q + row * P.V;
  const TreeDrawWeight w{d.c > 0.0, d.c};
  unsigned long long* sums = P.rec.at<unsigned long long>(b, kTreeRecSums);
  publish_chunk_sums<VEC4, NT>(prow, qrow, w, c0, c1, P.CS, P.V, sums);
  __syncthreads();   // every wave has published before the workgroup arrives
  if (tid == 0) s_last = arrive(P.rec.ticket(b), WPS - 1);
  __syncthreads();
  if (!s_last) return;
  const float uk = P.uniforms[(long long)b * P.N];
  const TreeDrawWeight prev{d.c_prev > 0.0, d.c_prev};
  const int token = finish_draw<VEC4>(sums, C, P.CS, P.V, uk, prow, qrow, w, prev,
                                      P.err, s_loc, s_cstar, s_red, s_int);
  if (tid == 0) P.out_ids[(long long)b * P.N + d.n] = token;
}

}  // namespace

// Workgroups that stream at least this many chunks load them non-temporally (see publish_chunk_sums).
constexpr int kNtChunks = 32;

template <bool LOGITS>
hipError_t launch_verify_t(const VerifyParams& p, bool vec4, hipStream_t stream, KTimer t) {
  const dim3 grid((unsigned)((long long)p.WPS * p.B));
  const bool nt = (p.C + p.WPS - 1) / p.WPS >= kNtChunks;
#define VAP_LAUNCH_VERIFY(V4, N)                                                                       \
  hipExtLaunchKernelGGL((spec_verify_kernel<V4, LOGITS, N>), grid, dim3(kThreads), 0, stream, t.start, t.stop, 0, p)
  if (vec4) {
    if (nt) VAP_LAUNCH_VERIFY(true, true); else VAP_LAUNCH_VERIFY(true, false);
  } else {
    if (nt) VAP_LAUNCH_VERIFY(false, true); else VAP_LAUNCH_VERIFY(false, false);
  }
#undef VAP_LAUNCH_VERIFY
  return hipGetLastError();
}

hipError_t launch_spec_verify(const VerifyParams& p, bool vec4, hipStream_t stream, KTimer t) {
  return launch_verify_t<false>(p, vec4, stream, t);
}

hipError_t launch_spec_verify_logits(const VerifyParams& p, bool vec4, hipStream_t stream, KTimer t) {
  return launch_verify_t<true>(p, vec4, stream, t);
}

hipError_t launch_logit_stats(const LogitStatsParams& p, bool vec4, int num_wg, hipStream_t stream, KTimer t) {
  const dim3 grid((unsigned)num_wg);
  const bool tlds = p.B <= kStatTempsLds;
#define VAP_LAUNCH_STATS(V4, TL)                                                                       \
  hipExtLaunchKernelGGL((logit_stats_kernel<V4, TL>), grid, dim3(kThreads), 0, stream, t.start, t.stop, 0, p)
  if (vec4) {
    if (tlds) VAP_LAUNCH_STATS(true, true); else VAP_LAUNCH_STATS(true, false);
  } else {
    if (tlds) VAP_LAUNCH_STATS(false, true); else VAP_LAUNCH_STATS(false, false);
  }
#undef VAP_LAUNCH_STATS
  return hipGetLastError();
}

hipError_t launch_tree_draw(const TreeDrawParams& p, bool vec4, hipStream_t stream, KTimer t) {
  const dim3 grid((unsigned)((long long)p.WPS * p.B));
  const bool nt = (p.C + p.WPS - 1) / p.WPS >= kNtChunks;
#define VAP_LAUNCH_DRAW(V4, N)                                                                         \
  hipExtLaunchKernelGGL((tree_draw_kernel<V4, N>), grid, dim3(kThreads), 0, stream, t.start, t.stop, 0, p)
  if (vec4) {
    if (nt) VAP_LAUNCH_DRAW(true, true); else VAP_LAUNCH_DRAW(true, false);
  } else {
    if (nt) VAP_LAUNCH_DRAW(false, true); else VAP_LAUNCH_DRAW(false, false);
  }
#undef VAP_LAUNCH_DRAW
  return hipGetLastError();
}

}  // namespace vap
