// Combine kernel of paged_attn_step: merges the partials of every unit of work that the main
// kernel split over several worker waves and writes the unit's output rows.
//
// A split unit's partials are (m_p, l_p, acc_p) per row: running max in log2 units, running
// sum and unnormalised output over one block range.  They merge as in flash-decoding's
// combine (the split-KV reduction the pages' long-context batches need -- tempatgunting.com
// article, section "Implementation Details That Affect Tail Latency"):
//     M = max_p m_p,   L = sum_p 2^(m_p - M) l_p,   out = sum_p 2^(m_p - M) acc_p / L,
// folded in a fixed order, so a step's output does not depend on timing.
//
// Layout of the work (the step is latency-bound: every partial was written by the previous
// kernel, so each dependent round trip to L2/MALL costs more than the bytes):
//  * one workgroup (NW = 2 waves for 16-row units, 8 for 32-row and 16 for 64-row units) per
//    K consecutive descriptors, loaded together; holder w's descriptor (a worker wave's share
//    or a pool piece) is valid when w holds the first block of a split unit, and then names
//    the last holder wb of part of it (holders are numbered in work order);
//  * 16 lanes per row, each lane D/16 consecutive dims (float4 loads), so a wave covers a
//    quad of 4 rows;
//  * nq = ceil(rows/4) quads (up to 16 for 64-row units); with nq >= NW each wave merges whole
//    quads (wave, wave + NW, ...); with nq < NW the partial list is split too: S = NW / nq
//    waves per quad take partials p, p+S, p+2S, ... and merge in LDS in wave order;
//  * up to kBatch partials are loaded before any is folded (one round trip per batch).
#include <algorithm>

#include "attn_internal.h"

namespace vap {
namespace {

constexpr int kBatch = 8;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

template <int DPL>
struct RowState {
  float M, L;
  float a[DPL];
};

// fold (m, l, v) into the running state s
template <int DPL>
__device__ __forceinline__ void fold(RowState<DPL>& s, float m, float l, const float (&v)[DPL]) {
  const float Mn = fmaxf(s.M, m);
  if (Mn == kNegInf) return;   // both empty
  const float fa = __builtin_amdgcn_exp2f(s.M - Mn), fb = __builtin_amdgcn_exp2f(m - Mn);
  s.L = s.L * fa + l * fb;
#pragma unroll
  for (int k = 0; k < DPL; ++k) s.a[k] = s.a[k] * fa + v[k] * fb;
  s.M = Mn;
}

// Merge the split unit that holder w's descriptor (d0, d1) opens; every wave of the workgroup
// calls it with the same descriptor.  NW waves per workgroup: 2 for 16-row units, 8 for
// 32-row units, 16 for 64-row units (16 quads).
template <int D, int NW>
__device__ __forceinline__ void combine_unit(const AttnParams& P, int w, int4 d0, int4 d1,
                                             float (&s_ml)[NW][64][2], float4 (&s_acc)[NW][D / 64][64]) {
  constexpr int kCombineWaves = NW;
  constexpr int DPL = D / 16;   // dims per lane
  constexpr int NV4 = DPL / 4;  // float4 loads per lane and partial
  const int kvh = d0.x, rg = d0.y, qoff = d0.z, Q = d0.w;
  const int wb = d1.x, slot_a = d1.y;
  const int G = P.G, RG = P.RG;
  const int nrows = min(RG, G * Q - rg * RG);
  const int n = wb - w + 1;              // partials of this unit, in holder (work) order
  const int nq = (nrows + 3) >> 2;
  const int S = nq >= kCombineWaves ? 1 : kCombineWaves / nq;

  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int li = lane & 15;

  // fold partials sub, sub+S, ... of the unit for row r into st (kBatch loads per round trip)
  auto fold_rows = [&](RowState<DPL>& st, int r, int sub) {
    st.M = kNegInf;
    st.L = 0.f;
#pragma unroll
    for (int k = 0; k < DPL; ++k) st.a[k] = 0.f;
    const int cnt = (n - sub + S - 1) / S;
    for (int i0 = 0; i0 < cnt; i0 += kBatch) {
      float2 ml[kBatch];
      float v[kBatch][DPL];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int i = min(i0 + j, cnt - 1);
        const int wp = w + sub + i * S;
        const long long prow = ((long long)wp * 2 + (wp == w ? slot_a : 0)) * RG + r;
        ml[j] = P.part_ml[prow];
        const float4* pa = reinterpret_cast<const float4*>(P.part_acc + prow * D + DPL * li);
#pragma unroll
        for (int t = 0; t < NV4; ++t) {
          const float4 x = pa[t];
          v[j][4 * t] = x.x;
          v[j][4 * t + 1] = x.y;
          v[j][4 * t + 2] = x.z;
          v[j][4 * t + 3] = x.w;
        }
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j)
        if (i0 + j < cnt) fold<DPL>(st, ml[j].x, ml[j].y, v[j]);
    }
  };
  auto write_row = [&](const RowState<DPL>& st, int r_raw) {
    if (r_raw >= nrows) return;
    const int row = rg * RG + r_raw;
    const int i = row / G;
    float* op = P.out + ((long long)(qoff + i) * P.Hq + kvh * G + (row - i * G)) * D + DPL * li;
    const float inv = 1.f / st.L;
#pragma unroll
    for (int t = 0; t < NV4; ++t)
      reinterpret_cast<float4*>(op)[t] =
          make_float4(st.a[4 * t] * inv, st.a[4 * t + 1] * inv, st.a[4 * t + 2] * inv, st.a[4 * t + 3] * inv);
  };

  RowState<DPL> st;
  if (S == 1) {
    // at least as many quads as waves: each wave takes quads wave, wave + NW, ... alone
    for (int quad = wave; quad < nq; quad += kCombineWaves) {
      const int r_raw = 4 * quad + (lane >> 4);
      fold_rows(st, min(r_raw, nrows - 1), 0);   // rows past the unit load a valid row, write nothing
      write_row(st, r_raw);
    }
    return;
  }

  // fewer quads than waves: S waves per quad split its partials and merge in LDS in wave order
  __syncthreads();                        // the previous unit's LDS reads are done
  const int quad = wave % nq;
  const int sub = wave / nq;
  const int r_raw = 4 * quad + (lane >> 4);
  if (sub < S) {
    fold_rows(st, min(r_raw, nrows - 1), sub);
  } else {
    st.M = kNegInf;
    st.L = 0.f;
#pragma unroll
    for (int k = 0; k < DPL; ++k) st.a[k] = 0.f;
  }
  s_ml[wave][lane][0] = st.M;
  s_ml[wave][lane][1] = st.L;
#pragma unroll
  for (int t = 0; t < NV4; ++t)
    s_acc[wave][t][lane] = make_float4(st.a[4 * t], st.a[4 * t + 1], st.a[4 * t + 2], st.a[4 * t + 3]);
  __syncthreads();
  if (sub != 0) return;                   // (no barrier follows within this unit)
  for (int t2 = 1; t2 < S; ++t2) {
    const int ow = quad + t2 * nq;
    float v[DPL];
#pragma unroll
    for (int t = 0; t < NV4; ++t) {
      const float4 x = s_acc[ow][t][lane];
      v[4 * t] = x.x;
      v[4 * t + 1] = x.y;
      v[4 * t + 2] = x.z;
      v[4 * t + 3] = x.w;
    }
    fold<DPL>(st, s_ml[ow][lane][0], s_ml[ow][lane][1], v);
  }
  write_row(st, r_raw);
}

// One workgroup per K consecutive descriptors (K chosen so that the grid takes at most two
// residency rounds): lanes 0 .. K-1 load them in one round trip, then the workgroup merges the units
// that valid ones open, in order.  Every holder's descriptor (worker waves' shares, then pool
// pieces) is written on every call, zeroed when it opens no split unit (including the waves
// past the step's work and the pool pieces the step does not use), so no other check is
// needed.
//
// With xcd_local, the workgroups that merge the worker waves' shares run on the XCDs that ran
// those waves.  The attention kernel gives XCD x the holders [x W/8, (x+1) W/8), and workgroup i
// goes to XCD i % 8, so workgroup i = 8 j + x (j < W/(8K)) takes the shares' descriptor group
// x W/(8K) + j and the rest take the pool pieces' groups in the same XCD-contiguous way.  The map
// is a permutation of the workgroups: which workgroup merges a unit changes, its result does not.
template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void attn_combine_kernel(const AttnParams P, int K, int xcd_local) {
  __shared__ float s_ml[NW][64][2];
  __shared__ float4 s_acc[NW][D / 64][64];
  const int lane = threadIdx.x & 63;
  int g = blockIdx.x;
  if (xcd_local) {
    const int G = (int)gridDim.x, nS = P.W / K;
    if (G % 8 == 0 && P.W % (8 * K) == 0 && nS <= G) {
      const int x = g % 8, j = g / 8, s = nS / 8;
      g = j < s ? x * s + j : nS + x * ((G - nS) / 8) + (j - s);
    }
  }
  const int w0 = g * K;
  const int nd = min(K, P.NH - w0);
  if (blockIdx.x == 0 && threadIdx.x == 0) P.hdr->pool_next = 0;   // the next step starts with a full pool
  int4 e0 = make_int4(0, 0, 0, 0), e1 = make_int4(0, 0, 0, 0);
  if (lane < nd) {
    const int4* dp = reinterpret_cast<const int4*>(P.desc) + 2 * (w0 + lane);
    e0 = dp[0];
    e1 = dp[1];
  }
  for (int i = 0; i < nd; ++i) {
    if (__builtin_amdgcn_readlane(e1.z, i) == 0) continue;
    const int4 d0 = make_int4(__builtin_amdgcn_readlane(e0.x, i), __builtin_amdgcn_readlane(e0.y, i),
                              __builtin_amdgcn_readlane(e0.z, i), __builtin_amdgcn_readlane(e0.w, i));
    const int4 d1 = make_int4(__builtin_amdgcn_readlane(e1.x, i), __builtin_amdgcn_readlane(e1.y, i), 1, 0);
    combine_unit<D, NW>(P, w0 + i, d0, d1, s_ml, s_acc);
  }
}

}  // namespace

hipError_t launch_attn_combine(const AttnParams& p, int D, int num_cus, bool xcd_local, hipStream_t stream) {
  // waves per workgroup: 2 for 16-row units (decode), 8 for 32-row units, 16 for 64-row units.
  // Most descriptors are empty; for decode batches the smaller workgroups measured faster
  // (less to dispatch, and four quads need no more waves).  K descriptors per workgroup keep
  // the grid within two residency rounds at 16 waves per CU (the D = 128 kernel's register
  // budget allows 4 waves per SIMD): a workgroup merges its units one after another, and
  // halving K from one round's worth took 4 us off the mixed batch's combine (more units in
  // flight at once); two-wave workgroups take at least 2 (fewer workgroups to dispatch
  // measured slightly faster).  xcd_local (decode- and verify-shaped batches) took about 1 us
  // off the verify step; the mixed and tree batches, whose prefill-like units sit on a few
  // XCDs, merged faster spread over all of them.
  const int nw = p.RG > 32 ? 16 : (p.RG > 16 ? 8 : 2);
  const long long resident = (long long)std::max(1, num_cus) * 16 * 2;
  const int K = (int)std::min<long long>(64, std::max<long long>(nw == 2 ? 2 : 1, ((long long)p.NH * nw + resident - 1) / resident));
  const dim3 grid((unsigned)((p.NH + K - 1) / K)), block(64 * nw);
  if (D == 64) {
    if (nw == 16) hipLaunchKernelGGL((attn_combine_kernel<64, 16>), grid, block, 0, stream, p, K, xcd_local ? 1 : 0);
    else if (nw == 8) hipLaunchKernelGGL((attn_combine_kernel<64, 8>), grid, block, 0, stream, p, K, xcd_local ? 1 : 0);
    else hipLaunchKernelGGL((attn_combine_kernel<64, 2>), grid, block, 0, stream, p, K, xcd_local ? 1 : 0);
  } else if (D == 128) {
    if (nw == 16) hipLaunchKernelGGL((attn_combine_kernel<128, 16>), grid, block, 0, stream, p, K, xcd_local ? 1 : 0);
    else if (nw == 8) hipLaunchKernelGGL((attn_combine_kernel<128, 8>), grid, block, 0, stream, p, K, xcd_local ? 1 : 0);
    else hipLaunchKernelGGL((attn_combine_kernel<128, 2>), grid, block, 0, stream, p, K, xcd_local ? 1 : 0);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace vap
