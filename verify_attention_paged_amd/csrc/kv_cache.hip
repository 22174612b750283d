// Writing a step's new K/V rows into the paged cache, and committing the accepted draft tokens
// after verification (gfx950).
//
// kv_append (tempatgunting.com article, section "Anatomy of the KV Cache: Memory Layout, Paging
// and Quantization Trade-offs"): the q_len new tokens of a sequence whose context length L
// already counts them sit at positions L - q_len .. L - 1, position j in row j % block_size of
// pool block table[j / block_size].  Their K and V rows ([total_q][Hkv][D] bf16, packed by
// sequence like the query rows) are written there.  For an 8-bit cache (same article, section
// "Quantization and Precision Choices for KV": per-token scales, asymmetric, separate for K and
// V) every (token, KV head) row of K and of V is quantised on its own in fp32:
//     lo = min(0, min x), hi = max(0, max x), scale = max((hi - lo) / 255, FLT_EPSILON),
//     zero = clamp(rint((0 - lo) / scale), 0, 255), code = clamp(rint(x * (1 / scale)) + zero, 0, 255)
// (IEEE division, round-half-even), and (scale, zero) stored beside the codes.
//
// kv_commit (same article, section "Speculative Decoding: Turning Verification Parallelism into
// Latency Wins": the KV of rejected draft tokens is rolled back): after verifying q_len rows with
// n drafts accepted the context becomes L - q_len + 1 + n.  For a draft tree the accepted nodes
// a_1 < ... < a_n are first moved from positions L - q_len + a_i to L - q_len + i, so that the
// kept tokens are contiguous; a chain needs no move.
//
// How.  Append: one launch; every workgroup first builds the exclusive prefix of q_lens in LDS
// (row r of the packed batch belongs to the sequence whose range holds r: binary search in LDS),
// then its waves take (row, head group) items with a grid stride.  A head row of D elements is
// spread over D/8 lanes holding 8 elements (16 bytes) of K and of V; the 8-bit path reduces min
// and max over those lanes with cross-lane shuffles.  Commit: one workgroup per sequence; the
// moved rows are staged through LDS in passes (all loads of a pass land before any store), and
// passes follow row order.  Row i's destination L - q_len + i can equal only the source of an
// earlier row j < i (a_j = i, since a_j >= j), which an earlier or the same pass has already
// read, so no source is overwritten before it is read.
#include <cfloat>

#include "vap_internal.h"

namespace vap {
namespace {

constexpr int kAppendThreads = 256;
constexpr int kCommitThreads = 256;
constexpr int kCommitStageChunks = 2048;   // 32 KB of 16-byte chunks staged per pass
constexpr int kAppendStagedSeqs = 4096;    // batches up to this size keep first new positions in LDS

__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ void unpack8(const uint4& u, float* x) {
  x[0] = bf16_lo(u.x); x[1] = bf16_hi(u.x);
  x[2] = bf16_lo(u.y); x[3] = bf16_hi(u.y);
  x[4] = bf16_lo(u.z); x[5] = bf16_hi(u.z);
  x[6] = bf16_lo(u.w); x[7] = bf16_hi(u.w);
}

// Affine uint8 quantisation of one head row spread over LPH lanes (8 elements each).
// Returns the 8 codes packed little-endian and the row's scale and zero point.
template <int LPH>
__device__ __forceinline__ uint2 quantize8(const float* x, float* scale_out, float* zero_out) {
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) {
    mn = fminf(mn, x[j]);
    mx = fmaxf(mx, x[j]);
  }
#pragma unroll
  for (int d = LPH / 2; d >= 1; d >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, d));
    mx = fmaxf(mx, __shfl_xor(mx, d));
  }
  const float lo = fminf(mn, 0.f);
  const float hi = fmaxf(mx, 0.f);
  const float scale = fmaxf((hi - lo) / 255.f, FLT_EPSILON);
  const float zero = fminf(fmaxf(rintf((0.f - lo) / scale), 0.f), 255.f);   // 0 - lo: +0 when lo = 0
  const float inv = 1.f / scale;
  uint32_t c[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) c[j] = (uint32_t)fminf(fmaxf(rintf(x[j] * inv) + zero, 0.f), 255.f);
  *scale_out = scale;
  *zero_out = zero;
  return make_uint2(c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24), c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24));
}

// s_start[s] = sum of clamp(q_lens[r], 0, T + 1) over r < s, saturated at T + 1, for s = 0 .. B.
// With s_base != nullptr also s_base[s] = ctx_len - q_len (the first new position), or -1 when the
// sequence's lengths are inconsistent.  Returns the unsaturated total on every thread.
__device__ long long build_row_starts(const KVAppendParams& p, int32_t* s_start, int32_t* s_base,
                                      long long* s_wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int B = p.B, T = p.T;
  for (int s = tid; s < B; s += kAppendThreads) {
    const int Q = p.q_lens[s];
    s_start[s] = min(max(Q, 0), T + 1);
    if (s_base != nullptr) {
      const int L = p.ctx_lens[s];
      s_base[s] = (Q >= 1 && Q <= L && (L - 1) / p.BS + 1 <= p.MB) ? L - Q : -1;
    }
  }
  __syncthreads();
  const int span = (B + kAppendThreads - 1) / kAppendThreads;
  const int s0 = tid * span;
  long long local = 0;
  for (int j = 0; j < span; ++j)
    if (s0 + j < B) local += s_start[s0 + j];
  long long incl = local;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const long long t = __shfl_up(incl, d);
    if (lane >= d) incl += t;
  }
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  long long run = incl - local, total = 0;
  for (int w = 0; w < kAppendThreads / 64; ++w) {
    if (w < wave) run += s_wsum[w];
    total += s_wsum[w];
  }
  for (int j = 0; j < span; ++j) {
    const int s = s0 + j;
    if (s < B) {
      const int qv = s_start[s];
      s_start[s] = (int)min(run, (long long)T + 1);
      run += qv;
    }
  }
  if (tid == 0) s_start[B] = (int)min(total, (long long)T + 1);
  __syncthreads();
  return total;
}

template <int D, bool U8>
__global__ __launch_bounds__(kAppendThreads) void kv_append_kernel(KVAppendParams p) {
  extern __shared__ int32_t s_lds[];     // [B + 1] row starts, then [B] first new positions
  __shared__ long long s_wsum[kAppendThreads / 64];
  constexpr int LPH = D / 8;             // lanes per head row
  constexpr int HPP = 64 / LPH;          // heads per wave pass
  const int lane = threadIdx.x & 63;
  const int B = p.B, T = p.T, Hkv = p.Hkv, BS = p.BS;
  const bool staged = B <= kAppendStagedSeqs;
  int32_t* s_start = s_lds;
  int32_t* s_base = staged ? s_lds + B + 1 : nullptr;

  const int passes = (Hkv + HPP - 1) / HPP;
  const long long items = (long long)T * passes;
  const int g = lane / LPH, sub = lane % LPH;
  const size_t plane = (size_t)p.NB * BS * Hkv * D;
  const long long stride = (long long)gridDim.x * (kAppendThreads / 64);
  long long it = (long long)blockIdx.x * (kAppendThreads / 64) + (threadIdx.x >> 6);
  // an item's new rows do not depend on the lengths: the first item's loads start before the scan
  auto load_rows = [&](long long item, uint4& k, uint4& v) {
    const int r = (int)(item / passes);
    const int h = (int)(item % passes) * HPP + g;
    if (item < items && h < Hkv) {
      const size_t src = ((size_t)r * Hkv + h) * D + sub * 8;
      k = *reinterpret_cast<const uint4*>(p.k_new + src);
      v = *reinterpret_cast<const uint4*>(p.v_new + src);
    }
  };
  uint4 kin = make_uint4(0, 0, 0, 0), vin = make_uint4(0, 0, 0, 0);
  load_rows(it, kin, vin);
  const long long total = build_row_starts(p, s_start, s_base, s_wsum);
  int derr = 0;
  if (blockIdx.x == 0 && threadIdx.x == 0 && total != T) derr |= VAP_DERR_TOTAL_Q;

  for (bool first = true; it < items; it += stride, first = false) {
    if (!first) load_rows(it, kin, vin);
    const int r = wave_uniform((int)(it / passes));
    const int h = (int)(it % passes) * HPP + g;
    if (r >= s_start[B]) continue;       // the lengths cover fewer rows than total_q
    int lo = 0, hi = B;                  // s_start[lo] <= r < s_start[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_start[mid] <= r) lo = mid; else hi = mid;
    }
    const int s = wave_uniform(lo);
    int base;
    if (staged) {
      base = s_base[s];
    } else {
      const int L = p.ctx_lens[s], Q = p.q_lens[s];
      base = (Q >= 1 && Q <= L && (L - 1) / BS + 1 <= p.MB) ? L - Q : -1;
    }
    base = wave_uniform(base);
    if (base < 0) {
      derr |= VAP_DERR_LENS;
      continue;
    }
    const int pos = base + r - s_start[s];
    const int blk = p.tables[(size_t)s * p.MB + pos / BS];
    if (blk < 0 || blk >= p.NB) {
      derr |= VAP_DERR_BLOCK_ID;
      continue;
    }
    if (h >= Hkv) continue;
    const int row = pos % BS;
    const size_t dst = (((size_t)blk * BS + row) * Hkv + h) * D + sub * 8;
    if constexpr (!U8) {
      uint16_t* pool = static_cast<uint16_t*>(p.kv);
      *reinterpret_cast<uint4*>(pool + dst) = kin;
      *reinterpret_cast<uint4*>(pool + plane + dst) = vin;
    } else {
      uint8_t* codes = static_cast<uint8_t*>(p.kv);
      float xk[8], xv[8];
      unpack8(kin, xk);
      unpack8(vin, xv);
      float ks, kz, vs, vz;
      const uint2 ck = quantize8<LPH>(xk, &ks, &kz);
      const uint2 cv = quantize8<LPH>(xv, &vs, &vz);
      *reinterpret_cast<uint2*>(codes + dst) = ck;
      *reinterpret_cast<uint2*>(codes + plane + dst) = cv;
      if (sub == 0)
        *reinterpret_cast<float4*>(p.kv_scales + (((size_t)blk * Hkv + h) * BS + row) * 4) = make_float4(ks, kz, vs, vz);
    }
  }
  if (derr) atomicOr(p.err, derr);
}

template <bool U8>
__global__ __launch_bounds__(kCommitThreads) void kv_commit_kernel(KVCommitParams p) {
  __shared__ int32_t s_src[kMaxTreeNodes], s_dst[kMaxTreeNodes];   // pool slots blk * BS + row
  __shared__ int32_t s_nmove, s_keep;
  __shared__ uint4 s_stage[kCommitStageChunks];
  const int s = blockIdx.x, tid = threadIdx.x;
  const int BS = p.BS;
  if (tid < 64) {
    // wave 0 reads the sequence's lengths and path (in one round of loads) and decides everything
    const int32_t* path = p.path != nullptr ? p.path + (size_t)s * p.path_stride : nullptr;
    const int a = (path != nullptr && tid < min(p.path_stride, 64)) ? path[tid] : 0;
    const int L = p.ctx_lens[s], Q = p.q_lens[s], n = p.n_accepted[s];
    int derr = 0;
    bool ok = Q >= 1 && Q <= L && (L - 1) / BS + 1 <= p.MB && n >= 0 && n <= Q - 1;
    if (!ok) derr |= VAP_DERR_LENS;
    if (ok && p.path != nullptr && (n > kMaxTreeNodes - 1 || n > p.path_stride)) {
      ok = false;
      derr |= VAP_DERR_TREE;
    }
    bool mv = false;
    int src = 0, dst = 0;
    const int prev = __shfl_up(a, 1);
    if (ok && path != nullptr && tid < n) {
      if (a <= (tid ? prev : 0) || a > Q - 1) {
        derr |= VAP_DERR_TREE;
      } else if (a != tid + 1) {
        const int ps = L - Q + a, pd = L - Q + tid + 1;
        const int bs_ = p.tables[(size_t)s * p.MB + ps / BS];
        const int bd = p.tables[(size_t)s * p.MB + pd / BS];
        if (bs_ < 0 || bs_ >= p.NB || bd < 0 || bd >= p.NB) {
          derr |= VAP_DERR_BLOCK_ID;
        } else {
          mv = true;
          src = bs_ * BS + ps % BS;
          dst = bd * BS + pd % BS;
        }
      }
    }
    const bool any_err = __ballot(derr != 0) != 0;
    const uint64_t m = __ballot(mv);
    if (mv) {
      const int idx = __popcll(m & ((1ull << tid) - 1));
      s_src[idx] = src;
      s_dst[idx] = dst;
    }
    if (tid == 0) {
      s_nmove = any_err ? 0 : __popcll(m);
      s_keep = (ok && !any_err) ? L - Q + 1 + n : L;
    }
    if (derr) atomicOr(p.err, derr);
  }
  __syncthreads();

  const int nmove = s_nmove;
  const int row_bytes = p.Hkv * p.D * (U8 ? 1 : 2);
  const int cpp = row_bytes / 16;                        // 16-byte chunks per row and plane
  const int cpr = 2 * cpp + (U8 ? p.Hkv : 0);            // + one float4 of scales per head
  const size_t plane = (size_t)p.NB * BS * row_bytes;
  char* kv = static_cast<char*>(p.kv);
  auto chunk = [&](int slot, int k) -> uint4* {
    if (k < 2 * cpp) {
      const int pl = k >= cpp;
      return reinterpret_cast<uint4*>(kv + pl * plane + (size_t)slot * row_bytes + (size_t)(k - pl * cpp) * 16);
    }
    const int h = k - 2 * cpp;
    return reinterpret_cast<uint4*>(p.kv_scales + (((size_t)(slot / BS) * p.Hkv + h) * BS + slot % BS) * 4);
  };
  const int total = nmove * cpr;
  for (int c0 = 0; c0 < total; c0 += kCommitStageChunks) {
    const int cend = min(total, c0 + kCommitStageChunks);
    for (int c = c0 + tid; c < cend; c += kCommitThreads) s_stage[c - c0] = *chunk(s_src[c / cpr], c % cpr);
    __syncthreads();
    for (int c = c0 + tid; c < cend; c += kCommitThreads) *chunk(s_dst[c / cpr], c % cpr) = s_stage[c - c0];
    __syncthreads();
  }
  if (tid == 0) p.out_lens[s] = s_keep;
}

}  // namespace

size_t kv_append_lds_bytes(int B) { return (size_t)(B + 1 + (B <= kAppendStagedSeqs ? B : 0)) * sizeof(int32_t); }

hipError_t launch_kv_append(const KVAppendParams& p, int D, bool u8, int num_wg, hipStream_t stream, KTimer t) {
  const uint32_t lds = (uint32_t)kv_append_lds_bytes(p.B);
  const dim3 grid((unsigned)num_wg), block(kAppendThreads);
  if (D == 128) {
    if (u8) hipExtLaunchKernelGGL((kv_append_kernel<128, true>), grid, block, lds, stream, t.start, t.stop, 0, p);
    else hipExtLaunchKernelGGL((kv_append_kernel<128, false>), grid, block, lds, stream, t.start, t.stop, 0, p);
  } else {
    if (u8) hipExtLaunchKernelGGL((kv_append_kernel<64, true>), grid, block, lds, stream, t.start, t.stop, 0, p);
    else hipExtLaunchKernelGGL((kv_append_kernel<64, false>), grid, block, lds, stream, t.start, t.stop, 0, p);
  }
  return hipGetLastError();
}

hipError_t launch_kv_commit(const KVCommitParams& p, bool u8, hipStream_t stream, KTimer t) {
  const dim3 grid((unsigned)p.B), block(kCommitThreads);
  if (u8) hipExtLaunchKernelGGL((kv_commit_kernel<true>), grid, block, 0, stream, t.start, t.stop, 0, p);
  else hipExtLaunchKernelGGL((kv_commit_kernel<false>), grid, block, 0, stream, t.start, t.stop, 0, p);
  return hipGetLastError();
}

}  // namespace vap
