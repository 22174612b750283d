// Main attention kernel of paged_attn_step (gfx950); partials of split units are merged by
// the combine kernel (attn_combine.hip).
//
// What is computed: for every query row of every sequence, softmax(scale * q k^T) v over the
// keys the row may see, reading K and V through the sequence's block table (position j lives
// in pool block table[j / block_size] at row j % block_size -- tempatgunting.com article,
// section "Anatomy of the KV Cache: Memory Layout, Paging and Quantization Trade-offs").  Row
// i of a sequence with ctx_len L and q_len Q sees keys 0 .. L-Q+i, so k+1 verify rows equal
// k+1 sequential decode steps (syslabs.in "Continuous Batching and Speculative Decoding: How
// Modern LLM Serving Engines Actually Work", section "The core idea").
//
// How (MI355X-first):
//  * Every workgroup of the main kernel first rebuilds the step's plan in LDS from
//    q_lens/ctx_lens (validation, packed-row offsets, per-sequence work); batches above 2048
//    sequences take the plan from a separate plan kernel instead.
//  * The work -- ceil(L/BS) KV blocks for each (sequence, KV head, row group) unit -- is split
//    evenly in blocks over W persistent worker waves, W being the number of waves the GPU
//    holds resident at once, so long-tail sequences spread over many waves and every CU
//    streams the same number of bytes.  A wave covers consecutive units and may cover only
//    part of one; then it writes a partial (running max, running sum, unnormalised rows) and
//    the combine kernel merges the partials of each split unit in wave order (flash-decoding's
//    combine) and writes its rows.
//  * One wave processes all rows of a unit at once: the G query heads of a GQA group times
//    the q_len rows, up to 16 * NRT rows (NRT = 1, 2 or 4 row tiles: decode, verify / mixed,
//    and batches averaging 48 or more rows per KV head such as token trees and prefill
//    chunks).  Every K and V byte a unit needs is loaded once from HBM, straight into MFMA
//    operand registers (16 bytes per lane per load), and serves all those rows.  A wave keeps
//    two 16-token tiles in flight (a two-stage register pipeline); three waves per CU (twice
//    that for prefill-heavy batches) already saturate the memory system for this access
//    pattern.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_16x16x32_bf16: the K tile is
//    the A operand (lane = token, 16 contiguous bytes per lane), the query rows the B operand.
//    Each lane then holds one query row and four tokens, so a row's softmax statistics live
//    in the four lanes {c, c+16, c+32, c+48}: a row max takes two cross-lane exchanges and the
//    accumulator rescale is lane-local.
//  * The output is accumulated transposed too, O^T += V^T P^T (v_mfma_f32_16x16x16bf16_1k):
//    the S^T accumulator already is the P^T operand; P (fp32) is split into bf16 hi + lo parts
//    that together keep ~16 mantissa bits; V^T comes from the 16-byte V loads by byte
//    permutes.  P never leaves registers.
//  * Only edge tiles (segment end, causal region of verify/prefill rows) are masked, and the
//    masking is select-based: tokens past the segment -- including a block's unused tail,
//    which may hold anything, even NaN -- get probability 0 and a zeroed V operand.
#include "attn_internal.h"

#include <type_traits>

// Tuning knobs: waves per SIMD the register allocation must allow (occupancy).
#ifndef VAP_ATTN_WAVES_1RT
#define VAP_ATTN_WAVES_1RT 3     // waves per SIMD with one 16-row tile per unit
#endif
#ifndef VAP_ATTN_WAVES_2RT
#define VAP_ATTN_WAVES_2RT 2     // waves per SIMD with two 16-row tiles per unit
#endif
// P.V of units with an even number of 16-row tiles (bf16 cache) on the 32x32x16 bf16 MFMA
#ifndef VAP_PV32
#define VAP_PV32 1
#endif

namespace vap {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x16(uint2 a, uint2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}
// gfx950 runs this one at the full bf16 rate (16x16x16 above at half of it)
__device__ __forceinline__ f32x16 mfma32x32x16(uint4 a, uint4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Output accumulators of a unit of NRT 16-row tiles.  16x16 layout: lane (c, g) holds rows
// 16 rt + c, dims (D/16)(4g + r) + jt in v[rt][jt][r].  32x32 layout (PV32, NRT even): lane
// (h, a, c) = 32 h + 16 a + c holds row 32 rp + 16 a + c in v[rp][jt][4q + e], dim
// (D/2)(q & 1) + (D/4) h + (D/16) e + 2 jt + (q >> 1).
template <int D, int NRT, bool PV32>
struct Acc {
  f32x4 v[NRT][D / 16];
};
template <int D, int NRT>
struct Acc<D, NRT, true> {
  f32x16 v[NRT / 2][D / 32];
};
template <int NRT, bool KV8>
constexpr bool pv32() { return VAP_PV32 != 0 && !KV8 && NRT % 2 == 0; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Keeps the instruction scheduler from moving code across a pipeline stage boundary (it would
// otherwise hoist a tile's math up to its loads and serialise the pipeline).
__device__ __forceinline__ void stage_fence() { __builtin_amdgcn_sched_barrier(0); }

// ---------------------------------------------------------------------------------------
// in-workgroup plan
// ---------------------------------------------------------------------------------------

// A lane's value moved by DPP (row shifts and broadcasts, a VALU operand modifier) in 32-bit
// pieces; lanes without a source, or outside ROW_MASK, read 0
template <int CTRL, int ROW_MASK, typename T>
__device__ __forceinline__ T dpp_move(T x) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit values");
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROW_MASK, 0xf, false));
  } else {
    const unsigned long long u = __builtin_bit_cast(unsigned long long, x);
    const unsigned lo = (unsigned)__builtin_amdgcn_update_dpp(0, (int)(unsigned)u, CTRL, ROW_MASK, 0xf, false);
    const unsigned hi = (unsigned)__builtin_amdgcn_update_dpp(0, (int)(unsigned)(u >> 32), CTRL, ROW_MASK, 0xf, false);
    return __builtin_bit_cast(T, ((unsigned long long)hi << 32) | lo);
  }
}

// Exclusive workgroup scan of one integer per thread (DPP steps inside each wave: 1, 2, 4 and 8
// lanes within 16-lane rows, then the row totals).  s_tmp is written before the barrier and read
// after it; the caller puts a barrier between this and the next write of s_tmp.
template <typename T>
__device__ __forceinline__ T wg_exclusive_scan(T x, T* s_tmp, T& total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;        // waves in this workgroup (at most kWavesPerWG)
  T incl = x;
  incl += dpp_move<0x111, 0xf>(incl);    // row_shr:1
  incl += dpp_move<0x112, 0xf>(incl);    // row_shr:2
  incl += dpp_move<0x114, 0xf>(incl);    // row_shr:4
  incl += dpp_move<0x118, 0xf>(incl);    // row_shr:8
  incl += dpp_move<0x142, 0xa>(incl);    // row_bcast:15 into rows 1 and 3
  incl += dpp_move<0x143, 0xc>(incl);    // row_bcast:31 into rows 2 and 3
  if (lane == 63) s_tmp[wv] = incl;
  __syncthreads();
  T before = 0;
  total = 0;
#pragma unroll
  for (int i = 0; i < kWavesPerWG; ++i) {
    if (i < nw) {
      if (i < wv) before += s_tmp[i];
      total += s_tmp[i];
    }
  }
  return before + incl - x;
}


__device__ void build_plan_lds(const AttnParams& P, int* s_L, int* s_Q, int* s_qoff, int* s_off) {
  __shared__ long long s_t64[kWavesPerWG];
  __shared__ int s_t32[kWavesPerWG];
  const int tid = threadIdx.x;
  const long long cap = (long long)P.MB * P.BS;
  long long carry_q = 0;
  int carry_w = 0;
  int err = 0;
  for (int base = 0; base < P.B; base += (int)blockDim.x) {
    const int s = base + tid;
    int Q = 0, L = 0;
    if (s < P.B) {
      Q = P.q_lens[s];
      L = P.ctx_lens[s];
    }
    const long long qc = (s < P.B && Q > 0) ? (long long)Q : 0;
    long long qtot;
    const long long qoff = wg_exclusive_scan<long long>(qc, s_t64, qtot) + carry_q;
    bool valid = false;
    if (s < P.B) {
      if (Q < 1 || L < Q || (long long)L > cap) err |= VAP_DERR_LENS;
      else if (qoff + Q > P.total_q) err |= VAP_DERR_TOTAL_Q;
      else valid = true;
    }
    const int work = valid ? (P.UH + (L + P.BS - 1) / P.BS) * ((P.G * Q + P.RG - 1) / P.RG) * P.Hkv : 0;
    int wtot;
    const int woff = wg_exclusive_scan<int>(work, s_t32, wtot) + carry_w;
    if (s < P.B) {
      s_L[s] = valid ? L : 0;
      s_Q[s] = valid ? Q : 1;
      s_qoff[s] = valid ? (int)qoff : 0;
      s_off[s] = woff;
    }
    carry_q += qtot;
    carry_w += wtot;
    __syncthreads();                     // s_t64 and s_t32 are written again by the next pass
  }
  if (tid == 0) {
    s_off[P.B] = carry_w;
    if (carry_q != (long long)P.total_q) err |= VAP_DERR_TOTAL_Q;
  }
  if (err && blockIdx.x == 0) atomicOr(&P.hdr->err, err);
  __syncthreads();
}

// ---------------------------------------------------------------------------------------
// one 16-token tile: loads and math
// ---------------------------------------------------------------------------------------

// A tile is 16 consecutive tokens of one block (tiles start at multiples of 16).
//   K: the A operands of S^T = K Q^T (v_mfma_f32_16x16x32_bf16) are, at lane (c, g), token c,
//      dims 32*kk + 8*g .. +7; in S^T lane (c, g) then holds row c at tokens 4g + r.  At
//      D = 128 (bf16) K is loaded like V -- lane (c, g) loads tokens 4g + r, bytes 16c .. +15,
//      so each load instruction reads four whole 256-byte head rows -- and reaches the operand
//      layout through a wave-private LDS tile (kKViaLds below).  Loaded directly in the operand
//      layout, each instruction reads 64 bytes of 16 rows (half cache lines), which measured
//      about 11% slower in a no-math gather over a decode batch (5.9 against 6.6 TB/s).
//   V: lane (c, g) loads, for its tokens 4g + r (r = 0..3), the D/16 consecutive dims
//      (D/16)*c .. +D/16-1 (16 bytes at D = 128, 8 at D = 64).
//   Output tile jt (16 dims x 16 rows) holds dim (D/16)*m + jt at its row m, so lane (c, g)'s
//   V^T operand for tile jt (v_mfma_f32_16x16x16bf16_1k, k-slots 4g + r = tokens 4g + r) is
//   16-bit word jt of its four V loads, and its P^T operand is exactly its four S^T values.
constexpr int kTile = 16;
constexpr int kXCDs = 8;    // accelerator complex dies of an MI355X, each with its own L2

template <int D, bool KV8>
struct KVTile;

template <int D>
struct KVTile<D, false> {
  bf16x8 ka[D / 32];       // K: operand layout, or (kKViaLds at D = 128) as loaded, ka[r] = tokens 4g + r
  uint32_t vw[4][D / 32];
};

#ifndef VAP_K_VIA_LDS
#define VAP_K_VIA_LDS 1
#endif
constexpr bool kKViaLds = VAP_K_VIA_LDS != 0;
constexpr int kKRow = 17;   // LDS row of one token: 16 chunks of 16 bytes and one chunk of padding

template <int D>
constexpr bool k_via_lds() { return kKViaLds && D == 128; }

// 8-bit cache: lane (c, g) holds the K codes of token c, dims (D/4) g .. +D/4-1; the V codes of
// tokens 4g + r, dims (D/16) c .. +D/16-1; and (k_scale, k_zero, v_scale, v_zero) of tokens
// 4g + r (r = 0..3).
template <int D>
struct KVTile<D, true> {
  uint32_t kc[D / 16];
  uint32_t vc[4][D / 64];
  float4 sc[4];
};

// Raw buffer loads: the tile's block base lives in a buffer resource in scalar registers (it
// is uniform over the wave), so a lane needs one 32-bit offset register per plane instead of
// a 64-bit address per load.  Loads past the resource's range return zeros.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
constexpr int kBufFlags = 0x00020000;   // raw (untyped) dword access
// Cache policy of the bf16 K/V loads of a unit that is the only reader of its K/V (its
// sequence's rows for that KV head fit one unit, as in decode and verify batches):
// non-temporal (nt).  Those bytes are read once per step, and streaming reads with this
// policy run markedly closer to the HBM peak on MI355X than default-policy reads.  Units
// whose K/V other units of the same step read again (prefill chunks split into several row
// groups) keep the default policy, so the re-reads can hit in L2.  The 8-bit cache measured
// no gain from nt and keeps the default.
#ifndef VAP_KV_LOAD_POLICY
#define VAP_KV_LOAD_POLICY 2
#endif
#ifndef VAP_KV8_LOAD_POLICY
#define VAP_KV8_LOAD_POLICY 0
#endif
#ifndef VAP_KV8_SCALE_POLICY
#define VAP_KV8_SCALE_POLICY 0
#endif
constexpr int kKVOnce = VAP_KV_LOAD_POLICY;
constexpr int kKV8 = VAP_KV8_LOAD_POLICY;
constexpr int kKV8S = VAP_KV8_SCALE_POLICY;

// base and bytes are uniform over the wave; readfirstlane states it, so the resource stays in
// scalar registers (a resource the compiler thinks divergent costs a loop around every load)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* ub = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, __builtin_amdgcn_readfirstlane(bytes), kBufFlags);
}

// vo_k = c * tok_bytes + 16 * g, vo_v = 4 * g * tok_bytes + 2 * (D/16) * c: fixed per lane.
// A tile that is not live gets an empty range: its loads return zeros without a memory access,
// which lets the pipelined loop issue loads unconditionally.
template <int D, int BS, int POLICY>
__device__ __forceinline__ void load_tile(KVTile<D, false>& t, const uint16_t* kbase, const uint16_t* vbase,
                                          long long tok_stride, int tg, int blk, int vo_k, int vo_v, bool live) {
  constexpr int NKK = D / 32;
  const long long row0 = (long long)blk * BS + (tg % BS);
  const int tok_bytes = (int)tok_stride * 2;
  const int range = live ? kTile * tok_bytes : 0;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + row0 * tok_stride, range);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + row0 * tok_stride, range);
  if constexpr (k_via_lds<D>()) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      t.ka[r] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, vo_v, r * tok_bytes, POLICY));
  } else {
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      t.ka[kk] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, vo_k + 64 * kk, 0, POLICY));
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if constexpr (D == 128) {
      const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rv, vo_v, r * tok_bytes, POLICY);
      t.vw[r][0] = x[0]; t.vw[r][1] = x[1]; t.vw[r][2] = x[2]; t.vw[r][3] = x[3];
    } else {
      const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(rv, vo_v, r * tok_bytes, POLICY);
      t.vw[r][0] = x[0]; t.vw[r][1] = x[1];
    }
  }
}

// 8-bit tile: codes and scales through buffer resources built from the wave-uniform block
// base (empty range when the tile is not live).  vo_k = c * tok_bytes + (D/4) g,
// vo_v = 4 g * tok_bytes + (D/16) c, vo_s = 64 g; sblk = floats per block of the scale array.
template <int D, int BS>
__device__ __forceinline__ void load_tile8(KVTile<D, true>& t, const uint8_t* kbase, const uint8_t* vbase,
                                           const float* sbase, long long sblk, int tok_bytes, int tg, int blk,
                                           int vo_k, int vo_v, int vo_s, bool live) {
  const long long row0 = (long long)blk * BS + (tg % BS);
  const int range = live ? kTile * tok_bytes : 0;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + row0 * tok_bytes, range);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + row0 * tok_bytes, range);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(sbase + (long long)blk * sblk + (tg % BS) * 4, live ? kTile * 16 : 0);
#pragma unroll
  for (int h = 0; h < D / 64; ++h) {
    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rk, vo_k + 16 * h, 0, kKV8);
    t.kc[4 * h] = x[0]; t.kc[4 * h + 1] = x[1]; t.kc[4 * h + 2] = x[2]; t.kc[4 * h + 3] = x[3];
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if constexpr (D == 128) {
      const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(rv, vo_v, r * tok_bytes, kKV8);
      t.vc[r][0] = x[0]; t.vc[r][1] = x[1];
    } else {
      t.vc[r][0] = __builtin_amdgcn_raw_buffer_load_b32(rv, vo_v, r * tok_bytes, kKV8);
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r)
    t.sc[r] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rs, vo_s, 16 * r, kKV8S));
}

// Which keys a lane's rows may see: key positions up to lim (L - Q + the row's node index), and
// of the new rows (positions >= base = L - Q) only those set in the row's tree mask (all ones
// for causal rows).
template <int NRT>
struct RowVis {
  int lim[NRT];
  uint64_t tmask[NRT];
  int base;
  __device__ __forceinline__ bool sees(int rt, int tok) const {
    return tok <= lim[rt] && (tok < base || ((tmask[rt] >> ((tok - base) & 63)) & 1ull));
  }
};

// Max over the four lanes {c, c+16, c+32, c+48} holding one row: two lane swaps (odd/even
// 16-lane rows, then the two 32-lane halves), no LDS round trip.
__device__ __forceinline__ float row_max4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// x0 on the lanes of even 16-lane rows, x1 on odd rows, for per-row values that all lanes (c, g)
// of one c hold alike (row maxima, sums, output rows): the odd rows take x1 from their even
// neighbour.  A plain select between two array elements would be turned into a dynamic index,
// which puts the array in scratch memory.
__device__ __forceinline__ uint32_t pick_row(uint32_t x0, uint32_t x1) {
  return __builtin_amdgcn_permlane16_swap(x0, x1, false, false)[0];
}
__device__ __forceinline__ float pick_row(float x0, float x1) {
  return __uint_as_float(pick_row(__float_as_uint(x0), __float_as_uint(x1)));
}

// two floats to packed bf16, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Softmax reference: a row's exponentials are taken against m_run, which moves only when the
// row's running max exceeds it by more than kRescaleLog2 (so P <= 2^kRescaleLog2); the
// running sum and the accumulator always share m_run, so the result is the same up to
// rounding, and most tiles skip the accumulator rescale.
constexpr float kRescaleLog2 = 8.f;

template <int D, int NRT, bool MASKED, bool PV32>
__device__ __forceinline__ void compute_tile(const KVTile<D, false>& t, int tg, int t_end, const RowVis<NRT>& vis,
                                             const bf16x8 (&qb)[NRT][D / 32], float scale_log2,
                                             float (&m_run)[NRT], float (&l_run)[NRT],
                                             Acc<D, NRT, PV32>& acc, int g, uint4* klds) {
  constexpr int NKK = D / 32;
  constexpr int NJT = D / 16;
  // K in the operand layout: through this wave's LDS tile when it was loaded as whole rows
  // (written and read back by the same wave: its LDS accesses complete in order, no barrier)
  bf16x8 ka[NKK];
  if constexpr (k_via_lds<D>()) {
    const int c = threadIdx.x & 15;
#pragma unroll
    for (int r = 0; r < 4; ++r) klds[(4 * g + r) * kKRow + c] = __builtin_bit_cast(uint4, t.ka[r]);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) ka[kk] = as_bf16x8(klds[c * kKRow + 4 * kk + g]);
  } else {
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) ka[kk] = t.ka[kk];
  }
  f32x4 sc[NRT];
  bool ok[NRT][4];
  float mx[NRT];
  bool grow = false;
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    sc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) sc[rt] = mfma16x16x32(ka[kk], qb[rt][kk], sc[rt]);
    float m = kNegInf;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (MASKED) {
        const int tok = tg + 4 * g + r;
        ok[rt][r] = (tok < t_end) && vis.sees(rt, tok);
        m = ok[rt][r] ? fmaxf(m, sc[rt][r]) : m;
      } else {
        m = fmaxf(m, sc[rt][r]);
      }
    }
    mx[rt] = row_max4(m) * scale_log2;     // scale_log2 > 0
    grow = grow || (mx[rt] > m_run[rt] + kRescaleLog2);
  }
  if (__builtin_amdgcn_ballot_w64(grow) != 0) {   // uniform branch
    float alpha[NRT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      const float m_new = fmaxf(m_run[rt], mx[rt]);
      alpha[rt] = (m_new == kNegInf) ? 1.f : fast_exp2(m_run[rt] - m_new);
      l_run[rt] *= alpha[rt];
      m_run[rt] = m_new;
    }
    if constexpr (PV32) {
#pragma unroll
      for (int rp = 0; rp < NRT / 2; ++rp) {
        const float al = pick_row(alpha[2 * rp], alpha[2 * rp + 1]);   // this lane's row: tile 2 rp + (g & 1)
#pragma unroll
        for (int jt = 0; jt < D / 32; ++jt) acc.v[rp][jt] *= al;
      }
    } else {
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int jt = 0; jt < NJT; ++jt) acc.v[rt][jt] *= alpha[rt];
    }
  }
  uint2 ph[NRT], pl[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const float ref = (m_run[rt] == kNegInf) ? 0.f : m_run[rt];
    float pv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pv[r] = fast_exp2(sc[rt][r] * scale_log2 - ref);
      if (MASKED) pv[r] = ok[rt][r] ? pv[r] : 0.f;
    }
    l_run[rt] += (pv[0] + pv[1]) + (pv[2] + pv[3]);
    // P = hi + lo, both bf16: ~16 significant bits for the output product
    const uint32_t h01 = pack_bf16(pv[0], pv[1]), h23 = pack_bf16(pv[2], pv[3]);
    const uint32_t l01 = pack_bf16(pv[0] - __uint_as_float(h01 << 16), pv[1] - __uint_as_float(h01 & 0xffff0000u));
    const uint32_t l23 = pack_bf16(pv[2] - __uint_as_float(h23 << 16), pv[3] - __uint_as_float(h23 & 0xffff0000u));
    ph[rt] = make_uint2(h01, h23);
    pl[rt] = make_uint2(l01, l23);
  }
  if constexpr (PV32) {
    // O^T (32 dims x 32 rows) += V^T (32 dims x 16 tokens) P^T (16 tokens x 32 rows).  Lane
    // (h, a, c) supplies tokens 8h .. 8h+7: P^T of row 16a + c of the pair, and V of dim
    // (D/16) c + 2 jt + a.  It holds tokens 8h + 4a .. +3 of both tiles' rows c and both dims,
    // so one swap between 16-lane rows a = 0 and a = 1 completes each operand.
    uint4 pbh[NRT / 2], pbl[NRT / 2];
#pragma unroll
    for (int rp = 0; rp < NRT / 2; ++rp) {
      const auto h0 = __builtin_amdgcn_permlane16_swap(ph[2 * rp].x, ph[2 * rp + 1].x, false, false);
      const auto h1 = __builtin_amdgcn_permlane16_swap(ph[2 * rp].y, ph[2 * rp + 1].y, false, false);
      const auto l0 = __builtin_amdgcn_permlane16_swap(pl[2 * rp].x, pl[2 * rp + 1].x, false, false);
      const auto l1 = __builtin_amdgcn_permlane16_swap(pl[2 * rp].y, pl[2 * rp + 1].y, false, false);
      pbh[rp] = make_uint4(h0[0], h1[0], h0[1], h1[1]);
      pbl[rp] = make_uint4(l0[0], l1[0], l0[1], l1[1]);
    }
#pragma unroll
    for (int jt = 0; jt < D / 32; ++jt) {
      uint32_t src[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        src[r] = t.vw[r][jt];
        if (MASKED) src[r] = (tg + 4 * g + r < t_end) ? src[r] : 0u;
      }
      // even dim (kept by a = 0) and odd dim (kept by a = 1) of this lane's four tokens
      const auto e0 = __builtin_amdgcn_permlane16_swap(__builtin_amdgcn_perm(src[1], src[0], 0x05040100u),
                                                       __builtin_amdgcn_perm(src[1], src[0], 0x07060302u), false, false);
      const auto e1 = __builtin_amdgcn_permlane16_swap(__builtin_amdgcn_perm(src[3], src[2], 0x05040100u),
                                                       __builtin_amdgcn_perm(src[3], src[2], 0x07060302u), false, false);
      const uint4 va = make_uint4(e0[0], e1[0], e0[1], e1[1]);
#pragma unroll
      for (int rp = 0; rp < NRT / 2; ++rp) {
        acc.v[rp][jt] = mfma32x32x16(va, pbh[rp], acc.v[rp][jt]);
        acc.v[rp][jt] = mfma32x32x16(va, pbl[rp], acc.v[rp][jt]);
      }
    }
  } else {
#pragma unroll
    for (int jt = 0; jt < NJT; ++jt) {
      const uint32_t sel = (jt & 1) ? 0x07060302u : 0x05040100u;
      uint32_t src[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        src[r] = t.vw[r][jt >> 1];
        if (MASKED) src[r] = (tg + 4 * g + r < t_end) ? src[r] : 0u;
      }
      const uint2 vt = make_uint2(__builtin_amdgcn_perm(src[1], src[0], sel), __builtin_amdgcn_perm(src[3], src[2], sel));
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        acc.v[rt][jt] = mfma16x16x16(vt, ph[rt], acc.v[rt][jt]);
        acc.v[rt][jt] = mfma16x16x16(vt, pl[rt], acc.v[rt][jt]);
      }
    }
  }
}

// Sum over the four lanes {c, c+16, c+32, c+48} holding one row (fixed order).
__device__ __forceinline__ float row_sum4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// byte i of w as a float (an 8-bit code is exact in fp32 and in bf16)
__device__ __forceinline__ float code_f32(uint32_t w, int i) { return (float)((w >> (8 * i)) & 0xffu); }

// The four codes of a word as floats: unsigned integers (8-bit cache) or, for F8, E4M3 values
// (the FP8 cache; gfx950's packed conversion decodes OCP E4M3, two codes per instruction).  Both
// are exact in bf16, so the tile's bf16 MFMAs stay exact in their inputs.
template <bool F8>
__device__ __forceinline__ void codes_f32(uint32_t w, float (&f)[4]) {
  if constexpr (F8) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    f[0] = lo[0]; f[1] = lo[1]; f[2] = hi[0]; f[3] = hi[1];
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = code_f32(w, i);
  }
}

// Two E4M3 codes (bytes 0-1, or 2-3 for HI) of a word straight to two bf16 values: gfx950's
// scaled conversion with scale 1.  A probe on the GPU matched it bit for bit against the f32
// conversion then rounding to bf16 on all 256 codes; every E4M3 value is exact in bf16.
template <bool HI>
__device__ __forceinline__ uint32_t fp8_pair_bf16(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, HI));
}

// One tile of the 8-bit cache.  With x = s (c - z) per token: the score of token j is
// s_k,j (q.c_j - z_k,j sum(q)), so the K codes go to the MFMA as they are (exact in bf16) and
// the per-token scale is applied to the 16 scores; the output is
// sum_j p_j s_v,j c_j - sum_j p_j s_v,j z_v,j, so P is scaled by s_v per token and the second
// sum is kept per row (o_run, subtracted at the end).
template <int D, int NRT, bool MASKED, bool F8>
__device__ __forceinline__ void compute_tile8(const KVTile<D, true>& t, int tg, int t_end, const RowVis<NRT>& vis,
                                              const bf16x8 (&qb)[NRT][D / 32], const float (&qsum)[NRT],
                                              float scale_log2, float (&m_run)[NRT], float (&l_run)[NRT],
                                              float (&o_run)[NRT], f32x4 (&acc)[NRT][D / 16], int g) {
  constexpr int NKK = D / 32;
  constexpr int NJT = D / 16;
  bf16x8 ka[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    uint4 u;
    if constexpr (F8) {
      u = make_uint4(fp8_pair_bf16<false>(t.kc[2 * kk]), fp8_pair_bf16<true>(t.kc[2 * kk]),
                     fp8_pair_bf16<false>(t.kc[2 * kk + 1]), fp8_pair_bf16<true>(t.kc[2 * kk + 1]));
    } else {
      float a[4], b[4];
      codes_f32<F8>(t.kc[2 * kk], a);
      codes_f32<F8>(t.kc[2 * kk + 1], b);
      u = make_uint4(pack_bf16(a[0], a[1]), pack_bf16(a[2], a[3]), pack_bf16(b[0], b[1]), pack_bf16(b[2], b[3]));
    }
    ka[kk] = as_bf16x8(u);
  }
  float sv[NRT][4];
  bool ok[NRT][4];
  float mx[NRT];
  bool grow = false;
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    f32x4 raw = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) raw = mfma16x16x32(ka[kk], qb[rt][kk], raw);
    float m = kNegInf;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sv[rt][r] = t.sc[r].x * fmaf(-t.sc[r].y, qsum[rt], raw[r]);
      if (MASKED) {
        const int tok = tg + 4 * g + r;
        ok[rt][r] = (tok < t_end) && vis.sees(rt, tok);
        m = ok[rt][r] ? fmaxf(m, sv[rt][r]) : m;
      } else {
        m = fmaxf(m, sv[rt][r]);
      }
    }
    mx[rt] = row_max4(m) * scale_log2;
    grow = grow || (mx[rt] > m_run[rt] + kRescaleLog2);
  }
  if (__builtin_amdgcn_ballot_w64(grow) != 0) {   // uniform branch
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      const float m_new = fmaxf(m_run[rt], mx[rt]);
      const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m_run[rt] - m_new);
      l_run[rt] *= alpha;
      o_run[rt] *= alpha;
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt) acc[rt][jt] *= alpha;
      m_run[rt] = m_new;
    }
  }
  uint2 ph[NRT], pl[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const float ref = (m_run[rt] == kNegInf) ? 0.f : m_run[rt];
    float pv[4], pw[4];
    float o = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pv[r] = fast_exp2(sv[rt][r] * scale_log2 - ref);
      pw[r] = pv[r] * t.sc[r].z;
      float oz = pw[r] * t.sc[r].w;
      if (MASKED) {
        pv[r] = ok[rt][r] ? pv[r] : 0.f;
        pw[r] = ok[rt][r] ? pw[r] : 0.f;
        oz = ok[rt][r] ? oz : 0.f;
      }
      o += oz;
    }
    l_run[rt] += (pv[0] + pv[1]) + (pv[2] + pv[3]);
    o_run[rt] += o;
    const uint32_t h01 = pack_bf16(pw[0], pw[1]), h23 = pack_bf16(pw[2], pw[3]);
    const uint32_t l01 = pack_bf16(pw[0] - __uint_as_float(h01 << 16), pw[1] - __uint_as_float(h01 & 0xffff0000u));
    const uint32_t l23 = pack_bf16(pw[2] - __uint_as_float(h23 << 16), pw[3] - __uint_as_float(h23 & 0xffff0000u));
    ph[rt] = make_uint2(h01, h23);
    pl[rt] = make_uint2(l01, l23);
  }
#pragma unroll
  for (int jt = 0; jt < NJT; ++jt) {
    uint2 vt;
    if constexpr (F8) {
      // byte jt % 4 of tokens r = 0, 1 (and 2, 3) side by side, with the next byte after them,
      // so one conversion gives the pair for dim jt and the other for dim jt + 1
      const int wi = jt >> 2, kb = jt & 2;
      const uint32_t sel = (uint32_t)kb | ((uint32_t)(4 + kb) << 8) | ((uint32_t)(kb + 1) << 16) |
                           ((uint32_t)(5 + kb) << 24);
      const uint32_t w01 = __builtin_amdgcn_perm(t.vc[1][wi], t.vc[0][wi], sel);
      const uint32_t w23 = __builtin_amdgcn_perm(t.vc[3][wi], t.vc[2][wi], sel);
      vt = (jt & 1) ? make_uint2(fp8_pair_bf16<true>(w01), fp8_pair_bf16<true>(w23))
                    : make_uint2(fp8_pair_bf16<false>(w01), fp8_pair_bf16<false>(w23));
    } else {
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float f[4];
        codes_f32<F8>(t.vc[r][jt >> 2], f);
        v[r] = f[jt & 3];
      }
      vt = make_uint2(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]));
    }
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      acc[rt][jt] = mfma16x16x16(vt, ph[rt], acc[rt][jt]);
      acc[rt][jt] = mfma16x16x16(vt, pl[rt], acc[rt][jt]);
    }
  }
}

// ---------------------------------------------------------------------------------------
// one segment: a contiguous block range of one unit
// ---------------------------------------------------------------------------------------

struct Segment {
  int s, kvh, rg, unit, ub, seg, nb, soff;
  int L, Q, qoff;
  bool whole;
  int slot;   // 0 = first segment of this wave, 1 = its last
};

// A unit split across waves is merged by the combine kernel; the wave holding its first block
// describes it (the others' segments follow in waves wa+1 .. wb, each in slot 0).
struct SplitDesc {
  int kvh, rg, qoff, Q;   // to place the unit's rows
  int wb, slot_a, valid, pad;
};

// Lane (c, g) holds, for row rt*16+c, dim (D/16)*(4g + r) + jt in acc[rt][jt][r]: for each r,
// D/16 consecutive dims starting at (D/4)*g + (D/16)*r.
template <int D, int NRT>
__device__ __forceinline__ void write_rows(float* out, const int (&out_row)[NRT], const f32x4 (&acc)[NRT][D / 16],
                                           const float (&lsum)[NRT], int g) {
  constexpr int NJT = D / 16;
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    if (out_row[rt] >= 0) {
      const float inv = 1.f / lsum[rt];
      float* op = out + (long long)out_row[rt] * D + (D / 4) * g;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int j4 = 0; j4 < NJT; j4 += 4) {
          *reinterpret_cast<float4*>(op + NJT * r + j4) =
              make_float4(acc[rt][j4][r] * inv, acc[rt][j4 + 1][r] * inv, acc[rt][j4 + 2][r] * inv,
                          acc[rt][j4 + 3][r] * inv);
        }
      }
    }
  }
}

// One row pair of 32x32 accumulators (PV32): lane (h, a, c) writes its row's dims (D/2) b +
// (D/4) h + (D/16) e + o for b < 2, e < 4, o < D/16 (element o of that run is v[o >> 1]
// [4 (2 (o & 1) + b) + e]) at row + (D/4) h.  Output rows are scaled by 1/l, partials by 1.
template <int D>
__device__ __forceinline__ void store_row32(float* row, const f32x16 (&v)[D / 32], float mul, int lane) {
  float* op = row + (D / 4) * (lane >> 5);
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int o = 0; o < D / 16; o += 4) {
        const f32x4 x = {v[o >> 1][4 * b + e], v[o >> 1][4 * (2 + b) + e], v[(o >> 1) + 1][4 * b + e],
                         v[(o >> 1) + 1][4 * (2 + b) + e]};
        *reinterpret_cast<f32x4*>(op + (D / 2) * b + (D / 16) * e + o) = x * mul;
      }
}

template <int D, int NRT>
__device__ __forceinline__ void unit_rows(const AttnParams& P, int kvh, int rg, int Q, int qoff, int c,
                                          int (&out_row)[NRT], int& nrows) {
  const int G = P.G;
  nrows = min(16 * NRT, G * Q - rg * 16 * NRT);
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const int r = rt * 16 + c;
    const int row = rg * 16 * NRT + r;
    const int i = row / G;
    out_row[rt] = (r < nrows) ? (qoff + i) * P.Hq + kvh * G + (row - i * G) : -1;
  }
}

template <int D, int BS, int NRT, bool KV8, bool ONCE, bool F8 = false>
__device__ void process_segment(const AttnParams& P, const Segment& sg, int h, int W, int T1, int PS,
                                int lane, int c, int g, SplitDesc& desc, uint4* klds) {
  constexpr int NKK = D / 32;
  constexpr int NJT = D / 16;
  constexpr int RG = 16 * NRT;
  constexpr bool PV32 = pv32<NRT, KV8>();
  const int G = P.G;
  const int row0 = sg.rg * RG;
  const int t_start = sg.ub * BS;
  const int t_end = min(sg.L, (sg.ub + sg.seg) * BS);
  // tokens <= full_until are visible to every row (tree rows: the committed prefix only)
  const int full_until = P.tree_mask ? sg.L - sg.Q - 1 : sg.L - sg.Q;
  const int32_t* trow = P.tables + (long long)sg.s * P.MB;
  const long long tok_stride = (long long)P.Hkv * D;
  const uint16_t* kbase = P.kpool + (long long)sg.kvh * D;
  const uint16_t* vbase = P.vpool + (long long)sg.kvh * D;
  const int vo_k = KV8 ? c * (int)tok_stride + (D / 4) * g : c * (int)tok_stride * 2 + 16 * g;
  const int vo_v = KV8 ? 4 * g * (int)tok_stride + (D / 16) * c : 4 * g * (int)tok_stride * 2 + 2 * (D / 16) * c;
  const int jend = sg.ub + sg.seg;
  // 8-bit cache: codes have the bf16 pool's shape with one byte per element
  const uint8_t* kbase8 = KV8 ? P.kcodes + (long long)sg.kvh * D : nullptr;
  const uint8_t* vbase8 = KV8 ? P.vcodes + (long long)sg.kvh * D : nullptr;
  const float* sbase8 = KV8 ? P.kv_scales + (long long)sg.kvh * BS * 4 : nullptr;
  const long long sblk = (long long)P.Hkv * BS * 4;
  const int vo_s = 64 * g;

  int out_row[NRT];
  int nrows;
  unit_rows<D, NRT>(P, sg.kvh, sg.rg, sg.Q, sg.qoff, c, out_row, nrows);

  // query rows of this unit as B operands: lane holds row rt*16+c, dims 32*kk + 8*g .. +7
  // (8-bit cache: dims (D/4)*g + 8*kk .. +7, matching the K code layout), and for the 8-bit
  // cache the row sums of q (the zero points' term of the scores)
  bf16x8 qb[NRT][NKK];
  float qsum[NRT];
  RowVis<NRT> vis;
  vis.base = sg.L - sg.Q;
  int derr = 0;
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const int node = (row0 + rt * 16 + c) / G;
    vis.lim[rt] = sg.L - sg.Q + node;
    vis.tmask[rt] = ~0ull;
    if (P.tree_mask != nullptr && out_row[rt] >= 0) {
      // a tree row sees itself and nodes before it only (topological order, at most 64 nodes)
      const uint64_t m = P.tree_mask[sg.qoff + node];
      const uint64_t allowed = (node >= 63) ? ~0ull : ((2ull << node) - 1);
      if (sg.Q > 64) {
        derr |= VAP_DERR_TREE;                 // cannot be a tree: keep the row causal
      } else {
        if (!((m >> node) & 1ull) || (m & ~allowed)) derr |= VAP_DERR_TREE;
        vis.tmask[rt] = (m & allowed) | (1ull << node);
      }
    }
    const uint16_t* qp = P.q + (long long)(out_row[rt] >= 0 ? out_row[rt] : 0) * D + (KV8 ? (D / 4) * g : 8 * g);
    float qs = 0.f;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const uint4 v = out_row[rt] >= 0 ? ld16(qp + (KV8 ? 8 * kk : 32 * kk)) : make_uint4(0, 0, 0, 0);
      qb[rt][kk] = as_bf16x8(v);
      if constexpr (KV8) {
        const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) qs += __uint_as_float(wv[e] << 16) + __uint_as_float(wv[e] & 0xffff0000u);
      }
    }
    qsum[rt] = KV8 ? row_sum4(qs) : 0.f;
  }

  float m_run[NRT], l_run[NRT], o_run[NRT];
  Acc<D, NRT, PV32> acc;
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    m_run[rt] = kNegInf;
    l_run[rt] = 0.f;
    o_run[rt] = 0.f;
  }
  if constexpr (PV32) {
#pragma unroll
    for (int rp = 0; rp < NRT / 2; ++rp)
#pragma unroll
      for (int jt = 0; jt < D / 32; ++jt) acc.v[rp][jt] = f32x16{};
  } else {
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt) acc.v[rt][jt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // The tile loop walks the segment in windows of 64 KV blocks.  A window's pool block ids are
  // loaded once (one per lane) before its tiles, so no vector load inside the tile loop depends
  // on a branch.
  constexpr int kWinBlocks = 64;
  constexpr int kWinTiles = kWinBlocks * BS / kTile;
  const int ntiles = (t_end - t_start + kTile - 1) / kTile;
  // Tiles that need no mask form a prefix: tile i (first token t_start + 16 i) needs none when
  // it ends inside the segment and every row sees all its tokens.
  const int last_free = min(t_end - kTile, full_until - (kTile - 1)) - t_start;
  const int n_unmasked = last_free < 0 ? 0 : min(ntiles, last_free / kTile + 1);
  for (int wt = 0; wt < ntiles; wt += kWinTiles) {
    const int wbase = sg.ub + wt * kTile / BS;    // first block of the window
    int win;
    {
      const int j = wbase + lane;
      win = (j < jend) ? trow[j] : 0;
      if (j < jend && (unsigned)win >= (unsigned)P.num_blocks) {
        derr |= VAP_DERR_BLOCK_ID;
        win = 0;
      }
    }
    const int nt = min(kWinTiles, ntiles - wt);
    const int tw0 = t_start + wt * kTile;          // first token of the window
    auto issue = [&](KVTile<D, KV8>& X, int i, bool live) {
      const int ic = min(i, nt - 1);
      const int tg = tw0 + ic * kTile;
      const int blk = __builtin_amdgcn_readlane(win, tg / BS - wbase);
      if constexpr (KV8)
        load_tile8<D, BS>(X, kbase8, vbase8, sbase8, sblk, (int)tok_stride, tg, blk, vo_k, vo_v, vo_s, live);
      else
        load_tile<D, BS, ONCE ? kKVOnce : 0>(X, kbase, vbase, tok_stride, tg, blk, vo_k, vo_v, live);
    };
    auto compute = [&](const KVTile<D, KV8>& X, int i, auto masked) {
      if constexpr (KV8)
        compute_tile8<D, NRT, decltype(masked)::value, F8>(X, tw0 + i * kTile, t_end, vis, qb, qsum, P.scale_log2,
                                                       m_run, l_run, o_run, acc.v, g);
      else
        compute_tile<D, NRT, decltype(masked)::value, PV32>(X, tw0 + i * kTile, t_end, vis, qb, P.scale_log2, m_run,
                                                            l_run, acc, g, klds);
    };
    // Unmasked tiles first, then the masked suffix: two loops rather than a branch per tile,
    // which would make the compiler keep a second copy of the accumulators.  Both loops are
    // one two-stage pipeline: tile i+1 is in flight while tile i is computed, across the hand-
    // over too (the unmasked loop's last issue loads the first masked tile); the two buffers
    // rotate and every load is issued unconditionally (a tile that is not live gets an empty
    // range), so the compiler never has to drain the load counter at a branch.
    const int nu = min(nt, max(0, n_unmasked - wt));
    if constexpr (!KV8) {
      KVTile<D, KV8> ta, tb;
      issue(ta, 0, true);
      int i = 0;
      for (; i + 1 < nu; i += 2) {      // both tiles of a pair are always computed
        issue(tb, i + 1, true);
        stage_fence();
        compute(ta, i, std::false_type{});
        stage_fence();
        issue(ta, i + 2, i + 2 < nt);   // the next pair's first tile, the odd last one, or a masked one
        stage_fence();
        compute(tb, i + 1, std::false_type{});
        stage_fence();
      }
      if (i < nu) {                     // the odd last unmasked tile; the first masked one goes in flight
        issue(tb, i + 1, i + 1 < nt);
        stage_fence();
        compute(ta, i, std::false_type{});
        stage_fence();
        ta = tb;
        ++i;
      }
      // ta holds tile i, the first masked tile (if any)
      for (; i + 1 < nt; i += 2) {
        issue(tb, i + 1, true);
        stage_fence();
        compute(ta, i, std::true_type{});
        stage_fence();
        issue(ta, i + 2, i + 2 < nt);
        stage_fence();
        compute(tb, i + 1, std::true_type{});
        stage_fence();
      }
      if (i < nt) compute(ta, i, std::true_type{});
    } else {
      // 8-bit cache: the masked tiles one at a time (a second buffer there spills registers)
      if (nu > 0) {
        KVTile<D, KV8> ta, tb;
        issue(ta, 0, true);
        int i = 0;
        for (; i + 1 < nu; i += 2) {
          issue(tb, i + 1, true);
          stage_fence();
          compute(ta, i, std::false_type{});
          stage_fence();
          issue(ta, i + 2, i + 2 < nu);
          stage_fence();
          compute(tb, i + 1, std::false_type{});
          stage_fence();
        }
        if (i < nu) compute(ta, i, std::false_type{});
      }
      for (int i = nu; i < nt; ++i) {
        KVTile<D, KV8> t0;
        issue(t0, i, true);
        compute(t0, i, std::true_type{});
      }
    }
  }
  if (derr) atomicOr(&P.hdr->err, derr);      // any lane: errors are per table entry / row

  float lsum[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    float l = l_run[rt];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    lsum[rt] = l;
    if constexpr (KV8) {            // subtract the zero points' share from every output dim
      const float osum = row_sum4(o_run[rt]);
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt) acc.v[rt][jt] -= osum;
    }
  }
  if constexpr (PV32) {
    // lane (h, a, c) holds row 32 rp + 16 a + c of the unit, that is row c of tile 2 rp + a
    if (sg.whole) {
#pragma unroll
      for (int rp = 0; rp < NRT / 2; ++rp) {
        const int orow = (int)pick_row((uint32_t)out_row[2 * rp], (uint32_t)out_row[2 * rp + 1]);
        if (orow >= 0)
          store_row32<D>(P.out + (long long)orow * D, acc.v[rp], 1.f / pick_row(lsum[2 * rp], lsum[2 * rp + 1]), lane);
      }
      return;
    }
    // partial: this segment's (max, sum, unnormalised rows) in its slot, natural dim order; the
    // combine kernel reads them after this kernel has finished
#pragma unroll
    for (int rp = 0; rp < NRT / 2; ++rp) {
      const int r_in_unit = 32 * rp + 16 * (g & 1) + c;
      if (r_in_unit < nrows) {
        const long long prow = ((long long)h * 2 + sg.slot) * RG + r_in_unit;
        store_row32<D>(P.part_acc + prow * D, acc.v[rp], 1.f, lane);
        if (lane < 32)
          P.part_ml[prow] = make_float2(pick_row(m_run[2 * rp], m_run[2 * rp + 1]), pick_row(lsum[2 * rp], lsum[2 * rp + 1]));
      }
    }
  } else {
    if (sg.whole) {
      write_rows<D, NRT>(P.out, out_row, acc.v, lsum, g);
      return;
    }
    // partial: store this segment's (max, sum, unnormalised rows) in its slot, rows in natural
    // dim order; the combine kernel reads them after this kernel has finished
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      const int r_in_unit = rt * 16 + c;
      if (r_in_unit < nrows) {
        const long long prow = ((long long)h * 2 + sg.slot) * RG + r_in_unit;
        float* pp = P.part_acc + prow * D + (D / 4) * g;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
          for (int j4 = 0; j4 < NJT; j4 += 4)
            *reinterpret_cast<float4*>(pp + NJT * r + j4) =
                make_float4(acc.v[rt][j4][r], acc.v[rt][j4 + 1][r], acc.v[rt][j4 + 2][r], acc.v[rt][j4 + 3][r]);
        }
        if (g == 0) P.part_ml[prow] = make_float2(m_run[rt], lsum[rt]);
      }
    }
  }
  if (sg.ub == 0) {
    // this holder opens the unit: holders h .. wb hold its segments, this one in slot sg.slot;
    // wb holds the unit's last block x = U1 - 1 (a wave's share below T1, a pool piece above)
    const long long U1 = (long long)sg.soff + (long long)(sg.unit + 1) * (P.UH + sg.nb);
    desc.kvh = sg.kvh;
    desc.rg = sg.rg;
    desc.qoff = sg.qoff;
    desc.Q = sg.Q;
    desc.wb = (U1 <= T1) ? (int)((U1 * W - 1) / T1) : W + (int)((U1 - 1 - T1) / PS);
    desc.slot_a = sg.slot;
    desc.valid = 1;
  }
}

template <int D, int BS, int NRT, bool LDS_PLAN, bool KV8, bool F8>
__global__ __launch_bounds__(kAttnThreads, NRT == 1 ? VAP_ATTN_WAVES_1RT : (NRT == 2 ? VAP_ATTN_WAVES_2RT : 1)) void attn_main_kernel(const AttnParams P) {
  extern __shared__ int s_mem[];
  // each wave's K transpose tile (bf16 cache at D = 128 only)
  __shared__ uint4 s_klds[(!KV8 && k_via_lds<D>()) ? kWavesPerWG * kTile * kKRow : 1];
  uint4* const klds = s_klds + ((!KV8 && k_via_lds<D>()) ? (threadIdx.x >> 6) * kTile * kKRow : 0);
  const int lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  // Holder of this wave, XCD-aware: the GPU dispatches workgroup i to XCD i % kXCDs, and each XCD
  // has its own L2, so each XCD takes a contiguous range of holders.  Units that read the same K/V
  // (the row groups of a prefill chunk's KV head) are consecutive in work order and then share
  // one L2.  Which wave runs which holder changes nothing else (results are bitwise the same).
  int wg = blockIdx.x;
  if (gridDim.x % kXCDs == 0) wg = (int)(blockIdx.x % kXCDs) * (int)(gridDim.x / kXCDs) + (int)(blockIdx.x / kXCDs);
  const int w = uniform(wg * (blockDim.x >> 6) + (threadIdx.x >> 6));

  // per-sequence tables: in this workgroup's LDS (ds_read, counted apart from the vector loads
  // in flight) or, for very large batches, in global memory written by the plan kernel
  if constexpr (LDS_PLAN) build_plan_lds(P, s_mem, s_mem + P.B, s_mem + 2 * P.B, s_mem + 3 * P.B);
  auto plan_L = [&](int i) { if constexpr (LDS_PLAN) return s_mem[i]; else return P.g_L[i]; };
  auto plan_Q = [&](int i) { if constexpr (LDS_PLAN) return s_mem[P.B + i]; else return P.g_Q[i]; };
  auto plan_qoff = [&](int i) { if constexpr (LDS_PLAN) return s_mem[2 * P.B + i]; else return P.q_off[i]; };
  auto plan_off = [&](int i) { if constexpr (LDS_PLAN) return s_mem[3 * P.B + i]; else return P.seq_off[i]; };

  const int TB = uniform(plan_off(P.B));
  const int W = min(P.W, TB);
  if (LDS_PLAN && blockIdx.x == 0 && threadIdx.x == 0) P.hdr->total_work = TB;
  // Pool: the last NP pieces of PS work blocks, for bf16 steps of 16-row units with at least
  // 32 work blocks per wave (then W = P.W and the pool holders W .. W+NP-1 follow the last
  // share's holder directly)
  const int PS = max(1, P.pool_piece);
  int NP = 0;
  if (LDS_PLAN && !KV8 && NRT == 1 && P.pool_max > 0 && TB >= 32 * P.W)
    NP = min(P.pool_max, (int)((long long)TB * P.pool_pct / 100) / PS);
  const int T1 = TB - NP * PS;
  // descriptors of the pool holders this step leaves unused (every holder's is written)
  for (int hh = P.W + NP + w; hh < P.NH; hh += P.W)
    if (lane == 0) reinterpret_cast<int4*>(P.desc)[2 * hh + 1] = make_int4(0, 0, 0, 0);
  if (w >= W) {                          // no workgroup barrier below this point
    if (lane == 0) reinterpret_cast<int4*>(P.desc)[2 * w + 1] = make_int4(0, 0, 0, 0);
    return;
  }

  // This wave's own share (holder w), then pool pieces (holder W + k) while any are left: one
  // range per pass, so the segment code is instantiated once.
  int h = w;
  long long b0 = (long long)w * T1 / W;
  long long b1 = (long long)(w + 1) * T1 / W;
  while (true) {
    int s;
    if constexpr (LDS_PLAN) {
      int lo = 0, hi = P.B;              // largest s with off[s] <= b0
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (plan_off(mid) <= b0) lo = mid; else hi = mid - 1;
      }
      s = uniform(lo);
    } else {
      s = uniform(P.wave_seq[w]);        // (no pool on this path: b0 is this wave's share)
    }

    SplitDesc desc = {0, 0, 0, 0, 0, 0, 0, 0};
    int pos = (int)b0;
    bool first = true;
    while (pos < b1) {
      const int soff = uniform(plan_off(s));
      const int send = uniform(plan_off(s + 1));
      if (pos >= send) { ++s; continue; }
      Segment sg;
      sg.s = s;
      sg.L = uniform(plan_L(s));
      sg.Q = uniform(plan_Q(s));
      sg.qoff = uniform(plan_qoff(s));
      sg.soff = soff;
      sg.nb = (sg.L + BS - 1) / BS;
      const int ns = P.UH + sg.nb;        // work blocks per unit
      const int nrg = (P.G * sg.Q + 16 * NRT - 1) / (16 * NRT);
      const int local = pos - soff;
      sg.unit = local / ns;
      const int uoff = local - sg.unit * ns;
      if (uoff < P.UH) {                  // inside the unit's virtual blocks: start at its KV
        pos += P.UH - uoff;
        continue;
      }
      sg.ub = uoff - P.UH;
      sg.seg = min(sg.nb - sg.ub, (int)(b1 - pos));
      sg.kvh = sg.unit / nrg;
      sg.rg = sg.unit - sg.kvh * nrg;
      sg.whole = (sg.ub == 0) && (sg.seg == sg.nb);
      sg.slot = first ? 0 : 1;
      if constexpr (KV8)
        process_segment<D, BS, NRT, true, false, F8>(P, sg, h, W, T1, PS, lane, c, g, desc, klds);
      else if (nrg > 1)                   // K/V read again by the sequence's other row groups
        process_segment<D, BS, NRT, false, false>(P, sg, h, W, T1, PS, lane, c, g, desc, klds);
      else
        process_segment<D, BS, NRT, false, true>(P, sg, h, W, T1, PS, lane, c, g, desc, klds);
      pos += sg.seg;
      first = false;
    }
    if (lane == 0) {
      int4* dp = reinterpret_cast<int4*>(P.desc) + 2 * h;
      dp[0] = make_int4(desc.kvh, desc.rg, desc.qoff, desc.Q);
      dp[1] = make_int4(desc.wb, desc.slot_a, desc.valid, 0);
    }
    if (NP == 0) return;
    int k = 0;
    if (lane == 0) k = __hip_atomic_fetch_add(&P.hdr->pool_next, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    k = uniform(__shfl(k, 0));
    if (k >= NP) return;
    h = W + k;
    b0 = T1 + (long long)k * PS;
    b1 = b0 + PS;
  }
}

template <int D, int BS, int NRT, bool LDS_PLAN, bool KV8, bool F8>
hipError_t launch_main_t(const AttnParams& p, int num_wg, int wg_waves, hipStream_t stream, KTimer t) {
  const size_t lds = LDS_PLAN ? attn_main_lds_bytes(p.B) : 0;
  hipExtLaunchKernelGGL((attn_main_kernel<D, BS, NRT, LDS_PLAN, KV8, F8>), dim3(num_wg), dim3(64 * wg_waves),
                        (uint32_t)lds, stream, t.start, t.stop, 0, p);
  return hipGetLastError();
}

}  // namespace

size_t attn_main_lds_bytes(int B) { return size_t(4 * B + 1) * sizeof(int); }

#define VAP_ATTN_VARIANTS(X) \
  X(64, 16, 1) X(64, 16, 2) X(64, 16, 4) X(64, 32, 1) X(64, 32, 2) X(64, 32, 4) \
  X(128, 16, 1) X(128, 16, 2) X(128, 16, 4) X(128, 32, 1) X(128, 32, 2) X(128, 32, 4)

// kv: 0 = bf16 cache, 1 = 8-bit integer codes, 2 = FP8 (E4M3) codes
template <int d, int bs, int nrt, bool lds>
hipError_t launch_main_kv(const AttnParams& p, int kv, int num_wg, int wg_waves, hipStream_t stream, KTimer t) {
  if (kv == 1) return launch_main_t<d, bs, nrt, lds, true, false>(p, num_wg, wg_waves, stream, t);
  if (kv == 2) return launch_main_t<d, bs, nrt, lds, true, true>(p, num_wg, wg_waves, stream, t);
  return launch_main_t<d, bs, nrt, lds, false, false>(p, num_wg, wg_waves, stream, t);
}

hipError_t launch_attn_main(const AttnParams& p, int D, int BS, int NRT, int kv, int num_wg, int wg_waves,
                            hipStream_t stream, KTimer t) {
  if (wg_waves < 1 || wg_waves > kWavesPerWG) return hipErrorInvalidValue;
  const bool lds = p.B <= kLdsPlanMaxSeqs;
#define X(d, bs, nrt)                                                                           \
  if (D == d && BS == bs && NRT == nrt)                                                         \
    return lds ? launch_main_kv<d, bs, nrt, true>(p, kv, num_wg, wg_waves, stream, t)           \
               : launch_main_kv<d, bs, nrt, false>(p, kv, num_wg, wg_waves, stream, t);
  VAP_ATTN_VARIANTS(X)
#undef X
  return hipErrorInvalidValue;
}

const void* attn_main_kernel_ptr(int D, int BS, int NRT, bool lds_plan, bool kv8) {
#define X(d, bs, nrt)                                                                          \
  if (D == d && BS == bs && NRT == nrt) {                                                      \
    if (kv8)                                                                                   \
      return lds_plan ? reinterpret_cast<const void*>(&attn_main_kernel<d, bs, nrt, true, true, false>) \
                      : reinterpret_cast<const void*>(&attn_main_kernel<d, bs, nrt, false, true, false>); \
    return lds_plan ? reinterpret_cast<const void*>(&attn_main_kernel<d, bs, nrt, true, false, false>) \
                    : reinterpret_cast<const void*>(&attn_main_kernel<d, bs, nrt, false, false, false>); \
  }
  VAP_ATTN_VARIANTS(X)
#undef X
  return nullptr;
}

}  // namespace vap
