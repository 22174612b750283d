// Attention kernel of paged_attn_step (gfx950).
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
//  * One launch.  Every workgroup first rebuilds the step's plan in LDS from q_lens/ctx_lens
//    (validation, packed-row offsets, per-sequence work); batches above 2048 sequences take
//    the plan from a separate plan kernel instead.
//  * The work -- ceil(L/BS) KV blocks for each (sequence, KV head, row group) unit -- is split
//    evenly in blocks over W persistent worker waves, so long-tail sequences spread over many
//    waves and every CU streams the same number of bytes.  A wave covers consecutive units and
//    may cover only part of one; then it writes a partial (running max, running sum,
//    unnormalised output) and the last wave of that unit to arrive merges the partials
//    (flash-decoding's combine, in wave order) and writes the output.  No second kernel.
//  * One wave processes all rows of a unit at once: the G query heads of a GQA group times
//    the q_len rows (up to 16 * NRT rows).  Every K and V byte is loaded once from HBM,
//    straight into MFMA operand registers, and serves all those rows.  The next 32-token tile
//    is loaded while the current one is computed (register double buffering).
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_16x16x32_bf16: the K tile is
//    the A operand (lane = token, 16 contiguous bytes per lane), the query rows the B operand.
//    Each lane then holds one query row and four tokens, so a row's softmax statistics live
//    in the four lanes {c, c+16, c+32, c+48}: a row max takes two cross-lane exchanges and the
//    accumulator rescale is lane-local.
//  * The output is accumulated transposed too, O^T += V^T P^T: P (fp32) is split into
//    bf16 hi + lo parts that together keep ~16 mantissa bits; V^T is built from 4-byte loads
//    (two dims of one token) with byte permutes.  P never leaves registers.
//  * Only edge tiles (segment end, causal region of verify/prefill rows) are masked, and the
//    masking is select-based: tokens past the segment -- including a block's unused tail,
//    which may hold anything, even NaN -- get probability 0 and a zeroed V operand.
#include "vap_internal.h"

// Tuning knobs: waves per SIMD the register allocation must allow (occupancy), and the depth
// of the register pipeline (tiles in flight per wave: 2 or 3).
#ifndef VAP_ATTN_WAVES_1RT
#define VAP_ATTN_WAVES_1RT 3     // waves per SIMD with one 16-row tile per unit
#endif
#ifndef VAP_ATTN_WAVES_2RT
#define VAP_ATTN_WAVES_2RT 2     // waves per SIMD with two 16-row tiles per unit
#endif
#ifndef VAP_ATTN_STAGES
#define VAP_ATTN_STAGES 1
#endif

namespace vap {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint2 ld8(const uint16_t* p) { return *reinterpret_cast<const uint2*>(p); }
__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x16(uint2 a, uint2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

// bf16 bits of a finite float, round to nearest even
__device__ __forceinline__ uint32_t bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// token offset (0..31 inside a 32-token tile) of element e of lane group g in the MFMA
// k-slots shared by the P^T (B) and V^T (A) operands of the output product
__device__ __forceinline__ int tile_token(int g, int e) { return (e < 4) ? (4 * g + e) : (12 + 4 * g + e); }

// ---------------------------------------------------------------------------------------
// in-workgroup plan
// ---------------------------------------------------------------------------------------

template <typename T>
__device__ __forceinline__ T wg_exclusive_scan(T x, T* s_tmp, T& total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  T incl = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const T y = __shfl_up(incl, d);
    if (lane >= d) incl += y;
  }
  if (lane == 63) s_tmp[wv] = incl;
  __syncthreads();
  T before = 0;
  total = 0;
#pragma unroll
  for (int i = 0; i < kWavesPerWG; ++i) {
    if (i < wv) before += s_tmp[i];
    total += s_tmp[i];
  }
  __syncthreads();
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
  for (int base = 0; base < P.B; base += kAttnThreads) {
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
    const int work = valid ? ((L + P.BS - 1) / P.BS) * ((P.G * Q + P.RG - 1) / P.RG) * P.Hkv : 0;
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
  }
  if (tid == 0) {
    s_off[P.B] = carry_w;
    if (carry_q != (long long)P.total_q) err |= VAP_DERR_TOTAL_Q;
  }
  if (err && blockIdx.x == 0) atomicOr(&P.hdr->err, err);
  __syncthreads();
}

// ---------------------------------------------------------------------------------------
// one 32-token tile: loads and math
// ---------------------------------------------------------------------------------------

// A tile is 16 consecutive tokens of one block (tiles start at multiples of 16).
//   K: lane (c, g) loads token c, dims 32*kk + 8*g .. +7 -> A operands of S^T = K Q^T
//      (v_mfma_f32_16x16x32_bf16); in S^T lane (c, g) then holds row c at tokens 4g + r.
//   V: lane (c, g) loads, for its tokens 4g + r (r = 0..3), the D/16 consecutive dims
//      (D/16)*c .. +D/16-1 (16 bytes at D = 128, 8 at D = 64).
//   Output tile jt (16 dims x 16 rows) holds dim (D/16)*m + jt at its row m, so lane (c, g)'s
//   V^T operand for tile jt (v_mfma_f32_16x16x16bf16_1k, k-slots 4g + r = tokens 4g + r) is
//   16-bit word jt of its four V loads, and its P^T operand is exactly its four S^T values.
constexpr int kTile = 16;

template <int D>
struct KVTile {
  bf16x8 ka[D / 32];
  uint32_t vw[4][D / 32];
};

template <int D, int BS>
__device__ __forceinline__ void load_tile(KVTile<D>& t, const uint16_t* kbase, const uint16_t* vbase,
                                          long long tok_stride, int tg, int blk, int c, int g) {
  constexpr int NKK = D / 32;
  const long long row0 = (long long)blk * BS + (tg % BS);
  const uint16_t* kp = kbase + (row0 + c) * tok_stride + 8 * g;
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) t.ka[kk] = as_bf16x8(ld16(kp + 32 * kk));
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint16_t* vp = vbase + (row0 + 4 * g + r) * tok_stride + (D / 16) * c;
    if constexpr (D == 128) {
      const uint4 x = ld16(vp);
      t.vw[r][0] = x.x; t.vw[r][1] = x.y; t.vw[r][2] = x.z; t.vw[r][3] = x.w;
    } else {
      const uint2 x = ld8(vp);
      t.vw[r][0] = x.x; t.vw[r][1] = x.y;
    }
  }
}

template <int D, int NRT, bool MASKED>
__device__ __forceinline__ void compute_tile(const KVTile<D>& t, int tg, int t_end, const int (&lim)[NRT],
                                             const bf16x8 (&qb)[NRT][D / 32], float scale_log2,
                                             float (&m_run)[NRT], float (&l_run)[NRT],
                                             f32x4 (&acc)[NRT][D / 16], int g) {
  constexpr int NKK = D / 32;
  constexpr int NJT = D / 16;
  uint2 ph[NRT], pl[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) sc = mfma16x16x32(t.ka[kk], qb[rt][kk], sc);
    float sv[4];
    bool ok[4];
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sv[r] = sc[r] * scale_log2;
      if (MASKED) {
        const int tok = tg + 4 * g + r;
        ok[r] = (tok < t_end) && (tok <= lim[rt]);
        mx = ok[r] ? fmaxf(mx, sv[r]) : mx;
      } else {
        mx = fmaxf(mx, sv[r]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run[rt], mx);
    const float ref = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run[rt] - ref);
    float pv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pv[r] = fast_exp2(sv[r] - ref);
      if (MASKED) pv[r] = ok[r] ? pv[r] : 0.f;
    }
    l_run[rt] = l_run[rt] * alpha + ((pv[0] + pv[1]) + (pv[2] + pv[3]));
    m_run[rt] = m_new;
#pragma unroll
    for (int jt = 0; jt < NJT; ++jt) acc[rt][jt] *= alpha;
    uint32_t h[4], lo[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      h[r] = bf16_bits(pv[r]);
      lo[r] = bf16_bits(pv[r] - __uint_as_float(h[r] << 16));
    }
    ph[rt] = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
    pl[rt] = make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
  }
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

template <int D, int BS, int NRT>
__device__ void process_segment(const AttnParams& P, const Segment& sg, int w, int W, int TB,
                                int lane, int c, int g, SplitDesc& desc) {
  constexpr int NKK = D / 32;
  constexpr int NJT = D / 16;
  constexpr int RG = 16 * NRT;
  const int G = P.G;
  const int row0 = sg.rg * RG;
  const int t_start = sg.ub * BS;
  const int t_end = min(sg.L, (sg.ub + sg.seg) * BS);
  const int full_until = sg.L - sg.Q;   // tokens <= this are visible to every row
  const int32_t* trow = P.tables + (long long)sg.s * P.MB;
  const long long tok_stride = (long long)P.Hkv * D;
  const uint16_t* kbase = P.kpool + (long long)sg.kvh * D;
  const uint16_t* vbase = P.vpool + (long long)sg.kvh * D;
  const int jend = sg.ub + sg.seg;

  int out_row[NRT];
  int nrows;
  unit_rows<D, NRT>(P, sg.kvh, sg.rg, sg.Q, sg.qoff, c, out_row, nrows);

  // query rows of this unit as B operands: lane holds row rt*16+c, dims 32*kk + 8*g .. +7
  bf16x8 qb[NRT][NKK];
  int lim[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    lim[rt] = sg.L - sg.Q + (row0 + rt * 16 + c) / G;
    const uint16_t* qp = P.q + (long long)(out_row[rt] >= 0 ? out_row[rt] : 0) * D + 8 * g;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const uint4 v = out_row[rt] >= 0 ? ld16(qp + 32 * kk) : make_uint4(0, 0, 0, 0);
      qb[rt][kk] = as_bf16x8(v);
    }
  }

  float m_run[NRT], l_run[NRT];
  f32x4 acc[NRT][NJT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    m_run[rt] = kNegInf;
    l_run[rt] = 0.f;
#pragma unroll
    for (int jt = 0; jt < NJT; ++jt) acc[rt][jt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // The tile loop walks the segment in windows of 64 KV blocks.  A window's pool block ids are
  // loaded once (one per lane) before its tiles, so no vector load inside the tile loop depends
  // on a branch.  Each wave keeps VAP_ATTN_STAGES tiles in flight; latency is mostly hidden by
  // the other waves of the CU (up to 16).
  int derr = 0;
  constexpr int kWinBlocks = 64;
  constexpr int kWinTiles = kWinBlocks * BS / kTile;
  const int ntiles = (t_end - t_start + kTile - 1) / kTile;
  for (int wt = 0; wt < ntiles; wt += kWinTiles) {
    const int wbase = sg.ub + wt * kTile / BS;    // first block of the window
    int win;
    {
      const int j = wbase + lane;
      win = (j < jend) ? trow[j] : 0;
      if (j < jend && (unsigned)win >= (unsigned)P.num_blocks) {
        derr = VAP_DERR_BLOCK_ID;
        win = 0;
      }
    }
    const int nt = min(kWinTiles, ntiles - wt);
    const int tw0 = t_start + wt * kTile;          // first token of the window
    auto issue = [&](KVTile<D>& X, int i) {
      const int tg = tw0 + i * kTile;
      load_tile<D, BS>(X, kbase, vbase, tok_stride, tg, __builtin_amdgcn_readlane(win, tg / BS - wbase), c, g);
    };
    auto compute = [&](const KVTile<D>& X, int i) {
      const int tg = tw0 + i * kTile;
      if (tg + kTile > t_end || tg + kTile - 1 > full_until)
        compute_tile<D, NRT, true>(X, tg, t_end, lim, qb, P.scale_log2, m_run, l_run, acc, g);
      else
        compute_tile<D, NRT, false>(X, tg, t_end, lim, qb, P.scale_log2, m_run, l_run, acc, g);
    };
#if VAP_ATTN_STAGES >= 2
    KVTile<D> t0, t1;
    issue(t0, 0);
    int i = 0;
    bool done = false;
    while (i + 1 < nt) {             // two buffers in rotation, no register copies
      issue(t1, i + 1);
      compute(t0, i);
      ++i;
      if (i + 1 >= nt) { compute(t1, i); done = true; break; }
      issue(t0, i + 1);
      compute(t1, i);
      ++i;
    }
    if (!done) compute(t0, i);
#else
    for (int i = 0; i < nt; ++i) {
      KVTile<D> t0;
      issue(t0, i);
      compute(t0, i);
    }
#endif
  }
  if (derr && lane == 0) atomicOr(&P.hdr->err, derr);

  float lsum[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    float l = l_run[rt];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    lsum[rt] = l;
  }
  if (sg.whole) {
    write_rows<D, NRT>(P.out, out_row, acc, lsum, g);
    return;
  }
  // partial: store this segment's (max, sum, unnormalised rows) in its slot, rows in natural
  // dim order; the combine kernel reads them after this kernel has finished
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const int r_in_unit = rt * 16 + c;
    if (r_in_unit < nrows) {
      const long long prow = ((long long)w * 2 + sg.slot) * RG + r_in_unit;
      float* pp = P.part_acc + prow * D + (D / 4) * g;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int j4 = 0; j4 < NJT; j4 += 4)
          *reinterpret_cast<float4*>(pp + NJT * r + j4) =
              make_float4(acc[rt][j4][r], acc[rt][j4 + 1][r], acc[rt][j4 + 2][r], acc[rt][j4 + 3][r]);
      }
      if (g == 0) P.part_ml[prow] = make_float2(m_run[rt], lsum[rt]);
    }
  }
  if (sg.ub == 0) {
    // this wave opens the unit: waves w .. wb hold its segments, this one in slot sg.slot
    const long long U1 = (long long)sg.soff + (long long)(sg.unit + 1) * sg.nb;
    desc.kvh = sg.kvh;
    desc.rg = sg.rg;
    desc.qoff = sg.qoff;
    desc.Q = sg.Q;
    desc.wb = (int)((U1 * W - 1) / TB);
    desc.slot_a = sg.slot;
    desc.valid = 1;
  }
}

template <int D, int BS, int NRT, bool LDS_PLAN>
__global__ __launch_bounds__(kAttnThreads, NRT == 1 ? VAP_ATTN_WAVES_1RT : VAP_ATTN_WAVES_2RT) void attn_main_kernel(const AttnParams P) {
  extern __shared__ int s_mem[];
  const int lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  const int w = uniform(blockIdx.x * kWavesPerWG + (threadIdx.x >> 6));

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
  if (w >= W) {                          // no workgroup barrier below this point
    if (lane == 0) reinterpret_cast<int4*>(P.desc)[2 * w + 1] = make_int4(0, 0, 0, 0);
    return;
  }
  const long long b0 = (long long)w * TB / W;
  const long long b1 = (long long)(w + 1) * TB / W;

  int s;
  if constexpr (LDS_PLAN) {
    int lo = 0, hi = P.B;                // largest s with off[s] <= b0
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (plan_off(mid) <= b0) lo = mid; else hi = mid - 1;
    }
    s = uniform(lo);
  } else {
    s = uniform(P.wave_seq[w]);
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
    const int nrg = (P.G * sg.Q + 16 * NRT - 1) / (16 * NRT);
    const int local = pos - soff;
    sg.unit = local / sg.nb;
    sg.ub = local - sg.unit * sg.nb;
    sg.seg = min(sg.nb - sg.ub, (int)(b1 - pos));
    sg.kvh = sg.unit / nrg;
    sg.rg = sg.unit - sg.kvh * nrg;
    sg.whole = (sg.ub == 0) && (sg.seg == sg.nb);
    sg.slot = first ? 0 : 1;
    process_segment<D, BS, NRT>(P, sg, w, W, TB, lane, c, g, desc);
    pos += sg.seg;
    first = false;
  }
  if (lane == 0) {
    int4* dp = reinterpret_cast<int4*>(P.desc) + 2 * w;
    dp[0] = make_int4(desc.kvh, desc.rg, desc.qoff, desc.Q);
    dp[1] = make_int4(desc.wb, desc.slot_a, desc.valid, 0);
  }
}

// Combine kernel: one workgroup per split unit (described by the wave w holding its first
// block); wave j of the workgroup takes rows j, j+4, ... and lane l dims (D/64)*l .. +D/64-1.
// Per row it folds the partials p = w .. wb in wave order with flash-decoding's combine
// (running max M, sum L = sum 2^(m_p - M) l_p, rows sum 2^(m_p - M) acc_p), loading
// kCombineBatch partials per round trip; out = rows / L.
constexpr int kCombineThreads = 256;
constexpr int kCombineBatch = 8;

template <int D>
__global__ __launch_bounds__(kCombineThreads) void attn_combine_kernel(const AttnParams P) {
  constexpr int DPL = D / 64;
  const int w = blockIdx.x;
  const int TB = P.hdr->total_work;
  if (w >= min(P.W, TB)) return;
  const int4* dp = reinterpret_cast<const int4*>(P.desc) + 2 * w;
  const int4 d1 = dp[1];
  if (d1.z == 0) return;
  const int4 d0 = dp[0];
  const int kvh = d0.x, rg = d0.y, qoff = d0.z, Q = d0.w;
  const int wb = d1.x, slot_a = d1.y;
  const int G = P.G, RG = P.RG;
  const int nrows = min(RG, G * Q - rg * RG);
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  for (int r = wave; r < nrows; r += kCombineThreads / 64) {
    float M = kNegInf, L = 0.f;
    float a[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k) a[k] = 0.f;
    for (int p0 = w; p0 <= wb; p0 += kCombineBatch) {
      float2 ml[kCombineBatch];
      float v[kCombineBatch][DPL];
#pragma unroll
      for (int j = 0; j < kCombineBatch; ++j) {
        const int wp = p0 + j;
        if (wp <= wb) {
          const long long prow = ((long long)wp * 2 + (wp == w ? slot_a : 0)) * RG + r;
          ml[j] = P.part_ml[prow];
          const float* pa = P.part_acc + prow * D + DPL * lane;
          if constexpr (DPL == 2) {
            const float2 x = *reinterpret_cast<const float2*>(pa);
            v[j][0] = x.x;
            v[j][1] = x.y;
          } else {
            v[j][0] = pa[0];
          }
        }
      }
#pragma unroll
      for (int j = 0; j < kCombineBatch; ++j) {
        if (p0 + j <= wb) {
          const float Mn = fmaxf(M, ml[j].x);
          if (Mn != kNegInf) {
            const float fa = fast_exp2(M - Mn), fb = fast_exp2(ml[j].x - Mn);
            L = L * fa + ml[j].y * fb;
#pragma unroll
            for (int k = 0; k < DPL; ++k) a[k] = a[k] * fa + v[j][k] * fb;
            M = Mn;
          }
        }
      }
    }
    const int row = rg * RG + r;
    const int i = row / G;
    float* op = P.out + ((long long)(qoff + i) * P.Hq + kvh * G + (row - i * G)) * D + DPL * lane;
    const float inv = 1.f / L;
    if constexpr (DPL == 2) {
      *reinterpret_cast<float2*>(op) = make_float2(a[0] * inv, a[1] * inv);
    } else {
      op[0] = a[0] * inv;
    }
  }
}

template <int D, int BS, int NRT, bool LDS_PLAN>
hipError_t launch_main_t(const AttnParams& p, int num_wg, hipStream_t stream) {
  const size_t lds = LDS_PLAN ? attn_main_lds_bytes(p.B) : 0;
  hipLaunchKernelGGL((attn_main_kernel<D, BS, NRT, LDS_PLAN>), dim3(num_wg), dim3(kAttnThreads), lds, stream, p);
  return hipGetLastError();
}

}  // namespace

size_t attn_main_lds_bytes(int B) { return size_t(4 * B + 1) * sizeof(int); }

#define VAP_ATTN_VARIANTS(X) \
  X(64, 16, 1) X(64, 16, 2) X(64, 32, 1) X(64, 32, 2) \
  X(128, 16, 1) X(128, 16, 2) X(128, 32, 1) X(128, 32, 2)

hipError_t launch_attn_main(const AttnParams& p, int D, int BS, int NRT, int num_wg, hipStream_t stream) {
  const bool lds = p.B <= kLdsPlanMaxSeqs;
#define X(d, bs, nrt)                                                          \
  if (D == d && BS == bs && NRT == nrt)                                        \
    return lds ? launch_main_t<d, bs, nrt, true>(p, num_wg, stream)            \
               : launch_main_t<d, bs, nrt, false>(p, num_wg, stream);
  VAP_ATTN_VARIANTS(X)
#undef X
  return hipErrorInvalidValue;
}

hipError_t launch_attn_combine(const AttnParams& p, int D, hipStream_t stream) {
  if (D == 64) {
    hipLaunchKernelGGL(attn_combine_kernel<64>, dim3(p.W), dim3(kCombineThreads), 0, stream, p);
  } else if (D == 128) {
    hipLaunchKernelGGL(attn_combine_kernel<128>, dim3(p.W), dim3(kCombineThreads), 0, stream, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

const void* attn_main_kernel_ptr(int D, int BS, int NRT, bool lds_plan) {
#define X(d, bs, nrt)                                                                        \
  if (D == d && BS == bs && NRT == nrt)                                                      \
    return lds_plan ? reinterpret_cast<const void*>(&attn_main_kernel<d, bs, nrt, true>)     \
                    : reinterpret_cast<const void*>(&attn_main_kernel<d, bs, nrt, false>);
  VAP_ATTN_VARIANTS(X)
#undef X
  return nullptr;
}

}  // namespace vap
