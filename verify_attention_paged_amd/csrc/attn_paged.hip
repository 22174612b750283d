// Attention kernel of paged_attn_step and its split-merge kernel (gfx950).
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
//  * Work is split evenly in KV blocks over W persistent worker waves (the plan kernel's
//    partition), so long-tail sequences are spread over many waves and every CU streams the
//    same number of bytes.  A unit of work is (sequence, KV head, row group); a wave covers
//    consecutive units and may cover only part of one, in which case it writes a partial
//    (running max, running sum, unnormalised output) for the merge kernel.
//  * One wave processes all rows of a unit at once: the G query heads of the GQA group times
//    the q_len rows (up to 16 * NRT rows).  Every K and V byte is loaded once from HBM, straight
//    into MFMA operand registers, and serves all those rows; nothing is staged through LDS.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_16x16x32_bf16: the K tile is
//    the A operand (lane = token, 16 contiguous bytes per lane -> 64-byte runs per token row),
//    the query rows are the B operand.  In the result each lane holds one query row and four
//    tokens, so the online-softmax statistics of a row live in the four lanes {c, c+16, c+32,
//    c+48}: a row max needs two cross-lane exchanges and rescaling the accumulator is local.
//  * The output is accumulated transposed too, O^T += V^T P^T: P (fp32) is split into
//    bf16 hi + lo parts that together keep ~16 mantissa bits, and V^T is built from 4-byte
//    loads (two dims of one token) with byte permutes.  The softmax probabilities therefore
//    never leave registers.
//  * Masking is select-based: tokens past the segment (including a block's unused tail,
//    which may hold anything, even NaN) get probability 0 and their V operand is zeroed.
#include "vap_internal.h"

namespace vap {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ uint4 ld16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ uint32_t ld4(const uint16_t* p) {
  return *reinterpret_cast<const uint32_t*>(p);
}
__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// bf16 bits of a finite float, round to nearest even
__device__ __forceinline__ uint32_t bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// token offset (0..31 inside a 32-token tile) of element e of lane group g in the MFMA
// k-slots shared by the P^T (B) and V^T (A) operands of the output product
__device__ __forceinline__ int tile_token(int g, int e) { return (e < 4) ? (4 * g + e) : (12 + 4 * g + e); }

template <int D, int BS, int NRT>
__device__ __forceinline__ void process_segment(const AttnParams& P, int s, int kvh, int rg,
                                                int ub, int seg, bool whole, int w, int slot,
                                                int c, int g) {
  constexpr int NKK = D / 32;   // 32-dim slices of the score contraction
  constexpr int NJT = D / 16;   // 16-dim output tiles
  constexpr int RG = 16 * NRT;

  const int L = P.ctx_lens[s];
  const int Q = P.q_lens[s];
  const int qoff = P.q_off[s];
  const int G = P.G;
  const int row0 = rg * RG;
  const int nrows = min(RG, G * Q - row0);
  const int t_start = ub * BS;
  const int t_end = min(L, (ub + seg) * BS);
  const int32_t* trow = P.tables + (long long)s * P.MB;
  const long long tok_stride = (long long)P.Hkv * D;
  const uint16_t* kbase = P.kpool + (long long)kvh * D;
  const uint16_t* vbase = P.vpool + (long long)kvh * D;

  // query rows of this unit as B operands: lane holds row rt*16+c, dims 32*kk + 8*g .. +7
  bf16x8 qb[NRT][NKK];
  int lim[NRT];
  int out_row[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const int r = rt * 16 + c;
    const bool ok = r < nrows;
    const int row = row0 + r;
    const int i = row / G;
    const int h = kvh * G + (row - i * G);
    lim[rt] = L - Q + i;
    out_row[rt] = ok ? (qoff + i) * P.Hq + h : -1;
    const uint16_t* qp = P.q + (long long)(ok ? out_row[rt] : 0) * D + 8 * g;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const uint4 v = ok ? ld16(qp + 32 * kk) : make_uint4(0, 0, 0, 0);
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

  int derr = 0;
  for (int tg = t_start; tg < t_end; tg += kTokTile) {
    // pool blocks of the two 16-token halves (wave-uniform); a half past the segment reuses
    // the first half's block so that every address stays inside a valid block
    int blk0 = trow[tg / BS];
    int blk1 = (tg + 16 < t_end) ? trow[(tg + 16) / BS] : blk0;
    if ((unsigned)blk0 >= (unsigned)P.num_blocks) { derr = VAP_DERR_BLOCK_ID; blk0 = 0; }
    if ((unsigned)blk1 >= (unsigned)P.num_blocks) { derr = VAP_DERR_BLOCK_ID; blk1 = 0; }

    // K tile as A operands: lane c holds token tg + st*16 + c, dims 32*kk + 8*g .. +7
    bf16x8 ka[2][NKK];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int blk = st ? blk1 : blk0;
      const int rib = (tg + st * 16) % BS + c;
      const uint16_t* kp = kbase + ((long long)blk * BS + rib) * tok_stride + 8 * g;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) ka[st][kk] = as_bf16x8(ld16(kp + 32 * kk));
    }
    // V tile: lane loads, for its 8 tokens, the two dims 32*mm + 2c, +1 (4 bytes each)
    uint32_t vw[8][NKK];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int tr = tile_token(g, e);
      const int blk = (e < 4) ? blk0 : blk1;
      const uint16_t* vp = vbase + ((long long)blk * BS + (tg + tr) % BS) * tok_stride + 2 * c;
      const bool okv = tg + tr < t_end;
#pragma unroll
      for (int mm = 0; mm < NKK; ++mm) {
        const uint32_t x = ld4(vp + 32 * mm);
        vw[e][mm] = okv ? x : 0u;
      }
    }

    // V^T A operands: tile 2*mm holds dims 32*mm + 2*(l%16), tile 2*mm+1 the next dim
    bf16x8 vt[NJT];
#pragma unroll
    for (int mm = 0; mm < NKK; ++mm) {
      uint4 ev, od;
      ev.x = __builtin_amdgcn_perm(vw[1][mm], vw[0][mm], 0x05040100u);
      ev.y = __builtin_amdgcn_perm(vw[3][mm], vw[2][mm], 0x05040100u);
      ev.z = __builtin_amdgcn_perm(vw[5][mm], vw[4][mm], 0x05040100u);
      ev.w = __builtin_amdgcn_perm(vw[7][mm], vw[6][mm], 0x05040100u);
      od.x = __builtin_amdgcn_perm(vw[1][mm], vw[0][mm], 0x07060302u);
      od.y = __builtin_amdgcn_perm(vw[3][mm], vw[2][mm], 0x07060302u);
      od.z = __builtin_amdgcn_perm(vw[5][mm], vw[4][mm], 0x07060302u);
      od.w = __builtin_amdgcn_perm(vw[7][mm], vw[6][mm], 0x07060302u);
      vt[2 * mm] = as_bf16x8(ev);
      vt[2 * mm + 1] = as_bf16x8(od);
    }

#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        s0 = mfma16x16x32(ka[0][kk], qb[rt][kk], s0);
        s1 = mfma16x16x32(ka[1][kk], qb[rt][kk], s1);
      }
      // lane holds row rt*16+c at tokens tile_token(g, e): e < 4 in s0, e >= 4 in s1
      float sv[8];
      bool ok[8];
      float mx = kNegInf;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int tok = tg + tile_token(g, e);
        ok[e] = (tok < t_end) && (tok <= lim[rt]);
        sv[e] = ((e < 4) ? s0[e] : s1[e - 4]) * P.scale_log2;
        mx = ok[e] ? fmaxf(mx, sv[e]) : mx;
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run[rt], mx);
      const float ref = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run[rt] - ref);
      float psum = 0.f;
      uint32_t hb[8], lb[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pe = ok[e] ? fast_exp2(sv[e] - ref) : 0.f;
        psum += pe;
        hb[e] = bf16_bits(pe);
        lb[e] = bf16_bits(pe - __uint_as_float(hb[e] << 16));
      }
      l_run[rt] = l_run[rt] * alpha + psum;
      m_run[rt] = m_new;
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt) acc[rt][jt] *= alpha;
      const bf16x8 ph = as_bf16x8(make_uint4(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16),
                                             hb[4] | (hb[5] << 16), hb[6] | (hb[7] << 16)));
      const bf16x8 pl = as_bf16x8(make_uint4(lb[0] | (lb[1] << 16), lb[2] | (lb[3] << 16),
                                             lb[4] | (lb[5] << 16), lb[6] | (lb[7] << 16)));
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt) {
        acc[rt][jt] = mfma16x16x32(vt[jt], ph, acc[rt][jt]);
        acc[rt][jt] = mfma16x16x32(vt[jt], pl, acc[rt][jt]);
      }
    }
  }
  if (derr) atomicOr(&P.hdr->err, derr);

  // lane (c, g) holds, for row rt*16+c, dims 32*mm + 8*g + 2*r + par in acc[rt][2*mm+par][r]
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    float l = l_run[rt];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const int r_in_unit = rt * 16 + c;
    if (whole) {
      if (out_row[rt] >= 0) {
        const float inv = 1.f / l;
        float* op = P.out + (long long)out_row[rt] * D + 8 * g;
#pragma unroll
        for (int mm = 0; mm < NKK; ++mm) {
          const f32x4 a = acc[rt][2 * mm], b = acc[rt][2 * mm + 1];
          *reinterpret_cast<float4*>(op + 32 * mm) = make_float4(a[0] * inv, b[0] * inv, a[1] * inv, b[1] * inv);
          *reinterpret_cast<float4*>(op + 32 * mm + 4) = make_float4(a[2] * inv, b[2] * inv, a[3] * inv, b[3] * inv);
        }
      }
    } else if (r_in_unit < nrows) {
      const long long prow = ((long long)w * 2 + slot) * RG + r_in_unit;
      float* pp = P.part_acc + prow * D + 8 * g;
#pragma unroll
      for (int mm = 0; mm < NKK; ++mm) {
        const f32x4 a = acc[rt][2 * mm], b = acc[rt][2 * mm + 1];
        *reinterpret_cast<float4*>(pp + 32 * mm) = make_float4(a[0], b[0], a[1], b[1]);
        *reinterpret_cast<float4*>(pp + 32 * mm + 4) = make_float4(a[2], b[2], a[3], b[3]);
      }
      if (g == 0) P.part_ml[prow] = make_float2(m_run[rt], l);
    }
  }
}

template <int D, int BS, int NRT>
__global__ __launch_bounds__(kAttnThreads) void attn_main_kernel(const AttnParams P) {
  const int lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(blockIdx.x * kWavesPerWG + (threadIdx.x >> 6));
  const int W = P.W;
  const int TB = P.hdr->total_work;
  const long long b0 = (long long)w * TB / W;
  const long long b1 = (long long)(w + 1) * TB / W;
  int4 desc = make_int4(-1, 0, 0, 0);
  if (b0 < b1) {
    int s = P.wave_seq[w];
    int pos = (int)b0;
    bool first = true;
    while (pos < b1) {
      const int soff = P.seq_off[s];
      const int send = P.seq_off[s + 1];
      if (pos >= send) { ++s; continue; }
      const int nb = P.nblk[s];
      const int nrg = P.n_rg[s];
      const int local = pos - soff;
      const int unit = local / nb;
      const int ub = local - unit * nb;
      const int seg = min(nb - ub, (int)(b1 - pos));
      const int kvh = unit / nrg;
      const int rg = unit - kvh * nrg;
      const bool whole = (ub == 0) && (seg == nb);
      const int slot = first ? 0 : 1;
      process_segment<D, BS, NRT>(P, s, kvh, rg, ub, seg, whole, w, slot, c, g);
      if (!whole && ub == 0) {
        // this wave opens a unit that continues into later waves: it owns the merge
        const long long U1 = (long long)soff + (long long)(unit + 1) * nb;
        const int wb = (int)((U1 * W - 1) / TB);
        desc = make_int4(s, unit, wb, slot);
      }
      pos += seg;
      first = false;
    }
  }
  if (lane == 0) P.desc[w] = desc;
}

// Merge the partials of every unit that was split across waves: for each row,
// M = max_p m_p, out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p, in wave order.
template <int D>
__global__ __launch_bounds__(kAttnThreads) void attn_reduce_kernel(const AttnParams P) {
  constexpr int DPL = D / 64;   // dims per lane
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(blockIdx.x * kWavesPerWG + (threadIdx.x >> 6));
  if (w >= P.W) return;
  const int4 d = P.desc[w];
  if (d.x < 0) return;
  const int s = d.x, unit = d.y, wb = d.z, slot_a = d.w;
  const int nrg = P.n_rg[s];
  const int kvh = unit / nrg;
  const int rg = unit - kvh * nrg;
  const int Q = P.q_lens[s];
  const int qoff = P.q_off[s];
  const int G = P.G;
  const int RG = P.RG;
  const int nrows = min(RG, G * Q - rg * RG);
  const int TB = P.hdr->total_work;
  const int W = P.W;

  for (int r = 0; r < nrows; ++r) {
    float M = kNegInf;
    for (int wp = w; wp <= wb; ++wp) {
      if (wp != w && (long long)wp * TB / W == (long long)(wp + 1) * TB / W) continue;  // empty wave
      const int sl = (wp == w) ? slot_a : 0;
      M = fmaxf(M, P.part_ml[((long long)wp * 2 + sl) * RG + r].x);
    }
    float lsum = 0.f;
    float o[DPL];
#pragma unroll
    for (int j = 0; j < DPL; ++j) o[j] = 0.f;
    for (int wp = w; wp <= wb; ++wp) {
      if (wp != w && (long long)wp * TB / W == (long long)(wp + 1) * TB / W) continue;
      const int sl = (wp == w) ? slot_a : 0;
      const long long prow = ((long long)wp * 2 + sl) * RG + r;
      const float2 ml = P.part_ml[prow];
      const float sc = (ml.x == kNegInf) ? 0.f : fast_exp2(ml.x - M);
      lsum += ml.y * sc;
      const float* pa = P.part_acc + prow * D + lane * DPL;
#pragma unroll
      for (int j = 0; j < DPL; ++j) o[j] += sc * pa[j];
    }
    const int row = rg * RG + r;
    const int i = row / G;
    const int h = kvh * G + (row - i * G);
    float* op = P.out + ((long long)(qoff + i) * P.Hq + h) * D + lane * DPL;
    const float inv = 1.f / lsum;
#pragma unroll
    for (int j = 0; j < DPL; ++j) op[j] = o[j] * inv;
  }
}

template <int D, int BS, int NRT>
hipError_t launch_main_t(const AttnParams& p, int num_wg, hipStream_t stream) {
  hipLaunchKernelGGL((attn_main_kernel<D, BS, NRT>), dim3(num_wg), dim3(kAttnThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

#define VAP_ATTN_VARIANTS(X) \
  X(64, 16, 1) X(64, 16, 2) X(64, 32, 1) X(64, 32, 2) \
  X(128, 16, 1) X(128, 16, 2) X(128, 32, 1) X(128, 32, 2)

hipError_t launch_attn_main(const AttnParams& p, int D, int BS, int NRT, int num_wg, hipStream_t stream) {
#define X(d, bs, nrt) if (D == d && BS == bs && NRT == nrt) return launch_main_t<d, bs, nrt>(p, num_wg, stream);
  VAP_ATTN_VARIANTS(X)
#undef X
  return hipErrorInvalidValue;
}

const void* attn_main_kernel_ptr(int D, int BS, int NRT) {
#define X(d, bs, nrt) if (D == d && BS == bs && NRT == nrt) return reinterpret_cast<const void*>(&attn_main_kernel<d, bs, nrt>);
  VAP_ATTN_VARIANTS(X)
#undef X
  return nullptr;
}

hipError_t launch_attn_reduce(const AttnParams& p, int D, hipStream_t stream) {
  const int num_wg = (p.W + kWavesPerWG - 1) / kWavesPerWG;
  if (D == 64) {
    hipLaunchKernelGGL(attn_reduce_kernel<64>, dim3(num_wg), dim3(kAttnThreads), 0, stream, p);
  } else if (D == 128) {
    hipLaunchKernelGGL(attn_reduce_kernel<128>, dim3(num_wg), dim3(kAttnThreads), 0, stream, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace vap
