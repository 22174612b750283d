// Attention kernels' internal declarations: workspace layout, parameters, launchers (not part
// of the C ABI).
#pragma once

#include "vap_common.h"

namespace vap {

constexpr int kMaxSeqs = 8192;      // plan kernel keeps per-sequence work offsets in LDS
constexpr int kPlanThreads = 1024;
constexpr int kAttnThreads = 256;   // at most 4 independent worker waves per workgroup
constexpr int kWavesPerWG = kAttnThreads / 64;


// ---------------------------------------------------------------------------------------
// Attention workspace layout (all offsets 256-byte aligned).
//   [0, 256)   header: sticky err word, total work blocks, next pool piece to claim
//   desc       int32 [NH][8]      split-unit descriptor written for every holder (below):
//              {kv head, row group, first packed row of the sequence, q_len,
//               last holder of part of the unit, slot of this holder's partial, valid, 0};
//              valid = 0 when the holder has the first block of no split unit.  Read by
//              the combine kernel.  A unit has at most 64 rows (RG = 16, 32 or 64).
//   g_L, g_Q   int32 [B]          per-sequence lengths (g_L = 0 for a skipped sequence)   \  only
//   q_off      int32 [B]          first packed row of each sequence                        |  for
//   seq_off    int32 [B+1]        exclusive prefix of per-sequence work                   |  B >
//   wave_seq   int32 [W]          sequence holding each worker wave's first work block    /  2048
//   part_ml    float2 [NH][2][RG]     (running max in log2 units, running sum) per row
//   part_acc   float  [NH][2][RG][D]  unnormalised output per row
// A unit of work is (sequence, KV head, row group).  Its work is UH + ceil(L/BS) blocks: UH
// virtual blocks stand for the fixed cost of starting a unit (its query rows and block-table
// window are dependent loads), followed by its ceil(L/BS) KV blocks.  The work blocks are cut
// into ranges, each with its own holder index (partial slots and descriptor), in work order:
//   * holders 0 .. W'-1, W' = min(W, TB): worker wave w's own share [w*T1/W', (w+1)*T1/W');
//   * holders W .. W+NP-1: NP pool pieces of PS blocks covering [T1, TB), T1 = TB - NP*PS,
//     which waves that have finished their share claim one at a time (header pool_next).
// NP = 0 (T1 = TB) unless the step (bf16 cache, 16-row units) has at least 32 work blocks per
// wave (then W' = W and the pool follows the last share without a gap); NP <= pool_max,
// NH = W + pool_max.  A range that
// starts inside a unit's virtual blocks begins at the unit's first KV block.
// ---------------------------------------------------------------------------------------
constexpr int kMaxWaves = 16384;
constexpr int kLdsPlanMaxSeqs = 2048;   // above this the plan kernel builds the tables

struct AttnHeader {
  int32_t err;
  int32_t total_work;   // TB: total work blocks of the step (plan kernel path)
  int32_t pool_next;    // next pool piece to claim; zero between calls (the combine kernel resets it)
  int32_t pad;
};

struct AttnLayout {
  size_t desc, g_L, g_Q, q_off, seq_off, wave_seq, part_ml, part_acc, total;
};

inline AttnLayout attn_layout(int B, int W, int RG, int D, int NH) {
  AttnLayout L;
  size_t o = 256;
  L.desc = o;      o = align256(o + size_t(NH) * 32);
  L.g_L = o;       o = align256(o + size_t(B) * 4);
  L.g_Q = o;       o = align256(o + size_t(B) * 4);
  L.q_off = o;     o = align256(o + size_t(B) * 4);
  L.seq_off = o;   o = align256(o + size_t(B + 1) * 4);
  L.wave_seq = o;  o = align256(o + size_t(W) * 4);
  L.part_ml = o;   o = align256(o + size_t(NH) * 2 * RG * 8);
  L.part_acc = o;  o = align256(o + size_t(NH) * 2 * RG * D * 4);
  L.total = o;
  return L;
}

struct AttnParams {
  const uint16_t* q;        // bf16 [T][Hq][D]
  const uint16_t* kpool;    // bf16 [NB][BS][Hkv][D]
  const uint16_t* vpool;    // bf16 [NB][BS][Hkv][D]
  const uint8_t* kcodes;    // 8-bit cache: uint8 [NB][BS][Hkv][D] codes of K and of V
  const uint8_t* vcodes;
  const float* kv_scales;   // 8-bit cache: fp32 [NB][Hkv][BS][4] (k_scale, k_zero, v_scale, v_zero)
  const uint64_t* tree_mask;   // [T] ancestor masks of tree rows, or nullptr (causal rows)
  const int32_t* tables;    // [B][MB]
  const int32_t* ctx_lens;  // [B]
  const int32_t* q_lens;    // [B]
  float* out;               // fp32 [T][Hq][D]
  int32_t B, Hq, Hkv, G, num_blocks, MB, total_q;
  int32_t W;                // worker waves launched
  int32_t RG;               // rows per unit (16 * row tiles)
  int32_t BS;               // block size (the attention kernel also templates it)
  int32_t UH;               // setup cost of a unit, in work blocks (see the layout comment)
  int32_t NH;               // holders: W worker waves, then pool_max pool pieces
  int32_t pool_max;         // pool pieces at most (0: static shares only)
  int32_t pool_pct;         // share of the step's work put in the pool, in percent
  int32_t pool_piece;       // work blocks per pool piece
  float scale_log2;         // softmax scale * log2(e)
  AttnHeader* hdr;
  int32_t* desc;
  int32_t* g_L;
  int32_t* g_Q;
  int32_t* q_off;
  int32_t* seq_off;
  int32_t* wave_seq;
  float2* part_ml;
  float* part_acc;
};

// launchers (attn_plan.hip, attn_paged.hip, attn_combine.hip); return hipError_t of the launch
hipError_t launch_attn_plan(const AttnParams& p, hipStream_t stream);
// kv: 0 = bf16 cache, 1 = 8-bit integer codes, 2 = FP8 (E4M3) codes
hipError_t launch_attn_main(const AttnParams& p, int D, int BS, int NRT, int kv, int num_wg, int wg_waves,
                            hipStream_t stream, KTimer t = {});
// xcd_local: merge each worker wave's shares on the XCD that ran that wave (see the kernel)
hipError_t launch_attn_combine(const AttnParams& p, int D, int num_cus, bool xcd_local, hipStream_t stream);
const void* attn_main_kernel_ptr(int D, int BS, int NRT, bool lds_plan, bool kv8);
size_t attn_main_lds_bytes(int B);

}  // namespace vap
