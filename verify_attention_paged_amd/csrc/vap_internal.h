// Internal declarations shared by the HIP sources of the library (not part of the C ABI).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "vap.h"

namespace vap {

// Timing events of one launch (both null when the kernel timer is off).  The launchers pass them
// to hipExtLaunchKernelGGL, which stamps the kernel's own start and end, so the interval excludes
// the wait between the previous kernel's end and this kernel's first wave.
struct KTimer {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

constexpr int kMaxSeqs = 8192;      // plan kernel keeps per-sequence work offsets in LDS
constexpr int kPlanThreads = 1024;
constexpr int kAttnThreads = 256;   // 4 independent worker waves per workgroup
constexpr int kWavesPerWG = kAttnThreads / 64;


// ---------------------------------------------------------------------------------------
// Attention workspace layout (all offsets 256-byte aligned).
//   [0, 256)   header: sticky err word, total work blocks
//   desc       int32 [W][8]       split-unit descriptor written by every worker wave:
//              {kv head, row group, first packed row of the sequence, q_len,
//               last wave holding part of the unit, slot of this wave's partial, valid, 0};
//              valid = 0 when the wave holds the first block of no split unit.  Read by
//              the combine kernel.  A unit has at most 32 rows (RG = 16 or 32).
//   g_L, g_Q   int32 [B]          per-sequence lengths (g_L = 0 for a skipped sequence)   \  only
//   q_off      int32 [B]          first packed row of each sequence                        |  for
//   seq_off    int32 [B+1]        exclusive prefix of per-sequence work                   |  B >
//   wave_seq   int32 [W]          sequence holding each worker wave's first work block    /  2048
//   part_ml    float2 [W][2][RG]      (running max in log2 units, running sum) per row
//   part_acc   float  [W][2][RG][D]   unnormalised output per row
// A unit of work is (sequence, KV head, row group).  Its work is UH + ceil(L/BS) blocks: UH
// virtual blocks stand for the fixed cost of starting a unit (its query rows and block-table
// window are dependent loads), followed by its ceil(L/BS) KV blocks.  Worker wave w owns work
// blocks [w*TB/W', (w+1)*TB/W') with W' = min(W, TB); a wave whose range starts inside a
// unit's virtual blocks begins at the unit's first KV block.
// ---------------------------------------------------------------------------------------
constexpr int kMaxWaves = 16384;
constexpr int kLdsPlanMaxSeqs = 2048;   // above this the plan kernel builds the tables

struct AttnHeader {
  int32_t err;
  int32_t total_work;   // TB: total work blocks of the step (plan kernel path)
  int32_t pad[2];
};

struct AttnLayout {
  size_t desc, g_L, g_Q, q_off, seq_off, wave_seq, part_ml, part_acc, total;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline AttnLayout attn_layout(int B, int W, int RG, int D) {
  AttnLayout L;
  size_t o = 256;
  L.desc = o;      o = align256(o + size_t(W) * 32);
  L.g_L = o;       o = align256(o + size_t(B) * 4);
  L.g_Q = o;       o = align256(o + size_t(B) * 4);
  L.q_off = o;     o = align256(o + size_t(B) * 4);
  L.seq_off = o;   o = align256(o + size_t(B + 1) * 4);
  L.wave_seq = o;  o = align256(o + size_t(W) * 4);
  L.part_ml = o;   o = align256(o + size_t(W) * 2 * RG * 8);
  L.part_acc = o;  o = align256(o + size_t(W) * 2 * RG * D * 4);
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

// ---------------------------------------------------------------------------------------
// Verification workspace layout.
//   [0, 256)            header: err word
//   [256, ...)          chunk_sums: double [B][C], per-chunk residual / bonus row sums
//   [..., end)          tickets: int32, ticket of sequence b at end - 4*(b+1) (growing down
//                       from the end, so its place does not depend on B).  Arrival counters
//                       return to 0 at the end of every call.  Because every call checks
//                       bytes >= 256 + B*(256*8 + 4), a call's tickets never overlap the chunk
//                       sums an earlier call (any B) left behind.
// ---------------------------------------------------------------------------------------
constexpr int kMaxChunks = 256;
constexpr long long kMaxVerifySeqs = 1LL << 22;

inline size_t verify_bytes(long long B) {
  return align256(256 + (size_t)B * (kMaxChunks * 8 + 4));
}

// Statistics of (a chunk of) one logit row z at temperature T > 0: m = max z, argmax = its first
// index, S = sum_x 2^((z_x - m) * log2(e) / T) (fp64).  At T = 0 only m and argmax are set.
struct LogitRowStat {
  double S;
  float m;
  int32_t argmax;
};

struct VerifyParams {
  const float* p;
  const float* q;
  const int32_t* draft_ids;
  const float* uniforms;
  int32_t* out_ids;
  int32_t* n_accepted;
  int32_t B, k, V;
  int32_t C;        // chunks per row
  int32_t CS;       // elements per chunk (multiple of 4)
  int32_t* err;
  int32_t* tickets_end;   // ticket of sequence b is tickets_end[-(b + 1)]
  double* chunk_sums;
  // verification from logits: p and q hold target and draft logits, temps the per-sequence
  // temperature, part the statistics kernel's per-chunk partials ([B(2k+1)][C1])
  const float* temps = nullptr;
  const LogitRowStat* part = nullptr;
  int32_t C1 = 0;
};

// ---------------------------------------------------------------------------------------
// Verification-from-logits workspace layout (R = B(2k+1) rows, C1 = ceil(V / kStatChunk)).
//   [0, 256)        header: err word
//   part            LogitRowStat [R][C1]: per-chunk (max, first argmax, sum of exponentials
//                   relative to the chunk's max), written by the statistics kernel and merged
//                   by every verification workgroup for its own sequence
//   chunk_sums      double [B][kMaxChunks]
//   tickets         int32 [B], growing down from the end (sequence b at end - 4(b+1)); they
//                   return to 0 at the end of every call.
// The data lies in the first half of the workspace and the tickets in the second half (the
// size required is twice the larger of the two), so no call's tickets ever overlap data an
// earlier call of another shape left behind.
// ---------------------------------------------------------------------------------------
constexpr int kStatChunk = 2048;        // tokens per statistics item (32 per lane of a wave)
constexpr int kStatMaxChunks = 512;     // V <= 2^20
#ifndef VAP_STAT_WAVES_PER_CU
#define VAP_STAT_WAVES_PER_CU 8
#endif
constexpr int kStatWavesPerCU = VAP_STAT_WAVES_PER_CU;   // persistent statistics waves

struct LogitsLayout {
  size_t part, chunk_sums, data_end, tickets, total;
};

inline LogitsLayout logits_layout(long long B, int k, int V) {
  LogitsLayout L;
  const long long R = B * (2 * k + 1);
  const long long C1 = (V + kStatChunk - 1) / kStatChunk;
  size_t o = 256;
  L.part = o;        o = align256(o + (size_t)(R * C1) * sizeof(LogitRowStat));
  L.chunk_sums = o;  o = align256(o + (size_t)B * kMaxChunks * 8);
  L.data_end = o;
  L.tickets = (size_t)B * 4;
  L.total = 2 * align256(L.data_end > L.tickets ? L.data_end : L.tickets);
  return L;
}

struct LogitStatsParams {
  const float* zp;          // [B][k+1][V] target logits
  const float* zq;          // [B][k][V] draft logits
  const float* temps;       // [B]
  LogitRowStat* part;       // [B * (2k+1)][C] per-chunk partials (rows: k+1 target, then k draft)
  int32_t B, k, V;
  int32_t C;                // chunks per row (ceil(V / kStatChunk) <= kStatMaxChunks)
  int32_t* err;
};

// launchers (defined in the .hip files); return hipError_t of the launch
hipError_t launch_attn_plan(const AttnParams& p, hipStream_t stream);
hipError_t launch_attn_main(const AttnParams& p, int D, int BS, int NRT, bool kv8, int num_wg, hipStream_t stream,
                            KTimer t = {});
hipError_t launch_attn_combine(const AttnParams& p, int D, hipStream_t stream);
const void* attn_main_kernel_ptr(int D, int BS, int NRT, bool lds_plan, bool kv8);
size_t attn_main_lds_bytes(int B);
hipError_t launch_spec_verify(const VerifyParams& p, bool vec4, hipStream_t stream, KTimer t = {});
hipError_t launch_spec_verify_logits(const VerifyParams& p, bool vec4, hipStream_t stream, KTimer t = {});
hipError_t launch_logit_stats(const LogitStatsParams& p, bool vec4, int num_wg, hipStream_t stream, KTimer t = {});
hipError_t launch_fill_zero(void* dst, size_t bytes, hipStream_t stream);
hipError_t launch_stream_copy(void* dst, const void* src, size_t bytes, hipStream_t stream);
hipError_t launch_stream_read(const void* src, size_t bytes, void* sink, hipStream_t stream);

// ---------------------------------------------------------------------------------------
// Tree verification: one workgroup per sequence, no workspace beyond the error word.
// ---------------------------------------------------------------------------------------
constexpr int kMaxTreeNodes = 64;

struct TreeVerifyParams {
  const float* p;           // [B][N][V] target rows per node
  const float* q;           // [B][N][V] draft rows per node (the children's proposal)
  const int32_t* parents;   // [B][N]
  const int32_t* tokens;    // [B][N]
  const float* uniforms;    // [B][N]
  int32_t* out_ids;         // [B][N]
  int32_t* out_path;        // [B][N]
  int32_t* n_accepted;      // [B]
  int32_t B, N, V;
  bool vec4;                // V % 4 == 0 and p, q 16-byte aligned
  int32_t* err;
};

hipError_t launch_tree_verify(const TreeVerifyParams& p, hipStream_t stream, KTimer t = {});

// ---- KV append / commit ----------------------------------------------------------------------

struct KVAppendParams {
  const uint16_t* k_new;    // [T][Hkv][D] bf16, rows packed by sequence
  const uint16_t* v_new;
  void* kv;                 // bf16 pool [2][NB][BS][Hkv][D], or uint8 codes of the same shape
  float* kv_scales;         // 8-bit only: [NB][Hkv][BS][4] = (k_scale, k_zero, v_scale, v_zero)
  const int32_t* tables;    // [B][MB]
  const int32_t* ctx_lens;  // [B], counting the new rows
  const int32_t* q_lens;    // [B]
  int32_t B, Hkv, BS, NB, MB, T;
  int32_t* err;
};

struct KVCommitParams {
  void* kv;
  float* kv_scales;         // 8-bit only
  const int32_t* tables;
  const int32_t* ctx_lens;
  const int32_t* q_lens;
  const int32_t* path;      // [B][path_stride] accepted node indices, or nullptr for a chain
  int32_t path_stride;
  const int32_t* n_accepted;
  int32_t* out_lens;        // may alias ctx_lens
  int32_t B, Hkv, D, BS, NB, MB;
  int32_t* err;
};

size_t kv_append_lds_bytes(int B);
hipError_t launch_kv_append(const KVAppendParams& p, int D, bool u8, int num_wg, hipStream_t stream, KTimer t = {});
hipError_t launch_kv_commit(const KVCommitParams& p, bool u8, hipStream_t stream, KTimer t = {});

}  // namespace vap
