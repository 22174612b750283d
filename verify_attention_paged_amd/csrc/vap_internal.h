// Internal declarations of the library's other kernels (verification, tree verification,
// logits, KV append/commit, utilities), plus the attention declarations (not part of the C ABI).
#pragma once

#include "attn_internal.h"

namespace vap {

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
constexpr int kStatWavesPerWG = 4;                       // 256-thread statistics workgroups

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
hipError_t launch_spec_verify(const VerifyParams& p, bool vec4, hipStream_t stream, KTimer t = {});
hipError_t launch_spec_verify_logits(const VerifyParams& p, bool vec4, hipStream_t stream, KTimer t = {});
hipError_t launch_logit_stats(const LogitStatsParams& p, bool vec4, int num_wg, hipStream_t stream, KTimer t = {});
hipError_t launch_fill_zero(void* dst, size_t bytes, hipStream_t stream);
hipError_t launch_stream_copy(void* dst, const void* src, size_t bytes, hipStream_t stream);
hipError_t launch_stream_read(const void* src, size_t bytes, void* sink, hipStream_t stream);

// ---------------------------------------------------------------------------------------
// Tree verification: S workgroups per sequence walk it in lockstep (S = 1 for large batches).
// ---------------------------------------------------------------------------------------
constexpr int kMaxTreeNodes = 64;
constexpr int kMaxTreeParts = 16;   // workgroups per sequence in the walk
constexpr int kTreeRoundTokens = 4 * 8 * 1024;   // tokens one walk workgroup loads per round of a pass

// Where the walk of one sequence ended: the final draw is from max(0, p - c q) of node `node`
// (c = 0: p itself), or, if those weights are all zero, from max(0, p - c_prev q) (a walk that
// ends in a rejection skips the pass that would have checked this); its token goes to
// out_ids[b][n].
struct TreeDraw {
  double c;
  double c_prev;
  int32_t node;
  int32_t n;
  int32_t arrivals; // the walk's arrivals on the sequence's ticket (S * passes when S > 1, else 0)
  int32_t pad;
};

// ---------------------------------------------------------------------------------------
// Tree verification workspace layout.
//   [0, 256)                 header: err word
//   [256, 256 + 32B)         TreeDraw [B], written by the walk, read by the draw kernel
//   [256 + 32B, +2048B)      chunk_sums: double [B][kMaxChunks]; during the walk, the first
//                            2 * kMaxTreeParts of each sequence's row hold the parts' partial sums
// A sequence's ticket first counts the walk's arrivals (its parts arrive once per residual
// pass), then the draw kernel's chunks; the draw's last chunk resets it to 0.
//   [..., end)               tickets: int32, sequence b at end - 4(b+1); they return to 0
// Every call checks bytes >= 256 + 2084 B, so a call's tickets never overlap data an earlier
// call (any B) left behind (the same argument as for the verification workspace).
// ---------------------------------------------------------------------------------------
inline size_t tree_verify_bytes(long long B) { return align256(256 + (size_t)B * (32 + kMaxChunks * 8 + 4)); }

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
  TreeDraw* draws;          // [B], written at the end of the walk
  int32_t S;                // workgroups per sequence (1 .. kMaxTreeParts)
  double* xch;              // partial-sum slots: sequence b at xch + b * xch_stride, [2][S]
  int32_t xch_stride;
  int32_t* tickets_end;     // sequence b's ticket is tickets_end[-(b + 1)] (zero at the start of a call)
};

struct TreeDrawParams {
  const float* p;
  const float* q;
  const float* uniforms;    // [B][N]: uniforms[b][0] drives the final draw
  int32_t* out_ids;         // [B][N]: entry n of sequence b receives the drawn token
  const TreeDraw* draws;
  int32_t B, N, V;
  int32_t C, CS;            // chunks per row and their length (multiple of 4, <= 4096)
  double* chunk_sums;       // [B][C]
  int32_t* tickets_end;     // ticket of sequence b is tickets_end[-(b + 1)]
  int32_t* err;
};

hipError_t launch_tree_verify(const TreeVerifyParams& p, hipStream_t stream, KTimer t = {});
hipError_t launch_tree_draw(const TreeDrawParams& p, bool vec4, hipStream_t stream, KTimer t = {});

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
