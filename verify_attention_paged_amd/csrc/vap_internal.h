// Internal declarations of the library's other kernels (verification, tree verification,
// logits, KV append/commit, utilities), plus the attention declarations (not part of the C ABI).
#pragma once

#include "attn_internal.h"

namespace vap {

// ---------------------------------------------------------------------------------------
// Per-sequence records of the verification workspaces.  Sequence b owns the record at
// base + b * stride; its first 4 bytes are the sequence's arrival ticket, which only the ticket
// logic ever writes and which is zero between calls (the last arrival of a call resets it).
// A ticket's place depends on b alone, and no call writes data over any record's ticket, so a
// zero-filled workspace serves calls of any batch size, k, vocabulary and workspace_bytes
// (at or above what each call needs), in stream order, without being cleared again.
// ---------------------------------------------------------------------------------------
constexpr int kMaxChunks = 256;
constexpr long long kMaxVerifySeqs = 1LL << 22;

struct SeqRecords {
  char* base;
  long long stride;
  __host__ __device__ int32_t* ticket(long long b) const { return reinterpret_cast<int32_t*>(base + b * stride); }
  // data of record b, `off` bytes in (off >= 16 keeps it clear of the ticket)
  template <typename T>
  __host__ __device__ T* at(long long b, int off) const { return reinterpret_cast<T*>(base + b * stride + off); }
};

// Workgroup index in sequence-major order, XCD-aware: the GPU deals workgroup i to XCD i % 8
// and each XCD has its own L2, so each XCD takes a contiguous range of indices.  The workgroups
// of one sequence then share an L2: a draw's last workgroup rescans a chunk that a sibling
// streamed from that L2 instead of from HBM, and the tree walk's workgroups exchange their chunk
// sums within one XCD.
constexpr int kXCDs = 8;
__device__ __forceinline__ int seq_major_index() {
  if (gridDim.x % kXCDs != 0) return blockIdx.x;
  return (int)(blockIdx.x % kXCDs) * (int)(gridDim.x / kXCDs) + (int)(blockIdx.x / kXCDs);
}

// Cross-lane moves of the verifiers' reductions and scans through DPP (row shifts and row
// broadcasts): a modifier on a VALU move, where __shfl_* takes one LDS-crossbar round trip
// (ds_bpermute) per 32-bit half.  Lanes without a source, or outside ROW_MASK, read 0.  The
// wave must be fully active.
constexpr int kDppRowShr = 0x110, kDppWaveShr1 = 0x138, kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ double dpp_f64(double x) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(x);
  const unsigned lo = (unsigned)__builtin_amdgcn_update_dpp(0, (int)(unsigned)u, CTRL, ROW_MASK, 0xf, false);
  const unsigned hi = (unsigned)__builtin_amdgcn_update_dpp(0, (int)(unsigned)(u >> 32), CTRL, ROW_MASK, 0xf, false);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}
// Sum over lanes 0 .. lane, in a fixed order: steps of 1, 2, 4, 8 lanes inside each 16-lane
// row, then row 0's total into row 1 and row 2's into row 3, then lane 31's into rows 2 and 3.
__device__ __forceinline__ double wave_incl_scan(double x) {
  x += dpp_f64<kDppRowShr + 1>(x);
  x += dpp_f64<kDppRowShr + 2>(x);
  x += dpp_f64<kDppRowShr + 4>(x);
  x += dpp_f64<kDppRowShr + 8>(x);
  x += dpp_f64<kDppRowBcast15, 0xa>(x);
  x += dpp_f64<kDppRowBcast31, 0xc>(x);
  return x;
}
__device__ __forceinline__ double lane_value(double x, int lane) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(x);
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)u, lane);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(u >> 32), lane);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}
// Sum of x over the wave, on every lane (fixed order)
__device__ __forceinline__ double wave_total(double x) { return lane_value(wave_incl_scan(x), 63); }

// Publishing an fp64 value to other workgroups through a workspace slot.  The slot holds the
// complement of the value's bits and is zero between calls, so a reader can tell a value that
// is not yet visible (zero) from any value: no value published here has all 64 bits set (the
// values are sums of non-negative weights converted from fp32, and the low 29 bits of a NaN
// that comes from fp32 are zero).  Writer and reader use agent-scope atomic accesses to the
// slot itself and nothing else: the reader spins until the slot is nonzero, which per-location
// coherence guarantees it eventually sees once the writer has stored, and no ordering between
// different locations is assumed (so no cache-wide writeback or invalidate is needed).  The
// spin is bounded as a guard; it never runs out while the writer has already stored (the
// callers only read slots whose writer has arrived or is resident).
constexpr int kSlotSpinMax = 1 << 18;

__device__ __forceinline__ void publish_slot(unsigned long long* slot, double v) {
  __hip_atomic_store(slot, ~(unsigned long long)__double_as_longlong(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The published value, waiting until it is visible; *timed_out is set if the guard ran out
// (the value then reads 0).
__device__ __forceinline__ double read_slot(unsigned long long* slot, bool* timed_out) {
  unsigned long long x = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int it = 0; x == 0ull; ++it) {
    if (it >= kSlotSpinMax) {
      *timed_out = true;
      return 0.0;
    }
    __builtin_amdgcn_s_sleep(1);
    x = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return __longlong_as_double((long long)~x);
}

__device__ __forceinline__ void clear_slot(unsigned long long* slot) {
  __hip_atomic_store(slot, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// spec_verify workspace:
//   [0, 256)   header: err word
//   records    [B] of kVerifyRec bytes: ticket, then at +16 the published chunk sums [C]
//              (C <= kMaxChunks) of the row the sequence draws from (zero between calls)
constexpr int kVerifyRecSums = 16;
constexpr size_t kVerifyRec = kVerifyRecSums + 8 * kMaxChunks;

inline size_t verify_bytes(long long B) { return align256(256 + (size_t)B * kVerifyRec); }

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
  int32_t WPS;      // workgroups per sequence (each takes G = ceil(C / WPS) consecutive chunks)
  int32_t* err;
  SeqRecords rec;   // sequence b: ticket, and its chunk sums at +kVerifyRecSums
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
//   records         [B] of kVerifyRec bytes, as for spec_verify (ticket, chunk sums)
// The records' place depends on k and V, so an earlier call of another shape may have left
// data under this call's tickets and slots: the statistics kernel, which runs first, zeroes
// the ones this call uses.
// ---------------------------------------------------------------------------------------
constexpr int kStatChunk = 2048;        // tokens per statistics item (32 per lane of a wave)
constexpr int kStatMaxChunks = 512;     // V <= 2^20
#ifndef VAP_STAT_WAVES_PER_CU
#define VAP_STAT_WAVES_PER_CU 8
#endif
constexpr int kStatWavesPerCU = VAP_STAT_WAVES_PER_CU;   // persistent statistics waves
constexpr int kStatWavesPerWG = 4;                       // 256-thread statistics workgroups

struct LogitsLayout {
  size_t part, records, total;
};

inline LogitsLayout logits_layout(long long B, int k, int V) {
  LogitsLayout L;
  const long long R = B * (2 * k + 1);
  const long long C1 = (V + kStatChunk - 1) / kStatChunk;
  size_t o = 256;
  L.part = o;     o = align256(o + (size_t)(R * C1) * sizeof(LogitRowStat));
  L.records = o;  o = align256(o + (size_t)B * kVerifyRec);
  L.total = o;
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
  SeqRecords rec;           // the verification's records: their tickets and first VC slots are zeroed here
  int32_t VC;               // verification chunks per row
};

// launchers (defined in the .hip files); return hipError_t of the launch
hipError_t launch_spec_verify(const VerifyParams& p, bool vec4, hipStream_t stream, KTimer t = {});
hipError_t launch_spec_verify_logits(const VerifyParams& p, bool vec4, hipStream_t stream, KTimer t = {});
hipError_t launch_logit_stats(const LogitStatsParams& p, bool vec4, int num_wg, hipStream_t stream, KTimer t = {});
hipError_t launch_fill_zero(void* dst, size_t bytes, hipStream_t stream);

// Vocabulary chunking of a verification draw over B sequences on a GPU of `cus` CUs: C chunks of
// CS tokens per row (C <= kMaxChunks slots; CS a multiple of 4, at most kDrawPiece = 1024 while
// the vocabulary allows, else up to 4096), about eight chunks per CU over the batch.  One wave
// sums a chunk (in pieces of kDrawPiece tokens) and publishes it; the selecting workgroup holds
// one chunk in registers.  WPS workgroups per sequence each take G = ceil(C / WPS) consecutive
// chunks, their four waves taking every fourth: about four workgroups per CU over the batch, and
// at least four chunks per workgroup.
constexpr int kDrawPiece = 1024;
struct DrawChunks {
  int C, CS, WPS;
};

inline DrawChunks draw_chunks(long long B, long long V, int cus) {
  long long C = (8LL * cus + B - 1) / B;
  const long long cmax = (V + 255) / 256 < kMaxChunks ? (V + 255) / 256 : kMaxChunks;
  C = C < 1 ? 1 : (C > cmax ? cmax : C);
  const long long cmin = (V + kDrawPiece - 1) / kDrawPiece;
  if (C < cmin) C = cmin < kMaxChunks ? cmin : kMaxChunks;
  if (C < (V + 4095) / 4096) C = (V + 4095) / 4096;
  long long CS = (V + C - 1) / C;
  CS = (CS + 3) / 4 * 4;
  C = (V + CS - 1) / CS;
  long long WPS = (4LL * cus + B - 1) / B;
  const long long wmax = (C + 3) / 4;
  WPS = WPS < 1 ? 1 : (WPS > wmax ? wmax : WPS);
  const long long G = (C + WPS - 1) / WPS;
  WPS = (C + G - 1) / G;          // no workgroup without a chunk
  return DrawChunks{(int)C, (int)CS, (int)WPS};
}

// Host side of spec_verify with its records (kVerifyRec bytes per sequence, tickets and slots
// zero) at `records` and its device error word at `err`: checks the call and launches the
// kernel; returns a VAP_* code (api.cpp, shared by spec_verify and spec_verify_static).
int verify_dispatch(const float* p, const float* q, const int32_t* draft_ids, const float* uniforms,
                    int32_t* out_ids, int32_t* n_accepted, int32_t num_seqs, int32_t k, int32_t vocab,
                    char* records, int32_t* err, hipStream_t stream);
// Records a host-side error for vap_last_error_message(); returns `code`.
int host_error(int code, const char* msg);
hipError_t launch_stream_copy(void* dst, const void* src, size_t bytes, hipStream_t stream);
hipError_t launch_stream_read(const void* src, size_t bytes, void* sink, hipStream_t stream);

// ---------------------------------------------------------------------------------------
// Tree verification: a walk (S workgroups per sequence walking together and sharing its
// vocabulary-wide sums), then the final draw.
// ---------------------------------------------------------------------------------------
constexpr int kMaxTreeNodes = 64;
constexpr int kWalkPasses = 16;   // residual sums of a walk that its workgroups share
constexpr int kWalkChunks = 16;   // each such sum is split into this many chunk sums at most
constexpr int kMaxWalkWgs = 16;   // workgroups per sequence at most

// Chunks of the walk's residual sums: kWalkChunks at most, each a multiple of 4096 elements (so
// a 1024-thread workgroup takes whole float4s), the last one possibly shorter.
struct WalkChunks {
  int32_t C, CS;
};
inline __host__ __device__ WalkChunks walk_chunks(int V) {
  const int per = (V + kWalkChunks - 1) / kWalkChunks;
  const int CS = ((per + 4095) / 4096) * 4096;
  return WalkChunks{(V + CS - 1) / CS, CS};
}

// Where the walk of one sequence ended: the final draw is from max(0, p - c q) of node `node`
// (c = 0: p itself), or, if those weights are all zero, from max(0, p - c_prev q) (a walk that
// ends in a rejection skips the pass that would have checked this); its token goes to
// out_ids[b][n].
struct TreeDraw {
  double c;
  double c_prev;
  int32_t node;
  int32_t n;
  int32_t passes;   // shared sums of the walk (their slots are cleared by the draw kernel)
  int32_t pad;
};

// ---------------------------------------------------------------------------------------
// Tree verification workspace layout.
//   [0, 256)       header: err word
//   records        [B] of kTreeRec bytes:
//     +0              the sequence's ticket (the draw kernel's chunks arrive on it; its last
//                     chunk resets it to 0)
//     +kTreeRecDraw   TreeDraw, written by the walk, read by the draw kernel
//     +kTreeRecSums   published slots [kMaxChunks]: the draw's chunk sums (zero between calls,
//                     see publish_slot)
//     +kTreeRecWalk   published slots [kWalkPasses][kWalkChunks]: the chunk sums of the walk's
//                     shared residual sums sum_x max(0, p - c q) (zero between calls: the draw
//                     kernel clears what the walk used)
// ---------------------------------------------------------------------------------------
constexpr int kTreeRecDraw = 16;
constexpr int kTreeRecSums = kTreeRecDraw + (int)sizeof(TreeDraw);
constexpr int kTreeRecWalk = kTreeRecSums + 8 * kMaxChunks;
constexpr size_t kTreeRec = kTreeRecWalk + 8 * kWalkPasses * kWalkChunks;
static_assert(kTreeRecSums % 16 == 0 && kTreeRecWalk % 16 == 0 && kTreeRec % 16 == 0,
              "tree record fields stay 16-byte aligned");

inline size_t tree_verify_bytes(long long B) { return align256(256 + (size_t)B * kTreeRec); }

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
  int32_t S;                // workgroups walking each sequence together
  int32_t wait_ticks;       // how long a workgroup waits for another chunk sum (100 MHz ticks)
  int32_t* err;
  SeqRecords rec;           // TreeDraw of each sequence, written at the end of its walk; walk slots
};

struct TreeDrawParams {
  const float* p;
  const float* q;
  const float* uniforms;    // [B][N]: uniforms[b][0] drives the final draw
  int32_t* out_ids;         // [B][N]: entry n of sequence b receives the drawn token
  int32_t B, N, V;
  int32_t C, CS;            // chunks per row and their length (multiple of 4, <= 4096)
  int32_t WPS;              // workgroups per sequence (each takes G = ceil(C / WPS) consecutive chunks)
  SeqRecords rec;           // ticket, TreeDraw, chunk sums [C]
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
