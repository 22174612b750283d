/*
 * vap.h -- C ABI of the paged decode/verify attention and speculative verification library
 * for AMD Instinct MI355X (gfx950).
 *
 * Two operations form one continuous-batching step's data-parallel work:
 *
 *   paged_attn_step  attention of a ragged batch of query rows over a paged KV cache.  The KV
 *                    cache is a pool of fixed-size blocks and each sequence owns a block table
 *                    mapping logical blocks to pool blocks (tempatgunting.com article,
 *                    section "Anatomy of the KV Cache: Memory Layout, Paging and Quantization
 *                    Trade-offs"; syslabs.in "Continuous Batching and Speculative Decoding: How
 *                    Modern LLM Serving Engines Actually Work", section "PagedAttention: making
 *                    the KV cache schedulable").  A sequence brings 1 decode row, k+1 verify
 *                    rows, or a prefill chunk; the rows are causal among themselves, so k+1
 *                    verify rows equal k+1 sequential decodes (syslabs.in, section "The core
 *                    idea").
 *
 *   spec_verify      speculative-decoding verification by modified rejection sampling: accept
 *                    draft x_i when r_i <= min(1, p_i(x_i)/q_i(x_i)); on the first rejection
 *                    draw the replacement from max(0, p - q) normalised; if every draft is
 *                    accepted draw a bonus token from p_k (neuralmasteryai.com "Continuous
 *                    Batching & Speculative Decoding", section "The Modified Rejection Sampling
 *                    Algorithm"; syslabs.in, section "The core idea").
 *
 * Around them, kv_append writes the step's new K/V rows into the cache before the attention,
 * and kv_commit keeps the accepted draft tokens' rows (moving a tree's accepted path into
 * place) and sets the committed lengths after verification.
 *
 * Conventions shared by every entry point:
 *   - Data pointers are DEVICE pointers owned by the caller.  The library never allocates,
 *     frees or synchronises device memory on these paths (vap_get_device_error is the only
 *     call that synchronises).  Inputs are read-only; outputs are fully overwritten.
 *   - `stream` is a hipStream_t passed as void* (NULL = the legacy default stream).  All work
 *     is enqueued on it, in order.
 *   - Return value: VAP_OK (0) or a negative VAP_E* code for an error detected on the host,
 *     in which case nothing was enqueued -- except VAP_EHIP, a kernel launch that failed after
 *     the call's earlier kernels were enqueued; the workspace must then be zero-filled again
 *     before its next use (a step leaves per-call state there, such as claim counters, that
 *     only its last kernel resets).  vap_last_error_message() describes the last host error
 *     of the calling thread.
 *   - Errors found in the data on the device (a block id outside the pool, inconsistent
 *     lengths, a draft id outside the vocabulary) never fault: the kernels clamp, OR a
 *     VAP_DERR_* bit into a sticky word at the start of the workspace, and leave the affected
 *     outputs unspecified (but written only inside the output arrays).
 *   - A workspace must be zero-filled before its first use (vap_workspace_init, or any
 *     zero-filled allocation); every call leaves it reusable by later calls of the same entry
 *     point with any sizes and any workspace_bytes at or above what each call needs (per-call
 *     state such as arrival tickets sits at offsets that depend on neither).  Calls that share
 *     a workspace must be ordered (same stream, or synchronised).  A workspace serves one kind
 *     of call (the paged_attn_step family, spec_verify, spec_verify_logits or
 *     spec_verify_tree); kv_append and kv_commit touch only the sticky error word and may
 *     share any of them.
 */
#ifndef VAP_H_
#define VAP_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* host-side return codes */
#define VAP_OK 0
#define VAP_EINVAL (-1)  /* null pointer, unsupported or inconsistent sizes            */
#define VAP_ENOSPC (-2)  /* workspace smaller than the required minimum                */
#define VAP_EHIP (-3)    /* a HIP runtime call or kernel launch failed                  */
#define VAP_ENODEV (-4)  /* no usable gfx950 device is current                          */

/* device-side data error bits (sticky, OR-ed into the workspace's first 32-bit word) */
#define VAP_DERR_BLOCK_ID 0x1  /* block table entry outside [0, num_blocks) inside a context */
#define VAP_DERR_LENS 0x2      /* q_len < 1, q_len > ctx_len, or ctx_len > table capacity     */
#define VAP_DERR_TOTAL_Q 0x4   /* sum of q_lens differs from total_q                          */
#define VAP_DERR_DRAFT_ID 0x8  /* draft id outside [0, vocab)                                  */
#define VAP_DERR_EMPTY_ROW 0x10 /* the row to sample from has no positive weight              */
#define VAP_DERR_TREE 0x20      /* tree mask without the row's own bit or with bits past it, or
                                   a tree of more than 64 rows (the row is then repaired: own
                                   bit set, later bits cleared; or kept causal)              */
#define VAP_DERR_TEMP 0x40      /* temperature negative or not finite (the sequence is greedy)  */
#define VAP_DERR_SYNC 0x80      /* spec_verify, spec_verify_logits and spec_verify_tree's draw: a
                                   workgroup reading a value that another workgroup of the same
                                   call has already stored waited past a guard of about a
                                   quarter of a second (never expected: the guard only keeps
                                   every wait finite)                                          */

/*
 * Shape of one attention step.
 *   num_seqs            B, 0 <= B <= 8192
 *   num_q_heads         Hq, a multiple of num_kv_heads
 *   num_kv_heads        Hkv >= 1 (query head h reads KV head h / (Hq/Hkv))
 *   head_dim            D, 64 or 128
 *   block_size          tokens per KV block, 16 or 32
 *   num_blocks          blocks in the KV pool
 *   max_blocks_per_seq  width of a block-table row
 *   total_q             T = number of packed query rows (must equal the sum of q_lens)
 *   scale               softmax scale; 0 means 1/sqrt(head_dim)
 */
typedef struct vap_attn_shape {
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t total_q;
  float scale;
} vap_attn_shape;

/* Workspace bytes paged_attn_step needs for `shape` on the current device (0 on bad shape).
 * A smaller workspace (but at least the minimum reported by vap_attn_workspace_min_bytes)
 * also works: the library then partitions the work into fewer pieces. */
size_t vap_attn_workspace_bytes(const vap_attn_shape* shape);
size_t vap_attn_workspace_min_bytes(const vap_attn_shape* shape);

/*
 * paged_attn_step -- attention for one ragged batch over a paged KV cache.
 *
 *   q             bf16 [total_q][Hq][D]; rows packed by sequence, sequences in order, so
 *                 sequence s owns rows [sum_{r<s} q_lens[r], ... + q_lens[s]).
 *   kv_pool       bf16 [2][num_blocks][block_size][Hkv][D]; plane 0 holds K, plane 1 holds V.
 *   block_tables  int32 [num_seqs][max_blocks_per_seq]; entry j of row s is the pool block
 *                 of logical block j of sequence s.  Entries past ceil(ctx_len/block_size)
 *                 are never read (any value, e.g. -1).  Rows may share blocks.
 *   ctx_lens      int32 [num_seqs]; L_s, the number of cached tokens INCLUDING this step's
 *                 q_len new tokens (whose K and V are already in the pool).
 *   q_lens        int32 [num_seqs]; Q_s >= 1.  Row i of sequence s sits at position
 *                 L_s - Q_s + i and attends keys 0 .. L_s - Q_s + i.
 *   out           fp32 [total_q][Hq][D]; softmax(scale * q k^T) v per row and head.
 *   workspace     device scratch of workspace_bytes (see vap_attn_workspace_bytes).
 *
 * Enqueues the attention kernel and a combine kernel for the units split across worker waves
 * on `stream` (preceded by a plan kernel when num_seqs > 2048).
 */
int paged_attn_step(const void* q, const void* kv_pool, const int32_t* block_tables,
                    const int32_t* ctx_lens, const int32_t* q_lens, float* out,
                    const vap_attn_shape* shape, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * paged_attn_step_u8 -- paged_attn_step over an 8-bit KV cache, dequantised inside the kernel
 * (tempatgunting.com article, section "Quantization and Precision Choices for KV": INT8 KV with
 * per-token or per-head scale factors, asymmetric, separate scales for K and V).
 *
 *   kv_codes   uint8 [2][num_blocks][block_size][Hkv][D]; plane 0 holds K, plane 1 holds V.
 *   kv_scales  fp32 [num_blocks][Hkv][block_size][4] = (k_scale, k_zero, v_scale, v_zero) for
 *              each cached token and KV head.  The value of code c is scale * (c - zero).
 *
 * Everything else (shape, q, tables, lengths, out, workspace and its size, errors) is as for
 * paged_attn_step; the same workspace serves both.  All pointers 16-byte aligned.  Scales of
 * rows past ctx_len are never read.
 */
int paged_attn_step_u8(const void* q, const void* kv_codes, const float* kv_scales,
                       const int32_t* block_tables, const int32_t* ctx_lens, const int32_t* q_lens,
                       float* out, const vap_attn_shape* shape, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * paged_attn_step_fp8 -- paged_attn_step_u8 with FP8 codes: each byte of kv_codes is an OCP FP8
 * E4M3 value (sign, 4-bit exponent with bias 7, 3-bit mantissa; subnormals; no infinities), and
 * element = scale * (e4m3 - zero) with the same per-token, per-KV-head kv_scales layout
 * (tempatgunting.com article, section "Quantization and Precision Choices for KV": FP8 or INT8
 * KV with per-head or per-token scale factors, dequantised inside the attention kernel).  A
 * symmetric FP8 cache stores zero points of 0.  Everything else (shape, q, tables, lengths, out,
 * workspace, errors) is as for paged_attn_step_u8; the same workspace serves both.
 */
int paged_attn_step_fp8(const void* q, const void* kv_codes, const float* kv_scales, const int32_t* block_tables,
                        const int32_t* ctx_lens, const int32_t* q_lens, float* out, const vap_attn_shape* shape,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_attn_step_tree -- paged_attn_step where each sequence's q_len new rows are the nodes of
 * a draft token tree verified in one pass under a tree attention mask (neuralmasteryai.com
 * "Continuous Batching & Speculative Decoding", section "4. Tree Attention & Medusa Heads").
 *
 *   tree_mask  uint64 [total_q], 8-byte aligned.  Nodes are numbered 0 .. q_len-1 within their
 *              sequence in an order where ancestors come first; node i sits at position
 *              L - q_len + i.  Bit j of node i's mask is set when node i attends node j: its
 *              ancestors and itself (so only bits 0 .. i).  Every node also attends the whole
 *              committed prefix, positions 0 .. L - q_len - 1.  A chain (mask of node i =
 *              bits 0 .. i) is the causal verify of paged_attn_step.  q_len <= 64.
 *   kv, kv_scales  a bf16 pool as for paged_attn_step when kv_scales is NULL, else 8-bit codes
 *              and their scales as for paged_attn_step_u8.
 *
 * A mask without its own bit or with bits past its node, or a sequence of more than 64 rows,
 * sets VAP_DERR_TREE; the row then uses its mask with its own bit set and later bits cleared
 * (or stays causal past 64 rows).  Everything else is as for paged_attn_step.
 */
int paged_attn_step_tree(const void* q, const void* kv, const float* kv_scales, const int32_t* block_tables,
                         const int32_t* ctx_lens, const int32_t* q_lens, const uint64_t* tree_mask, float* out,
                         const vap_attn_shape* shape, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes spec_verify needs (0 on bad sizes). */
size_t vap_verify_workspace_bytes(int32_t num_seqs, int32_t k, int32_t vocab);

/*
 * spec_verify -- modified rejection sampling for a batch of speculative drafts.
 *
 *   p           fp32 [B][k+1][V]  target probabilities at the k draft positions and the
 *                                 bonus position (used as given; need not sum to 1)
 *   q           fp32 [B][k][V]    draft probabilities (may be NULL when k == 0)
 *   draft_ids   int32 [B][k]      draft tokens (may be NULL when k == 0)
 *   uniforms    fp32 [B][k+1]     values in (0,1): uniforms[b][i] is r_i for i < k and
 *                                 uniforms[b][k] drives the final draw
 *   out_ids     int32 [B][k+1]    accepted drafts, then the drawn token, then -1 padding
 *   n_accepted  int32 [B]         number of accepted drafts n in [0, k]
 *   0 <= B <= 2^22, 0 <= k <= 64, 1 <= V <= 2^20.
 *
 * Per sequence: x_i is accepted iff p_i(x_i) > 0 and r_i * q_i(x_i) <= p_i(x_i) (exact in
 * fp64); the first rejection at n stops the tests.  The emitted token is drawn from
 * w = max(0, p_n - q_n) (n < k) or w = p_k (n == k) by inverse CDF in ascending token id:
 * t = uniforms[b][k] * Z with Z = sum(w) in fp64, and the token is the smallest x whose
 * running sum exceeds t.  If Z == 0 the row p_n is used instead.  A draft id outside [0,V)
 * is rejected and sets VAP_DERR_DRAFT_ID.
 */
int spec_verify(const float* p, const float* q, const int32_t* draft_ids, const float* uniforms,
                int32_t* out_ids, int32_t* n_accepted, int32_t num_seqs, int32_t k, int32_t vocab,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * spec_verify_static -- spec_verify without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).
 *
 *   p, q, draft_ids, uniforms, out_ids, n_accepted, num_seqs, k, vocab  as for spec_verify,
 *                  with 0 <= num_seqs <= 4096 (VAP_EINVAL above: use spec_verify).
 *   device_error   NULL, or a caller-owned device int32 into which the kernel ORs the
 *                  VAP_DERR_* bits of the call (it is not cleared first).
 *
 * The scratch is a static device array of the library (8,454,400 bytes, one per device), looked up
 * and zero-filled at the first call on each device; nothing is allocated or freed by any call.
 * Every call on a device uses the same array, so calls on one device must not overlap in time
 * (one stream, or synchronised).  Results are those of spec_verify.
 */
int spec_verify_static(const float* p, const float* q, const int32_t* draft_ids, const float* uniforms,
                       int32_t* out_ids, int32_t* n_accepted, int32_t num_seqs, int32_t k, int32_t vocab,
                       int32_t* device_error, void* stream);

/* Workspace bytes spec_verify_logits needs (0 on bad sizes). */
size_t vap_verify_logits_workspace_bytes(int32_t num_seqs, int32_t k, int32_t vocab);

/*
 * spec_verify_logits -- spec_verify from logits: temperature, softmax and the verification in
 * one pass over the logits, without writing probability rows (tempatgunting.com article,
 * section "Speculative Decoding: Turning Verification Parallelism into Latency Wins": the
 * verify pass returns logits [k+1][vocab] and tokens are sampled from logits).
 *
 *   target_logits  fp32 [B][k+1][V]   logits at the k draft positions and the bonus position
 *   draft_logits   fp32 [B][k][V]     the draft model's logits (may be NULL when k == 0)
 *   temperatures   fp32 [B]           sampling temperature T per sequence
 *   draft_ids, uniforms, out_ids, n_accepted, B, k, V  as for spec_verify (V <= 2^20)
 *
 * With T > 0: p_i = softmax(target_logits_i / T) and q_i = softmax(draft_logits_i / T), and
 * spec_verify's rule runs on them.  Every probability the rule needs is evaluated in fp64 as
 * 2^((z - max z) log2(e) / T) / S, S being the row's fp64 sum of those terms.  With T = 0
 * (greedy, exact token matching: tempatgunting.com article, section "Frequently Asked
 * Questions"): draft x_i is accepted while it is the first argmax of target row i; the
 * emitted token is the first argmax of target row n; draft logits are not read.  A negative
 * or non-finite T sets VAP_DERR_TEMP and the sequence is treated as greedy.  Logits must be
 * finite or -inf, with at least one finite entry per row.
 *
 * Two kernels on `stream`: row statistics (max, argmax, sum of exponentials) of all rows,
 * then the verification.  The workspace (vap_verify_logits_workspace_bytes) serves
 * spec_verify_logits calls only.
 */
int spec_verify_logits(const float* target_logits, const float* draft_logits, const int32_t* draft_ids,
                       const float* uniforms, const float* temperatures, int32_t* out_ids, int32_t* n_accepted,
                       int32_t num_seqs, int32_t k, int32_t vocab, void* workspace, size_t workspace_bytes,
                       void* stream);

/* Zero-fill `bytes` of a workspace on `stream` (a fill kernel, no memset node). */
int vap_workspace_init(void* workspace, size_t bytes, void* stream);

/* Synchronise `stream` and read the sticky VAP_DERR_* bits of a workspace into *err_out;
 * clear them afterwards when `clear` is nonzero. */
int vap_get_device_error(void* workspace, void* stream, int32_t* err_out, int clear);

/* Static text for a VAP_* return code. */
const char* vap_strerror(int code);

/* Detail of the calling thread's last host-side error ("" if none). */
const char* vap_last_error_message(void);

/* Workspace bytes spec_verify_tree needs for num_seqs sequences (0 on bad sizes). */
size_t vap_tree_verify_workspace_bytes(int32_t num_seqs);

/*
 * spec_verify_tree -- verify a draft token tree per sequence (modified rejection sampling,
 * neuralmasteryai.com "Continuous Batching & Speculative Decoding", sections "The Modified
 * Rejection Sampling Algorithm" and "4. Tree Attention & Medusa Heads").
 *
 *   p          fp32 [B][N][V]  target next-token distribution after each node
 *   q          fp32 [B][N][V]  draft distribution each node's children were drawn from
 *   parents    int32 [B][N]    parent of each node: -1 for node 0 (the last committed token),
 *                              0 <= parent[i] < i otherwise
 *   tokens     int32 [B][N]    draft token of each node (entry 0 unused)
 *   uniforms   fp32 [B][N]     in (0,1): uniforms[i] decides node i's accept test (i > 0),
 *                              uniforms[0] the final draw
 *   out_ids    int32 [B][N]    accepted tokens along the path, then the drawn token, then -1
 *   out_path   int32 [B][N]    accepted node indices along the path, then -1
 *   n_accepted int32 [B]       number of accepted draft nodes
 *   1 <= N <= 64, 1 <= V <= 2^20.
 *
 * Per sequence: at the current node, its children are tested in index order; child c with
 * token x passes when p_cur(x) > 0 and uniforms[c] * q(x) <= p_cur(x) (q = the current node's
 * draft row, decided in fp64).  After a rejection p_cur becomes max(0, p_cur - q), normalised
 * (unchanged when it sums to 0).  The first child that passes is accepted and the walk moves to
 * it with p_cur = its target row.  With no child left, one token is drawn from p_cur (inverse
 * CDF in ascending token id, t = uniforms[0] * sum).  A chain-shaped tree gives spec_verify's
 * result.  Invalid parents set VAP_DERR_TREE (the node is then nobody's child); draft ids
 * outside the vocabulary VAP_DERR_DRAFT_ID (rejected).  Two kernels on `stream`: the walk (up
 * to 16 workgroups per sequence, which take the same decisions and share the chunks of each
 * residual sum through the workspace; none ever waits on another for more than a short bounded
 * time, after which it computes the missing chunks itself), then the final draw spread over the
 * GPU, which also zeroes what the walk left in the workspace.  Results do not depend on how
 * many workgroups walk.  The workspace (zero-filled before first use) serves spec_verify_tree
 * calls only.
 */
int spec_verify_tree(const float* p, const float* q, const int32_t* parents, const int32_t* tokens,
                     const float* uniforms, int32_t* out_ids, int32_t* out_path, int32_t* n_accepted,
                     int32_t num_seqs, int32_t num_nodes, int32_t vocab, void* workspace,
                     size_t workspace_bytes, void* stream);

/* Workspace bytes kv_append and kv_commit need: they use only the sticky error word at its
 * start, so the workspace of the step's paged_attn_step (used in stream order) serves too. */
size_t vap_kv_workspace_bytes(void);

/*
 * kv_append -- write one step's new K and V rows into the paged cache (tempatgunting.com
 * article, section "Anatomy of the KV Cache: Memory Layout, Paging and Quantization
 * Trade-offs"), before paged_attn_step reads them.
 *
 *   k_new, v_new  bf16 [total_q][Hkv][D], 16-byte aligned; rows packed by sequence exactly as
 *                 the query rows of paged_attn_step (sequence s owns q_lens[s] rows).
 *   kv            the pool, written in place: bf16 [2][num_blocks][block_size][Hkv][D] when
 *                 kv_scales is NULL, else uint8 codes of the same shape.
 *   kv_scales     NULL, or fp32 [num_blocks][Hkv][block_size][4] written in place (as for
 *                 paged_attn_step_u8).
 *   block_tables, ctx_lens, q_lens, shape  as for paged_attn_step: ctx_lens already count the
 *                 new rows, so row i of sequence s goes to position ctx_len - q_len + i.
 *
 * The 8-bit cache stores each (token, KV head) row of K and of V on its own (tempatgunting.com
 * article, section "Quantization and Precision Choices for KV": per-token, asymmetric, separate
 * for K and V), computed in fp32 from the bf16 input x (D values):
 *   lo = min(0, min x), hi = max(0, max x), scale = max((hi - lo) / 255, FLT_EPSILON),
 *   zero = clamp(rint((0 - lo) / scale), 0, 255), code = clamp(rint(x * (1 / scale)) + zero, 0, 255)
 * with IEEE division and round-half-even; inputs must be finite.  Nothing but the new rows'
 * entries (and their scales) is written.  Rows whose sequence has inconsistent lengths
 * (VAP_DERR_LENS) or a block id outside the pool (VAP_DERR_BLOCK_ID) are skipped; a sum of
 * q_lens other than total_q sets VAP_DERR_TOTAL_Q.  Rows of different sequences must not map to
 * the same slot.  One kernel on `stream`.
 */
int kv_append(const void* k_new, const void* v_new, void* kv, float* kv_scales, const int32_t* block_tables,
              const int32_t* ctx_lens, const int32_t* q_lens, const vap_attn_shape* shape, void* workspace,
              size_t workspace_bytes, void* stream);

/*
 * kv_commit -- keep the accepted draft tokens of a verified step and drop the rest
 * (tempatgunting.com article, section "Speculative Decoding: Turning Verification Parallelism
 * into Latency Wins": the rejected tokens' KV is rolled back).
 *
 *   kv, kv_scales  the pool as for kv_append, updated in place.
 *   block_tables, ctx_lens, q_lens, shape  those of the verified step (the q_len rows are the
 *                  last committed token and the drafts, at positions ctx_len - q_len ...).
 *   path           NULL for a chain of drafts (nothing moves), or int32 [num_seqs][path_stride]:
 *                  the accepted tree nodes a_1 < a_2 < ... < a_n (node i at position
 *                  ctx_len - q_len + i; spec_verify_tree's out_path).  Node a_i's K, V (and
 *                  scales) move to position ctx_len - q_len + i, so the kept tokens are
 *                  contiguous.  With a path, n <= min(63, path_stride).
 *   n_accepted     int32 [num_seqs], n in [0, q_len - 1].
 *   out_ctx_lens   int32 [num_seqs] = ctx_len - q_len + 1 + n: the committed length (the last
 *                  committed token and the n accepted drafts).  May be ctx_lens itself.
 *
 * Slots past the committed length keep stale entries; they are never read.  A sequence with
 * inconsistent lengths or n (VAP_DERR_LENS), a path that is not increasing within [1, q_len - 1]
 * (VAP_DERR_TREE) or a block id outside the pool (VAP_DERR_BLOCK_ID) is left unchanged with
 * out_ctx_len = ctx_len.  One workgroup per sequence on `stream`.
 */
int kv_commit(void* kv, float* kv_scales, const int32_t* block_tables, const int32_t* ctx_lens, const int32_t* q_lens,
              const int32_t* path, int32_t path_stride, const int32_t* n_accepted, int32_t* out_ctx_lens,
              const vap_attn_shape* shape, void* workspace, size_t workspace_bytes, void* stream);

/* ---- measurement helpers (not part of the step) ------------------------------------------ */

/* Kernel timer.  While enabled, every paged_attn_step times its attention kernel (kind 0),
 * every spec_verify its kernel (kind 1), spec_verify_tree its walk (kind 2) and its final
 * draw (kind 7), kv_append (kind 3) and kv_commit (kind 4) theirs, and spec_verify_logits its
 * statistics kernel (kind 5) and its verification kernel (kind 6); into a ring of 4096 event
 * pairs per kind.  The events are stamped
 * by the kernel launch itself (hipExtLaunchKernelGGL), so each pair spans the kernel's execution
 * without the wait before its first wave.  vap_timer_read synchronises on the recorded
 * events, returns the summed milliseconds and the number of pairs, and resets the ring when
 * `reset` is nonzero. */
int vap_timer_enable(int on);
int vap_timer_read(int kind, double* total_ms, int32_t* count, int reset);

/* Plain streaming copy kernel (16-byte loads and stores) of `bytes` (a multiple of 16) from
 * src to dst on `stream`; used to measure the achievable HBM copy rate and to calibrate the
 * hardware byte counters. */
int vap_stream_copy(void* dst, const void* src, size_t bytes, void* stream);

/* Plain streaming read kernel over `bytes` (a multiple of 16) of src: the achievable HBM read
 * rate.  Writes at most one 16-byte value per workgroup into `sink` (16-byte aligned, room for
 * 16 * (8 * number of CUs) bytes) only if a checksum matches a sentinel, so the loads cannot be
 * elided. */
int vap_stream_read(const void* src, size_t bytes, void* sink, void* stream);

/* Number of compute units of the current device and its gfx arch name ("gfx950"). */
int vap_device_info(int32_t* num_cus, char* arch_name, size_t arch_name_len);

#ifdef __cplusplus
}
#endif

#endif /* VAP_H_ */
