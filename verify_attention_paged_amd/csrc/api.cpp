// Host side of the C ABI declared in include/vap.h: argument validation, workspace carving,
// kernel dispatch, error reporting and the measurement helpers.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <mutex>
#include <string>

#include "vap_internal.h"

namespace {

using namespace vap;

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return VAP_OK;
}

// ---- per-device facts ------------------------------------------------------------------

struct DevInfo {
  bool probed = false;
  bool gfx950 = false;
  int num_cus = 0;
  char arch[64] = {0};
  int attn_occ[2][2][3][2] = {};   // workgroups per CU of the attention kernel [D128][BS32][NRT 1/2/4][KV8]
};

constexpr int kMaxDevices = 64;
std::mutex g_mu;
DevInfo g_dev[kMaxDevices];

const DevInfo* device_info() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  DevInfo& d = g_dev[dev];
  if (!d.probed) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return nullptr;
    d.num_cus = prop.multiProcessorCount;
    std::strncpy(d.arch, prop.gcnArchName, sizeof(d.arch) - 1);
    d.gfx950 = std::strncmp(d.arch, "gfx950", 6) == 0;
    for (int a = 0; a < 2; ++a)
      for (int b = 0; b < 2; ++b)
        for (int c = 0; c < 3; ++c)
          for (int k8 = 0; k8 < 2; ++k8) {
            int nb = 0;
            // occupancy with the largest in-workgroup plan (LDS never binds before registers)
            const void* f = attn_main_kernel_ptr(a ? 128 : 64, b ? 32 : 16, 1 << c, true, k8 != 0);
            if (f == nullptr ||
                hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, f, kAttnThreads,
                                                              attn_main_lds_bytes(kLdsPlanMaxSeqs)) != hipSuccess ||
                nb < 1)
              nb = 1;
            d.attn_occ[a][b][c][k8] = nb;
          }
    d.probed = true;
  }
  return &d;
}

// ---- kernel timer ------------------------------------------------------------------------

constexpr int kTimerSlots = 4096;
constexpr int kTimerKinds = 8;   // attention, spec_verify, spec_verify_tree walk, kv_append, kv_commit,
                                  // logit statistics, verification from logits, tree draw
struct Timer {
  bool on = false;
  bool created = false;
  hipEvent_t start[kTimerKinds][kTimerSlots];
  hipEvent_t stop[kTimerKinds][kTimerSlots];
  int count[kTimerKinds] = {};
};
Timer g_timer;

// Events for the next timed launch of `kind` (null pair when the timer is off or its ring is
// full); timer_commit keeps them once the launch has been enqueued.
KTimer timer_slot(int kind) {
  KTimer t;
  if (g_timer.on && g_timer.count[kind] < kTimerSlots) {
    t.start = g_timer.start[kind][g_timer.count[kind]];
    t.stop = g_timer.stop[kind][g_timer.count[kind]];
  }
  return t;
}

void timer_commit(int kind, const KTimer& t, hipError_t launch) {
  if (t.start != nullptr && launch == hipSuccess) ++g_timer.count[kind];
}

// ---- attention shape checks ---------------------------------------------------------------

// Fixed cost of starting a unit of work, in work blocks: a few 16-token tiles of streaming
// time (its query rows and block-table window are dependent loads that the tile pipeline
// cannot hide).  Counting it balances waves that start many short units.  Measured best:
// 2 tiles for one-tile (decode) units over bf16 K/V, 4 over the 8-bit cache (its tiles cost
// more math), 12 for units of several row tiles (verify rows, trees, prefill chunks).
#ifndef VAP_UNIT_SETUP_TILES_1RT
#define VAP_UNIT_SETUP_TILES_1RT 2
#endif
#ifndef VAP_UNIT_SETUP_TILES_KV8
#define VAP_UNIT_SETUP_TILES_KV8 4
#endif
#ifndef VAP_UNIT_SETUP_TILES_NRT
#define VAP_UNIT_SETUP_TILES_NRT 12
#endif
int unit_setup_blocks(int block_size, int nrt, bool kv8) {
  const int tiles = kv8 ? VAP_UNIT_SETUP_TILES_KV8 : (nrt == 1 ? VAP_UNIT_SETUP_TILES_1RT : VAP_UNIT_SETUP_TILES_NRT);
  return std::max(1, tiles * 16 / block_size);
}

struct AttnPlanChoice {
  int D, BS, NRT, RG, G;
  bool kv8;
  int rows_per_seq;   // total_q / num_seqs, rounded down
};

int check_attn_shape(const vap_attn_shape* s, AttnPlanChoice* c) {
  if (s == nullptr) return fail(VAP_EINVAL, "shape is NULL");
  if (s->num_seqs < 0 || s->num_seqs > kMaxSeqs)
    return fail(VAP_EINVAL, "num_seqs=%d outside [0, %d]", s->num_seqs, kMaxSeqs);
  if (s->num_kv_heads < 1 || s->num_q_heads < 1 || s->num_q_heads % s->num_kv_heads)
    return fail(VAP_EINVAL, "num_q_heads=%d must be a positive multiple of num_kv_heads=%d",
                s->num_q_heads, s->num_kv_heads);
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(VAP_EINVAL, "head_dim=%d not supported (64 or 128)", s->head_dim);
  if (s->block_size != 16 && s->block_size != 32)
    return fail(VAP_EINVAL, "block_size=%d not supported (16 or 32)", s->block_size);
  if (s->num_blocks < 1 || s->max_blocks_per_seq < 1)
    return fail(VAP_EINVAL, "num_blocks=%d and max_blocks_per_seq=%d must be >= 1", s->num_blocks,
                s->max_blocks_per_seq);
  if (s->total_q < 0) return fail(VAP_EINVAL, "total_q=%d < 0", s->total_q);
  if (!(std::isfinite(s->scale) && s->scale >= 0.f)) return fail(VAP_EINVAL, "scale must be finite and >= 0");
  c->kv8 = false;
  c->rows_per_seq = s->num_seqs > 0 ? s->total_q / s->num_seqs : 0;
  c->D = s->head_dim;
  c->BS = s->block_size;
  c->G = s->num_q_heads / s->num_kv_heads;
  // decode-only batches (one row per sequence) with at most 16 rows per KV head use one
  // 16-row MFMA tile per unit; batches averaging 48 or more rows per KV head and sequence
  // (token trees, prefill chunks) use four (64 rows per unit, so K/V are read once for up to
  // 64 rows); everything else uses two (32 rows per unit)
  const long long rows_per_kvh = s->num_seqs > 0 ? (long long)c->G * s->total_q / s->num_seqs : 0;
  c->NRT = (s->total_q == s->num_seqs && c->G <= 16) ? 1 : (rows_per_kvh >= 48 ? 4 : 2);
  c->RG = 16 * c->NRT;
  const long long cap = (long long)s->max_blocks_per_seq * s->block_size;
  if (cap * s->num_q_heads >= (1LL << 31))
    return fail(VAP_EINVAL, "max_blocks_per_seq*block_size*num_q_heads exceeds 2^31");
  if ((long long)s->total_q * s->num_q_heads >= (1LL << 31))
    return fail(VAP_EINVAL, "total_q*num_q_heads exceeds 2^31");
  const long long rows_groups = ((long long)c->G * s->total_q + c->RG - 1) / c->RG + s->num_seqs;
  if ((long long)s->num_kv_heads * (s->max_blocks_per_seq + std::max(unit_setup_blocks(c->BS, c->NRT, false), unit_setup_blocks(c->BS, c->NRT, true))) * rows_groups >= (1LL << 31) - 1)
    return fail(VAP_EINVAL, "work of the step may exceed 2^31 blocks");
  return VAP_OK;
}

// Worker waves: one workgroup per CU for decode- and verify-shaped batches.  Each wave keeps
// two tiles in flight; at that depth the memory system is already saturated for this access
// pattern, so more waves only add latency to every dependent load (and partials to merge).
// Batches averaging 8 or more query rows per sequence (prefill chunks) make the MFMA work per
// byte large enough that a second workgroup per CU pays.
#ifndef VAP_WAVES_PER_SIMD_DECODE
#define VAP_WAVES_PER_SIMD_DECODE 1
#endif
#ifndef VAP_WAVES_PER_SIMD_PREFILL
#define VAP_WAVES_PER_SIMD_PREFILL 2
#endif
// Waves per attention workgroup: three for decode- and verify-shaped batches over bf16 K/V,
// four otherwise.  With two tiles in flight per wave, three waves per CU already saturate HBM
// for the bf16 gather: against four, the kernel was about 1 us faster and the step 1.5-2 us
// faster (a quarter fewer partials to merge).  The 8-bit cache's heavier tile math and
// prefill batches want the fourth wave (8-bit decode 43.5 against 50.6 us, mixed batch 346
// against 364 us).
#ifndef VAP_DECODE_WG_WAVES
#define VAP_DECODE_WG_WAVES 3
#endif
int attn_wg_waves(const AttnPlanChoice& c) { return (!c.kv8 && c.rows_per_seq < 8) ? VAP_DECODE_WG_WAVES : kWavesPerWG; }

int worker_waves(const DevInfo* d, const AttnPlanChoice& c) {
  const int occ = d->attn_occ[c.D == 128][c.BS == 32][c.NRT == 1 ? 0 : (c.NRT == 2 ? 1 : 2)][c.kv8 ? 1 : 0];
  const int per_cu = c.rows_per_seq >= 8 ? VAP_WAVES_PER_SIMD_PREFILL : VAP_WAVES_PER_SIMD_DECODE;
  return std::min(kMaxWaves, d->num_cus * std::min(occ, per_cu) * attn_wg_waves(c));
}

// Pool of the attention step: the last VAP_POOL_PCT percent of the work, in pieces of
// VAP_POOL_PIECE work blocks, is left out of the worker waves' static shares; waves that
// finish their share early take the pieces one at a time, so slow waves end sooner.  At most
// one piece per two worker waves.  The kernel uses it for bf16 steps of 16-row units with at
// least 32 work blocks per wave: with fewer blocks per wave, with the 8-bit cache's cheaper
// blocks, or with 32- and 64-row units (whose restart loads more query rows and leaves a
// larger partial to merge), a piece's restart cost as much as the balance gained or more.
#ifndef VAP_POOL_PCT
#define VAP_POOL_PCT 10
#endif
#ifndef VAP_POOL_PIECE
#define VAP_POOL_PIECE 12
#endif
int pool_max(int W) { return VAP_POOL_PCT > 0 ? W / 2 : 0; }

AttnLayout layout_of(int B, int W, const AttnPlanChoice& c) {
  return attn_layout(B, W, c.RG, c.D, W + pool_max(W));
}

// Shape and pointer checks shared by kv_append and kv_commit.
int check_kv_call(const vap_attn_shape* shape, const void* kv, const float* kv_scales, const void* workspace,
                  size_t workspace_bytes) {
  AttnPlanChoice c;
  const int rc = check_attn_shape(shape, &c);
  if (rc != VAP_OK) return rc;
  if ((long long)shape->num_blocks * shape->block_size >= (1LL << 31))
    return fail(VAP_EINVAL, "num_blocks*block_size exceeds 2^31");
  if (shape->num_seqs == 0) return VAP_OK;
  if (!kv || !workspace) return fail(VAP_EINVAL, "NULL data pointer");
  if ((reinterpret_cast<uintptr_t>(kv) | reinterpret_cast<uintptr_t>(kv_scales)) & 15)
    return fail(VAP_EINVAL, "the KV pool and its scales must be 16-byte aligned");
  if (workspace_bytes < vap_kv_workspace_bytes())
    return fail(VAP_ENOSPC, "workspace of %zu bytes is below %zu", workspace_bytes, vap_kv_workspace_bytes());
  if (reinterpret_cast<uintptr_t>(workspace) & 15) return fail(VAP_EINVAL, "workspace must be 16-byte aligned");
  return VAP_OK;
}

const DevInfo* gfx950_or_null() {
  const DevInfo* d = device_info();
  return (d != nullptr && d->gfx950) ? d : nullptr;
}

}  // namespace

namespace vap {

int host_error(int code, const char* msg) { return fail(code, "%s", msg); }

int verify_dispatch(const float* p, const float* q, const int32_t* draft_ids, const float* uniforms,
                    int32_t* out_ids, int32_t* n_accepted, int32_t num_seqs, int32_t k, int32_t vocab,
                    char* records, int32_t* err, hipStream_t stream) {
  if (num_seqs < 0 || num_seqs > kMaxVerifySeqs)
    return fail(VAP_EINVAL, "num_seqs=%d outside [0, %lld]", num_seqs, kMaxVerifySeqs);
  if (k < 0 || k > 64) return fail(VAP_EINVAL, "k=%d outside [0, 64]", k);
  if (vocab < 1) return fail(VAP_EINVAL, "vocab=%d < 1", vocab);
  if ((long long)vocab > (long long)kMaxChunks * 4096)
    return fail(VAP_EINVAL, "vocab=%d above %d", vocab, kMaxChunks * 4096);
  if (num_seqs == 0) return ok();
  if (!p || !uniforms || !out_ids || !n_accepted || !records || !err || (k > 0 && (!q || !draft_ids)))
    return fail(VAP_EINVAL, "NULL data pointer");
  const DevInfo* d = device_info();
  if (d == nullptr || !d->gfx950) return fail(VAP_ENODEV, "current device is not gfx950 (%s)", d ? d->arch : "none");

  const DrawChunks ch = draw_chunks(num_seqs, vocab, d->num_cus);
  VerifyParams P;
  P.p = p;
  P.q = q;
  P.draft_ids = draft_ids;
  P.uniforms = uniforms;
  P.out_ids = out_ids;
  P.n_accepted = n_accepted;
  P.B = num_seqs;
  P.k = k;
  P.V = vocab;
  P.C = ch.C;
  P.CS = ch.CS;
  P.WPS = ch.WPS;
  P.err = err;
  P.rec = SeqRecords{records, (long long)kVerifyRec};
  const bool vec4 = (vocab % 4 == 0) &&
                    ((reinterpret_cast<uintptr_t>(p) | reinterpret_cast<uintptr_t>(k ? q : p)) & 15) == 0;
  const KTimer t = timer_slot(1);
  hipError_t e = launch_spec_verify(P, vec4, stream, t);
  timer_commit(1, t, e);
  if (e != hipSuccess) return fail(VAP_EHIP, "spec_verify launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace vap

extern "C" {

const char* vap_strerror(int code) {
  switch (code) {
    case VAP_OK: return "ok";
    case VAP_EINVAL: return "invalid argument";
    case VAP_ENOSPC: return "workspace too small";
    case VAP_EHIP: return "HIP runtime error";
    case VAP_ENODEV: return "no gfx950 device is current";
    default: return "unknown error";
  }
}

const char* vap_last_error_message(void) { return g_last_error.c_str(); }

size_t vap_attn_workspace_bytes(const vap_attn_shape* shape) {
  AttnPlanChoice c;
  if (check_attn_shape(shape, &c) != VAP_OK) return 0;
  const DevInfo* d = device_info();
  // one workspace serves the bf16 and the 8-bit cache: size it for the larger launch
  int W = 256 * kWavesPerWG * 2;
  if (d) {
    AttnPlanChoice c8 = c;
    c8.kv8 = true;
    W = std::max(worker_waves(d, c), worker_waves(d, c8));
  }
  return layout_of(shape->num_seqs, W, c).total;
}

size_t vap_attn_workspace_min_bytes(const vap_attn_shape* shape) {
  AttnPlanChoice c;
  if (check_attn_shape(shape, &c) != VAP_OK) return 0;
  return layout_of(shape->num_seqs, kWavesPerWG, c).total;
}

}  // extern "C"

namespace {

// Shared body of the bf16 and 8-bit entry points: kv_scales == nullptr selects the bf16 pool.
int attn_step(const void* q, const void* kv, const float* kv_scales, const int32_t* block_tables,
              const int32_t* ctx_lens, const int32_t* q_lens, const uint64_t* tree_mask, float* out,
              const vap_attn_shape* shape, void* workspace, size_t workspace_bytes, void* stream_, bool kv8,
              bool fp8 = false) {
  AttnPlanChoice c;
  int rc = check_attn_shape(shape, &c);
  if (rc != VAP_OK) return rc;
  c.kv8 = kv8;
  const vap_attn_shape& s = *shape;
  if (s.num_seqs == 0) {
    if (s.total_q != 0) return fail(VAP_EINVAL, "num_seqs=0 but total_q=%d", s.total_q);
    return ok();
  }
  if (!q || !kv || !block_tables || !ctx_lens || !q_lens || !out || !workspace || (kv8 && !kv_scales))
    return fail(VAP_EINVAL, "NULL data pointer");
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(kv) | reinterpret_cast<uintptr_t>(kv_scales) |
       reinterpret_cast<uintptr_t>(out) | reinterpret_cast<uintptr_t>(workspace)) & 15)
    return fail(VAP_EINVAL, "q, the KV pool, its scales, out and workspace must be 16-byte aligned");
  const DevInfo* d = device_info();
  if (d == nullptr || !d->gfx950) return fail(VAP_ENODEV, "current device is not gfx950 (%s)", d ? d->arch : "none");

  // worker waves: as many as stay resident, fewer if the workspace is smaller
  int W = worker_waves(d, c);
  if (layout_of(s.num_seqs, W, c).total > workspace_bytes) {
    int lo = kWavesPerWG, hi = W;
    if (layout_of(s.num_seqs, lo, c).total > workspace_bytes)
      return fail(VAP_ENOSPC, "workspace of %zu bytes is below the minimum %zu", workspace_bytes,
                  layout_of(s.num_seqs, lo, c).total);
    while (lo < hi) {
      const int mid = (lo + hi + 1) / 2;
      if (layout_of(s.num_seqs, mid, c).total <= workspace_bytes) lo = mid; else hi = mid - 1;
    }
    W = lo;
  }
  const int wg_waves = attn_wg_waves(c);
  W = std::max(wg_waves, (W / wg_waves) * wg_waves);
  const AttnLayout lay = layout_of(s.num_seqs, W, c);
  char* ws = static_cast<char*>(workspace);

  AttnParams P;
  P.q = static_cast<const uint16_t*>(q);
  const size_t plane = (size_t)s.num_blocks * s.block_size * s.num_kv_heads * s.head_dim;
  P.kpool = kv8 ? nullptr : static_cast<const uint16_t*>(kv);
  P.vpool = kv8 ? nullptr : P.kpool + plane;
  P.kcodes = kv8 ? static_cast<const uint8_t*>(kv) : nullptr;
  P.vcodes = kv8 ? P.kcodes + plane : nullptr;
  P.kv_scales = kv8 ? kv_scales : nullptr;
  P.tree_mask = tree_mask;
  P.tables = block_tables;
  P.ctx_lens = ctx_lens;
  P.q_lens = q_lens;
  P.out = out;
  P.B = s.num_seqs;
  P.Hq = s.num_q_heads;
  P.Hkv = s.num_kv_heads;
  P.G = c.G;
  P.num_blocks = s.num_blocks;
  P.MB = s.max_blocks_per_seq;
  P.total_q = s.total_q;
  P.W = W;
  P.RG = c.RG;
  P.BS = c.BS;
  P.UH = unit_setup_blocks(c.BS, c.NRT, kv8);
  P.pool_max = pool_max(W);
  P.NH = W + P.pool_max;
  P.pool_pct = VAP_POOL_PCT;
  P.pool_piece = VAP_POOL_PIECE;
  const float scale = s.scale > 0.f ? s.scale : 1.0f / std::sqrt((float)s.head_dim);
  P.scale_log2 = scale * 1.4426950408889634f;
  P.hdr = reinterpret_cast<AttnHeader*>(ws);
  P.desc = reinterpret_cast<int32_t*>(ws + lay.desc);
  P.g_L = reinterpret_cast<int32_t*>(ws + lay.g_L);
  P.g_Q = reinterpret_cast<int32_t*>(ws + lay.g_Q);
  P.q_off = reinterpret_cast<int32_t*>(ws + lay.q_off);
  P.seq_off = reinterpret_cast<int32_t*>(ws + lay.seq_off);
  P.wave_seq = reinterpret_cast<int32_t*>(ws + lay.wave_seq);
  P.part_ml = reinterpret_cast<float2*>(ws + lay.part_ml);
  P.part_acc = reinterpret_cast<float*>(ws + lay.part_acc);

  hipStream_t stream = static_cast<hipStream_t>(stream_);
  hipError_t e = hipSuccess;
  if (s.num_seqs > kLdsPlanMaxSeqs) {
    e = launch_attn_plan(P, stream);
    if (e != hipSuccess) return fail(VAP_EHIP, "plan launch: %s", hipGetErrorString(e));
  }
  const KTimer t = timer_slot(0);
  e = launch_attn_main(P, c.D, c.BS, c.NRT, kv8 ? (fp8 ? 2 : 1) : 0, W / wg_waves, wg_waves, stream, t);
  timer_commit(0, t, e);
  if (e != hipSuccess) return fail(VAP_EHIP, "attention launch: %s", hipGetErrorString(e));
  e = launch_attn_combine(P, c.D, d->num_cus, c.rows_per_seq < 8, stream);
  if (e != hipSuccess) return fail(VAP_EHIP, "combine launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int paged_attn_step(const void* q, const void* kv_pool, const int32_t* block_tables,
                    const int32_t* ctx_lens, const int32_t* q_lens, float* out,
                    const vap_attn_shape* shape, void* workspace, size_t workspace_bytes,
                    void* stream) {
  return attn_step(q, kv_pool, nullptr, block_tables, ctx_lens, q_lens, nullptr, out, shape, workspace,
                   workspace_bytes, stream, false);
}

int paged_attn_step_u8(const void* q, const void* kv_codes, const float* kv_scales,
                       const int32_t* block_tables, const int32_t* ctx_lens, const int32_t* q_lens,
                       float* out, const vap_attn_shape* shape, void* workspace, size_t workspace_bytes,
                       void* stream) {
  return attn_step(q, kv_codes, kv_scales, block_tables, ctx_lens, q_lens, nullptr, out, shape, workspace,
                   workspace_bytes, stream, true);
}

int paged_attn_step_fp8(const void* q, const void* kv_codes, const float* kv_scales, const int32_t* block_tables,
                        const int32_t* ctx_lens, const int32_t* q_lens, float* out, const vap_attn_shape* shape,
                        void* workspace, size_t workspace_bytes, void* stream) {
  return attn_step(q, kv_codes, kv_scales, block_tables, ctx_lens, q_lens, nullptr, out, shape, workspace,
                   workspace_bytes, stream, true, true);
}

int paged_attn_step_tree(const void* q, const void* kv, const float* kv_scales, const int32_t* block_tables,
                         const int32_t* ctx_lens, const int32_t* q_lens, const uint64_t* tree_mask, float* out,
                         const vap_attn_shape* shape, void* workspace, size_t workspace_bytes, void* stream) {
  if (shape != nullptr && shape->num_seqs > 0 && tree_mask == nullptr) return fail(VAP_EINVAL, "NULL tree_mask");
  if (reinterpret_cast<uintptr_t>(tree_mask) & 7) return fail(VAP_EINVAL, "tree_mask must be 8-byte aligned");
  return attn_step(q, kv, kv_scales, block_tables, ctx_lens, q_lens, tree_mask, out, shape, workspace,
                   workspace_bytes, stream, kv_scales != nullptr);
}

size_t vap_verify_workspace_bytes(int32_t num_seqs, int32_t k, int32_t vocab) {
  if (num_seqs < 0 || num_seqs > kMaxVerifySeqs || k < 0 || k > 64 || vocab < 1) return 0;
  return verify_bytes(num_seqs);
}

int spec_verify(const float* p, const float* q, const int32_t* draft_ids, const float* uniforms,
                int32_t* out_ids, int32_t* n_accepted, int32_t num_seqs, int32_t k, int32_t vocab,
                void* workspace, size_t workspace_bytes, void* stream_) {
  if (num_seqs > 0 && !workspace) return fail(VAP_EINVAL, "NULL data pointer");
  if (num_seqs > 0 && num_seqs <= kMaxVerifySeqs && k >= 0 && k <= 64 && vocab >= 1 &&
      workspace_bytes < vap_verify_workspace_bytes(num_seqs, k, vocab))
    return fail(VAP_ENOSPC, "workspace of %zu bytes is below %zu", workspace_bytes,
                vap_verify_workspace_bytes(num_seqs, k, vocab));
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return fail(VAP_EINVAL, "workspace must be 256-byte aligned");
  char* ws = static_cast<char*>(workspace);
  return vap::verify_dispatch(p, q, draft_ids, uniforms, out_ids, n_accepted, num_seqs, k, vocab, ws + 256,
                              reinterpret_cast<int32_t*>(ws), static_cast<hipStream_t>(stream_));
}

size_t vap_verify_logits_workspace_bytes(int32_t num_seqs, int32_t k, int32_t vocab) {
  if (num_seqs < 0 || num_seqs > kMaxVerifySeqs || k < 0 || k > 64 || vocab < 1 || vocab > kMaxChunks * 4096) return 0;
  return logits_layout(num_seqs, k, vocab).total;
}

int spec_verify_logits(const float* target_logits, const float* draft_logits, const int32_t* draft_ids,
                       const float* uniforms, const float* temperatures, int32_t* out_ids, int32_t* n_accepted,
                       int32_t num_seqs, int32_t k, int32_t vocab, void* workspace, size_t workspace_bytes,
                       void* stream_) {
  if (num_seqs < 0 || num_seqs > kMaxVerifySeqs)
    return fail(VAP_EINVAL, "num_seqs=%d outside [0, %lld]", num_seqs, kMaxVerifySeqs);
  if (k < 0 || k > 64) return fail(VAP_EINVAL, "k=%d outside [0, 64]", k);
  if (vocab < 1 || vocab > kMaxChunks * 4096) return fail(VAP_EINVAL, "vocab=%d outside [1, %d]", vocab, kMaxChunks * 4096);
  if (num_seqs == 0) return ok();
  if (!target_logits || !uniforms || !temperatures || !out_ids || !n_accepted || !workspace ||
      (k > 0 && (!draft_logits || !draft_ids)))
    return fail(VAP_EINVAL, "NULL data pointer");
  const LogitsLayout lay = logits_layout(num_seqs, k, vocab);
  if (workspace_bytes < lay.total)
    return fail(VAP_ENOSPC, "workspace of %zu bytes is below %zu", workspace_bytes, lay.total);
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return fail(VAP_EINVAL, "workspace must be 256-byte aligned");
  const long long R = (long long)num_seqs * (2 * k + 1);
  const long long C1 = ((long long)vocab + kStatChunk - 1) / kStatChunk;
  if (C1 > kStatMaxChunks) return fail(VAP_EINVAL, "vocab=%d needs more than %d statistics chunks", vocab, kStatMaxChunks);
  if (R * C1 + (long long)kStatWavesPerCU * 1024 >= (1LL << 31)) return fail(VAP_EINVAL, "too many logit rows");
  const DevInfo* d = device_info();
  if (d == nullptr || !d->gfx950) return fail(VAP_ENODEV, "current device is not gfx950 (%s)", d ? d->arch : "none");

  char* ws = static_cast<char*>(workspace);
  const SeqRecords rec{ws + lay.records, (long long)kVerifyRec};
  const bool vec4 = (vocab % 4 == 0) && ((reinterpret_cast<uintptr_t>(target_logits) |
                                           reinterpret_cast<uintptr_t>(k ? draft_logits : target_logits)) & 15) == 0;
  LogitStatsParams S;
  S.zp = target_logits;
  S.zq = draft_logits;
  S.temps = temperatures;
  S.part = reinterpret_cast<LogitRowStat*>(ws + lay.part);
  S.B = num_seqs;
  S.k = k;
  S.V = vocab;
  S.C = (int)C1;
  S.err = reinterpret_cast<int32_t*>(ws);
  S.rec = rec;
  // persistent statistics waves: kStatWavesPerCU per CU, no more than there are items
  const long long stat_waves = std::min(R * C1, (long long)d->num_cus * kStatWavesPerCU);
  const int stat_wg = (int)((stat_waves + kStatWavesPerWG - 1) / kStatWavesPerWG);

  // verification chunks: as spec_verify
  const DrawChunks ch = draw_chunks(num_seqs, vocab, d->num_cus);
  VerifyParams P;
  P.p = target_logits;
  P.q = draft_logits;
  P.draft_ids = draft_ids;
  P.uniforms = uniforms;
  P.out_ids = out_ids;
  P.n_accepted = n_accepted;
  P.B = num_seqs;
  P.k = k;
  P.V = vocab;
  P.C = ch.C;
  P.CS = ch.CS;
  P.WPS = ch.WPS;
  P.err = reinterpret_cast<int32_t*>(ws);
  P.rec = rec;
  S.VC = ch.C;
  P.temps = temperatures;
  P.part = S.part;
  P.C1 = (int)C1;

  hipStream_t stream = static_cast<hipStream_t>(stream_);
  const KTimer t1 = timer_slot(5);
  hipError_t e = launch_logit_stats(S, vec4, stat_wg, stream, t1);
  timer_commit(5, t1, e);
  if (e != hipSuccess) return fail(VAP_EHIP, "logit statistics launch: %s", hipGetErrorString(e));
  const KTimer t2 = timer_slot(6);
  e = launch_spec_verify_logits(P, vec4, stream, t2);
  timer_commit(6, t2, e);
  if (e != hipSuccess) return fail(VAP_EHIP, "spec_verify_logits launch: %s", hipGetErrorString(e));
  return ok();
}

// A workgroup of the tree walk waits for the other workgroups' chunk sums only while they keep
// arriving: at most this long without a new one (100 MHz ticks: 6 us), then it computes the rest
// itself.
#ifndef VAP_WALK_WAIT_TICKS
#define VAP_WALK_WAIT_TICKS 600
#endif

size_t vap_tree_verify_workspace_bytes(int32_t num_seqs) {
  if (num_seqs < 0 || num_seqs > kMaxVerifySeqs) return 0;
  return tree_verify_bytes(num_seqs);
}

int spec_verify_tree(const float* p, const float* q, const int32_t* parents, const int32_t* tokens,
                     const float* uniforms, int32_t* out_ids, int32_t* out_path, int32_t* n_accepted,
                     int32_t num_seqs, int32_t num_nodes, int32_t vocab, void* workspace,
                     size_t workspace_bytes, void* stream_) {
  if (num_seqs < 0 || num_seqs > kMaxVerifySeqs)
    return fail(VAP_EINVAL, "num_seqs=%d outside [0, %lld]", num_seqs, kMaxVerifySeqs);
  if (num_nodes < 1 || num_nodes > kMaxTreeNodes)
    return fail(VAP_EINVAL, "num_nodes=%d outside [1, %d]", num_nodes, kMaxTreeNodes);
  if (vocab < 1 || vocab > kMaxChunks * 4096) return fail(VAP_EINVAL, "vocab=%d outside [1, %d]", vocab, kMaxChunks * 4096);
  if (num_seqs == 0) return ok();
  if (!p || !q || !parents || !tokens || !uniforms || !out_ids || !out_path || !n_accepted || !workspace)
    return fail(VAP_EINVAL, "NULL data pointer");
  if (workspace_bytes < vap_tree_verify_workspace_bytes(num_seqs))
    return fail(VAP_ENOSPC, "workspace of %zu bytes is below %zu", workspace_bytes,
                vap_tree_verify_workspace_bytes(num_seqs));
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return fail(VAP_EINVAL, "workspace must be 256-byte aligned");
  const DevInfo* d = device_info();
  if (d == nullptr || !d->gfx950) return fail(VAP_ENODEV, "current device is not gfx950 (%s)", d ? d->arch : "none");
  char* ws = static_cast<char*>(workspace);
  TreeVerifyParams P;
  P.p = p;
  P.q = q;
  P.parents = parents;
  P.tokens = tokens;
  P.uniforms = uniforms;
  P.out_ids = out_ids;
  P.out_path = out_path;
  P.n_accepted = n_accepted;
  P.B = num_seqs;
  P.N = num_nodes;
  P.V = vocab;
  P.vec4 = (vocab % 4 == 0) && ((reinterpret_cast<uintptr_t>(p) | reinterpret_cast<uintptr_t>(q)) & 15) == 0;
  P.err = reinterpret_cast<int32_t*>(ws);
  P.rec = SeqRecords{ws + 256, (long long)kTreeRec};
  // workgroups walking each sequence together: up to two 1024-thread workgroups per CU in all,
  // and no more than a shared sum has chunks
  P.S = std::max(1, std::min({kMaxWalkWgs, walk_chunks(vocab).C, 2 * d->num_cus / num_seqs}));
  P.wait_ticks = VAP_WALK_WAIT_TICKS;

  // draw chunks: as spec_verify
  const DrawChunks ch = draw_chunks(num_seqs, vocab, d->num_cus);
  TreeDrawParams D;
  D.p = p;
  D.q = q;
  D.uniforms = uniforms;
  D.out_ids = out_ids;
  D.B = num_seqs;
  D.N = num_nodes;
  D.V = vocab;
  D.C = ch.C;
  D.CS = ch.CS;
  D.WPS = ch.WPS;
  D.rec = P.rec;
  D.err = P.err;

  hipStream_t stream = static_cast<hipStream_t>(stream_);
  const KTimer t = timer_slot(2);
  hipError_t e = launch_tree_verify(P, stream, t);
  timer_commit(2, t, e);
  if (e != hipSuccess) return fail(VAP_EHIP, "tree verify launch: %s", hipGetErrorString(e));
  const KTimer t2 = timer_slot(7);
  e = launch_tree_draw(D, P.vec4, stream, t2);
  timer_commit(7, t2, e);
  if (e != hipSuccess) return fail(VAP_EHIP, "tree draw launch: %s", hipGetErrorString(e));
  return ok();
}

size_t vap_kv_workspace_bytes(void) { return 256; }

int kv_append(const void* k_new, const void* v_new, void* kv, float* kv_scales, const int32_t* block_tables,
              const int32_t* ctx_lens, const int32_t* q_lens, const vap_attn_shape* shape, void* workspace,
              size_t workspace_bytes, void* stream_) {
  int rc = check_kv_call(shape, kv, kv_scales, workspace, workspace_bytes);
  if (rc != VAP_OK) return rc;
  const vap_attn_shape& s = *shape;
  if (s.num_seqs == 0) {
    if (s.total_q != 0) return fail(VAP_EINVAL, "num_seqs=0 but total_q=%d", s.total_q);
    return ok();
  }
  if (!block_tables || !ctx_lens || !q_lens || (s.total_q > 0 && (!k_new || !v_new)))
    return fail(VAP_EINVAL, "NULL data pointer");
  if ((reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new)) & 15)
    return fail(VAP_EINVAL, "k_new and v_new must be 16-byte aligned");
  const DevInfo* d = gfx950_or_null();
  if (d == nullptr) return fail(VAP_ENODEV, "current device is not gfx950");
  KVAppendParams P;
  P.k_new = static_cast<const uint16_t*>(k_new);
  P.v_new = static_cast<const uint16_t*>(v_new);
  P.kv = kv;
  P.kv_scales = kv_scales;
  P.tables = block_tables;
  P.ctx_lens = ctx_lens;
  P.q_lens = q_lens;
  P.B = s.num_seqs;
  P.Hkv = s.num_kv_heads;
  P.BS = s.block_size;
  P.NB = s.num_blocks;
  P.MB = s.max_blocks_per_seq;
  P.T = s.total_q;
  P.err = static_cast<int32_t*>(workspace);
  // one wave per (row, group of 64 / (D / 8) heads); at most two workgroups per CU, each of
  // which rebuilds the row starts of the whole batch in LDS
  const int hpp = 64 / (s.head_dim / 8);
  const long long items = (long long)s.total_q * ((s.num_kv_heads + hpp - 1) / hpp);
  const long long wg = std::max(1LL, std::min((items + 3) / 4, 2LL * d->num_cus));
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  const KTimer t = timer_slot(3);
  const hipError_t e = launch_kv_append(P, s.head_dim, kv_scales != nullptr, (int)wg, stream, t);
  timer_commit(3, t, e);
  if (e != hipSuccess) return fail(VAP_EHIP, "kv_append launch: %s", hipGetErrorString(e));
  return ok();
}

int kv_commit(void* kv, float* kv_scales, const int32_t* block_tables, const int32_t* ctx_lens, const int32_t* q_lens,
              const int32_t* path, int32_t path_stride, const int32_t* n_accepted, int32_t* out_ctx_lens,
              const vap_attn_shape* shape, void* workspace, size_t workspace_bytes, void* stream_) {
  int rc = check_kv_call(shape, kv, kv_scales, workspace, workspace_bytes);
  if (rc != VAP_OK) return rc;
  const vap_attn_shape& s = *shape;
  if (s.num_seqs == 0) return ok();
  if (!block_tables || !ctx_lens || !q_lens || !n_accepted || !out_ctx_lens) return fail(VAP_EINVAL, "NULL data pointer");
  if (path != nullptr && path_stride < 1) return fail(VAP_EINVAL, "path_stride=%d < 1", path_stride);
  if (gfx950_or_null() == nullptr) return fail(VAP_ENODEV, "current device is not gfx950");
  KVCommitParams P;
  P.kv = kv;
  P.kv_scales = kv_scales;
  P.tables = block_tables;
  P.ctx_lens = ctx_lens;
  P.q_lens = q_lens;
  P.path = path;
  P.path_stride = path_stride;
  P.n_accepted = n_accepted;
  P.out_lens = out_ctx_lens;
  P.B = s.num_seqs;
  P.Hkv = s.num_kv_heads;
  P.D = s.head_dim;
  P.BS = s.block_size;
  P.NB = s.num_blocks;
  P.MB = s.max_blocks_per_seq;
  P.err = static_cast<int32_t*>(workspace);
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  const KTimer t = timer_slot(4);
  const hipError_t e = launch_kv_commit(P, kv_scales != nullptr, stream, t);
  timer_commit(4, t, e);
  if (e != hipSuccess) return fail(VAP_EHIP, "kv_commit launch: %s", hipGetErrorString(e));
  return ok();
}

int vap_workspace_init(void* workspace, size_t bytes, void* stream) {
  if (!workspace) return fail(VAP_EINVAL, "NULL workspace");
  if (bytes == 0) return ok();
  const hipError_t e = launch_fill_zero(workspace, bytes, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(VAP_EHIP, "fill launch: %s", hipGetErrorString(e));
  return ok();
}

int vap_get_device_error(void* workspace, void* stream_, int32_t* err_out, int clear) {
  if (!workspace || !err_out) return fail(VAP_EINVAL, "NULL pointer");
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  hipError_t e = hipStreamSynchronize(stream);
  if (e == hipSuccess) e = hipMemcpy(err_out, workspace, sizeof(int32_t), hipMemcpyDeviceToHost);
  if (e == hipSuccess && clear) {
    e = launch_fill_zero(workspace, sizeof(int32_t), stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
  }
  if (e != hipSuccess) return fail(VAP_EHIP, "reading the error word: %s", hipGetErrorString(e));
  return ok();
}

int vap_timer_enable(int on) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (on && !g_timer.created) {
    for (int k = 0; k < kTimerKinds; ++k)
      for (int i = 0; i < kTimerSlots; ++i) {
        if (hipEventCreate(&g_timer.start[k][i]) != hipSuccess || hipEventCreate(&g_timer.stop[k][i]) != hipSuccess)
          return fail(VAP_EHIP, "hipEventCreate failed");
      }
    g_timer.created = true;
  }
  g_timer.on = on != 0;
  return ok();
}

int vap_timer_read(int kind, double* total_ms, int32_t* count, int reset) {
  if (kind < 0 || kind >= kTimerKinds || !total_ms || !count) return fail(VAP_EINVAL, "bad timer arguments");
  double sum = 0.0;
  const int n = g_timer.count[kind];
  for (int i = 0; i < n; ++i) {
    float ms = 0.f;
    if (hipEventSynchronize(g_timer.stop[kind][i]) != hipSuccess ||
        hipEventElapsedTime(&ms, g_timer.start[kind][i], g_timer.stop[kind][i]) != hipSuccess)
      return fail(VAP_EHIP, "reading timer events failed");
    sum += ms;
  }
  *total_ms = sum;
  *count = n;
  if (reset) g_timer.count[kind] = 0;
  return ok();
}

int vap_stream_copy(void* dst, const void* src, size_t bytes, void* stream) {
  if (!dst || !src) return fail(VAP_EINVAL, "NULL pointer");
  if ((bytes & 15) || ((reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(src)) & 15))
    return fail(VAP_EINVAL, "bytes and pointers must be multiples of 16");
  const hipError_t e = launch_stream_copy(dst, src, bytes, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(VAP_EHIP, "copy launch: %s", hipGetErrorString(e));
  return ok();
}

int vap_stream_read(const void* src, size_t bytes, void* sink, void* stream) {
  if (!src || !sink) return fail(VAP_EINVAL, "NULL pointer");
  if ((bytes & 15) || ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(sink)) & 15))
    return fail(VAP_EINVAL, "bytes and pointers must be multiples of 16");
  const hipError_t e = launch_stream_read(src, bytes, sink, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(VAP_EHIP, "read launch: %s", hipGetErrorString(e));
  return ok();
}

int vap_device_info(int32_t* num_cus, char* arch_name, size_t arch_name_len) {
  const DevInfo* d = device_info();
  if (d == nullptr) return fail(VAP_ENODEV, "no current HIP device");
  if (num_cus) *num_cus = d->num_cus;
  if (arch_name && arch_name_len) {
    std::strncpy(arch_name, d->arch, arch_name_len - 1);
    arch_name[arch_name_len - 1] = 0;
  }
  return ok();
}

}  // extern "C"
