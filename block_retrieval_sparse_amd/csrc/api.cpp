// C-ABI entry points of libbrs: argument validation on the host, then kernel
// launches on the caller's stream.  No call allocates device memory.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "brs_internal.h"

// Workspace of brs_retrieval_step_static: one array per GPU, held from the
// library's load until the process ends.  Host code must not use this name as
// an address (on the host it is only a stand-in for the symbol); the device
// address comes from hipGetSymbolAddress, per device.
constexpr size_t kStaticScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

thread_local char g_err[512] = "";
thread_local hipEvent_t g_prof_start = nullptr;
thread_local hipEvent_t g_prof_stop = nullptr;

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return BRS_OK;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(BRS_E_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_memory(const brs_memory* m) {
  if (!m) return fail(BRS_E_INVAL, "memory descriptor is NULL");
  if (m->dtype != BRS_F32 && m->dtype != BRS_BF16) return fail(BRS_E_INVAL, "dtype %d", m->dtype);
  if (m->rep_dtype != BRS_F32 && m->rep_dtype != BRS_BF16)
    return fail(BRS_E_INVAL, "rep_dtype %d", m->rep_dtype);
  if (m->rep_mode < BRS_REP_MEAN || m->rep_mode > BRS_REP_ATTNSCORE)
    return fail(BRS_E_INVAL, "rep_mode %d", m->rep_mode);
  if (m->reserved != 0) return fail(BRS_E_INVAL, "reserved field must be 0");
  if (m->batch < 1 || m->n_kv_heads < 1 || m->head_dim < 1 || m->block_size < 1 ||
      m->reps_per_block < 1 || m->rep_dim < 1 || m->rep_heads < 1)
    return fail(BRS_E_INVAL, "sizes must be >= 1");
  if (m->row_stride < m->head_dim) return fail(BRS_E_INVAL, "row_stride < head_dim");
  if ((m->row_stride * brs::elem_bytes(m->dtype)) % 4 != 0)
    return fail(BRS_E_INVAL, "row_stride * element size must be a multiple of 4 bytes");
  if (m->capacity < 0 || m->capacity > INT32_MAX) return fail(BRS_E_INVAL, "capacity out of range");
  if (m->length < 0 || m->length > m->capacity) return fail(BRS_E_INVAL, "length out of range");
  const bool embed = m->rep_mode == BRS_REP_EMBED;
  if (m->rep_heads != (embed ? 1 : m->n_kv_heads))
    return fail(BRS_E_INVAL, "rep_heads must be %d for this rep_mode", embed ? 1 : m->n_kv_heads);
  if (!embed && (m->rep_dim != m->head_dim || m->rep_dtype != m->dtype))
    return fail(BRS_E_INVAL, "rep_dim/rep_dtype must equal head_dim/dtype unless rep_mode is EMBED");
  if ((m->rep_mode == BRS_REP_MEAN || embed) && m->reps_per_block != 1)
    return fail(BRS_E_INVAL, "reps_per_block must be 1 for MEAN and EMBED");
  const bool ranked = m->rep_mode == BRS_REP_TOPNORM || m->rep_mode == BRS_REP_ATTNSCORE;
  if (ranked && (m->reps_per_block > m->block_size || m->reps_per_block > 64))
    return fail(BRS_E_INVAL, "TOPNORM and ATTNSCORE need reps_per_block <= min(block_size, 64)");
  if (ranked && m->block_size > 1024)
    return fail(BRS_E_UNSUPPORTED, "TOPNORM and ATTNSCORE support block_size <= 1024");
  if (!m->k || !m->v || !m->reps) return fail(BRS_E_INVAL, "k, v and reps must be non-NULL");
  if (!aligned(m->k, 16) || !aligned(m->v, 16) || !aligned(m->reps, 16))
    return fail(BRS_E_INVAL, "k, v and reps must be 16-byte aligned");
  return BRS_OK;
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int static_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(BRS_E_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(BRS_E_HIP, "hipGetSymbolAddress(scratch) gave NULL");
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return BRS_OK;
}

void eligible(int64_t N, int64_t B, int64_t S, int64_t W, int64_t* lo, int64_t* hi) {
  // Tokens outside the sinks and the window are [S, N - W); block b meets
  // them iff floor(S/B) <= b < ceil((N-W)/B); it must also be complete.
  const int64_t nb = N / B;
  int64_t l = S / B;
  if (l > nb) l = nb;
  int64_t h = l;
  if (N - W > S) {
    h = (N - W + B - 1) / B;
    if (h > nb) h = nb;
    if (h < l) h = l;
  }
  *lo = l;
  *hi = h;
}

}  // namespace

extern "C" {

int brs_version(void) { return BRS_VERSION; }

const char* brs_last_error(void) { return g_err; }

int brs_memory_check(const brs_memory* m) {
  int rc = check_memory(m);
  return rc ? rc : ok();
}

int brs_eligible_range(const brs_memory* m, int64_t n_sink, int64_t window, int64_t* lo,
                       int64_t* hi) {
  int rc = check_memory(m);
  if (rc) return rc;
  if (n_sink < 0 || window < 0) return fail(BRS_E_INVAL, "n_sink and window must be >= 0");
  if (!lo || !hi) return fail(BRS_E_INVAL, "lo/hi must be non-NULL");
  eligible(m->length, m->block_size, n_sink, window, lo, hi);
  return ok();
}

int brs_mem_append(brs_memory* m, const void* k_new, const void* v_new, int64_t n_new,
                   const void* reps_new, void* stream) {
  int rc = check_memory(m);
  if (rc) return rc;
  if (n_new < 0) return fail(BRS_E_INVAL, "n_new < 0");
  if (n_new == 0) return ok();
  if (m->length + n_new > m->capacity)
    return fail(BRS_E_CAPACITY, "length %lld + n_new %lld > capacity %lld", (long long)m->length,
                (long long)n_new, (long long)m->capacity);
  if (!k_new || !v_new) return fail(BRS_E_INVAL, "k_new/v_new must be non-NULL");
  const int es = brs::elem_bytes(m->dtype);
  if (!aligned(k_new, es) || !aligned(v_new, es)) return fail(BRS_E_INVAL, "k_new/v_new misaligned");
  const int64_t b0 = m->length / m->block_size;
  const int64_t b1 = (m->length + n_new) / m->block_size;
  const bool given = m->rep_mode == BRS_REP_GIVEN || m->rep_mode == BRS_REP_EMBED;
  if (given && b1 > b0 && !reps_new)
    return fail(BRS_E_INVAL, "reps_new required: this append completes %lld block(s)", (long long)(b1 - b0));
  if (given && b1 > b0 && !aligned(reps_new, brs::elem_bytes(m->rep_dtype)))
    return fail(BRS_E_INVAL, "reps_new misaligned");
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = brs::launch_kv_append(*m, k_new, v_new, n_new, s);
  if (e != hipSuccess) return hip_fail(e, "kv_append");
  if (b1 > b0 && m->rep_mode != BRS_REP_ATTNSCORE) {  // ATTNSCORE: built by brs_reps_from_mass
    brs_memory after = *m;
    after.length = m->length + n_new;
    e = brs::launch_rep_build(after, b0, b1, reps_new, s);
    if (e != hipSuccess) return hip_fail(e, "rep_build");
  }
  m->length += n_new;
  return ok();
}

int brs_score_blocks(const brs_memory* m, const void* qrep, int32_t n_score_heads, int64_t lo,
                     int64_t hi, float* scores, void* stream) {
  int rc = check_memory(m);
  if (rc) return rc;
  const int64_t nb = m->length / m->block_size;
  if (lo < 0 || hi < lo || hi > nb)
    return fail(BRS_E_INVAL, "need 0 <= lo <= hi <= %lld (complete blocks)", (long long)nb);
  if (!qrep || !scores) return fail(BRS_E_INVAL, "qrep/scores must be non-NULL");
  if (!aligned(scores, 4)) return fail(BRS_E_INVAL, "scores misaligned");
  hipStream_t s = (hipStream_t)stream;
  if (m->rep_mode == BRS_REP_EMBED) {
    if (n_score_heads != 1) return fail(BRS_E_INVAL, "cosine scoring has one score head per sequence");
    if (!aligned(qrep, brs::elem_bytes(m->rep_dtype))) return fail(BRS_E_INVAL, "qrep misaligned");
    if (hi == lo) return ok();
    hipError_t e = brs::launch_score_cosine(*m, qrep, lo, hi, scores, s);
    return e == hipSuccess ? ok() : hip_fail(e, "score_cosine");
  }
  if (n_score_heads < 1 || n_score_heads % m->n_kv_heads != 0)
    return fail(BRS_E_INVAL, "n_score_heads must be a positive multiple of n_kv_heads");
  if (n_score_heads / m->n_kv_heads > 32) return fail(BRS_E_UNSUPPORTED, "more than 32 query heads per kv head");
  if (!aligned(qrep, brs::elem_bytes(m->dtype))) return fail(BRS_E_INVAL, "q misaligned");
  if (hi == lo) return ok();
  hipError_t e = brs::launch_score_dot(*m, qrep, n_score_heads, lo, hi, scores, false, s);
  return e == hipSuccess ? ok() : hip_fail(e, "score_dot");
}

int brs_score_blocks_group(const brs_memory* m, const void* q, int32_t n_q_heads, int64_t lo, int64_t hi,
                           float* scores, void* stream) {
  int rc = check_memory(m);
  if (rc) return rc;
  if (m->rep_mode == BRS_REP_EMBED) return fail(BRS_E_INVAL, "group scores need dot scoring (rep_mode != EMBED)");
  const int64_t nb = m->length / m->block_size;
  if (lo < 0 || hi < lo || hi > nb)
    return fail(BRS_E_INVAL, "need 0 <= lo <= hi <= %lld (complete blocks)", (long long)nb);
  if (!q || !scores) return fail(BRS_E_INVAL, "q/scores must be non-NULL");
  if (!aligned(scores, 4)) return fail(BRS_E_INVAL, "scores misaligned");
  if (n_q_heads < 1 || n_q_heads % m->n_kv_heads != 0)
    return fail(BRS_E_INVAL, "n_q_heads must be a positive multiple of n_kv_heads");
  if (n_q_heads / m->n_kv_heads > 32) return fail(BRS_E_UNSUPPORTED, "more than 32 query heads per kv head");
  if (!aligned(q, brs::elem_bytes(m->dtype))) return fail(BRS_E_INVAL, "q misaligned");
  if (hi == lo) return ok();
  hipError_t e = brs::launch_score_dot(*m, q, n_q_heads, lo, hi, scores, true, (hipStream_t)stream);
  return e == hipSuccess ? ok() : hip_fail(e, "score_dot (group)");
}

int brs_select_topk(const float* scores, int32_t batch, int32_t n_heads, int64_t blocks_stride,
                    int64_t lo, int64_t hi, int32_t k, int32_t* idx, float* vals, void* stream) {
  if (!scores || !idx) return fail(BRS_E_INVAL, "scores/idx must be non-NULL");
  if (batch < 1 || n_heads < 1) return fail(BRS_E_INVAL, "batch and n_heads must be >= 1");
  if (k < 1 || k > 2048) return fail(BRS_E_UNSUPPORTED, "k must be in [1, 2048]");
  if (lo < 0 || hi < lo || hi > blocks_stride) return fail(BRS_E_INVAL, "need 0 <= lo <= hi <= blocks_stride");
  if (hi - lo > (1 << 20)) return fail(BRS_E_UNSUPPORTED, "more than 2^20 candidates");
  if (!aligned(scores, 4) || !aligned(idx, 4) || (vals && !aligned(vals, 4)))
    return fail(BRS_E_INVAL, "misaligned pointer");
  hipError_t e = brs::launch_select_topk(scores, batch, n_heads, blocks_stride, lo, hi, k, idx, vals,
                                         (hipStream_t)stream);
  return e == hipSuccess ? ok() : hip_fail(e, "select_topk");
}

static int attn_setup(const brs_memory* m, int32_t n_q_heads, int32_t n_q, int32_t idx_heads, int32_t k,
                      int64_t n_sink, int64_t window, float scale, brs::AttnGeom& g) {
  int rc = check_memory(m);
  if (rc) return rc;
  if (n_q_heads < 1 || n_q_heads % m->n_kv_heads != 0)
    return fail(BRS_E_INVAL, "n_q_heads must be a positive multiple of n_kv_heads");
  if (n_q < 1 || n_q > m->length) return fail(BRS_E_INVAL, "need 1 <= n_q <= length");
  if (idx_heads != 1 && idx_heads != m->n_kv_heads && idx_heads != n_q_heads)
    return fail(BRS_E_INVAL, "idx_heads must be 1, n_kv_heads or n_q_heads");
  if (k < 0) return fail(BRS_E_INVAL, "k < 0");
  if (n_sink < 0 || window < 0) return fail(BRS_E_INVAL, "n_sink and window must be >= 0");
  if (!isfinite(scale)) return fail(BRS_E_INVAL, "scale must be finite");
  if (n_sink == 0 && window == 0 && k == 0) return fail(BRS_E_EMPTY, "no sinks, no window and k = 0");
  const int G = n_q_heads / m->n_kv_heads;
  if (G > 32) return fail(BRS_E_UNSUPPORTED, "more than 32 query heads per kv head");
  g = brs::AttnGeom{};
  g.batch = m->batch;
  g.hq = n_q_heads;
  g.hkv = m->n_kv_heads;
  g.group = G;
  g.n_q = n_q;
  g.d = m->head_dim;
  g.row_stride = m->row_stride;
  g.dtype = m->dtype;
  g.N = (int)m->length;
  g.B = m->block_size;
  g.nb = (int)(m->length / m->block_size);
  const int64_t S = n_sink < m->length ? n_sink : m->length;
  g.sink_end = (int)S;
  const int64_t ws = m->length - window;
  g.win_start = (int)(ws > S ? ws : S);
  g.idx_heads = idx_heads;
  g.k = k;
  g.head_stride = m->capacity * (int64_t)m->row_stride;
  g.qscale = scale * 1.4426950408889634f;
  if (!brs::attn_geometry(g)) return fail(BRS_E_UNSUPPORTED, "attention shape not supported");
  return BRS_OK;
}

int brs_attention_workspace_bytes(const brs_memory* m, int32_t n_q_heads, int32_t n_q,
                                  int32_t idx_heads, int32_t k, int64_t n_sink, int64_t window,
                                  size_t* bytes) {
  if (!bytes) return fail(BRS_E_INVAL, "bytes must be non-NULL");
  *bytes = 0;
  brs::AttnGeom g;
  int rc = attn_setup(m, n_q_heads, n_q, idx_heads, k, n_sink, window, 1.0f, g);
  if (rc) return rc;
  *bytes = g.total;
  return ok();
}

// plan (unless the split kernels build it themselves), then the attention kernels
static int run_attention(const brs::AttnGeom& g, const brs_memory* m, const void* q, const int32_t* idx,
                         float* out, float* lse, void* workspace, hipStream_t s) {
  hipEvent_t e0 = g_prof_start, e1 = g_prof_stop;
  g_prof_start = g_prof_stop = nullptr;
  hipError_t e;
  if (!g.local_plan && !g.slot && !g.prefill) {
    e = brs::launch_attn_plan(g, idx, workspace, out, s);
    if (e != hipSuccess) return hip_fail(e, "attn_plan");
  }
  if (g.prefill) {
    e = brs::launch_attn_prefill(g, m->k, m->v, q, idx, out, lse, s, e0, e1);
    if (e != hipSuccess) return hip_fail(e, "attn_prefill");
    return ok();
  }
  e = brs::launch_attn_split(g, m->k, m->v, q, idx, workspace, out, s, e0, e1);
  if (e != hipSuccess) return hip_fail(e, "attn_split");
  e = brs::launch_attn_merge(g, workspace, out, lse, s);
  if (e != hipSuccess) return hip_fail(e, "attn_merge");
  return ok();
}

static int check_attention_buffers(const brs::AttnGeom& g, const void* q, const int32_t* idx, int32_t k, float* out,
                                   float* lse, void* workspace, size_t workspace_bytes) {
  if (!q || !out) return fail(BRS_E_INVAL, "q/out must be non-NULL");
  if (lse && !aligned(lse, 4)) return fail(BRS_E_INVAL, "lse misaligned");
  if (k > 0 && !idx) return fail(BRS_E_INVAL, "idx must be non-NULL when k > 0");
  if (!aligned(q, 16) || !aligned(out, 16)) return fail(BRS_E_INVAL, "q/out must be 16-byte aligned");
  if (idx && !aligned(idx, 4)) return fail(BRS_E_INVAL, "idx misaligned");
  if (!workspace || workspace_bytes < g.total)
    return fail(BRS_E_WORKSPACE, "workspace of %zu bytes needed", g.total);
  if (!aligned(workspace, 256)) return fail(BRS_E_WORKSPACE, "workspace must be 256-byte aligned");
  return BRS_OK;
}

int brs_retrieval_attention(const brs_memory* m, const void* q, int32_t n_q_heads, int32_t n_q,
                            const int32_t* idx, int32_t idx_heads, int32_t k, int64_t n_sink,
                            int64_t window, float scale, float* out, float* lse, void* workspace,
                            size_t workspace_bytes, void* stream) {
  brs::AttnGeom g;
  int rc = attn_setup(m, n_q_heads, n_q, idx_heads, k, n_sink, window, scale, g);
  if (rc) return rc;
  rc = check_attention_buffers(g, q, idx, k, out, lse, workspace, workspace_bytes);
  if (rc) return rc;
  return run_attention(g, m, q, idx, out, lse, workspace, (hipStream_t)stream);
}

// the selection lists of a step: 1 for cosine scores; n_q_heads or
// n_kv_heads (group scores) for dot scores
static int step_select_heads(const brs_memory* m, int32_t n_q_heads, int32_t select_heads) {
  if (m->rep_mode == BRS_REP_EMBED) {
    if (select_heads != 1) return fail(BRS_E_INVAL, "cosine scoring makes one selection per sequence: select_heads = 1");
    return BRS_OK;
  }
  if (select_heads != n_q_heads && select_heads != m->n_kv_heads)
    return fail(BRS_E_INVAL, "select_heads must be n_q_heads or n_kv_heads for dot scoring");
  return BRS_OK;
}

int brs_retrieval_step(const brs_memory* m, const void* q, int32_t n_q_heads, int32_t n_q, const void* qrep,
                       int32_t select_heads, int32_t k, int64_t n_sink, int64_t window, float scale, float* scores,
                       int32_t* idx, float* vals, float* out, float* lse, void* workspace, size_t workspace_bytes,
                       void* stream) {
  int rc = check_memory(m);
  if (rc) return rc;
  const bool cosine = m->rep_mode == BRS_REP_EMBED;
  if (n_q_heads < 1 || n_q_heads % m->n_kv_heads != 0)
    return fail(BRS_E_INVAL, "n_q_heads must be a positive multiple of n_kv_heads");
  rc = step_select_heads(m, n_q_heads, select_heads);
  if (rc) return rc;
  const int32_t hs = select_heads;
  const bool grouped = !cosine && hs != n_q_heads;
  int64_t lo = 0, hi = 0;
  rc = brs_eligible_range(m, n_sink, window, &lo, &hi);
  if (rc) return rc;
  brs::AttnGeom g;
  rc = attn_setup(m, n_q_heads, n_q, hs, k, n_sink, window, scale, g);
  if (rc) return rc;
  rc = check_attention_buffers(g, q, idx, k, out, lse, workspace, workspace_bytes);
  if (rc) return rc;
  if (k > 2048) return fail(BRS_E_UNSUPPORTED, "k must be at most 2048");
  if (k > 0) {
    if (!qrep || !scores) return fail(BRS_E_INVAL, "qrep/scores must be non-NULL when k > 0");
    if (!aligned(scores, 4) || (vals && !aligned(vals, 4))) return fail(BRS_E_INVAL, "scores/vals misaligned");
    if (!aligned(qrep, brs::elem_bytes(cosine ? m->rep_dtype : m->dtype))) return fail(BRS_E_INVAL, "qrep misaligned");
  }
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (k > 0) {
    const bool step = brs::step_supported(g, lo, hi, k);
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (step) {
      e0 = g_prof_start;
      e1 = g_prof_stop;
      g_prof_start = g_prof_stop = nullptr;
    }
    if (hi > lo) {
      // measurement: the step kernel's interval starts when the score kernel
      // completes (an event attached to the step launch itself is stamped
      // when its dispatch is processed, while the score kernel may still run)
      if (e0) {
        brs::set_score_stop_event(e0);
        e0 = nullptr;
      }
      e = cosine ? brs::launch_score_cosine(*m, qrep, lo, hi, scores, s)
                 : brs::launch_score_dot(*m, qrep, n_q_heads, lo, hi, scores, grouped, s);
      brs::set_score_stop_event(nullptr);
      if (e != hipSuccess) return hip_fail(e, "score_blocks");
    }
    const int64_t stride = m->capacity / m->block_size;
    if (step) {
      // selection and attention in one launch, then the merge
      e = brs::launch_attn_step(g, m->k, m->v, q, scores, stride, lo, hi, idx, vals, workspace, out, s, e0, e1);
      if (e != hipSuccess) return hip_fail(e, "select_topk + attention");
      e = brs::launch_attn_merge(g, workspace, out, lse, s);
      if (e != hipSuccess) return hip_fail(e, "attn_merge");
      return ok();
    }
    e = brs::launch_select_topk(scores, m->batch, hs, stride, lo, hi, k, idx, vals, s);
    if (e != hipSuccess) return hip_fail(e, "select_topk");
  }
  return run_attention(g, m, q, k > 0 ? idx : nullptr, out, lse, workspace, s);
}

int brs_retrieval_step_static(const brs_memory* m, const void* q, int32_t n_q_heads, int32_t n_q,
                              const void* qrep, int32_t select_heads, int32_t k, int64_t n_sink, int64_t window,
                              float scale, float* scores, int32_t* idx, float* vals, float* out, float* lse,
                              void* stream) {
  int rc = check_memory(m);
  if (rc) return rc;
  if (n_q_heads < 1 || n_q_heads % m->n_kv_heads != 0)
    return fail(BRS_E_INVAL, "n_q_heads must be a positive multiple of n_kv_heads");
  rc = step_select_heads(m, n_q_heads, select_heads);
  if (rc) return rc;
  brs::AttnGeom g;
  rc = attn_setup(m, n_q_heads, n_q, select_heads, k, n_sink, window, scale, g);
  if (rc) return rc;
  if (g.total > kStaticScratchBytes)
    return fail(BRS_E_UNSUPPORTED, "this step needs %zu bytes of workspace; the static scratch holds %zu",
                g.total, kStaticScratchBytes);
  void* ws = nullptr;
  rc = static_scratch(&ws);
  if (rc) return rc;
  return brs_retrieval_step(m, q, n_q_heads, n_q, qrep, select_heads, k, n_sink, window, scale, scores, idx, vals,
                            out, lse, ws, kStaticScratchBytes, stream);
}

size_t brs_static_scratch_bytes(void) { return kStaticScratchBytes; }

int brs_window_mass(const brs_memory* m, const void* q, int32_t n_q_heads, int32_t n_q, const float* lse,
                    int64_t window, float scale, float* mass, void* stream) {
  int rc = check_memory(m);
  if (rc) return rc;
  if (n_q_heads < 1 || n_q_heads % m->n_kv_heads != 0)
    return fail(BRS_E_INVAL, "n_q_heads must be a positive multiple of n_kv_heads");
  if (n_q < 1 || n_q > m->length) return fail(BRS_E_INVAL, "need 1 <= n_q <= length");
  if (window < 1) return fail(BRS_E_INVAL, "window must be >= 1");
  if (!isfinite(scale)) return fail(BRS_E_INVAL, "scale must be finite");
  if (!q || !lse || !mass) return fail(BRS_E_INVAL, "q, lse and mass must be non-NULL");
  if (!aligned(q, brs::elem_bytes(m->dtype)) || !aligned(lse, 4) || !aligned(mass, 4))
    return fail(BRS_E_INVAL, "misaligned pointer");
  const int64_t w0 = window < m->length ? m->length - window : 0;
  hipEvent_t e0 = g_prof_start, e1 = g_prof_stop;
  g_prof_start = g_prof_stop = nullptr;
  hipError_t e = brs::launch_window_mass(*m, q, n_q_heads, n_q, lse, w0, scale, mass, (hipStream_t)stream, e0, e1);
  return e == hipSuccess ? ok() : hip_fail(e, "window_mass");
}

int brs_reps_from_mass(const brs_memory* m, const float* mass, int64_t b0, int64_t b1, void* stream) {
  int rc = check_memory(m);
  if (rc) return rc;
  if (m->rep_mode != BRS_REP_ATTNSCORE) return fail(BRS_E_INVAL, "rep_mode must be ATTNSCORE");
  const int64_t nb = m->length / m->block_size;
  if (b0 < 0 || b1 < b0 || b1 > nb)
    return fail(BRS_E_INVAL, "need 0 <= b0 <= b1 <= %lld (complete blocks)", (long long)nb);
  if (!mass || !aligned(mass, 4)) return fail(BRS_E_INVAL, "mass must be non-NULL and 4-byte aligned");
  if (b1 == b0) return ok();
  hipError_t e = brs::launch_reps_from_mass(*m, mass, b0, b1, (hipStream_t)stream);
  return e == hipSuccess ? ok() : hip_fail(e, "reps_from_mass");
}

int brs_count_hits(const brs_memory* m, const int32_t* idx, int32_t idx_heads, int32_t k, int32_t* hits,
                   void* stream) {
  int rc = check_memory(m);
  if (rc) return rc;
  if (idx_heads < 1 || k < 0) return fail(BRS_E_INVAL, "need idx_heads >= 1 and k >= 0");
  if (k == 0) return ok();
  if (!idx || !hits || !aligned(idx, 4) || !aligned(hits, 4))
    return fail(BRS_E_INVAL, "idx/hits must be non-NULL and 4-byte aligned");
  hipError_t e = brs::launch_count_hits(*m, idx, idx_heads, k, hits, (hipStream_t)stream);
  return e == hipSuccess ? ok() : hip_fail(e, "count_hits");
}

int brs_mem_prune(const brs_memory* src, const int32_t* hits, brs_memory* dst, int32_t* dst_hits, int32_t* plan,
                  void* stream) {
  int rc = check_memory(src);
  if (rc) return rc;
  if (!dst) return fail(BRS_E_INVAL, "dst is NULL");
  brs_memory probe = *dst;
  probe.length = 0;
  rc = check_memory(&probe);
  if (rc) return rc;
  if (dst->dtype != src->dtype || dst->batch != src->batch || dst->n_kv_heads != src->n_kv_heads ||
      dst->head_dim != src->head_dim || dst->row_stride != src->row_stride || dst->block_size != src->block_size ||
      dst->reps_per_block != src->reps_per_block || dst->rep_dim != src->rep_dim ||
      dst->rep_heads != src->rep_heads || dst->rep_mode != src->rep_mode || dst->rep_dtype != src->rep_dtype ||
      dst->capacity != src->capacity)
    return fail(BRS_E_INVAL, "dst must have the geometry of src");
  if (dst->k == src->k || dst->v == src->v || dst->reps == src->reps)
    return fail(BRS_E_INVAL, "dst buffers must be distinct from src buffers");
  if (!hits || !plan || !aligned(hits, 4) || !aligned(plan, 4) || (dst_hits && !aligned(dst_hits, 4)))
    return fail(BRS_E_INVAL, "hits/plan must be non-NULL and 4-byte aligned");
  const int64_t B = src->block_size;
  const int64_t nb = src->length / B, tail = src->length - nb * B;
  const int64_t n10 = nb / 10, n_mid = nb - 2 * n10;
  int64_t budget = (src->capacity / 2 - tail) / B;
  if (budget < 0) budget = 0;
  int64_t keep_mid = budget - n10;
  keep_mid = keep_mid < 0 ? 0 : (keep_mid > n_mid ? n_mid : keep_mid);
  const int64_t n_evict = n_mid - keep_mid;
  const int64_t kept = nb - n10 - n_evict;
  if (n_mid > brs::prune_max_middle() || nb > brs::prune_max_blocks())
    return fail(BRS_E_UNSUPPORTED, "pruning supports up to %d middle blocks", brs::prune_max_middle());
  hipError_t e = brs::launch_prune(*src, *dst, hits, dst_hits, plan, (int)nb, (int)n10, (int)n_evict, (int)kept,
                                   (int)tail, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "prune");
  dst->length = kept * B + tail;
  return ok();
}

static int check_cache(const brs_memory* m, const brs_page_cache* c) {
  if (!c) return fail(BRS_E_INVAL, "cache descriptor is NULL");
  if (c->reserved != 0) return fail(BRS_E_INVAL, "cache reserved field must be 0");
  if (c->n_pages < 1 || c->n_pages > brs::cache_max_pages())
    return fail(BRS_E_UNSUPPORTED, "n_pages must be in [1, %d]", brs::cache_max_pages());
  if (!c->k || !c->v || !c->page_of_block || !c->page_block || !c->page_rows || !c->page_used)
    return fail(BRS_E_INVAL, "cache pointers must be non-NULL");
  if (!aligned(c->k, 16) || !aligned(c->v, 16)) return fail(BRS_E_INVAL, "cache k/v must be 16-byte aligned");
  if (!aligned(c->page_of_block, 4) || !aligned(c->page_block, 4) || !aligned(c->page_rows, 4) ||
      !aligned(c->page_used, 4))
    return fail(BRS_E_INVAL, "cache tables must be 4-byte aligned");
  if ((m->row_stride * brs::elem_bytes(m->dtype)) % 16 != 0)
    return fail(BRS_E_UNSUPPORTED, "a cached memory needs row_stride * element size to be a multiple of 16 bytes");
  if (m->capacity / m->block_size + 1 > brs::cache_max_blocks())
    return fail(BRS_E_UNSUPPORTED, "a cached memory holds at most %lld blocks", (long long)brs::cache_max_blocks() - 1);
  return BRS_OK;
}

int brs_cache_reset(const brs_memory* m, const brs_page_cache* c, void* stream) {
  int rc = check_memory(m);
  if (rc) return rc;
  rc = check_cache(m, c);
  if (rc) return rc;
  hipError_t e = brs::launch_cache_reset(*m, *c, (hipStream_t)stream);
  return e == hipSuccess ? ok() : hip_fail(e, "cache_reset");
}

int brs_cache_fetch(const brs_memory* m, const brs_page_cache* c, const int32_t* idx, int32_t idx_heads, int32_t k,
                    int64_t n_sink, int64_t window, int32_t step, int32_t* fetched, void* stream) {
  int rc = check_memory(m);
  if (rc) return rc;
  rc = check_cache(m, c);
  if (rc) return rc;
  if (k < 0 || n_sink < 0 || window < 0) return fail(BRS_E_INVAL, "k, n_sink and window must be >= 0");
  if (k > 0 && (!idx || !aligned(idx, 4))) return fail(BRS_E_INVAL, "idx must be non-NULL and 4-byte aligned");
  if (idx_heads < 1 || (idx_heads != 1 && idx_heads % m->n_kv_heads != 0))
    return fail(BRS_E_INVAL, "idx_heads must be 1 or a multiple of n_kv_heads");
  if (fetched && !aligned(fetched, 4)) return fail(BRS_E_INVAL, "fetched misaligned");
  const int64_t N = m->length, B = m->block_size;
  const int64_t S = n_sink < N ? n_sink : N;
  const int64_t ws0 = N - window;
  const int64_t ws = ws0 > S ? ws0 : S;
  const int64_t nbt = (N + B - 1) / B;
  const int64_t lists = idx_heads >= m->n_kv_heads ? idx_heads / m->n_kv_heads : 1;
  const int64_t need = (S + B - 1) / B + (ws < N ? nbt - ws / B : 0) + lists * k;
  if (need > c->n_pages)
    return fail(BRS_E_CAPACITY, "a step may need %lld blocks per kv head; the cache has %d pages", (long long)need,
                c->n_pages);
  hipError_t e = brs::launch_cache_fetch(*m, *c, k > 0 ? idx : nullptr, idx_heads, k, S, ws, step, fetched,
                                         (hipStream_t)stream);
  return e == hipSuccess ? ok() : hip_fail(e, "cache_fetch");
}

int brs_retrieval_attention_cached(const brs_memory* m, const brs_page_cache* c, const void* q, int32_t n_q_heads,
                                   int32_t n_q, const int32_t* idx, int32_t idx_heads, int32_t k, int64_t n_sink,
                                   int64_t window, float scale, float* out, float* lse, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  brs::AttnGeom g;
  int rc = attn_setup(m, n_q_heads, n_q, idx_heads, k, n_sink, window, scale, g);
  if (rc) return rc;
  rc = check_cache(m, c);
  if (rc) return rc;
  rc = check_attention_buffers(g, q, idx, k, out, lse, workspace, workspace_bytes);
  if (rc) return rc;
  g.pages = c->page_of_block;
  g.pages_stride = (int)(m->capacity / m->block_size + 1);
  g.head_stride = (int64_t)c->n_pages * m->block_size * m->row_stride;
  // the chunked-prefill kernel, or the slot kernels, both read K/V through the page table
  const bool prefill = g.prefill && brs::prefill_supported(g);
  if (!prefill && !g.slot)
    return fail(BRS_E_UNSUPPORTED, "a cached memory supports the slot-layout and chunked-prefill kernels only");
  hipEvent_t e0 = g_prof_start, e1 = g_prof_stop;
  g_prof_start = g_prof_stop = nullptr;
  hipStream_t s = (hipStream_t)stream;
  if (prefill) {
    hipError_t e = brs::launch_attn_prefill(g, c->k, c->v, q, idx, out, lse, s, e0, e1);
    return e == hipSuccess ? ok() : hip_fail(e, "attn_prefill (cached)");
  }
  hipError_t e = brs::launch_attn_split(g, c->k, c->v, q, idx, workspace, out, s, e0, e1);
  if (e != hipSuccess) return hip_fail(e, "attn_split (cached)");
  e = brs::launch_attn_merge(g, workspace, out, lse, s);
  if (e != hipSuccess) return hip_fail(e, "attn_merge");
  return ok();
}

int brs_profile_next_attention(void* start_event, void* stop_event) {
  if ((start_event == nullptr) != (stop_event == nullptr))
    return fail(BRS_E_INVAL, "pass both events or neither");
  g_prof_start = (hipEvent_t)start_event;
  g_prof_stop = (hipEvent_t)stop_event;
  return ok();
}

}  // extern "C"
