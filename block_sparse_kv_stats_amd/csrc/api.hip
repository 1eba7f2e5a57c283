// C ABI of libcknv: argument validation, workspace plan, kernel launches.
// Validation runs before any HIP call; on error nothing is enqueued.
#include <math.h>

#include <mutex>

#include "cknv_internal.h"
#include "step_config.h"

namespace cknv {

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static int check_shape(const cknv_shape* sh) {
  if (!sh) return CKNV_EINVAL;
  if (sh->S < 1 || sh->H < 1 || sh->G < 1 || sh->d < 1 || sh->r < 1 || sh->cap_blocks < 1)
    return CKNV_EINVAL;
  if (sh->block != kBlock) return CKNV_EUNSUPPORTED;
  if (sh->d != 64 && sh->d != 128) return CKNV_EUNSUPPORTED;
  if (sh->G != 1 && sh->G != 2 && sh->G != 4 && sh->G != 8) return CKNV_EUNSUPPORTED;
  if (sh->r > sh->d || sh->d % sh->r != 0) return CKNV_EUNSUPPORTED;
  if (sh->flags & ~CKNV_FLAGS_ALL) return CKNV_EUNSUPPORTED;
  if ((long long)sh->S * sh->H > (1 << 20)) return CKNV_EUNSUPPORTED;
  return CKNV_OK;
}

static int check_cache(const cknv_cache* c) {
  if (!c || !c->k || !c->v || !c->kbar || !c->dbar || !c->cnt || !c->vbar || !c->seq_len)
    return CKNV_EINVAL;
  return CKNV_OK;
}

int make_plan(const cknv_shape* sh, int max_blocks, int budget_tokens, Plan* p) {
  int st = check_shape(sh);
  if (st) return st;
  if (max_blocks < 1) return CKNV_EINVAL;
  if (max_blocks > sh->cap_blocks) return CKNV_ENOSPACE;
  if (budget_tokens < 3 * kBlock) return CKNV_EINVAL;  // must hold the forced set
  const int G = sh->G, d = sh->d, r = sh->r;
  Plan q{};
  q.U = sh->S * sh->H;
  q.NBmax = max_blocks;
  q.rows = score_rows(G);
  q.bpw = 4 * q.rows;
  q.NG = (max_blocks + q.bpw - 1) / q.bpw;
  q.Kb = budget_tokens / kBlock;
  q.C = (max_blocks + kScoreWaves * q.bpw - 1) / (kScoreWaves * q.bpw);
  const int per_wg = kWaves;  // kept blocks per attend workgroup (one per wave)
  q.P = (q.Kb + per_wg - 1) / per_wg;
  const int pc = (q.C + kMaxChunksPerAttendWG - 1) / kMaxChunksPerAttendWG;
  q.P = q.P > pc ? q.P : pc;
  int bpw = (max_blocks + kDenseMaxWGs - 1) / kDenseMaxWGs;
  bpw = bpw > kDenseBlocksPerWG ? bpw : kDenseBlocksPerWG;
  q.Pd = (max_blocks + bpw - 1) / bpw;
  q.kpw = step_kept_per_wave(q.U, q.Kb);
  q.Pf = (q.Kb + kStepAttendWaves * q.kpw - 1) / (kStepAttendWaves * q.kpw);
  const size_t W = (size_t)rec_words(d);
  size_t off = 0;
  q.off_grp = off;
  off = align256(off + (size_t)q.U * q.NG * G * 2 * 4);
  q.off_u = off;
  off = align256(off + (size_t)q.U * max_blocks * G * 4);
  q.off_comp = off;
  off = align256(off + (size_t)q.U * q.C * G * W * 4);
  q.off_attp = off;
  off = align256(off + (size_t)q.U * q.P * G * W * 4);
  q.off_dense = off;
  off = align256(off + (size_t)q.U * q.Pd * G * W * 4);
  q.off_t0 = off;
  off = align256(off + (size_t)sh->S * 4);
  q.off_fpart = off;
  off = align256(off + (size_t)q.U * q.Pf * G * W * 4);
  q.off_fphdr = off;
  off = align256(off + (size_t)q.U * G * q.Pf * 2 * 4);
  q.off_finfo = off;
  off = align256(off + (size_t)q.U * G * 2 * 4);
  q.off_hdr = off;
  off = align256(off + (size_t)q.U * q.C * G * 2 * 4);
  q.pstride = q.Pf > kFlatParts ? 1 + (q.Pf + kPartGroup - 1) / kPartGroup : 1;
  q.off_pcnt = off;
  off = align256(off + (size_t)q.U * q.pstride * 4);
  q.total = off;
  if (max_blocks > kSelThreads * kSelKeysPerThread) return CKNV_EUNSUPPORTED;
  *p = q;
  return CKNV_OK;
}

static int hip_status(hipError_t e) { return e == hipSuccess ? CKNV_OK : CKNV_EHIP; }

}  // namespace cknv

using namespace cknv;

extern "C" {

int cknv_workspace_size(const cknv_shape* shape, int32_t max_blocks, int32_t budget_tokens,
                        size_t* bytes) {
  if (!bytes) return CKNV_EINVAL;
  Plan p;
  const int st = make_plan(shape, max_blocks, budget_tokens, &p);
  if (st) return st;
  *bytes = p.total;
  return CKNV_OK;
}

int cknv_workspace_init(const cknv_shape* shape, int32_t max_blocks, int32_t budget_tokens,
                        void* ws, size_t ws_bytes, void* stream) {
  Plan p;
  int st = make_plan(shape, max_blocks, budget_tokens, &p);
  if (st) return st;
  if (!ws) return CKNV_EINVAL;
  if (ws_bytes < p.total) return CKNV_ENOSPACE;
  return hip_status(launch_zero_u32(static_cast<uint32_t*>(ws), p.total / 4, (hipStream_t)stream));
}

int cknv_append(const cknv_shape* shape, const cknv_cache* cache, const uint16_t* new_k,
                const uint16_t* new_v, void* stream) {
  int st = check_shape(shape);
  if (st) return st;
  if ((st = check_cache(cache))) return st;
  if (!new_k || !new_v) return CKNV_EINVAL;
  AppendArgs a{cache->k, cache->v, cache->kbar, cache->dbar, cache->cnt, cache->vbar,
               cache->seq_len, new_k, new_v, shape->S, shape->H, shape->r, shape->cap_blocks};
  return hip_status(launch_append(shape->d, a, (hipStream_t)stream));
}

int cknv_build_summaries(const cknv_shape* shape, const cknv_cache* cache, int32_t max_blocks,
                         void* stream) {
  int st = check_shape(shape);
  if (st) return st;
  if ((st = check_cache(cache))) return st;
  if (max_blocks < 1) return CKNV_EINVAL;
  if (max_blocks > shape->cap_blocks) return CKNV_ENOSPACE;
  BuildArgs a{cache->k, cache->v, cache->kbar, cache->dbar, cache->cnt, cache->vbar,
              cache->seq_len, shape->S, shape->H, shape->r, shape->cap_blocks, max_blocks};
  return hip_status(launch_build(shape->d, a, shape->S * shape->H, (hipStream_t)stream));
}

int cknv_score_select(const cknv_shape* shape, const cknv_cache* cache, const float* q,
                      int32_t budget_tokens, int32_t max_blocks, float* scores, int32_t* sel,
                      int32_t* n_sel, void* ws, size_t ws_bytes, void* stream) {
  Plan p;
  int st = make_plan(shape, max_blocks, budget_tokens, &p);
  if (st) return st;
  if ((st = check_cache(cache))) return st;
  if (!q || !sel || !n_sel || !ws) return CKNV_EINVAL;
  if (ws_bytes < p.total) return CKNV_ENOSPACE;
  char* w = static_cast<char*>(ws);
  ScoreArgs a{};
  a.kbar = cache->kbar; a.dbar = cache->dbar; a.cnt = cache->cnt; a.vbar = cache->vbar;
  a.seq_len = cache->seq_len; a.q = q;
  a.grp = reinterpret_cast<float*>(w + p.off_grp);
  a.u = reinterpret_cast<float*>(w + p.off_u);
  a.comp = reinterpret_cast<float*>(w + p.off_comp);
  a.hdr = reinterpret_cast<float*>(w + p.off_hdr);
  a.S = shape->S; a.H = shape->H; a.r = shape->r; a.cap_blocks = shape->cap_blocks;
  a.max_blocks = max_blocks; a.NG = p.NG; a.C = p.C; a.rows = p.rows;
  a.xcd = (p.U % 8) == 0;
  a.flags = (int)shape->flags;
  a.isd = 1.0f / sqrtf((float)shape->d);
  hipError_t e = launch_score(shape->d, shape->G, a, p.U, (hipStream_t)stream);
  if (e != hipSuccess) return CKNV_EHIP;
  SelectArgs sa{};
  sa.seq_len = cache->seq_len; sa.grp = a.grp; sa.u = a.u; sa.hdr = a.hdr; sa.C = p.C;
  sa.scores = scores; sa.sel = sel; sa.n_sel = n_sel;
  sa.H = shape->H; sa.cap_blocks = shape->cap_blocks; sa.max_blocks = max_blocks; sa.NG = p.NG;
  sa.Kb = p.Kb; sa.bpw_shift = p.bpw == 8 ? 3 : 4;
  return hip_status(launch_select(shape->G, sa, p.U, (hipStream_t)stream));
}

static int decode_score_impl(const Plan& p, const cknv_shape* shape, const cknv_cache* cache,
                             const uint16_t* new_k, const uint16_t* new_v, const float* q,
                             int32_t max_blocks, char* w, void* stream) {
  ScoreArgs a{};
  a.kbar = cache->kbar; a.dbar = cache->dbar; a.cnt = cache->cnt; a.vbar = cache->vbar;
  a.seq_len = cache->seq_len; a.q = q;
  a.grp = reinterpret_cast<float*>(w + p.off_grp);
  a.u = reinterpret_cast<float*>(w + p.off_u);
  a.comp = reinterpret_cast<float*>(w + p.off_comp);
  a.hdr = reinterpret_cast<float*>(w + p.off_hdr);
  a.S = shape->S; a.H = shape->H; a.r = shape->r; a.cap_blocks = shape->cap_blocks;
  a.max_blocks = max_blocks; a.NG = p.NG; a.C = p.C; a.rows = p.rows;
  a.xcd = (p.U % 8) == 0;
  a.closed_only = 1;
  a.nfresh = p.U;
  a.k = cache->k; a.v = cache->v; a.new_k = new_k; a.new_v = new_v;
  a.t0_out = reinterpret_cast<int32_t*>(w + p.off_t0);
  a.finfo = reinterpret_cast<float*>(w + p.off_finfo);
  a.pcnt = reinterpret_cast<uint32_t*>(w + p.off_pcnt);
  a.pstride = p.pstride;
  a.flags = (int)shape->flags;
  a.isd = 1.0f / sqrtf((float)shape->d);
  return hip_status(launch_score(shape->d, shape->G, a, p.U, (hipStream_t)stream));
}

// Where a pointer lies for device dev: 0 its device memory, 1 pinned host
// memory it maps at the same address, -1 anything else (pageable host memory
// included; the error the runtime records for it is cleared).
static int mem_where(const void* ptr, int dev) {
  hipPointerAttribute_t at{};
  if (hipPointerGetAttributes(&at, ptr) != hipSuccess) {
    (void)hipGetLastError();
    return -1;
  }
  if (at.type == hipMemoryTypeDevice) return at.device == dev ? 0 : -1;
  if (at.type == hipMemoryTypeHost) return at.devicePointer == ptr ? 1 : -1;
  return -1;
}

static int decode_finish_impl(const Plan& p, const cknv_shape* shape, const cknv_cache* cache,
                              const float* q, int32_t max_blocks, float* scores, int32_t* sel,
                              int32_t* n_sel, float* out, float* lse, char* w, void* stream) {
  StepArgs sa{};
  sa.k = cache->k; sa.v = cache->v; sa.kbar = cache->kbar; sa.dbar = cache->dbar;
  sa.cnt = cache->cnt; sa.vbar = cache->vbar; sa.seq_len = cache->seq_len;
  sa.t0 = reinterpret_cast<const int32_t*>(w + p.off_t0);
  sa.q = q;
  sa.finfo = reinterpret_cast<const float*>(w + p.off_finfo);
  sa.pcnt = reinterpret_cast<uint32_t*>(w + p.off_pcnt);
  sa.pstride = p.pstride;
  sa.grp = reinterpret_cast<const float*>(w + p.off_grp);
  sa.u = reinterpret_cast<const float*>(w + p.off_u);
  sa.comp = reinterpret_cast<const float*>(w + p.off_comp);
  sa.hdr = reinterpret_cast<const float*>(w + p.off_hdr);
  sa.scores = scores; sa.sel = sel; sa.n_sel = n_sel; sa.out = out; sa.lse = lse;
  sa.part = reinterpret_cast<float*>(w + p.off_fpart);
  sa.phdr = reinterpret_cast<float*>(w + p.off_fphdr);
  sa.S = shape->S; sa.H = shape->H; sa.r = shape->r; sa.cap_blocks = shape->cap_blocks;
  sa.max_blocks = max_blocks; sa.NG = p.NG; sa.C = p.C; sa.Kb = p.Kb; sa.P = p.Pf; sa.kpw = p.kpw;
  sa.bpw_shift = p.bpw == 8 ? 3 : 4;
  sa.xcd = (p.U % 8) == 0;
  sa.flags = (int)shape->flags;
  sa.isd = 1.0f / sqrtf((float)shape->d);
  return hip_status(launch_step(shape->d, shape->G, sa, p.U, (hipStream_t)stream));
}

static int decode_check(const cknv_shape* shape, const cknv_cache* cache, int32_t max_blocks,
                        int32_t budget_tokens, const void* ws, size_t ws_bytes, Plan* p) {
  int st = make_plan(shape, max_blocks, budget_tokens, p);
  if (st) return st;
  if ((st = check_cache(cache))) return st;
  if (!ws) return CKNV_EINVAL;
  if (ws_bytes < p->total) return CKNV_ENOSPACE;
  return CKNV_OK;
}

int cknv_decode_score(const cknv_shape* shape, const cknv_cache* cache, const uint16_t* new_k,
                      const uint16_t* new_v, const float* q, int32_t budget_tokens,
                      int32_t max_blocks, void* ws, size_t ws_bytes, void* stream) {
  Plan p;
  int st = decode_check(shape, cache, max_blocks, budget_tokens, ws, ws_bytes, &p);
  if (st) return st;
  if (!new_k || !new_v || !q) return CKNV_EINVAL;
  return decode_score_impl(p, shape, cache, new_k, new_v, q, max_blocks, static_cast<char*>(ws),
                           stream);
}

int cknv_decode_finish(const cknv_shape* shape, const cknv_cache* cache, const float* q,
                       int32_t budget_tokens, int32_t max_blocks, float* scores, int32_t* sel,
                       int32_t* n_sel, float* out, float* lse, void* ws, size_t ws_bytes,
                       void* stream) {
  Plan p;
  int st = decode_check(shape, cache, max_blocks, budget_tokens, ws, ws_bytes, &p);
  if (st) return st;
  if (!q || !sel || !n_sel || !out) return CKNV_EINVAL;
  return decode_finish_impl(p, shape, cache, q, max_blocks, scores, sel, n_sel, out, lse,
                            static_cast<char*>(ws), stream);
}

int cknv_decode_step(const cknv_shape* shape, const cknv_cache* cache, const uint16_t* new_k,
                     const uint16_t* new_v, const float* q, int32_t budget_tokens,
                     int32_t max_blocks, float* scores, int32_t* sel, int32_t* n_sel, float* out,
                     float* lse, void* ws, size_t ws_bytes, void* stream) {
  Plan p;
  int st = decode_check(shape, cache, max_blocks, budget_tokens, ws, ws_bytes, &p);
  if (st) return st;
  if (!new_k || !new_v || !q || !sel || !n_sel || !out) return CKNV_EINVAL;
  char* w = static_cast<char*>(ws);
  if ((st = decode_score_impl(p, shape, cache, new_k, new_v, q, max_blocks, w, stream))) return st;
  return decode_finish_impl(p, shape, cache, q, max_blocks, scores, sel, n_sel, out, lse, w,
                            stream);
}

// ---------------------------------------------------------------- no-allocation step
// cknv_decode_step_noalloc keeps its workspace in this file-scope device
// array instead of a caller's buffer. Each GPU the library runs on holds its
// own copy for the life of the process. In host code `scratch` names a
// host-side stand-in, never the device memory: the device address is taken
// once per device with hipGetSymbolAddress (that device current) and kept.
constexpr size_t kNoAllocScratchBytes = CKNV_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
struct DeviceScratch {
  void* ptr = nullptr;   // device address of this device's copy of `scratch`
  size_t plan_total = 0; // plan the step counters were last laid out for
  int plan_U = -1, plan_S = -1;
  size_t plan_pcnt = 0;
};
std::mutex g_scratch_mutex;
DeviceScratch g_scratch[kMaxDevices];
}  // namespace

// The current device's scratch address; on first use per device, or when the
// workspace layout changes, zero the step counters (by kernel, so that a
// caller may capture the call in a graph).
static int noalloc_workspace(const Plan& p, const cknv_shape* sh, void* stream, char** ws) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return CKNV_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return CKNV_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  DeviceScratch& d = g_scratch[dev];
  if (!d.ptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return CKNV_EHIP;
    d.ptr = ptr;
  }
  char* base = static_cast<char*>(d.ptr);
  if (d.plan_total != p.total || d.plan_U != p.U || d.plan_S != sh->S || d.plan_pcnt != p.off_pcnt) {
    const hipError_t e = launch_zero_u32(reinterpret_cast<uint32_t*>(base + p.off_pcnt),
                                         (size_t)p.U * p.pstride, (hipStream_t)stream);
    if (e != hipSuccess) return CKNV_EHIP;
    d.plan_total = p.total;
    d.plan_U = p.U;
    d.plan_S = sh->S;
    d.plan_pcnt = p.off_pcnt;
  }
  *ws = base;
  return CKNV_OK;
}

static int attend_common(const cknv_shape* shape, const cknv_cache* cache, const float* q,
                         const int32_t* sel, const int32_t* n_sel, int32_t budget_tokens,
                         int32_t max_blocks, float* out, float* lse, void* ws, size_t ws_bytes,
                         void* stream, bool dense) {
  Plan p;
  int st = make_plan(shape, max_blocks, budget_tokens, &p);
  if (st) return st;
  if ((st = check_cache(cache))) return st;
  if (!q || !out || !ws) return CKNV_EINVAL;
  if (!dense && (!sel || !n_sel)) return CKNV_EINVAL;
  if (ws_bytes < p.total) return CKNV_ENOSPACE;
  char* w = static_cast<char*>(ws);
  AttendArgs a{};
  a.k = cache->k; a.v = cache->v; a.kbar = cache->kbar; a.vbar = cache->vbar; a.cnt = cache->cnt;
  a.seq_len = cache->seq_len; a.q = q; a.sel = sel; a.n_sel = n_sel;
  a.out = out; a.lse = lse;
  a.comp = reinterpret_cast<const float*>(w + p.off_comp);
  a.part = reinterpret_cast<float*>(w + (dense ? p.off_dense : p.off_attp));
  a.S = shape->S; a.H = shape->H; a.cap_blocks = shape->cap_blocks; a.max_blocks = max_blocks;
  a.Kb = p.Kb; a.C = p.C; a.P = dense ? p.Pd : p.P;
  a.xcd = (p.U % 8) == 0;
  a.flags = (int)shape->flags;
  a.isd = 1.0f / sqrtf((float)shape->d);
  return hip_status(launch_attend(shape->d, shape->G, dense, a, p.U, (hipStream_t)stream));
}

int cknv_attend(const cknv_shape* shape, const cknv_cache* cache, const float* q,
                const int32_t* sel, const int32_t* n_sel, int32_t budget_tokens,
                int32_t max_blocks, float* out, float* lse, void* ws, size_t ws_bytes,
                void* stream) {
  return attend_common(shape, cache, q, sel, n_sel, budget_tokens, max_blocks, out, lse, ws,
                       ws_bytes, stream, false);
}

int cknv_dense_attend(const cknv_shape* shape, const cknv_cache* cache, const float* q,
                      int32_t budget_tokens, int32_t max_blocks, float* out, float* lse,
                      void* ws, size_t ws_bytes, void* stream) {
  return attend_common(shape, cache, q, nullptr, nullptr, budget_tokens, max_blocks, out, lse,
                       ws, ws_bytes, stream, true);
}

int cknv_decode_step_noalloc(const cknv_shape* shape, const cknv_cache* cache,
                             const uint16_t* new_k, const uint16_t* new_v, const float* q,
                             int32_t budget_tokens, int32_t max_blocks, float* scores,
                             int32_t* sel, int32_t* n_sel, float* out, float* lse, void* stream) {
  Plan p;
  int st = make_plan(shape, max_blocks, budget_tokens, &p);
  if (st) return st;
  if ((st = check_cache(cache))) return st;
  if (!new_k || !new_v || !q || !sel || !n_sel || !out) return CKNV_EINVAL;
  if (p.total > kNoAllocScratchBytes) return CKNV_ENOSPACE;
  char* w = nullptr;
  if ((st = noalloc_workspace(p, shape, stream, &w))) return st;
  if ((st = decode_score_impl(p, shape, cache, new_k, new_v, q, max_blocks, w, stream))) return st;
  return decode_finish_impl(p, shape, cache, q, max_blocks, scores, sel, n_sel, out, lse, w,
                            stream);
}

int cknv_kv_placement(const cknv_shape* shape, const cknv_cache* cache, int32_t* placement) {
  int st = check_shape(shape);
  if (st) return st;
  if ((st = check_cache(cache))) return st;
  if (!placement) return CKNV_EINVAL;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return CKNV_EHIP;
  }
  auto where = [dev](const void* ptr) { return mem_where(ptr, dev); };
  const int k = where(cache->k), v = where(cache->v);
  if (k < 0 || k != v) return CKNV_EINVAL;
  const int sm = where(cache->kbar);
  if (sm < 0 || where(cache->dbar) != sm || where(cache->cnt) != sm || where(cache->vbar) != sm)
    return CKNV_EINVAL;
  if (where(cache->seq_len) != 0) return CKNV_EINVAL;
  *placement = (k ? CKNV_KV_ON_HOST : 0) | (sm ? CKNV_SUMMARIES_ON_HOST : 0);
  return CKNV_OK;
}

const char* cknv_status_str(int status) {
  switch (status) {
    case CKNV_OK: return "CKNV_OK";
    case CKNV_EINVAL: return "CKNV_EINVAL: null pointer or invalid size";
    case CKNV_EUNSUPPORTED: return "CKNV_EUNSUPPORTED: shape not handled by the kernels";
    case CKNV_ENOSPACE: return "CKNV_ENOSPACE: workspace too small or max_blocks beyond capacity";
    case CKNV_EHIP: return "CKNV_EHIP: HIP launch or runtime error";
    default: return "unknown cknv status";
  }
}

}  // extern "C"
