// extern "C" entry points of libfvattn: argument validation on the host (nothing is
// enqueued unless every check passes), workspace carving, kernel launches.
#include <math.h>
#include <string.h>

#include <atomic>

#include "routing.h"

namespace fv {
int launch_pool(const void *x, int BH, int N, int d, int dtype, int block, double *out, hipStream_t st);
int launch_pool_k(const void *k, int BH, int N, int d, int dtype, int block_k, double *ksw, int32_t *zero0, int nzero0,
                  int32_t *zero1, int nzero1, int32_t *zero2, int nzero2, hipStream_t st);
size_t sasa_group_bytes(int R);
size_t sasa_hist_bytes(int R);
int launch_sasa(const double *imp, uint32_t *bitmask, int32_t *counts, int32_t *bsum, int32_t *head_load, int nkw,
                int nqb, int nkb, int BH, int R, int critical, double alpha, double tau, void *grp_buf,
                uint32_t *ghist, int32_t *tiecnt, int32_t *tiepre, int32_t *added_out, hipStream_t st);

int launch_csr(const int32_t *counts, const uint32_t *bitmask, const int32_t *bsum, int rows, int nkw, int nkb,
               int32_t *row_ptr, int32_t *col_idx, hipStream_t st);
int launch_plan(const int32_t *row_ptr, int rows, int nqb, int nkb, int G, int sched, int32_t *wl, int32_t *tmp,
                int32_t *counter, const int *sig, hipStream_t st);
int launch_attn_bf16(const void *q, const void *k, const void *v, void *o, int out_f32,
                     const int32_t *row_ptr,
                     const int32_t *col_idx, const int32_t *wl, int32_t *counter, int rows, int nqb, int nkb, int N,
                     int D, int BQ, int BK, int grid, uint64_t *trace, hipStream_t st);
int launch_attn_f32(const void *q, const void *k, const void *v, void *o, const int32_t *row_ptr,
                    const int32_t *col_idx, const int32_t *wl, int32_t *counter, int rows, int nqb, int nkb, int N,
                    int D, int BQ, int BK, uint64_t *trace, hipStream_t st);
}  // namespace fv

namespace {

constexpr int kMaxNkb = 4096;
constexpr int kMaxBH = 65535;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Shape {
  int B, H, N, d, bq, bk, BH, nqb, nkb, rows, nqbp, nkbp, nkw;
};

// Shape checks shared by every entry point.
int check_shape(int B, int H, int N, int d, int bq, int bk, Shape *s) {
  if (B <= 0 || H <= 0 || N <= 0) return FVATTN_ERR_INVALID;
  if (d != 64 && d != 128) return FVATTN_ERR_UNSUPPORTED;
  if (bq != 32 && bq != 64 && bq != 128) return FVATTN_ERR_UNSUPPORTED;
  if (bk != 32 && bk != 64) return FVATTN_ERR_UNSUPPORTED;
  const long long BH = (long long)B * H;
  if (BH > kMaxBH) return FVATTN_ERR_OVERFLOW;
  const long long nqb = (N + (long long)bq - 1) / bq, nkb = (N + (long long)bk - 1) / bk;
  if (nkb > kMaxNkb) return FVATTN_ERR_UNSUPPORTED;
  if (BH * nqb * nkb >= (1ll << 31)) return FVATTN_ERR_OVERFLOW;
  if (BH * (long long)N * d >= (1ll << 40)) return FVATTN_ERR_OVERFLOW;
  s->B = B; s->H = H; s->N = N; s->d = d; s->bq = bq; s->bk = bk;
  s->BH = (int)BH; s->nqb = (int)nqb; s->nkb = (int)nkb; s->rows = (int)(BH * nqb);
  s->nqbp = (int)((nqb + 15) / 16 * 16);
  s->nkbp = (int)((nkb + 15) / 16 * 16);
  s->nkw = (int)((nkb + 31) / 32);
  return FVATTN_OK;
}

struct RouteWs {
  uint32_t *status; // FVATTN_STATUS_* bits (first 4 bytes of the workspace)
  double *ksw;      // pooled K (the query blocks are pooled inside the select kernel)
  int32_t *counts;
  uint32_t *bitmask;
  int32_t *bsum;   // per-64-row sums of counts
  double *scr;     // score scratch of the large select (more than 1280 key blocks), else null
  int nblk;
  size_t bytes;
};

RouteWs route_ws_layout(const Shape &s, char *base) {
  RouteWs w;
  size_t off = 0;
  w.status = (uint32_t *)(base + off);
  off += 256;
  w.ksw = (double *)(base + off);
  off += align256((size_t)s.BH * s.nkbp * s.d * sizeof(double));
  w.counts = (int32_t *)(base + off);
  off += align256((size_t)s.rows * sizeof(int32_t));
  w.bitmask = (uint32_t *)(base + off);
  off += align256((size_t)s.rows * s.nkw * sizeof(uint32_t));
  w.nblk = (s.rows + 63) / 64;
  w.bsum = (int32_t *)(base + off);
  off += align256((size_t)w.nblk * sizeof(int32_t));
  w.scr = nullptr;
  if (s.nkb >= fv::kLargeSelMinNkb) {
    w.scr = (double *)(base + off);
    off += align256((size_t)fv::kLargeSelGrid * 16 * s.nkbp * sizeof(double));
  }
  w.bytes = off;
  return w;
}

// SASA workspace, after the routing workspace: importance of every block, per-group state,
// per-group histograms, per-row tie counts and running ranks.
struct SasaWs {
  double *imp;
  void *grp;
  uint32_t *ghist;
  int32_t *tiecnt, *tiepre;
  size_t bytes;   // including the routing workspace
};

SasaWs sasa_ws_layout(const Shape &s, int R, char *base) {
  SasaWs w;
  size_t off = align256(route_ws_layout(s, nullptr).bytes);
  w.imp = (double *)(base + off);
  off += align256((size_t)s.rows * s.nkb * sizeof(double));
  w.grp = base + off;
  off += align256(fv::sasa_group_bytes(R));
  w.ghist = (uint32_t *)(base + off);
  off += align256(fv::sasa_hist_bytes(R));
  w.tiecnt = (int32_t *)(base + off);
  off += align256((size_t)s.rows * sizeof(int32_t));
  w.tiepre = (int32_t *)(base + off);
  off += align256((size_t)s.rows * sizeof(int32_t));
  w.bytes = off;
  return w;
}

// Attention workspace: the plan's control block (fv::ctl), the work list and the sort scratch.
struct AttnWs {
  int32_t *counter, *worklist, *tmp;
  size_t bytes;
};

AttnWs attn_ws_layout(int rows, char *base) {
  AttnWs w;
  size_t off = 0;
  w.counter = (int32_t *)(base + off);
  off += align256(fv::ctl::kWords * sizeof(int32_t));
  w.worklist = (int32_t *)(base + off);
  off += align256((size_t)rows * sizeof(int32_t));
  w.tmp = (int32_t *)(base + off);
  off += align256((size_t)rows * sizeof(int32_t));
  w.bytes = off;
  return w;
}

bool dtype_ok(int dt) { return dt == FVATTN_BF16 || dt == FVATTN_F32; }

}  // namespace

extern "C" {

int fvattn_version(void) { return FVATTN_VERSION; }

const char *fvattn_strerror(int code) {
  switch (code) {
    case FVATTN_OK: return "ok";
    case FVATTN_ERR_INVALID: return "invalid argument (p outside (0,1], non-positive size or NULL pointer)";
    case FVATTN_ERR_UNSUPPORTED: return "unsupported head dim, block size, dtype or key-block count";
    case FVATTN_ERR_CAPACITY: return "CSR capacity below the worst-case number of kept blocks";
    case FVATTN_ERR_WORKSPACE: return "workspace smaller than required";
    case FVATTN_ERR_OVERFLOW: return "problem size overflows 32-bit indexing";
    case FVATTN_ERR_HIP: return "HIP launch failure";
    case FVATTN_ERR_MISMATCH: return "CSR shape does not match the attention arguments";
    case FVATTN_ERR_SCRATCH: return "more query-block rows than the no-allocation scratch holds (FVATTN_NOALLOC_MAX_ROWS)";
    default: return "unknown error code";
  }
}

int64_t fvattn_csr_max_nnz(int B, int H, int N, int block_q, int block_k) {
  Shape s;
  const int rc = check_shape(B, H, N, 64, block_q, block_k, &s);
  if (rc != FVATTN_OK) return rc;
  return (int64_t)s.rows * s.nkb;
}

size_t fvattn_route_ws_bytes(int B, int H, int N, int d, int block_q, int block_k) {
  Shape s;
  if (check_shape(B, H, N, d, block_q, block_k, &s) != FVATTN_OK) return 0;
  return route_ws_layout(s, nullptr).bytes;
}

size_t fvattn_attn_ws_bytes(int B, int H, int N, int d, int dtype, int block_q, int block_k) {
  Shape s;
  if (!dtype_ok(dtype) || check_shape(B, H, N, d, block_q, block_k, &s) != FVATTN_OK) return 0;
  return attn_ws_layout(s.rows, nullptr).bytes;
}

int fvattn_pool(const void *x, int BH, int N, int d, int dtype, int block, double *out, void *stream) {
  if (!dtype_ok(dtype)) return FVATTN_ERR_UNSUPPORTED;
  if (BH <= 0 || N <= 0) return FVATTN_ERR_INVALID;
  if (d != 64 && d != 128) return FVATTN_ERR_UNSUPPORTED;
  if (block != 32 && block != 64 && block != 128) return FVATTN_ERR_UNSUPPORTED;
  if (BH > kMaxBH) return FVATTN_ERR_OVERFLOW;
  if ((long long)BH * N * d >= (1ll << 40)) return FVATTN_ERR_OVERFLOW;
  if (x == nullptr || out == nullptr) return FVATTN_ERR_INVALID;
  return fv::launch_pool(x, BH, N, d, dtype, block, out, (hipStream_t)stream);
}

namespace {
// Validation of the routing options; FVATTN_OK or the error code.
int route_opts_check(const fvattn_route_opts &o) {
  if (o.mode == FVATTN_ROUTE_TOPP) {
    if (!(o.p > 0.0 && o.p <= 1.0)) return FVATTN_ERR_INVALID;  // also rejects NaN
    if (o.k_min < 1 || o.k_max < 0 || (o.k_max > 0 && o.k_max < o.k_min)) return FVATTN_ERR_INVALID;
  } else if (o.mode == FVATTN_ROUTE_TOPK) {
    if (o.topk < 1) return FVATTN_ERR_INVALID;
  } else {
    return FVATTN_ERR_INVALID;
  }
  if (o.window < 0) return FVATTN_ERR_INVALID;
  return FVATTN_OK;
}

// Pool, select (optionally writing the importance of every block) and, unless `csr_after`
// is false, the CSR.  Arguments already validated.
int route_core(const void *q, const void *k, const Shape &s, int N, int d, int dtype, int block_q, int block_k,
               const fvattn_route_opts &o, fvattn_csr *csr, const RouteWs &w, double *imp, bool csr_after,
               hipStream_t st) {
  int rc;
  csr->bh = s.BH; csr->n = N; csr->block_q = block_q; csr->block_k = block_k; csr->nqb = s.nqb; csr->nkb = s.nkb;
  fv::RouteLaunch r;
  r.q = q;
  r.k = k;
  r.ksw = w.ksw;
  r.BH = s.BH;
  r.N = N;
  r.d = d;
  r.dtype = dtype;
  r.bq = block_q;
  r.bk = block_k;
  r.nqb = s.nqb;
  r.nkb = s.nkb;
  r.nkw = s.nkw;
  r.p = o.mode == FVATTN_ROUTE_TOPP ? o.p : 1.0;
  r.counts = w.counts;
  r.bitmask = w.bitmask;
  r.head_load = csr->head_load;
  r.bsum = w.bsum;
  r.nbsum = w.nblk;
  r.sel = fv::SelOpts{o.mode, o.topk, o.k_min, o.k_max, o.window, block_q, block_k, N, imp};
  r.status = w.status;
  r.scr = w.scr;
  r.nkbp = s.nkbp;
  if ((rc = fv::launch_route(r, st)) != FVATTN_OK) return rc;
  if (!csr_after) return FVATTN_OK;
  return fv::launch_csr(w.counts, w.bitmask, w.bsum, s.rows, s.nkw, s.nkb, csr->row_ptr, csr->col_idx, st);
}
}  // namespace

int fvattn_route_ex(const void *q, const void *k, int B, int H, int N, int d, int dtype, int block_q,
                    int block_k, const fvattn_route_opts *opts, fvattn_csr *csr, void *ws, size_t ws_bytes,
                    void *stream) {
  if (!dtype_ok(dtype)) return FVATTN_ERR_UNSUPPORTED;
  if (opts == nullptr) return FVATTN_ERR_INVALID;
  Shape s;
  int rc = check_shape(B, H, N, d, block_q, block_k, &s);
  if (rc != FVATTN_OK) return rc;
  if ((rc = route_opts_check(*opts)) != FVATTN_OK) return rc;
  if (q == nullptr || k == nullptr || csr == nullptr || ws == nullptr) return FVATTN_ERR_INVALID;
  if (csr->row_ptr == nullptr || csr->col_idx == nullptr || csr->head_load == nullptr) return FVATTN_ERR_INVALID;
  if (csr->capacity < (int64_t)s.rows * s.nkb) return FVATTN_ERR_CAPACITY;
  const RouteWs w = route_ws_layout(s, (char *)ws);
  if (ws_bytes < w.bytes) return FVATTN_ERR_WORKSPACE;
  return route_core(q, k, s, N, d, dtype, block_q, block_k, *opts, csr, w, nullptr, true, (hipStream_t)stream);
}

size_t fvattn_route_sasa_ws_bytes(int B, int H, int N, int d, int block_q, int block_k, int groups) {
  Shape s;
  if (check_shape(B, H, N, d, block_q, block_k, &s) != FVATTN_OK) return 0;
  if (groups < 1 || groups > s.BH || groups > 1024) return 0;
  return sasa_ws_layout(s, groups, nullptr).bytes;
}

int fvattn_route_sasa(const void *q, const void *k, int B, int H, int N, int d, int dtype, int block_q,
                      int block_k, const fvattn_route_opts *ropts, const fvattn_sasa_opts *sopts, fvattn_csr *csr,
                      void *ws, size_t ws_bytes, void *stream) {
  if (!dtype_ok(dtype)) return FVATTN_ERR_UNSUPPORTED;
  if (ropts == nullptr || sopts == nullptr) return FVATTN_ERR_INVALID;
  Shape s;
  int rc = check_shape(B, H, N, d, block_q, block_k, &s);
  if (rc != FVATTN_OK) return rc;
  if ((rc = route_opts_check(*ropts)) != FVATTN_OK) return rc;
  const fvattn_sasa_opts &so = *sopts;
  if (so.groups < 1 || so.groups > s.BH || so.groups > 1024) return FVATTN_ERR_INVALID;
  if (!(so.alpha >= 0.0 && so.alpha <= 1.0) || !(so.tau >= 0.0 && so.tau <= 1.0)) return FVATTN_ERR_INVALID;
  if (so.critical < 0) return FVATTN_ERR_INVALID;
  if (q == nullptr || k == nullptr || csr == nullptr || ws == nullptr) return FVATTN_ERR_INVALID;
  if (csr->row_ptr == nullptr || csr->col_idx == nullptr || csr->head_load == nullptr) return FVATTN_ERR_INVALID;
  if (csr->capacity < (int64_t)s.rows * s.nkb) return FVATTN_ERR_CAPACITY;
  const SasaWs sw = sasa_ws_layout(s, so.groups, (char *)ws);
  if (ws_bytes < sw.bytes) return FVATTN_ERR_WORKSPACE;
  const RouteWs w = route_ws_layout(s, (char *)ws);
  hipStream_t st = (hipStream_t)stream;
  if ((rc = route_core(q, k, s, N, d, dtype, block_q, block_k, *ropts, csr, w, sw.imp, false, st)) != FVATTN_OK)
    return rc;
  if ((rc = fv::launch_sasa(sw.imp, w.bitmask, w.counts, w.bsum, csr->head_load, s.nkw, s.nqb, s.nkb, s.BH,
                            so.groups, so.critical, so.alpha, so.tau, sw.grp, sw.ghist, sw.tiecnt, sw.tiepre,
                            so.added, st)) != FVATTN_OK)
    return rc;
  return fv::launch_csr(w.counts, w.bitmask, w.bsum, s.rows, s.nkw, s.nkb, csr->row_ptr, csr->col_idx, st);
}

int fvattn_route(const void *q, const void *k, int B, int H, int N, int d, int dtype, int block_q, int block_k,
                 double p, fvattn_csr *csr, void *ws, size_t ws_bytes, void *stream) {
  fvattn_route_opts o{};
  o.mode = FVATTN_ROUTE_TOPP;
  o.p = p;
  o.k_min = 1;
  return fvattn_route_ex(q, k, B, H, N, d, dtype, block_q, block_k, &o, csr, ws, ws_bytes, stream);
}

size_t fvattn_worklist_ws_bytes(int rows) {
  if (rows <= 0) return 0;
  return attn_ws_layout(rows, nullptr).bytes;
}

namespace {
bool sched_known(int sched) {
  return sched == FVATTN_SCHED_LPT || sched == FVATTN_SCHED_IDENTITY || sched == FVATTN_SCHED_HEAD_LPT ||
         sched == FVATTN_SCHED_XCD || sched == FVATTN_SCHED_RLB || sched == FVATTN_SCHED_HEAD_DESC;
}
bool sched_by_head(int sched) {
  return sched == FVATTN_SCHED_HEAD_LPT || sched == FVATTN_SCHED_RLB || sched == FVATTN_SCHED_HEAD_DESC;
}
constexpr int kMaxPlanHeads = 4096;   // heads the head-ordered schedules rank on the device
}  // namespace

int fvattn_worklist(const fvattn_csr *csr, int schedule, int G, int32_t *worklist, void *ws, size_t ws_bytes,
                    void *stream) {
  if (csr == nullptr || worklist == nullptr || ws == nullptr || csr->row_ptr == nullptr) return FVATTN_ERR_INVALID;
  if (!sched_known(schedule)) return FVATTN_ERR_INVALID;
  if (G != 1 && G != 2 && G != 4) return FVATTN_ERR_INVALID;
  if (csr->bh <= 0 || csr->nqb <= 0 || csr->nkb <= 0) return FVATTN_ERR_INVALID;
  if (csr->nkb > kMaxNkb) return FVATTN_ERR_UNSUPPORTED;
  if (sched_by_head(schedule) && csr->bh > kMaxPlanHeads) return FVATTN_ERR_UNSUPPORTED;
  if ((long long)csr->bh * csr->nqb >= (1ll << 31) || (long long)csr->nqb * csr->nkb >= (1ll << 31))
    return FVATTN_ERR_OVERFLOW;
  const int rows = csr->bh * csr->nqb;
  const AttnWs w = attn_ws_layout(rows, (char *)ws);
  if (ws_bytes < w.bytes) return FVATTN_ERR_WORKSPACE;
  return fv::launch_plan(csr->row_ptr, rows, csr->nqb, csr->nkb, G, schedule, worklist, w.tmp, w.counter, nullptr,
                         (hipStream_t)stream);
}

int fvattn_ws_status(const void *ws, int which, uint32_t *status, void *stream) {
  if (ws == nullptr || status == nullptr || (which != 0 && which != 1)) return FVATTN_ERR_INVALID;
  const char *src = (const char *)ws + (which == 0 ? 0 : fv::ctl::kStatus * sizeof(int32_t));
  hipStream_t st = (hipStream_t)stream;
  if (hipMemcpyAsync(status, src, sizeof(uint32_t), hipMemcpyDeviceToHost, st) != hipSuccess) return FVATTN_ERR_HIP;
  if (hipStreamSynchronize(st) != hipSuccess) return FVATTN_ERR_HIP;
  return FVATTN_OK;
}

namespace {
// Argument checks shared by plan / run / sparse_attn (everything but the workspace).
int attn_arg_checks(const void *v, int B, int H, int N, int d, int dtype, const fvattn_csr *csr, Shape *s) {
  if (!dtype_ok(dtype)) return FVATTN_ERR_UNSUPPORTED;
  if (csr == nullptr) return FVATTN_ERR_INVALID;
  int rc = check_shape(B, H, N, d, csr->block_q, csr->block_k, s);
  if (rc != FVATTN_OK) return rc;
  if (v == nullptr) return FVATTN_ERR_INVALID;
  if (csr->row_ptr == nullptr || csr->col_idx == nullptr) return FVATTN_ERR_INVALID;
  if (csr->bh != s->BH || csr->n != N || csr->nqb != s->nqb || csr->nkb != s->nkb) return FVATTN_ERR_MISMATCH;
  return FVATTN_OK;
}

// The argument checks and the caller's workspace.  Returns the workspace layout through *w.
int attn_checks(const void *v, int B, int H, int N, int d, int dtype, const fvattn_csr *csr, Shape *s, void *ws,
                size_t ws_bytes, AttnWs *w) {
  int rc = attn_arg_checks(v, B, H, N, d, dtype, csr, s);
  if (rc != FVATTN_OK) return rc;
  if (ws == nullptr) return FVATTN_ERR_INVALID;
  *w = attn_ws_layout(s->rows, (char *)ws);
  if (ws_bytes < w->bytes) return FVATTN_ERR_WORKSPACE;
  return FVATTN_OK;
}

// FVATTN_SCHED_DEFAULT (any negative value): heads heaviest first (HEAD_DESC) while the plan can
// rank the heads on the device, else identity.
int resolve_sched(int sched, const Shape &s) {
  if (sched >= 0) return sched;
  return s.BH <= kMaxPlanHeads ? FVATTN_SCHED_HEAD_DESC : FVATTN_SCHED_IDENTITY;
}

int sched_ok(int sched, const Shape &s) {
  if (!sched_known(sched)) return FVATTN_ERR_INVALID;
  if (sched_by_head(sched) && s.BH > kMaxPlanHeads) return FVATTN_ERR_UNSUPPORTED;
  return FVATTN_OK;
}

// Query blocks per work unit: the bf16 kernel's units are 128 query rows; the float32 kernel's
// are single query blocks.
int unit_blocks(int dtype, int block_q) { return dtype == FVATTN_BF16 ? 128 / block_q : 1; }

// Signature of a plan: what the run kernels compare before consuming it.
void plan_sig(const Shape &s, int dtype, int sig[fv::ctl::kSigLen]) {
  const int G = unit_blocks(dtype, s.bq);
  sig[0] = s.BH * fv::cdiv(s.nqb, G);
  sig[1] = G;
  sig[2] = dtype;
  sig[3] = s.nqb;
  sig[4] = s.BH;
  sig[5] = s.nkb;
  sig[6] = s.N;
  sig[7] = fv::ctl::kMagic;
}

int run_checks(const void *q, const void *k, void *o, int dtype, const Shape &s, const fvattn_attn_opts *opts,
               int *grid, uint64_t **trace, int *out_dt) {
  if (q == nullptr || k == nullptr || o == nullptr) return FVATTN_ERR_INVALID;
  *grid = opts ? opts->grid : 0;
  if (*grid < 0) return FVATTN_ERR_INVALID;
  *trace = opts ? opts->trace : nullptr;
  if (*trace != nullptr) {
    const long long units = (long long)s.BH * fv::cdiv(s.nqb, unit_blocks(dtype, s.bq));
    if (opts->trace_cap < 4 * units) return FVATTN_ERR_INVALID;
  }
  *out_dt = (opts && opts->out_dtype >= 0) ? opts->out_dtype : dtype;
  if (!dtype_ok(*out_dt) || (dtype == FVATTN_F32 && *out_dt != FVATTN_F32)) return FVATTN_ERR_UNSUPPORTED;
  return FVATTN_OK;
}

int do_plan(const Shape &s, int dtype, const fvattn_csr *csr, int sched, const AttnWs &w, hipStream_t st) {
  int sig[fv::ctl::kSigLen];
  plan_sig(s, dtype, sig);
  return fv::launch_plan(csr->row_ptr, s.rows, s.nqb, s.nkb, sig[1], sched, w.worklist, w.tmp, w.counter, sig, st);
}

int do_run(const void *q, const void *k, const void *v, void *o, const Shape &s, int dtype, int out_dt,
           const fvattn_csr *csr, int grid, uint64_t *trace, const AttnWs &w, hipStream_t st) {
  if (dtype == FVATTN_F32)
    return fv::launch_attn_f32(q, k, v, o, csr->row_ptr, csr->col_idx, w.worklist, w.counter, s.rows, s.nqb, s.nkb,
                               s.N, s.d, csr->block_q, csr->block_k, trace, st);
  return fv::launch_attn_bf16(q, k, v, o, out_dt == FVATTN_F32, csr->row_ptr, csr->col_idx, w.worklist,
                              w.counter, s.rows, s.nqb, s.nkb, s.N, s.d, csr->block_q, csr->block_k, grid, trace,
                              st);
}
}  // namespace

int fvattn_attn_plan(const void *v, int B, int H, int N, int d, int dtype, const fvattn_csr *csr, int schedule,
                     void *ws, size_t ws_bytes, void *stream) {
  Shape s;
  AttnWs w;
  int rc = attn_checks(v, B, H, N, d, dtype, csr, &s, ws, ws_bytes, &w);
  if (rc != FVATTN_OK) return rc;
  schedule = resolve_sched(schedule, s);
  if ((rc = sched_ok(schedule, s)) != FVATTN_OK) return rc;
  return do_plan(s, dtype, csr, schedule, w, (hipStream_t)stream);
}

int fvattn_attn_run(const void *q, const void *k, const void *v, void *o, int B, int H, int N, int d, int dtype,
                    const fvattn_csr *csr, const fvattn_attn_opts *opts, void *ws, size_t ws_bytes, void *stream) {
  Shape s;
  AttnWs w;
  int rc = attn_checks(v, B, H, N, d, dtype, csr, &s, ws, ws_bytes, &w);
  if (rc != FVATTN_OK) return rc;
  int grid, out_dt;
  uint64_t *trace;
  if ((rc = run_checks(q, k, o, dtype, s, opts, &grid, &trace, &out_dt)) != FVATTN_OK) return rc;
  return do_run(q, k, v, o, s, dtype, out_dt, csr, grid, trace, w, (hipStream_t)stream);
}

int fvattn_sparse_attn(const void *q, const void *k, const void *v, void *o, int B, int H, int N, int d, int dtype,
                       const fvattn_csr *csr, const fvattn_attn_opts *opts, void *ws, size_t ws_bytes,
                       void *stream) {
  Shape s;
  AttnWs w;
  int rc = attn_checks(v, B, H, N, d, dtype, csr, &s, ws, ws_bytes, &w);
  if (rc != FVATTN_OK) return rc;
  const int sched = resolve_sched(opts ? opts->schedule : FVATTN_SCHED_DEFAULT, s);
  if ((rc = sched_ok(sched, s)) != FVATTN_OK) return rc;
  int grid, out_dt;
  uint64_t *trace;
  if ((rc = run_checks(q, k, o, dtype, s, opts, &grid, &trace, &out_dt)) != FVATTN_OK) return rc;
  hipStream_t st = (hipStream_t)stream;
  if ((rc = do_plan(s, dtype, csr, sched, w, st)) != FVATTN_OK) return rc;
  return do_run(q, k, v, o, s, dtype, out_dt, csr, grid, trace, w, st);
}

}  // extern "C"

// ---------------------------------------------------------------------------------------
// No-allocation variant of fvattn_sparse_attn: the attention workspace (plan control block,
// work list, sort scratch) is the static device array `scratch`, sized for
// FVATTN_NOALLOC_MAX_ROWS rows.  Host code never uses the array's name as a device address: on
// a device's first call the address is taken with hipGetSymbolAddress (with that device
// current) and kept per device.  The plan kernel writes every control word and work-list entry
// it later reads, so nothing needs clearing between calls.
// ---------------------------------------------------------------------------------------
namespace {
constexpr size_t kScratchBytes = 256 + 2 * (((size_t)FVATTN_NOALLOC_MAX_ROWS * sizeof(int32_t) + 255) & ~(size_t)255);
constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_addr[kMaxDevices];
}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
// Device address of this device's `scratch` (taken once per device).
int scratch_address(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return FVATTN_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return FVATTN_ERR_UNSUPPORTED;
  void *p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return FVATTN_ERR_HIP;
    g_scratch_addr[dev].store(p, std::memory_order_release);   // racing first calls store the same address
  }
  *out = p;
  return FVATTN_OK;
}
}  // namespace

extern "C" int fvattn_sparse_attn_noalloc(const void *q, const void *k, const void *v, void *o, int B, int H, int N,
                                          int d, int dtype, const fvattn_csr *csr, const fvattn_attn_opts *opts,
                                          void *stream) {
  // every argument check of fvattn_sparse_attn before the scratch address is taken
  Shape s;
  int rc = attn_arg_checks(v, B, H, N, d, dtype, csr, &s);
  if (rc != FVATTN_OK) return rc;
  if (s.rows > FVATTN_NOALLOC_MAX_ROWS || attn_ws_layout(s.rows, nullptr).bytes > kScratchBytes)
    return FVATTN_ERR_SCRATCH;
  const int sched = resolve_sched(opts ? opts->schedule : FVATTN_SCHED_DEFAULT, s);
  if ((rc = sched_ok(sched, s)) != FVATTN_OK) return rc;
  int grid, out_dt;
  uint64_t *trace;
  if ((rc = run_checks(q, k, o, dtype, s, opts, &grid, &trace, &out_dt)) != FVATTN_OK) return rc;
  void *ws = nullptr;
  if ((rc = scratch_address(&ws)) != FVATTN_OK) return rc;
  const AttnWs w = attn_ws_layout(s.rows, (char *)ws);
  hipStream_t st = (hipStream_t)stream;
  if ((rc = do_plan(s, dtype, csr, sched, w, st)) != FVATTN_OK) return rc;
  return do_run(q, k, v, o, s, dtype, out_dt, csr, grid, trace, w, st);
}
