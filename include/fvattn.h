/*
 * fvattn.h - C ABI of the Top-p block-sparse attention library for MI355X (gfx950).
 *
 * Method (FVAttn, PaperDaily summary "腾讯+中山大学新作：视频生成提速2.11×，靠的是RLB和SASA",
 * section "AI视频生成的阿喀琉斯之踵", Top-p routing paragraph): keys/values are cut into
 * fixed blocks; for each query block every key block gets an importance, blocks are ranked
 * in descending importance and the smallest prefix whose cumulative importance reaches p
 * is kept; softmax attention then runs over the kept blocks only.  Block importance uses
 * mean-pooled Q and K with a 1/sqrt(d) scale (tutorial page, section 5.2) followed by a
 * softmax over key blocks; ties in importance go to the lower block index.
 *
 * Conventions shared by every entry point
 *  - Tensors q, k, v, o are device pointers to contiguous [B, H, N, d] arrays (row-major,
 *    d fastest), the layout of the tutorial's block-sparse function (section 5.2).
 *  - Element type: FVATTN_BF16 (bfloat16; outputs rounded to nearest even) or FVATTN_F32.
 *  - Supported: d in {64, 128}; block_q in {32, 64, 128}; block_k in {32, 64};
 *    ceil(N / block_k) <= 4096 (262,144 tokens at 64-token key blocks).  Other values return
 *    FVATTN_ERR_UNSUPPORTED.
 *  - Row r of the routing is (b*H + h) * nqb + i for query block i; nqb = ceil(N/block_q),
 *    nkb = ceil(N/block_k).  The last block of each kind may be short (ragged): pooling
 *    averages its real tokens only, and padding never attends or is attended to.
 *  - Ownership: the caller owns every buffer, including workspaces; the library never
 *    allocates device memory and keeps no state between calls.
 *  - Asynchrony: compute calls validate their arguments on the host, enqueue kernels on
 *    `stream` (a hipStream_t; NULL = the default stream) and return without synchronising.
 *    Device outputs are valid once the stream has completed the work.
 *  - Errors: a validation failure returns its code before anything is enqueued; a failed
 *    launch returns FVATTN_ERR_HIP.  No C++ exception crosses the ABI.
 */
#ifndef FVATTN_H
#define FVATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FVATTN_VERSION 10100 /* 1.1.0 */

typedef enum fvattn_dtype { FVATTN_BF16 = 0, FVATTN_F32 = 1 } fvattn_dtype;

enum {
  FVATTN_OK = 0,
  FVATTN_ERR_INVALID = -1,     /* bad value: p outside (0,1] or NaN, B/H/N <= 0, NULL pointer */
  FVATTN_ERR_UNSUPPORTED = -2, /* d, block sizes, dtype or nkb outside the supported set     */
  FVATTN_ERR_CAPACITY = -3,    /* csr->capacity < fvattn_csr_max_nnz(...)                     */
  FVATTN_ERR_WORKSPACE = -4,   /* ws_bytes smaller than the matching *_ws_bytes() size        */
  FVATTN_ERR_OVERFLOW = -5,    /* B*H*nqb*nkb does not fit in int32                            */
  FVATTN_ERR_HIP = -6,         /* a HIP launch failed                                         */
  FVATTN_ERR_MISMATCH = -7,    /* CSR shape fields do not match the attention arguments       */
  FVATTN_ERR_SCRATCH = -8      /* problem larger than the static scratch of the no-allocation
                                  entry point (see fvattn_sparse_attn_noalloc)                 */
};

/*
 * Work-list orders for fvattn_worklist / fvattn_attn_plan / fvattn_sparse_attn.  A work unit is
 * G adjacent query blocks of one head; its work is the number of (query block, key block) pairs
 * its rows keep.  Head loads are the per-head loads of the FVAttn summary's RLB section.
 */
enum {
  FVATTN_SCHED_DEFAULT = -1, /* HEAD_DESC for up to 4096 heads, else IDENTITY                 */
  FVATTN_SCHED_LPT = 0,      /* units by work, longest first, ties by unit id                 */
  FVATTN_SCHED_IDENTITY = 1, /* units in ascending id (head-major) order                      */
  FVATTN_SCHED_HEAD_LPT = 2, /* heads by load (heaviest first, ties by id), a head's units
                                longest first                                                 */
  FVATTN_SCHED_XCD = 3,      /* units in id order cut into 8 contiguous ranges of equal work, one
                                per XCD (shared L2); an XCD that runs out takes units from the
                                others                                                        */
  FVATTN_SCHED_RLB = 4,      /* heads by load (heaviest first) each assigned to the XCD queue with
                                the least load so far (ties: lower XCD); a queue holds its heads in
                                assignment order, a head's units in id order; stealing as XCD.
                                The summary's RLB moves the heaviest heads first between ranks;
                                here the ranks are the 8 XCDs                                  */
  FVATTN_SCHED_HEAD_DESC = 5 /* heads by load (heaviest first, ties by id), a head's units in id
                                order, one queue                                               */
};

/* Bits of the device status words read by fvattn_ws_status (0 = no internal error). */
enum {
  FVATTN_STATUS_SELECT_NOCROSS = 1, /* routing: a row's radix search found no bin where the
                                       cumulative mass crosses its target; that row was kept
                                       whole.  Not expected to occur: an internal error.    */
  FVATTN_STATUS_PLAN_MISMATCH = 2   /* attention: the plan in the workspace was built for another
                                       dtype, CSR shape or unit size; nothing was computed    */
};

/*
 * Kept-block lists in CSR form, one row per (batch, head, query block).
 * All pointers are device memory allocated by the caller.  fvattn_route fills the shape
 * fields and the three arrays; fvattn_sparse_attn reads them and trusts the contents
 * (col_idx values in [0, nkb), ascending, row_ptr non-decreasing), so a CSR built by
 * other means (for example by a reference implementation) can be passed in.
 * nnz = row_ptr[rows].  head_load[bh] = number of kept (query block, key block) pairs of
 * that head: the per-head load of the FVAttn summary's RLB section (blocks a head must
 * compute, read off its sparse mask).
 */
typedef struct fvattn_csr {
  int32_t bh;        /* B*H                                             */
  int32_t n;         /* tokens per head                                 */
  int32_t block_q;   /* query block size                                */
  int32_t block_k;   /* key block size                                  */
  int32_t nqb;       /* ceil(n / block_q)                               */
  int32_t nkb;       /* ceil(n / block_k)                               */
  int32_t *row_ptr;  /* [bh*nqb + 1]                                    */
  int32_t *col_idx;  /* [capacity]; per row ascending key-block ids     */
  int64_t capacity;  /* elements available in col_idx                   */
  int32_t *head_load;/* [bh]                                            */
} fvattn_csr;

/*
 * Options of fvattn_sparse_attn; pass NULL for the defaults (FVATTN_SCHED_DEFAULT, library
 * grid, no trace).  The default order takes the heads heaviest first (the FVAttn summary's RLB
 * moves the heaviest heads first) and a head's units in id order: with one workgroup per CU the
 * units in flight then belong to one head, whose K/V tiles share the caches.  Measured on MI355X
 * it runs as fast as the identity order and faster than LPT, which balances CUs best but mixes
 * heads.
 *   schedule  one of FVATTN_SCHED_* (negative: FVATTN_SCHED_DEFAULT).
 *   grid      number of persistent workgroups; 0 = as many as stay resident.
 *   trace     optional device array of uint64.  Record t (t < units) describes the t-th work
 *             unit taken: {hardware id (XCC_ID << 32 | HW_ID), start clock, end clock, unit id},
 *             clocks from the 100 MHz constant-rate counter.  A unit is 128/block_q adjacent
 *             query blocks of one head for bf16 (128 query rows) and one query block for float32;
 *             units = B*H*ceil(nqb/(128/block_q)) resp. B*H*nqb.  Used to measure per-CU busy
 *             time; costs a few stores per unit.
 *   trace_cap uint64 elements available at trace; must be >= 4 * units when trace is not NULL
 *             (else FVATTN_ERR_INVALID).
 *   out_dtype element type of o: -1 = the input dtype; FVATTN_F32 = float32 output (the
 *             accumulator precision) for bf16 inputs.  With a bf16 output each value is the
 *             round-to-nearest-even of the float32 result.
 */
typedef struct fvattn_attn_opts {
  int32_t schedule;
  int32_t grid;
  uint64_t *trace;
  int64_t trace_cap;
  int32_t out_dtype;
  int32_t reserved;
} fvattn_attn_opts;

/* Routing variants of fvattn_route_ex. */
enum {
  FVATTN_ROUTE_TOPP = 0, /* Top-p: shortest prefix of the descending order with mass >= p  */
  FVATTN_ROUTE_TOPK = 1  /* fixed top-k: the first min(topk, nkb) blocks of that order      */
};

/*
 * Options of fvattn_route_ex.  The FVAttn summary contrasts Top-p routing with a fixed
 * Top-k; the tutorial's block-sparse section (5.2) keeps the top-k key blocks by pooled score
 * and adds a local window of neighbouring blocks.  Both use the same importance and the same
 * descending order (ties to the lower block index) as Top-p.
 *   mode    FVATTN_ROUTE_TOPP or FVATTN_ROUTE_TOPK
 *   p       Top-p threshold in (0, 1] (mode TOPP)
 *   topk    blocks per row, >= 1 (mode TOPK; more than nkb keeps every block)
 *   k_min   mode TOPP: the Top-p count is raised to at least k_min (>= 1) ...
 *   k_max   ... and lowered to at most k_max (0 = no upper bound; else >= k_min); the kept
 *           blocks are then the first clamp(count) blocks of the order
 *   window  >= 0: key blocks within `window` blocks of those that overlap the query block's
 *           tokens are always kept, in addition to the selection (0 = none).  With equal
 *           block sizes this is query block i's neighbours i-window .. i+window.
 */
typedef struct fvattn_route_opts {
  int32_t mode;
  int32_t topk;
  double p;
  int32_t k_min;
  int32_t k_max;
  int32_t window;
  int32_t reserved;
} fvattn_route_opts;

/* Library version (FVATTN_VERSION of the build). */
int fvattn_version(void);

/* Static string describing an error code. */
const char *fvattn_strerror(int code);

/* Worst-case CSR size B*H*nqb*nkb (every block kept), or a negative error code. */
int64_t fvattn_csr_max_nnz(int B, int H, int N, int block_q, int block_k);

/* Bytes of workspace fvattn_route needs (0 on invalid arguments).  Above 1280 key blocks it holds a
   score scratch of 256 x 16 rows x nkb doubles (up to 134 MB at 4096 key blocks). */
size_t fvattn_route_ws_bytes(int B, int H, int N, int d, int block_q, int block_k);

/* Bytes of workspace fvattn_sparse_attn needs (0 on invalid arguments). */
size_t fvattn_attn_ws_bytes(int B, int H, int N, int d, int dtype, int block_q, int block_k);

/*
 * Block mean-pooling (tutorial page, section 5.2: a block is summarised by the mean of its
 * tokens).  x: device [BH, N, d] of dtype; out: device float64 [BH, ceil(N/block), d], the
 * mean over each block's real tokens accumulated in float64.  This is the first step of
 * fvattn_route, exposed on its own.
 */
int fvattn_pool(const void *x, int BH, int N, int d, int dtype, int block, double *out,
                void *stream);

/*
 * Top-p routing (FVAttn summary, Top-p routing paragraph): pooled scores
 * s_ij = qbar_i . kbar_j / sqrt(d) (tutorial section 5.2), importance P_ij = softmax_j(s_ij),
 * descending order with ties to the lower index, kept set = shortest prefix whose
 * cumulative importance is >= p (p >= 1 keeps every block).  Scores, softmax and the cut
 * are evaluated in float64 (cumulative mass as exact 2^-52 fixed point).
 *   q, k       device [B, H, N, d] of dtype
 *   p          in (0, 1]
 *   csr        caller-filled pointers and capacity; shape fields are written
 *   ws         device workspace of at least fvattn_route_ws_bytes(...) bytes
 * The CSR is plain caller memory and may be applied to later q, k, v of the same shape: the
 * Baidu Cloud video-engine tutorial (step 2, dynamic sparse attention) refreshes the sparse
 * pattern only every few diffusion steps.  Attention over a given CSR is exact for any inputs.
 */
int fvattn_route(const void *q, const void *k, int B, int H, int N, int d, int dtype,
                 int block_q, int block_k, double p, fvattn_csr *csr, void *ws,
                 size_t ws_bytes, void *stream);

/*
 * fvattn_route with a routing variant (opts, not NULL; see fvattn_route_opts).  Same
 * arguments, outputs, workspace and errors as fvattn_route; invalid options return
 * FVATTN_ERR_INVALID.  fvattn_route(..., p, ...) equals fvattn_route_ex with
 * {FVATTN_ROUTE_TOPP, p, k_min = 1, k_max = 0, window = 0}.
 */
int fvattn_route_ex(const void *q, const void *k, int B, int H, int N, int d, int dtype, int block_q,
                    int block_k, const fvattn_route_opts *opts, fvattn_csr *csr, void *ws, size_t ws_bytes,
                    void *stream);

/*
 * Options of fvattn_route_sasa: SASA, slack-aware sparsity augmentation (FVAttn summary,
 * SASA section).  After load balancing every rank knows its kept-block count and the largest
 * one (the critical path); a rank with slack adds the highest-importance blocks that the
 * routing left out, from the candidates of all its heads, within its slack scaled by an
 * augmentation coefficient, and only when the slack passes a trigger threshold.  On one GPU
 * a rank is one of `groups` contiguous groups of the B*H heads (head h is in group
 * h*groups/(B*H)), the per-rank share of sequence parallelism.
 *   groups    1 .. min(B*H, 1024)
 *   critical  > 0: the critical path in kept blocks (for example the largest rank load
 *             gathered from the other ranks); 0: the largest group load
 *   alpha     augmentation coefficient in [0, 1]: a group adds floor(alpha * slack) blocks
 *   tau       trigger threshold in [0, 1]: only groups with slack >= tau * critical add blocks
 *   added     optional device int32[groups]: blocks added per group (NULL: not written)
 * Candidates of a group: its rows' unselected (row, key block) pairs, ordered by importance
 * (the routing's softmax over key blocks) descending, then row, then key block ascending.
 */
typedef struct fvattn_sasa_opts {
  int32_t groups;
  int32_t critical;
  double alpha;
  double tau;
  int32_t *added;
} fvattn_sasa_opts;

/* Bytes of workspace fvattn_route_sasa needs (0 on invalid arguments). */
size_t fvattn_route_sasa_ws_bytes(int B, int H, int N, int d, int block_q, int block_k, int groups);

/*
 * Routing (as fvattn_route_ex with ropts) followed by SASA (sopts); the CSR and head_load
 * hold the augmented kept sets.  Workspace: fvattn_route_sasa_ws_bytes(...) bytes.  Errors as
 * fvattn_route_ex; invalid SASA options return FVATTN_ERR_INVALID.  A group's augmented load
 * never exceeds the critical path.
 */
int fvattn_route_sasa(const void *q, const void *k, int B, int H, int N, int d, int dtype, int block_q,
                      int block_k, const fvattn_route_opts *ropts, const fvattn_sasa_opts *sopts,
                      fvattn_csr *csr, void *ws, size_t ws_bytes, void *stream);

/* Bytes of workspace fvattn_worklist needs for `rows` CSR rows (0 if rows <= 0). */
size_t fvattn_worklist_ws_bytes(int rows);

/*
 * Device-built work list (one-GPU analogue of the FVAttn summary's runtime load balancing:
 * the heaviest work is placed first).  Units of G adjacent query blocks of one head (G = 1: CSR
 * rows; the bf16 attention kernel uses G = 128 / block_q).  worklist: device int32
 * [B*H*ceil(nqb/G)] receives a permutation of the units in the requested FVATTN_SCHED_* order.
 * ws: device workspace of fvattn_worklist_ws_bytes(rows) bytes; its first 64 int32 are the
 * control block of a persistent consumer (tickets; for FVATTN_SCHED_XCD and FVATTN_SCHED_RLB
 * the per-XCD queue starts at int32 16 + x, x = 0..8).  G in {1, 2, 4}; the head-ordered
 * schedules (HEAD_LPT, RLB, HEAD_DESC) support up to 4096 heads.
 */
int fvattn_worklist(const fvattn_csr *csr, int schedule, int G, int32_t *worklist, void *ws, size_t ws_bytes,
                    void *stream);

/*
 * Status word left in a workspace by the last call that used it (FVATTN_STATUS_* bits; 0 = no
 * internal error).  which = 0: a routing workspace (fvattn_route, _ex, _sasa); which = 1: an
 * attention workspace (fvattn_attn_plan / _run / fvattn_sparse_attn).  Copies 4 bytes to the host
 * and synchronises `stream`.
 */
int fvattn_ws_status(const void *ws, int which, uint32_t *status, void *stream);

/*
 * Block-sparse attention (FVAttn summary: attention runs only over the kept blocks; the
 * sparse computation itself is exact): for each token t of query block i,
 *   o_t = sum_{s in T(i)} softmax_s(q_t . k_s / sqrt(d)) v_s,
 * T(i) = the real tokens of the key blocks listed in CSR row i.  bf16 inputs run on bf16
 * MFMA with float32 accumulation and online softmax (P rounded to bf16 for P.V); float32
 * inputs keep every step in float32.  Every row must list at least one block.
 *   q, k, v    device [B, H, N, d] of dtype
 *   o          device [B, H, N, d] of the output dtype (opts->out_dtype; default dtype),
 *              written for every real token
 *   csr        from fvattn_route or any valid CSR with matching shape fields
 *   opts       may be NULL
 *   ws         device workspace of at least fvattn_attn_ws_bytes(...) bytes
 * Equivalent to fvattn_attn_plan(opts->schedule) followed by fvattn_attn_run.
 */
int fvattn_sparse_attn(const void *q, const void *k, const void *v, void *o, int B, int H,
                       int N, int d, int dtype, const fvattn_csr *csr,
                       const fvattn_attn_opts *opts, void *ws, size_t ws_bytes, void *stream);

/*
 * First half of fvattn_sparse_attn: builds the work list of the CSR rows in `schedule`
 * order in `ws`.  The attention kernel reads q, k and v as given, so the plan depends on the
 * CSR only: it stays valid while the CSR and ws are unchanged, whatever q, k, v it later
 * meets.  v is not read; it must be non-NULL (the argument keeps the signature of
 * fvattn_sparse_attn's inputs).
 */
int fvattn_attn_plan(const void *v, int B, int H, int N, int d, int dtype, const fvattn_csr *csr,
                     int schedule, void *ws, size_t ws_bytes, void *stream);

/*
 * Second half of fvattn_sparse_attn: the attention kernel alone, consuming the plan held in
 * `ws` (enqueue fvattn_attn_plan on the same workspace first, in stream order).  May be
 * repeated on one plan; opts->schedule is ignored (the plan fixed the order).
 */
int fvattn_attn_run(const void *q, const void *k, const void *v, void *o, int B, int H, int N,
                    int d, int dtype, const fvattn_csr *csr, const fvattn_attn_opts *opts,
                    void *ws, size_t ws_bytes, void *stream);

/*
 * fvattn_sparse_attn without a workspace, for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  The plan
 * (control block, work list and sort scratch) lives in a static device array sized for
 * FVATTN_NOALLOC_MAX_ROWS rows (2 MiB), which the library holds on each GPU it runs on until the
 * process ends; B*H*ceil(N/block_q) > FVATTN_NOALLOC_MAX_ROWS returns FVATTN_ERR_SCRATCH before
 * anything is enqueued.  The device current on the calling thread must be the device of `stream`.
 * Every call on one GPU shares that GPU's array, which keeps the last call's plan: calls that
 * overlap on one GPU (several streams or host threads) race and must be serialised by the caller.
 * Calls no allocating routine.  Arguments, outputs and errors otherwise as fvattn_sparse_attn.
 */
#define FVATTN_NOALLOC_MAX_ROWS 262144
int fvattn_sparse_attn_noalloc(const void *q, const void *k, const void *v, void *o, int B, int H, int N, int d,
                               int dtype, const fvattn_csr *csr, const fvattn_attn_opts *opts, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FVATTN_H */
