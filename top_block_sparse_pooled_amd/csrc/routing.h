// Host/device interface of the routing kernels (route.hip), shared with the C ABI (abi.hip).
#pragma once
#include "common.h"

namespace fv {

// Routing variant of the select (see fvattn_route_opts): mode, top-k count, clamp of the Top-p
// count, local window, and the block geometry the window needs.
struct SelOpts {
  int mode, topk, k_min, k_max, window, bq, bk, N;
  double *imp;   // optional [rows][nkb]: importance P of every block (SASA candidates); EXT only
};

// Everything one routing launch needs (pooling, selection, the counters they share).
struct RouteLaunch {
  const void *q, *k;
  double *ksw;          // pooled keys (float64 MFMA operand order)
  int BH, N, d, dtype, bq, bk, nqb, nkb, nkw;
  double p;
  int32_t *counts;
  uint32_t *bitmask;
  int32_t *head_load, *bsum;
  int nbsum;
  SelOpts sel;
  uint32_t *status;
  double *scr;          // more than 1280 key blocks: kLargeSelGrid x 16 rows x nkbp scores, else unused
  int nkbp;             // key blocks rounded up to 16
};

// Workgroups of the select for more than 1280 key blocks; each owns 16 rows of score scratch.
constexpr int kLargeSelGrid = 256;
constexpr int kLargeSelMinNkb = 1281;

// Pooling of K (k_pool) and the selection (k_select, or k_select_large above 1280 key blocks).
int launch_route(const RouteLaunch &r, hipStream_t st);

}  // namespace fv
