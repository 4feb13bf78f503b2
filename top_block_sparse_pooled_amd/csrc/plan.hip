// Device-built work list of the attention kernels (the plan), and its control block.
//
// Method: the FVAttn summary page (PaperDaily, arXiv:2607.16190), section "RLB：不搞全局重洗…":
// runtime load balancing reads each head's load (its kept blocks) off the sparse mask and moves
// the heaviest heads first, from the most to the least loaded rank.  On one GPU the balanced
// resources are the compute units and the eight XCDs (each with its own L2); the work units are
// groups of adjacent query blocks of one head.
//
// A unit is G consecutive query blocks of one head (G = 1: a CSR row); unit u = bh * ngroups + g
// covers rows bh*nqb + g*G .. min(bh*nqb + g*G + G, (bh+1)*nqb) - 1, so its work (kept blocks) is
// one difference of row_ptr.  Orders (FVATTN_SCHED_*):
//   LPT       units by work descending, ties by unit id (a stable sort on the exact work);
//   IDENTITY  unit id order;
//   HEAD_LPT  heads by load descending (ties: head id), each head's units by work descending;
//   XCD       unit id order cut into 8 ranges of equal work, one per XCD, with stealing;
//   RLB       heads by load descending, each assigned in turn to the XCD queue with the least
//             load so far (ties: lower XCD); a queue holds its heads in assignment order, a head's
//             units in id order; a workgroup takes units from its own XCD's queue, then steals;
//   HEAD_DESC heads by load descending, units of a head in id order, one queue.
// Sorting: a stable least-significant-digit radix sort with 8-bit digits (per-wave histograms in
// LDS, bases by scan, scatter of 64-item chunks ranked with bit-sliced ballots), on one
// workgroup of 1024 threads.
#include "common.h"

namespace fv {

constexpr int kPlWaves = 16;
constexpr int kPlMaxHeads = 4096;   // heads the head-ordered schedules rank in LDS

struct PlanArgs {
  const int32_t *row_ptr;
  int rows, nqb, nkb, G, sched;
  int32_t *wl, *tmp, *counter;
  int sig[ctl::kSigLen];   // plan signature written to the control block
};

struct Units {
  const int32_t *row_ptr;
  int nqb, G, ngroups;
  __device__ __forceinline__ int work(int u) const {
    const int bh = u / ngroups, g = u - bh * ngroups;
    const int r0 = bh * nqb + g * G, r1 = min(r0 + G, (bh + 1) * nqb);
    return row_ptr[r1] - row_ptr[r0];
  }
  __device__ __forceinline__ int head_load(int h) const { return row_ptr[(h + 1) * nqb] - row_ptr[h * nqb]; }
};

struct PlanLds {
  int hist[kPlWaves][256];
  int scan[256];
  int wsum[4];
  int hkey[kPlMaxHeads];     // per head: its rank (head-ordered schedules)
  int ha[kPlMaxHeads], hb[kPlMaxHeads];   // head sort ping-pong; RLB: XCD and slot per head
  int xbase[9];
};

// Exclusive scan of s.scan[0..255] in place by threads 0..255 (all threads call).
__device__ void scan256(PlanLds &s) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int v = 0, incl = 0;
  if (tid < 256) {
    v = s.scan[tid];
    incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
  }
  __syncthreads();
  if (tid < 256 && lane == 63) s.wsum[w] = incl;
  __syncthreads();
  if (tid < 256) {
    int pre = 0;
    for (int ww = 0; ww < w; ++ww) pre += s.wsum[ww];
    s.scan[tid] = pre + incl - v;
  }
  __syncthreads();
}

// One stable pass (digit (key >> shift) & 255) of an LSD radix sort of n items: item i is
// src[i] (or i when src is null); dst receives the items ordered by digit, equal digits in input
// order.  Wave w owns the contiguous input segment w of kPlWaves.
template <class KeyF>
__device__ void lsd_pass(const int32_t *src, int32_t *dst, int n, int shift, KeyF key, PlanLds &s) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < kPlWaves * 256; i += 1024) (&s.hist[0][0])[i] = 0;
  __syncthreads();
  const int seg = cdiv(n, kPlWaves);
  const int lo = min(n, w * seg), hi = min(n, lo + seg);
  for (int i = lo + lane; i < hi; i += 64) {
    const int v = src ? src[i] : i;
    atomicAdd(&s.hist[w][(key(v) >> shift) & 255], 1);
  }
  __syncthreads();
  if (tid < 256) {
    int t = 0;
    for (int ww = 0; ww < kPlWaves; ++ww) t += s.hist[ww][tid];
    s.scan[tid] = t;
  }
  __syncthreads();
  scan256(s);
  if (tid < 256) {   // bin-major, wave-minor bases
    int run = s.scan[tid];
    for (int ww = 0; ww < kPlWaves; ++ww) {
      const int c = s.hist[ww][tid];
      s.hist[ww][tid] = run;
      run += c;
    }
  }
  __syncthreads();
  const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int c0 = lo; c0 < hi; c0 += 64) {
    const int i = c0 + lane;
    const bool act = i < hi;
    const int v = act ? (src ? src[i] : i) : 0;
    const int dg = act ? (key(v) >> shift) & 255 : 0;
    unsigned long long peers = __ballot(act);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const unsigned long long bb = __ballot(act && ((dg >> b) & 1));
      peers &= ((dg >> b) & 1) ? bb : ~bb;
    }
    const int rank = __popcll(peers & lt);
    int base = 0;
    if (act) base = s.hist[w][dg];
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    if (act) {
      dst[base + rank] = v;
      if (rank == 0) s.hist[w][dg] = base + __popcll(peers);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
}

// Stable sort of n items (0..n-1) by a key of `bits` bits, ending in out (tmp: scratch of n).
template <class KeyF>
__device__ void lsd_sort(int n, int bits, KeyF key, int32_t *out, int32_t *tmp, PlanLds &s) {
  int passes = cdiv(bits, 8);
  if (passes < 1) passes = 1;
  if (passes & 1) ++passes;   // an even count of passes ends in out
  const int32_t *src = nullptr;
  for (int p = 0; p < passes; ++p) {
    int32_t *dst = (p & 1) ? out : tmp;
    lsd_pass(src, dst, n, 8 * p, key, s);
    src = dst;
  }
}

__device__ __forceinline__ int bits_for(unsigned x) { return x == 0 ? 1 : 32 - __clz((int)x); }

__global__ __launch_bounds__(1024) void k_plan(PlanArgs a) {
  __shared__ PlanLds s;
  const int tid = threadIdx.x;
  const int nh = a.rows / a.nqb;
  const int ngroups = cdiv(a.nqb, a.G);
  const int units = nh * ngroups;
  const Units um{a.row_ptr, a.nqb, a.G, ngroups};
  int32_t *ctr = a.counter;
  const bool per_xcd = a.sched == FVATTN_SCHED_XCD || a.sched == FVATTN_SCHED_RLB;
  if (tid == 0 && ctr != nullptr) {
    ctr[ctl::kTicket] = 0;
    ctr[ctl::kExit] = 0;
    ctr[ctl::kPerXcd] = per_xcd ? 1 : 0;
    ctr[ctl::kStatus] = 0;
#pragma unroll
    for (int i = 0; i < ctl::kSigLen; ++i) ctr[ctl::kSig + i] = a.sig[i];
  }
  const int maxw = a.G * a.nkb;   // upper bound of a unit's work
  if (a.sched == FVATTN_SCHED_IDENTITY || a.sched == FVATTN_SCHED_XCD) {
    for (int u = tid; u < units; u += 1024) a.wl[u] = u;
    if (a.sched == FVATTN_SCHED_XCD && ctr != nullptr && tid < 9) {
      // range x starts at the first unit whose kept blocks begin at or after x/8 of the total
      const long long nnz = a.row_ptr[a.rows];
      const long long target = nnz * tid / 8;
      int lo = 0, hi = units;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        const int bh = mid / ngroups, g = mid - bh * ngroups;
        if (a.row_ptr[bh * a.nqb + g * a.G] < target) lo = mid + 1; else hi = mid;
      }
      const int start = tid == 8 ? units : lo;
      ctr[ctl::kXcdStart + tid] = start;
      if (tid < 8) ctr[ctl::kXcdTicket + tid] = start;
    }
    return;
  }
  if (a.sched == FVATTN_SCHED_LPT) {
    lsd_sort(units, bits_for((unsigned)maxw), [&](int u) { return maxw - um.work(u); }, a.wl, a.tmp, s);
    return;
  }
  // head-ordered schedules: rank heads by load descending, ties by head id (nh <= kPlMaxHeads)
  if (nh <= 1024) {
    // one pass: thread h counts the heads that go before it
    for (int h = tid; h < nh; h += 1024) s.hb[h] = um.head_load(h);
    __syncthreads();
    if (tid < nh) {
      const int lh = s.hb[tid];
      int rank = 0;
      for (int h2 = 0; h2 < nh; ++h2) {
        const int l2 = s.hb[h2];
        rank += (l2 > lh) || (l2 == lh && h2 < tid);
      }
      s.hkey[tid] = rank;
      s.ha[rank] = tid;
    }
  } else {
    const unsigned maxl = (unsigned)a.nqb * (unsigned)a.nkb;
    lsd_sort(nh, bits_for(maxl), [&](int h) { return (int)(maxl - (unsigned)um.head_load(h)); }, s.ha, s.hb, s);
    for (int r = tid; r < nh; r += 1024) s.hkey[s.ha[r]] = r;   // rank of each head
  }
  __syncthreads();
  if (a.sched == FVATTN_SCHED_HEAD_LPT) {
    const int hb = bits_for((unsigned)(nh - 1));
    const int wb = bits_for((unsigned)maxw);
    lsd_sort(units, hb + wb, [&](int u) { return (s.hkey[u / ngroups] << wb) | (maxw - um.work(u)); }, a.wl, a.tmp,
             s);
    return;
  }
  if (a.sched == FVATTN_SCHED_HEAD_DESC) {
    for (int u = tid; u < units; u += 1024) {
      const int h = u / ngroups, g = u - h * ngroups;
      a.wl[s.hkey[h] * ngroups + g] = u;
    }
    return;
  }
  // RLB: greedy assignment of the ranked heads to the 8 XCD queues (least load so far, ties to
  // the lower XCD); ha[h] = queue, hb[h] = slot of h in its queue
  if (tid == 0) {
    long long xl[8];
    int cnt[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      xl[x] = 0;
      cnt[x] = 0;
    }
    for (int r = 0; r < nh; ++r) {
      const int h = s.ha[r];
      int best = 0;
#pragma unroll
      for (int x = 1; x < 8; ++x)
        if (xl[x] < xl[best]) best = x;
      xl[best] += um.head_load(h);
      s.hb[r] = (best << 16) | cnt[best]++;   // queue and slot of the r-th ranked head
    }
    int run = 0;
    for (int x = 0; x < 8; ++x) {
      s.xbase[x] = run;
      run += cnt[x] * ngroups;
    }
    s.xbase[8] = run;
  }
  __syncthreads();
  for (int r = tid; r < nh; r += 1024) s.hkey[s.ha[r]] = s.hb[r];
  __syncthreads();
  for (int u = tid; u < units; u += 1024) {
    const int h = u / ngroups, g = u - h * ngroups;
    const int qs = s.hkey[h];
    a.wl[s.xbase[qs >> 16] + (qs & 0xffff) * ngroups + g] = u;
  }
  if (ctr != nullptr && tid < 9) {
    ctr[ctl::kXcdStart + tid] = s.xbase[tid];
    if (tid < 8) ctr[ctl::kXcdTicket + tid] = s.xbase[tid];
  }
}

int launch_plan(const int32_t *row_ptr, int rows, int nqb, int nkb, int G, int sched, int32_t *wl, int32_t *tmp,
                int32_t *counter, const int *sig, hipStream_t st) {
  PlanArgs a;
  a.row_ptr = row_ptr;
  a.rows = rows;
  a.nqb = nqb;
  a.nkb = nkb;
  a.G = G;
  a.sched = sched;
  a.wl = wl;
  a.tmp = tmp;
  a.counter = counter;
  for (int i = 0; i < ctl::kSigLen; ++i) a.sig[i] = sig ? sig[i] : 0;
  hipLaunchKernelGGL(k_plan, dim3(1), dim3(1024), 0, st, a);
  FV_CHECK_LAUNCH();
  return FVATTN_OK;
}

}  // namespace fv
