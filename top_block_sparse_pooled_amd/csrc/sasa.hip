// SASA, slack-aware sparsity augmentation, on one GPU.
//
// Method: FVAttn summary page (PaperDaily, arXiv:2607.16190), SASA section.  After load
// balancing each rank knows its own kept-block count and the largest one (the critical
// path); a rank with slack adds the highest-importance blocks that Top-p left out, taken from
// the candidates of all its heads in the routing's importance order, within its slack scaled
// by an augmentation coefficient, and only when the slack passes a trigger threshold.
//
// Here a rank is one of R contiguous groups of the layer's heads (head h is in group
// h*R/BH), the per-rank share of sequence parallelism; the critical path is the largest group
// load or a caller-given value.  The candidates of a group are its rows' unselected blocks,
// ordered by importance P (descending), then row, then key block (ascending).
//
// Kernels (all on the routing workspace: counts, kept bitmask, per-64-row sums, and the
// importance P of every block written by the routing's select pass):
//  * k_sasa_init     group loads, critical path, per-group budgets; radix state
//  * k_sasa_hist     per pass: histogram of the candidates' keys (float64 bit patterns of P,
//                    monotone for P >= 0) in each searching group's current range
//  * k_sasa_resolve  per pass: the bin where the count from the top reaches the budget;
//                    narrows the range (11-bit digits: 6 passes resolve any key in [0, 1])
//  * k_sasa_ties     candidates equal to a group's threshold key, per row; k_sasa_tiescan
//                    turns them into a per-group running rank in row order
//  * k_sasa_mark     adds the selected blocks to the kept bitmask, counts, loads and sums
#include "common.h"

namespace fv {

struct SasaGroup {
  unsigned long long lo, width, above, target;   // key range, candidates above it, budget
  int state;          // 0 searching, 1 unique threshold, 2 ties at key lo, 3 take all, 4 none
  int budget;
  long long load;     // group load before augmentation
};

__device__ __forceinline__ int group_of(int h, int R, int BH) { return (int)(((long long)h * R) / BH); }

// Radix passes over the candidates' keys use 11-bit digits (2048 bins): a key range of the
// whole [0, 1] (62 bits wide) resolves in at most 6 passes.
constexpr int kSasaBits = 11, kSasaBins = 1 << kSasaBits;
constexpr int kSasaPasses = (62 + kSasaBits - 1) / kSasaBits;

__device__ __forceinline__ int sasa_shift(unsigned long long width) {
  const unsigned long long wm1 = width - 1ull;
  return wm1 < (unsigned long long)kSasaBins ? 0 : 64 - __clzll((long long)wm1) - kSasaBits;
}

// One workgroup: group loads, critical path, budgets.
__global__ __launch_bounds__(1024) void k_sasa_init(const int32_t *__restrict__ head_load, int BH, int R,
                                                    int critical_in, double alpha, double tau, int nqb, int nkb,
                                                    SasaGroup *__restrict__ grp, uint32_t *__restrict__ ghist,
                                                    int32_t *__restrict__ added_out) {
  __shared__ long long s_load[1024];
  __shared__ int s_heads[1024];
  __shared__ long long s_crit;
  const int tid = threadIdx.x;
  for (int g = tid; g < R; g += 1024) {
    s_load[g] = 0;
    s_heads[g] = 0;
  }
  __syncthreads();
  for (int h = tid; h < BH; h += 1024) {
    const int g = group_of(h, R, BH);
    atomicAdd((unsigned long long *)&s_load[g], (unsigned long long)head_load[h]);
    atomicAdd(&s_heads[g], 1);
  }
  __syncthreads();
  if (tid == 0) {
    long long m = 0;
    for (int g = 0; g < R; ++g) m = s_load[g] > m ? s_load[g] : m;
    s_crit = critical_in > 0 ? (long long)critical_in : m;
  }
  __syncthreads();
  const long long crit = s_crit;
  for (int g = tid; g < R; g += 1024) {
    const long long L = s_load[g];
    const long long slack = crit - L;
    long long budget = 0;
    if (slack > 0 && (double)slack >= tau * (double)crit) budget = (long long)floor(alpha * (double)slack);
    const long long cands = (long long)s_heads[g] * nqb * nkb - L;
    if (budget > cands) budget = cands;
    SasaGroup G;
    G.lo = 0;
    G.width = (unsigned long long)__double_as_longlong(1.0) + 1ull;   // every P in [0, 1]
    G.above = 0;
    G.target = (unsigned long long)budget;
    G.state = budget <= 0 ? 4 : (budget == cands ? 3 : 0);
    G.budget = (int)budget;
    G.load = L;
    grp[g] = G;
    if (added_out != nullptr) added_out[g] = (int)budget;
  }
  for (size_t b = tid; b < (size_t)R * kSasaBins; b += 1024) ghist[b] = 0;
}

// grid = (cdiv(nqb, kRowsPerWg), BH), 256 threads: rows [i0, i0 + kRowsPerWg) of head bh.
constexpr int kRowsPerWg = 8;

__global__ __launch_bounds__(256) void k_sasa_hist(const double *__restrict__ imp, const uint32_t *__restrict__ bitmask,
                                                   int nkw, int nqb, int nkb, int R, int BH,
                                                   const SasaGroup *__restrict__ grp, uint32_t *__restrict__ ghist) {
  __shared__ uint32_t h[kSasaBins];
  const int bh = blockIdx.y, g = group_of(bh, R, BH);
  const SasaGroup G = grp[g];
  if (G.state != 0) return;   // uniform over the workgroup
  const int tid = threadIdx.x;
  for (int b = tid; b < kSasaBins; b += 256) h[b] = 0;
  __syncthreads();
  const int sh = sasa_shift(G.width);
  const int i0 = blockIdx.x * kRowsPerWg, i1 = min(i0 + kRowsPerWg, nqb);
  for (int i = i0; i < i1; ++i) {
    const size_t row = (size_t)bh * nqb + i;
    for (int j = tid; j < nkb; j += 256) {
      if ((bitmask[row * nkw + (j >> 5)] >> (j & 31)) & 1u) continue;   // already kept
      const unsigned long long key = (unsigned long long)__double_as_longlong(imp[row * nkb + j]);
      const unsigned long long off = key - G.lo;
      if (off < G.width) atomicAdd(&h[(int)(off >> sh)], 1u);
    }
  }
  __syncthreads();
  for (int b = tid; b < kSasaBins; b += 256)
    if (h[b] != 0) atomicAdd(&ghist[(size_t)g * kSasaBins + b], h[b]);
}

// One wave per group: find the bin where the count from the top reaches the budget (lane l
// holds bins 32 l .. 32 l + 31).
__global__ __launch_bounds__(256) void k_sasa_resolve(int R, SasaGroup *__restrict__ grp, uint32_t *__restrict__ ghist) {
  constexpr int PL = kSasaBins / 64;   // bins per lane
  const int lane = threadIdx.x & 63;
  const int g = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (g >= R) return;
  SasaGroup G = grp[g];
  if (G.state != 0) return;   // uniform over the wave
  uint32_t c[PL];
  unsigned long long cs = 0;
  uint32_t *hg = ghist + (size_t)g * kSasaBins + PL * lane;
#pragma unroll
  for (int q = 0; q < PL; ++q) {
    c[q] = hg[q];
    cs += c[q];
  }
  unsigned long long sm = cs;   // inclusive suffix sum over lanes (higher lanes: larger keys)
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned long long o = __shfl_down(sm, off);
    if (lane + off < 64) sm += o;
  }
  unsigned long long above = sm - cs;
  const int sh = sasa_shift(G.width);
#pragma unroll
  for (int q = PL - 1; q >= 0; --q) {
    const unsigned long long lo = G.above + above;
    if (c[q] > 0 && lo < G.target && G.target <= lo + c[q]) {
      SasaGroup N = G;
      N.above = lo;
      N.lo = G.lo + ((unsigned long long)(PL * lane + q) << sh);
      N.width = 1ull << sh;
      if (c[q] == 1) N.state = 1;
      else if (sh == 0) N.state = 2;
      grp[g] = N;
    }
    above += c[q];
  }
#pragma unroll
  for (int q = 0; q < PL; ++q) hg[q] = 0;   // ready for the next pass
}

// One wave per row: candidates equal to the group's threshold key (state 2).
__global__ __launch_bounds__(256) void k_sasa_ties(const double *__restrict__ imp, const uint32_t *__restrict__ bitmask,
                                                   int nkw, int nqb, int nkb, int R, int BH,
                                                   const SasaGroup *__restrict__ grp, int32_t *__restrict__ tiecnt) {
  const int lane = threadIdx.x & 63;
  const int bh = blockIdx.y, i = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= nqb) return;
  const size_t row = (size_t)bh * nqb + i;
  const SasaGroup G = grp[group_of(bh, R, BH)];
  int c = 0;
  if (G.state == 2) {
    for (int j = lane; j < nkb; j += 64) {
      const bool kept = (bitmask[row * nkw + (j >> 5)] >> (j & 31)) & 1u;
      const unsigned long long key = (unsigned long long)__double_as_longlong(imp[row * nkb + j]);
      c += (!kept && key == G.lo);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) c += __shfl_xor(c, off);
  }
  if (lane == 0) tiecnt[row] = c;
}

// One workgroup per group in state 2: exclusive running count of ties over the group's rows
// (heads of a group are contiguous, so are their rows).
__global__ __launch_bounds__(1024) void k_sasa_tiescan(const int32_t *__restrict__ tiecnt, int nqb, int R, int BH,
                                                       const SasaGroup *__restrict__ grp, int32_t *__restrict__ tiepre) {
  __shared__ int s_scan[1024];
  __shared__ int s_run;
  const int g = blockIdx.x, tid = threadIdx.x;
  if (grp[g].state != 2) return;
  // rows of group g: heads h with h*R/BH == g
  const int h0 = (int)(((long long)g * BH + R - 1) / R), h1 = (int)(((long long)(g + 1) * BH + R - 1) / R);
  const size_t r0 = (size_t)h0 * nqb, r1 = (size_t)h1 * nqb;
  if (tid == 0) s_run = 0;
  __syncthreads();
  for (size_t base = r0; base < r1; base += 1024) {
    const size_t row = base + tid;
    const int v = row < r1 ? tiecnt[row] : 0;
    s_scan[tid] = v;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int o = tid >= off ? s_scan[tid - off] : 0;
      __syncthreads();
      s_scan[tid] += o;
      __syncthreads();
    }
    if (row < r1) tiepre[row] = s_run + s_scan[tid] - v;
    __syncthreads();
    if (tid == 1023) s_run += s_scan[1023];
    __syncthreads();
  }
}

// One wave per row: add the selected candidates.
__global__ __launch_bounds__(256) void k_sasa_mark(const double *__restrict__ imp, uint32_t *__restrict__ bitmask,
                                                   int nkw, int nqb, int nkb, int R, int BH,
                                                   const SasaGroup *__restrict__ grp, const int32_t *__restrict__ tiepre,
                                                   int32_t *__restrict__ counts, int32_t *__restrict__ head_load,
                                                   int32_t *__restrict__ bsum) {
  __shared__ int s_add[4];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int bh = blockIdx.y, i = blockIdx.x * 4 + w;
  const SasaGroup G = grp[group_of(bh, R, BH)];
  if (G.state == 4) return;   // uniform over the workgroup (one head)
  int added = 0;
  if (i < nqb) {   // wave-uniform
    const size_t row = (size_t)bh * nqb + i;
    const unsigned long long need = G.target - G.above;   // ties to take (state 2)
    unsigned long long rank = G.state == 2 ? (unsigned long long)tiepre[row] : 0ull;
    // lane L holds words L and L + 64 of the row's kept mask (up to 4096 key blocks); the chunk
    // of key blocks 64c .. 64c+63 is words 2c and 2c + 1, in register c / 32 of lanes 2c % 64 and
    // 2c % 64 + 1
    uint32_t word[2], word0[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      word[q] = lane + 64 * q < nkw ? bitmask[row * nkw + lane + 64 * q] : 0u;
      word0[q] = word[q];
    }
    for (int j0 = 0; j0 < nkb; j0 += 64) {
      const int j = j0 + lane;
      const int q = j0 >> 11, wl = (j0 >> 5) & 63;   // register and first lane of this chunk
      const uint32_t src = (uint32_t)__shfl((int)(q ? word0[1] : word0[0]), wl + (lane >> 5));
      const bool kept = (src >> (j & 31)) & 1u;
      bool add = false, tie = false;
      if (j < nkb && !kept) {
        const unsigned long long key = (unsigned long long)__double_as_longlong(imp[row * nkb + j]);
        if (G.state == 3) add = true;
        else if (G.state == 1) add = key >= G.lo;
        else {   // state 2: strictly above the tie key, or a tie within the remaining need
          tie = key == G.lo;
          add = key > G.lo;
        }
      }
      if (G.state == 2) {
        const unsigned long long tb = __ballot(tie);
        const unsigned long long below = tb & ((1ull << lane) - 1ull);
        if (tie && rank + (unsigned long long)__popcll(below) < need) add = true;
        rank += (unsigned long long)__popcll(tb);
      }
      const unsigned long long ab = __ballot(add);
      added += __popcll(ab);
      if (lane == wl) word[q] |= (uint32_t)ab;
      if (lane == wl + 1) word[q] |= (uint32_t)(ab >> 32);
    }
#pragma unroll
    for (int q = 0; q < 2; ++q)
      if (lane + 64 * q < nkw && word[q] != word0[q]) bitmask[row * nkw + lane + 64 * q] = word[q];
    if (lane == 0 && added > 0) counts[row] += added;
  }
  // the workgroup's four rows: one load update for the head, at most two per-64-row sums
  if (lane == 0) s_add[w] = added;
  __syncthreads();
  if (threadIdx.x == 0) {
    const size_t row0 = (size_t)bh * nqb + blockIdx.x * 4;
    int tot = 0, c0 = 0, c1 = 0;
    for (int r = 0; r < 4; ++r) {
      tot += s_add[r];
      if (((row0 + r) >> 6) == (row0 >> 6)) c0 += s_add[r];
      else c1 += s_add[r];
    }
    if (tot > 0) atomicAdd(&head_load[bh], tot);
    if (c0 > 0) atomicAdd(&bsum[row0 >> 6], c0);
    if (c1 > 0) atomicAdd(&bsum[(row0 >> 6) + 1], c1);
  }
}

size_t sasa_group_bytes(int R) { return (size_t)R * sizeof(SasaGroup); }
size_t sasa_hist_bytes(int R) { return (size_t)R * kSasaBins * sizeof(uint32_t); }

int launch_sasa(const double *imp, uint32_t *bitmask, int32_t *counts, int32_t *bsum, int32_t *head_load, int nkw,
                int nqb, int nkb, int BH, int R, int critical, double alpha, double tau, void *grp_buf,
                uint32_t *ghist, int32_t *tiecnt, int32_t *tiepre, int32_t *added_out, hipStream_t st) {
  SasaGroup *grp = (SasaGroup *)grp_buf;
  hipLaunchKernelGGL(k_sasa_init, dim3(1), dim3(1024), 0, st, head_load, BH, R, critical, alpha, tau, nqb, nkb, grp,
                     ghist, added_out);
  FV_CHECK_LAUNCH();
  const dim3 gh(cdiv(nqb, kRowsPerWg), BH), gr(cdiv(R, 4)), gw(cdiv(nqb, 4), BH);
  for (int pass = 0; pass < kSasaPasses; ++pass) {
    hipLaunchKernelGGL(k_sasa_hist, gh, dim3(256), 0, st, imp, bitmask, nkw, nqb, nkb, R, BH, grp, ghist);
    FV_CHECK_LAUNCH();
    hipLaunchKernelGGL(k_sasa_resolve, gr, dim3(256), 0, st, R, grp, ghist);
    FV_CHECK_LAUNCH();
  }
  hipLaunchKernelGGL(k_sasa_ties, gw, dim3(256), 0, st, imp, bitmask, nkw, nqb, nkb, R, BH, grp, tiecnt);
  FV_CHECK_LAUNCH();
  hipLaunchKernelGGL(k_sasa_tiescan, dim3(R), dim3(1024), 0, st, tiecnt, nqb, R, BH, grp, tiepre);
  FV_CHECK_LAUNCH();
  hipLaunchKernelGGL(k_sasa_mark, gw, dim3(256), 0, st, imp, bitmask, nkw, nqb, nkb, R, BH, grp, tiepre, counts,
                     head_load, bsum);
  FV_CHECK_LAUNCH();
  return FVATTN_OK;
}

}  // namespace fv
