// Top-p routing on gfx950: block mean-pooling, pooled block scores, softmax over key
// blocks, descending order with ties to the lower index, cut at cumulative mass >= p,
// and compaction into a CSR of kept key blocks with per-head loads.
//
// Method: FVAttn summary page (PaperDaily, arXiv:2607.16190), Top-p routing paragraph of
// section "AI视频生成的阿喀琉斯之踵"; pooled scores with 1/sqrt(d): tutorial page, section 5.2.
//
// Design (gfx950):
//  * k_pool      HBM-bound pass over Q or K: each workgroup streams whole blocks with 16-byte
//                loads, accumulates in float64 (the mean of a block of bf16 values is then
//                exact up to the final division), and writes the pooled rows in the lane
//                order the float64 MFMA of k_select consumes (one 512-byte load per operand).
//  * k_select    one workgroup = 16 query blocks of one head, 4 waves.  Scores
//                qbar.kbar^T/sqrt(d) come from v_mfma_f64_16x16x4 and stay in registers
//                (wave w holds key tiles w, w+4, ...).  Softmax numerators e = exp(s - max)
//                in float64; masses as 2^-52 fixed point so every partial sum is exact and
//                order independent.  The descending order is never materialised: a radix
//                select over the float64 bit pattern of e (monotone for e >= 0) splits the
//                row's key range [e_min, 1] into 256 bins, walks the mass histogram from the
//                largest bin down, stops at the bin where the cumulative mass crosses p * Z,
//                and refines that bin the same way until one key remains.  That gives exactly the shortest
//                prefix of the (e descending, index ascending) order with mass >= p: elements
//                above the threshold key are all kept, and among keys equal to the threshold
//                the lowest indices are taken first.
//  * k_csr       exclusive scan of per-row counts (each workgroup sums the counts before its
//                range itself, no second pass) and expansion of the kept-bit masks into
//                ascending column indices.
#include "common.h"

namespace fv {

// Swizzled index of pooled element (block j, dim c) for the f64 MFMA operand layout:
// lane l of 16x16x4 supplies row (l % 16) and k-index (l / 16).
__device__ __forceinline__ size_t swz(int bh, int ngroups, int D, int j, int c) {
  return ((size_t)(bh * ngroups + (j >> 4)) * (D / 4) + (c >> 2)) * 64 + (j & 15) + 16 * (c & 3);
}

// ---------------------------------------------------------------------------------------
// k_pool: x [BH][N][D] -> mean of every block of `block` tokens (real tokens only), for one
// or two tensors (Q and K) in one launch.  Item = 16 consecutive blocks of one head of one
// tensor; grid = (groups of tensor 0 + groups of tensor 1, BH), 256 threads.  Wave w pools
// blocks w, w+4, w+8, w+12 of the group: lane l reads 16-byte chunk l % CPR of rows
// l / CPR + RPL*i (16 loads in flight per lane), accumulates in float64 and the lanes of a
// chunk are summed with cross-lane shuffles.  The 16 pooled rows are staged in LDS and
// written as one contiguous run: layout 1 is the swizzled float64 MFMA operand order of
// k_select (blocks past nb written as zero), layout 0 the plain [BH][nb][D] array.
// ---------------------------------------------------------------------------------------
struct PoolArgs {
  const void *x[2];
  double *out[2];
  int block[2], nb[2], ngrp[2];   // ngrp = ceil(nb / 16); ngrp[1] = 0 for one tensor
  int N, layout;
  int32_t *zero[2];               // zeroed by workgroup (0, 0) (may be null)
  int nzero[2];
};

template <typename T, int D>
__global__ __launch_bounds__(256) void k_pool(PoolArgs a) {
  constexpr int EPC = DT<T>::per16;   // elements per 16-byte chunk
  constexpr int CPR = D / EPC;        // chunks per row
  constexpr int RPL = 64 / CPR;       // rows covered by one wave-wide load
  constexpr int NLD = 16;             // loads in flight per lane
  constexpr int RPR = RPL * NLD;      // rows per round
  __shared__ double stage[16][D + 1];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int bh = blockIdx.y;
  int gx = blockIdx.x;
  const int t = gx < a.ngrp[0] ? 0 : 1;
  if (t) gx -= a.ngrp[0];
  if (blockIdx.x == 0 && bh == 0) {
    for (int z = 0; z < 2; ++z)
      if (a.zero[z] != nullptr)
        for (int i = tid; i < a.nzero[z]; i += 256) a.zero[z][i] = 0;
  }
  const T *xh = reinterpret_cast<const T *>(a.x[t]) + (size_t)bh * a.N * D;
  const int block = a.block[t], nb = a.nb[t], N = a.N;
  const int c = lane % CPR, r = lane / CPR;

  for (int jj = w; jj < 16; jj += 4) {
    const int j = gx * 16 + jj;
    double acc[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] = 0.0;
    int cnt = 1;
    if (j < nb) {
      const int s0 = j * block, e0 = min(s0 + block, N);
      cnt = e0 - s0;
      for (int base = s0; base < e0; base += RPR) {
        u32x4 buf[NLD];
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
          const int row = base + r + RPL * i;
          buf[i] = u32x4{0u, 0u, 0u, 0u};
          if (row < e0) buf[i] = *reinterpret_cast<const u32x4 *>(xh + (size_t)row * D + c * EPC);
        }
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
          float f[EPC];
          unpack16(buf[i], f, T());
#pragma unroll
          for (int e = 0; e < EPC; ++e) acc[e] += (double)f[e];
        }
      }
    }
#pragma unroll
    for (int off = CPR; off < 64; off <<= 1)
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[e] += __shfl_xor(acc[e], off);
    if (r == 0) {
#pragma unroll
      for (int e = 0; e < EPC; ++e) stage[jj][c * EPC + e] = (j < nb) ? acc[e] / (double)cnt : 0.0;
    }
  }
  __syncthreads();
  double *out = a.out[t];
  if (a.layout) {
    // region of (bh, group): element (block jj, dim c) at (c/4)*64 + jj + 16*(c%4)
    double *dst = out + ((size_t)bh * a.ngrp[t] + gx) * (D / 4) * 64;
    for (int idx = tid; idx < 16 * D; idx += 256) {
      const int jj = idx & 15, cc = ((idx >> 6) << 2) | ((idx >> 4) & 3);
      dst[idx] = stage[jj][cc];
    }
  } else {
    const int nrows = min(16, nb - gx * 16);
    double *dst = out + ((size_t)bh * nb + gx * 16) * D;
    for (int idx = tid; idx < nrows * D; idx += 256) dst[idx] = stage[idx / D][idx % D];
  }
}

// ---------------------------------------------------------------------------------------
// k_select: scores, softmax, Top-p cut for 16 query blocks of one head per item.
// Persistent: grid = min(resident workgroups, items), at least 8; 256 threads.
// MAXT = key tiles (of 16) per wave.
// Outputs counts[row] and the kept-bit mask bitmask[row][nkw]; adds loads to head_load.
// ---------------------------------------------------------------------------------------
constexpr int kMaxNkw = 40;  // 1280 key blocks

// Routing variant of k_select (see fvattn_route_opts): mode, top-k count, clamp of the Top-p
// count, local window, and the block geometry the window needs.
struct SelOpts {
  int mode, topk, k_min, k_max, window, bq, bk, N;
  double *imp;   // optional [rows][nkb]: importance P of every block (SASA candidates); EXT only
};


// NWV waves per workgroup (4, or 8 for more than 512 key blocks): wave w holds key tiles
// w, w + NWV, ... (MAXT of them).  EXT: routing variants (count searches, clamp, window).
template <int D, int MAXT, int NWV, bool EXT>
__global__ __launch_bounds__(64 * NWV, NWV == 4 ? 2 : 1) void k_select(const double *__restrict__ qsw,
                                                const double *__restrict__ ksw, int nqb, int nkb,
                                                double scale, double p, int32_t *__restrict__ counts,
                                                uint32_t *__restrict__ bitmask, int nkw,
                                                int32_t *__restrict__ head_load, int32_t *__restrict__ bsum,
                                                int BH, SelOpts sel) {
  constexpr int KS = D / 4;  // MFMA k-steps
  __shared__ uint32_t h_cnt[16][256];
  __shared__ unsigned long long h_mass[16][256];
  __shared__ uint32_t s_kept[16][kMaxNkw];
  __shared__ uint32_t s_ties[16][kMaxNkw];
  __shared__ double s_part[NWV][16];
  __shared__ unsigned long long s_zpart[NWV][16];
  __shared__ unsigned long long s_lo[16], s_width[16], s_above[16], s_target[16];
  __shared__ double s_minpart[NWV][16];
  __shared__ int s_state[16];   // 0 searching, 1 unique threshold, 2 ties, 3 keep all, 4 final
  __shared__ int s_bycnt[16];   // search by count instead of mass
  __shared__ unsigned long long s_lo0[16];
  __shared__ double s_invz[16];     // 1 / Z (importance P = e / Z)
  __shared__ uint32_t s_selcnt[16];
  __shared__ int s_any;

  constexpr int NT = 64 * NWV;      // threads
  constexpr int RPW = 16 / NWV;     // rows resolved per wave
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nqg = (nqb + 15) >> 4;
  const int nkt = (nkb + 15) >> 4;

  // Persistent loop over items (head bh, group g of 16 query blocks).  Workgroup b runs on
  // XCD b % 8 (round-robin dispatch); XCD x owns the x-th eighth of the items in head-major
  // order, so its L2 holds the pooled keys of only a few heads.  gridDim.x >= 8.
  const int items = BH * nqg;
  const int xcd = blockIdx.x & 7;
  const int nwx = ((int)gridDim.x - xcd + 7) >> 3;
  const int it_end = (int)((long long)items * (xcd + 1) / 8);
  for (int it = (int)((long long)items * xcd / 8) + (int)(blockIdx.x >> 3); it < it_end; it += nwx) {
  const int bh = it / nqg, g = it - bh * nqg;

  // ---- scores: S[i][j] = sum_c qbar[i][c] * kbar[j][c], i = lane/16 + 4v, j = 16t + lane%16
  d4 acc[MAXT];
#pragma unroll
  for (int k = 0; k < MAXT; ++k) acc[k] = d4{0.0, 0.0, 0.0, 0.0};
  {
    const double *qa = qsw + ((size_t)(bh * nqg + g) * KS) * 64 + lane;
    // k-step outer, tiles inner: MAXT independent accumulators, and the operands of step s+1
    // (one of qbar, MAXT of kbar) are in flight while step s runs.  Tiles past the last read a
    // valid tile (their key columns are >= nkb and ignored below), so the loop has no branches.
    const double *kb[MAXT];
#pragma unroll
    for (int k = 0; k < MAXT; ++k) kb[k] = ksw + ((size_t)(bh * nkt + min(w + NWV * k, nkt - 1)) * KS) * 64 + lane;
    double acur = qa[0], bcur[MAXT];
#pragma unroll
    for (int k = 0; k < MAXT; ++k) bcur[k] = kb[k][0];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      double anxt = 0.0, bnxt[MAXT];
      if (s + 1 < KS) {
        anxt = qa[(s + 1) * 64];
#pragma unroll
        for (int k = 0; k < MAXT; ++k) bnxt[k] = kb[k][(s + 1) * 64];
      }
#pragma unroll
      for (int k = 0; k < MAXT; ++k) acc[k] = __builtin_amdgcn_mfma_f64_16x16x4f64(acur, bcur[k], acc[k], 0, 0, 0);
      if (s + 1 < KS) {
        acur = anxt;
#pragma unroll
        for (int k = 0; k < MAXT; ++k) bcur[k] = bnxt[k];
      }
    }
  }

  // ---- row max over valid keys
  const int jl = lane & 15, ig = lane >> 4;
  double mx[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) mx[v] = -INFINITY;
#pragma unroll
  for (int k = 0; k < MAXT; ++k) {
    const int j = 16 * (w + NWV * k) + jl;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      acc[k][v] *= scale;
      if (j < nkb) mx[v] = fmax(mx[v], acc[k][v]);
    }
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) {
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) mx[v] = fmax(mx[v], __shfl_xor(mx[v], off, 16));
    if (jl == 0) s_part[w][ig + 4 * v] = mx[v];
  }
  __syncthreads();
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int r = ig + 4 * v;
    double m = s_part[0][r];
#pragma unroll
    for (int ww = 1; ww < NWV; ++ww) m = fmax(m, s_part[ww][r]);
    mx[v] = m;
  }

  // ---- e = exp(s - max) (in place), fixed-point masses, Z
  constexpr double kFix = 4503599627370496.0;  // 2^52
  unsigned long long zs[4] = {0, 0, 0, 0};
  double mn[4] = {1.0, 1.0, 1.0, 1.0};
#pragma unroll
  for (int k = 0; k < MAXT; ++k) {
    const int j = 16 * (w + NWV * k) + jl;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const double e = (j < nkb) ? exp(acc[k][v] - mx[v]) : 0.0;
      acc[k][v] = e;
      zs[v] += (unsigned long long)(e * kFix);
      if (j < nkb) mn[v] = fmin(mn[v], e);
    }
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) {
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) {
      zs[v] += __shfl_xor(zs[v], off, 16);
      mn[v] = fmin(mn[v], __shfl_xor(mn[v], off, 16));
    }
    if (jl == 0) {
      s_zpart[w][ig + 4 * v] = zs[v];
      s_minpart[w][ig + 4 * v] = mn[v];
    }
  }
  __syncthreads();
  // ---- per-row selection setup.  A row searches by mass (Top-p: the shortest prefix of the
  // descending order whose mass reaches p Z) or by count (top-k, or a clamped Top-p count):
  // the same radix walk over mass or count histograms.
  if (tid < 16) {
    const int r = tid;
    unsigned long long Z = 0;
    double emin = 1.0;
    for (int ww = 0; ww < NWV; ++ww) {
      Z += s_zpart[ww][r];
      emin = fmin(emin, s_minpart[ww][r]);
    }
    // search range of keys (float64 bit patterns of e, monotone for e >= 0): [e_min, 1.0]
    const unsigned long long lo = (unsigned long long)__double_as_longlong(emin);
    const bool live = (16 * g + r) < nqb;
    unsigned long long T;
    int st;
    if (EXT && sel.mode == FVATTN_ROUTE_TOPK) {
      T = (unsigned long long)sel.topk;
      st = (!live || sel.topk >= nkb) ? 3 : 0;
      s_bycnt[r] = 1;
    } else {
      T = (unsigned long long)ceil(p * (double)Z);
      if (T > Z) T = Z;
      if (T < 1) T = 1;
      st = (!live || p >= 1.0) ? 3 : 0;
      s_bycnt[r] = 0;
    }
    s_target[r] = T;
    s_lo0[r] = lo;
    if (EXT) s_invz[r] = Z > 0 ? 4503599627370496.0 / (double)Z : 0.0;   // 2^52 / fixed-point Z
    s_lo[r] = lo;
    s_width[r] = (unsigned long long)__double_as_longlong(1.0) + 1ull - lo;
    s_above[r] = 0;
    s_selcnt[r] = 0;
    s_state[r] = st;
  }
  __syncthreads();

  // Round 0 selects; with a clamp on the Top-p count, round 1 re-selects by count the rows
  // whose kept count lies outside [k_min, k_max] (other rows are final: state 4).
  const bool clamp = EXT && sel.mode != FVATTN_ROUTE_TOPK && (sel.k_min > 1 || sel.k_max > 0);
  for (int round = 0; round < (EXT ? 2 : 1); ++round) {
    // ---- radix select over the key range [lo, lo + width): each pass splits the range into
    // 256 equal digit bins (log-linear in e), finds the bin where the cumulative mass (or
    // count) from the top crosses the target, and narrows the range to that bin.  The first
    // range spans the row's own [e_min, 1], so elements spread over the bins.
  for (int pass = 0; pass < 8; ++pass) {
    if (tid == 0) {
      int any = 0;
      for (int r = 0; r < 16; ++r) any |= (s_state[r] == 0);
      s_any = any;
    }
    for (int i = tid; i < 16 * 256; i += NT) {
      (&h_cnt[0][0])[i] = 0;
      (&h_mass[0][0])[i] = 0;
    }
    __syncthreads();
    if (!s_any) break;
    unsigned long long rlo[4], rw[4];
    int rsh[4];
    bool act[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = ig + 4 * v;
      rlo[v] = s_lo[r];
      rw[v] = s_width[r];
      rsh[v] = digit_shift(rw[v]);
      act[v] = s_state[r] == 0;
    }
#pragma unroll
    for (int k = 0; k < MAXT; ++k) {
      const int j = 16 * (w + NWV * k) + jl;
      if (j < nkb) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const unsigned long long off = (unsigned long long)__double_as_longlong(acc[k][v]) - rlo[v];
          if (act[v] && off < rw[v]) {
            const int dg = (int)(off >> rsh[v]);
            const int r = ig + 4 * v;
            atomicAdd(&h_cnt[r][dg], 1u);
            atomicAdd(&h_mass[r][dg], (unsigned long long)(acc[k][v] * kFix));
          }
        }
      }
    }
    __syncthreads();
    // wave w resolves rows 4w .. 4w+3: find the digit where the mass crosses the target
    for (int rr = 0; rr < RPW; ++rr) {
      const int r = RPW * w + rr;
      if (s_state[r] != 0) continue;  // uniform across the wave
      // the walk runs over masses (Top-p) or counts (top-k, clamped count)
      const bool bc = EXT && s_bycnt[r] != 0;
      unsigned long long m4[4];
      uint32_t c4[4];
      unsigned long long ms = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        c4[q] = h_cnt[r][4 * lane + q];
        m4[q] = bc ? (unsigned long long)c4[q] : h_mass[r][4 * lane + q];
        ms += m4[q];
      }
      // exclusive suffix sums over lanes (higher lanes hold larger digits)
      unsigned long long sm = ms;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const unsigned long long om = __shfl_down(sm, off);
        if (lane + off < 64) sm += om;
      }
      unsigned long long above_m = sm - ms;  // mass of digits held by higher lanes
      const unsigned long long base = s_above[r];
      const unsigned long long T = s_target[r];
      const unsigned long long lo0 = s_lo[r], w0 = s_width[r];
      const int sh = digit_shift(w0);
      for (int q = 3; q >= 0; --q) {
        const unsigned long long lo = base + above_m;
        if (m4[q] > 0 && lo < T && T <= lo + m4[q]) {
          s_above[r] = lo;
          s_lo[r] = lo0 + ((unsigned long long)(4 * lane + q) << sh);
          s_width[r] = 1ull << sh;
          s_selcnt[r] = c4[q];
          if (c4[q] == 1) s_state[r] = 1;         // the threshold block is unique
          else if (sh == 0) s_state[r] = 2;       // several blocks share the threshold key
        }
        above_m += m4[q];
      }
    }
    __syncthreads();
  }

  // ---- mark kept blocks
  for (int i = tid; i < 16 * kMaxNkw; i += NT) {
    if (s_state[i / kMaxNkw] == 4) continue;   // final from the previous round
    (&s_kept[0][0])[i] = 0;
    (&s_ties[0][0])[i] = 0;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < MAXT; ++k) {
    const int j = 16 * (w + NWV * k) + jl;
    if (j < nkb) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = ig + 4 * v;
        const int st = s_state[r];
        if (st == 4) continue;
        const unsigned long long key = (unsigned long long)__double_as_longlong(acc[k][v]);
        const unsigned long long lo = s_lo[r], hi = lo + s_width[r];
        const uint32_t bit = 1u << (j & 31);
        const bool in_range = key >= lo && key < hi;
        if (st == 3 || key >= hi || (in_range && st == 1))
          atomicOr(&s_kept[r][j >> 5], bit);
        else if (in_range && st == 2)
          atomicOr(&s_ties[r][j >> 5], bit);
      }
    }
  }
  __syncthreads();
  // ties (identical importance): the lowest indices first, as many as the mass requires.
  // Every tied element has the same fixed-point mass; any holder publishes it.
  __shared__ unsigned long long s_mt[16];
#pragma unroll
  for (int k = 0; k < MAXT; ++k) {
    const int j = 16 * (w + NWV * k) + jl;
    if (j < nkb) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = ig + 4 * v;
        if (s_state[r] == 2 && (s_ties[r][j >> 5] >> (j & 31) & 1u))
          s_mt[r] = (unsigned long long)(acc[k][v] * kFix);  // identical for all ties
      }
    }
  }
  __syncthreads();
  for (int rr = 0; rr < RPW; ++rr) {
    const int r = RPW * w + rr;
    if (s_state[r] != 2) continue;
    const unsigned long long rem = s_target[r] - s_above[r];
    const unsigned long long mt = s_mt[r];
    const uint32_t ntie = s_selcnt[r];
    uint32_t need;
    if (EXT && s_bycnt[r])
      need = (uint32_t)min((unsigned long long)ntie, rem);   // count search: rem blocks
    else
      need = (mt == 0) ? ntie : (uint32_t)min((unsigned long long)ntie, (rem + mt - 1) / mt);
    uint32_t word = lane < nkw ? s_ties[r][lane] : 0u;
    const uint32_t pc = __popc(word);
    uint32_t incl = pc;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    const uint32_t excl = incl - pc;
    if (lane < nkw && excl < need) {
      uint32_t take = need - excl;
      uint32_t keep = 0, wd = word;
      while (wd && take) {
        const uint32_t b = wd & (0u - wd);
        keep |= b;
        wd ^= b;
        --take;
      }
      s_kept[r][lane] |= keep;
    }
  }
  __syncthreads();


  if constexpr (EXT) {
  if (!clamp || round == 1) break;
  for (int rr = 0; rr < RPW; ++rr) {
    const int r = RPW * w + rr;
    uint32_t word = lane < nkw ? s_kept[r][lane] : 0u;
    int c = __popc(word);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) c += __shfl_xor(c, off);
    if (lane == 0) {
      int tgt = max(c, sel.k_min);
      if (sel.k_max > 0) tgt = min(tgt, sel.k_max);
      tgt = min(tgt, nkb);
      if ((16 * g + r) < nqb && tgt != c) {
        s_bycnt[r] = 1;
        s_target[r] = (unsigned long long)tgt;
        s_lo[r] = s_lo0[r];
        s_width[r] = (unsigned long long)__double_as_longlong(1.0) + 1ull - s_lo0[r];
        s_above[r] = 0;
        s_selcnt[r] = 0;
        s_state[r] = tgt >= nkb ? 3 : 0;
      } else {
        s_state[r] = 4;
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    int any = 0;
    for (int r = 0; r < 16; ++r) any |= (s_state[r] != 4);
    s_any = any;
  }
  __syncthreads();
  if (!s_any) break;
  }
  }   // rounds

  if constexpr (EXT) {
    // importance of every block of the live rows: the candidates' order for SASA
    if (sel.imp != nullptr) {
#pragma unroll
      for (int k = 0; k < MAXT; ++k) {
        const int j = 16 * (w + NWV * k) + jl;
        if (j < nkb) {
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int r = ig + 4 * v;
            const int i = 16 * g + r;
            if (i < nqb) sel.imp[((size_t)bh * nqb + i) * nkb + j] = acc[k][v] * s_invz[r];
          }
        }
      }
    }
  }

  // ---- write counts, masks, loads (wave w: rows 4w..4w+3)
  for (int rr = 0; rr < RPW; ++rr) {
    const int r = RPW * w + rr;
    const int i = 16 * g + r;
    if (i >= nqb) continue;
    const size_t row = (size_t)bh * nqb + i;
    uint32_t word = lane < nkw ? s_kept[r][lane] : 0u;
    if (EXT && sel.window > 0 && lane < nkw) {
      // local window: key blocks within `window` of those overlapping the query block's tokens
      const int t0 = i * sel.bq, t1 = min(t0 + sel.bq, sel.N) - 1;
      const int ja = max(0, t0 / sel.bk - sel.window), jb = min(nkb - 1, t1 / sel.bk + sel.window);
      const int lo_j = max(ja, 32 * lane), hi_j = min(jb, 32 * lane + 31);
      if (lo_j <= hi_j) {
        const int nbits = hi_j - lo_j + 1;
        word |= (nbits == 32 ? 0xffffffffu : ((1u << nbits) - 1u)) << (lo_j - 32 * lane);
      }
    }
    if (lane < nkw) bitmask[row * nkw + lane] = word;
    int c = __popc(word);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) c += __shfl_xor(c, off);
    if (lane == 0) {
      counts[row] = c;
      atomicAdd(&head_load[bh], c);
      atomicAdd(&bsum[row >> 6], c);   // per-64-row sums for the CSR scan
    }
  }
  __syncthreads();   // LDS of this item fully consumed before the next item writes it
  }
}

// ---------------------------------------------------------------------------------------
// k_csr: row_ptr (exclusive scan of counts) and ascending col_idx from the kept masks.
// grid = cdiv(rows, 64), 256 threads: workgroup b owns rows [64b, 64b + 64); its offset is
// the sum of the per-64-row sums before it.  Each wave expands 16 rows, 64 key blocks per
// step: a ballot of the kept bits gives every kept block its output slot (coalesced writes).
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_csr(const int32_t *__restrict__ counts,
                                             const uint32_t *__restrict__ bitmask,
                                             const int32_t *__restrict__ bsum, int rows, int nkw, int nkb,
                                             int32_t *__restrict__ row_ptr, int32_t *__restrict__ col_idx) {
  __shared__ int s_red[4];
  __shared__ int s_rp[64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int b = blockIdx.x;
  const int r0 = b * 64;
  int part = 0;
  for (int i = tid; i < b; i += 256) part += bsum[i];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
  if (lane == 0) s_red[w] = part;
  __syncthreads();
  if (w == 0) {
    const int base = s_red[0] + s_red[1] + s_red[2] + s_red[3];
    const int row = r0 + lane;
    const int c = row < rows ? counts[row] : 0;
    int incl = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    const int rp = base + incl - c;
    s_rp[lane] = rp;
    if (row < rows) row_ptr[row] = rp;
    if (row == rows - 1) row_ptr[rows] = rp + c;
  }
  __syncthreads();
  const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int k = 0; k < 16; ++k) {
    const int rk = r0 + 16 * w + k;
    if (rk >= rows) break;
    int out = s_rp[16 * w + k];
    const uint32_t *bm = bitmask + (size_t)rk * nkw;
    for (int j0 = 0; j0 < nkb; j0 += 64) {
      const int j = j0 + lane;
      const bool kept = j < nkb && ((bm[j >> 5] >> (j & 31)) & 1u);
      const unsigned long long bal = __ballot(kept);
      if (kept) col_idx[out + __popcll(bal & lt)] = j;
      out += __popcll(bal);
    }
  }
}

// ---------------------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------------------
static int launch_pool_args(const PoolArgs &pa, int BH, int d, int dtype, hipStream_t st) {
  const dim3 grid(pa.ngrp[0] + pa.ngrp[1], BH);
  if (dtype == FVATTN_BF16) {
    if (d == 128) hipLaunchKernelGGL((k_pool<uint16_t, 128>), grid, dim3(256), 0, st, pa);
    else hipLaunchKernelGGL((k_pool<uint16_t, 64>), grid, dim3(256), 0, st, pa);
  } else {
    if (d == 128) hipLaunchKernelGGL((k_pool<float, 128>), grid, dim3(256), 0, st, pa);
    else hipLaunchKernelGGL((k_pool<float, 64>), grid, dim3(256), 0, st, pa);
  }
  FV_CHECK_LAUNCH();
  return FVATTN_OK;
}

int launch_pool(const void *x, int BH, int N, int d, int dtype, int block, double *out, hipStream_t st) {
  PoolArgs pa = {};
  pa.x[0] = x;
  pa.out[0] = out;
  pa.block[0] = block;
  pa.nb[0] = cdiv(N, block);
  pa.ngrp[0] = cdiv(pa.nb[0], 16);
  pa.N = N;
  pa.layout = 0;
  return launch_pool_args(pa, BH, d, dtype, st);
}

int launch_pool_qk(const void *q, const void *k, int BH, int N, int d, int dtype, int block_q, int block_k,
                   double *qsw, double *ksw, int32_t *zero0, int nzero0, int32_t *zero1, int nzero1,
                   hipStream_t st) {
  PoolArgs pa = {};
  pa.x[0] = q;
  pa.x[1] = k;
  pa.out[0] = qsw;
  pa.out[1] = ksw;
  pa.block[0] = block_q;
  pa.block[1] = block_k;
  for (int t = 0; t < 2; ++t) {
    pa.nb[t] = cdiv(N, pa.block[t]);
    pa.ngrp[t] = cdiv(pa.nb[t], 16);
  }
  pa.N = N;
  pa.layout = 1;
  pa.zero[0] = zero0;
  pa.nzero[0] = nzero0;
  pa.zero[1] = zero1;
  pa.nzero[1] = nzero1;
  return launch_pool_args(pa, BH, d, dtype, st);
}

template <int D, int MT, int NWV>
static int launch_select_mt(const double *qsw, const double *ksw, int BH, int nqb, int nkb, double p,
                            int32_t *counts, uint32_t *bitmask, int nkw, int32_t *head_load, int32_t *bsum,
                            const SelOpts &sel, hipStream_t st) {
  auto kern = (sel.mode != FVATTN_ROUTE_TOPP || sel.k_min > 1 || sel.k_max > 0 || sel.window > 0 ||
               sel.imp != nullptr)
                  ? k_select<D, MT, NWV, true>
                  : k_select<D, MT, NWV, false>;
  int cus = 0, occ = 0;
  if (device_cus(&cus) != 0) return FVATTN_ERR_HIP;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, 64 * NWV, 0) != hipSuccess) return FVATTN_ERR_HIP;
  const int items = cdiv(nqb, 16) * BH;
  int grid = cus * (occ > 0 ? occ : 1);
  if (grid > items) grid = items;
  if (grid < 8) grid = 8;   // every XCD range needs a worker
  const double scale = 1.0 / sqrt((double)D);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * NWV), 0, st, qsw, ksw, nqb, nkb, scale, p, counts, bitmask, nkw,
                     head_load, bsum, BH, sel);
  FV_CHECK_LAUNCH();
  return FVATTN_OK;
}

// Key tiles (of 16 blocks) per wave: up to 512 key blocks run on 4 waves with at most 8 tiles
// each; more (up to 1280) on 8 waves with at most 10 tiles each.
template <int D>
static int launch_select_d(const double *qsw, const double *ksw, int BH, int nqb, int nkb, double p,
                           int32_t *counts, uint32_t *bitmask, int nkw, int32_t *head_load, int32_t *bsum,
                           const SelOpts &sel, hipStream_t st) {
  const int nkt = cdiv(nkb, 16);
#define FV_SEL(MT, NWV) \
  return launch_select_mt<D, MT, NWV>(qsw, ksw, BH, nqb, nkb, p, counts, bitmask, nkw, head_load, bsum, sel, st)
  if (nkt <= 4) FV_SEL(1, 4);
  if (nkt <= 8) FV_SEL(2, 4);
  if (nkt <= 16) FV_SEL(4, 4);
  if (nkt <= 32) FV_SEL(8, 4);
  FV_SEL(10, 8);
#undef FV_SEL
}

int launch_select(const double *qsw, const double *ksw, int BH, int d, int nqb, int nkb, double p,
                  int32_t *counts, uint32_t *bitmask, int nkw, int32_t *head_load, int32_t *bsum, int mode, int topk,
                  int k_min, int k_max, int window, int bq, int bk, int N, double *imp, hipStream_t st) {
  const SelOpts sel{mode, topk, k_min, k_max, window, bq, bk, N, imp};
  if (d == 128) return launch_select_d<128>(qsw, ksw, BH, nqb, nkb, p, counts, bitmask, nkw, head_load, bsum, sel, st);
  return launch_select_d<64>(qsw, ksw, BH, nqb, nkb, p, counts, bitmask, nkw, head_load, bsum, sel, st);
}

int launch_csr(const int32_t *counts, const uint32_t *bitmask, const int32_t *bsum, int rows, int nkw, int nkb,
               int32_t *row_ptr, int32_t *col_idx, hipStream_t st) {
  hipLaunchKernelGGL(k_csr, dim3(cdiv(rows, 64)), dim3(256), 0, st, counts, bitmask, bsum, rows, nkw, nkb, row_ptr,
                     col_idx);
  FV_CHECK_LAUNCH();
  return FVATTN_OK;
}

}  // namespace fv
