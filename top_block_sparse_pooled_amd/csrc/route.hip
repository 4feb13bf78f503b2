// Top-p routing on gfx950: block mean-pooling, pooled block scores, softmax over key
// blocks, descending order with ties to the lower index, cut at cumulative mass >= p,
// and compaction into a CSR of kept key blocks with per-head loads.
//
// Method: FVAttn summary page (PaperDaily, arXiv:2607.16190), Top-p routing paragraph of
// section "AI视频生成的阿喀琉斯之踵"; pooled scores with 1/sqrt(d): tutorial page, section 5.2.
//
// Design (gfx950):
//  * k_pool      HBM-bound pass over K (and the exported pooling call): each workgroup streams
//                whole blocks with 16-byte loads, accumulates in float64 (the mean of a block
//                of bf16 values is then exact up to the final division), and writes the
//                pooled rows in the lane order the float64 MFMA of k_select consumes (one
//                512-byte load per operand).
//  * k_select    one item = 16 query blocks of one head (4 waves; 8 above 512 key blocks),
//                persistent.  The item pools its own query blocks into LDS (same summation
//                order as k_pool), so the raw Q reads overlap other workgroups' work.  Scores
//                qbar.kbar^T/sqrt(d) come from v_mfma_f64_16x16x4 and stay in registers (wave
//                w holds key tiles w, w + NWV, ...).  Softmax numerators e = exp(s - max) in
//                float64; masses as 2^-52 fixed point so every partial sum is exact and order
//                independent.  The rows then go to LDS and each wave resolves whole rows
//                alone: the descending order is never materialised; a radix select over the
//                float64 bit pattern of e (monotone for e >= 0) splits the row's key range
//                [e_min, 1] into 256 bins (a histogram private to the wave), walks the mass
//                histogram from the largest bin down, stops at the bin where the cumulative
//                mass crosses p * Z, and refines that bin the same way until one key remains.
//                That gives exactly the shortest prefix of the (e descending, index ascending)
//                order with mass >= p: elements above the threshold key are all kept, and
//                among keys equal to the threshold the lowest indices are taken first.
//  * k_csr       exclusive scan of per-row counts (a row's offset is the per-64-row sums
//                before its block plus a lane scan inside it, no second pass) and expansion
//                of the kept-bit masks into ascending column indices.
#include "common.h"

namespace fv {

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

// Means of the real tokens of NBK blocks j0, j0 + js, ... (block j: tokens [j block,
// min(j block + block, N))) of one head's rows xh, by one wave: lane l reads 16-byte chunk
// l % CPR of rows l / CPR + RPL i of every block (NBK x 16 loads in flight per lane),
// accumulates in float64, and the lanes of a chunk are summed with cross-lane shuffles.  Lanes
// l < CPR return dims l EPC .. l EPC + EPC - 1 of each block (zero for blocks >= nb).
template <typename T, int D, int NBK>
__device__ __forceinline__ void pool_blocks(const T *__restrict__ xh, int j0, int js, int block, int nb, int N,
                                            double (&mean)[NBK][DT<T>::per16]) {
  constexpr int EPC = DT<T>::per16;   // elements per 16-byte chunk
  constexpr int CPR = D / EPC;        // chunks per row
  constexpr int RPL = 64 / CPR;       // rows covered by one wave-wide load
  constexpr int NLD = 16;             // loads in flight per lane and block
  constexpr int RPR = RPL * NLD;      // rows per round
  const int lane = threadIdx.x & 63;
  const int c = lane % CPR, r = lane / CPR;
  double acc[NBK][EPC];
  int s0[NBK], e0[NBK];
#pragma unroll
  for (int b = 0; b < NBK; ++b) {
    const int j = j0 + b * js;
    s0[b] = j < nb ? j * block : 0;
    e0[b] = j < nb ? min(s0[b] + block, N) : 0;
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[b][e] = 0.0;
  }
  for (int base = 0; base < block; base += RPR) {
    u32x4 buf[NBK][NLD];
#pragma unroll
    for (int b = 0; b < NBK; ++b)
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const int row = s0[b] + base + r + RPL * i;
        buf[b][i] = u32x4{0u, 0u, 0u, 0u};
        if (row < e0[b]) buf[b][i] = *reinterpret_cast<const u32x4 *>(xh + (size_t)row * D + c * EPC);
      }
#pragma unroll
    for (int b = 0; b < NBK; ++b)
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        float f[EPC];
        unpack16(buf[b][i], f, T());
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[b][e] += (double)f[e];
      }
  }
#pragma unroll
  for (int b = 0; b < NBK; ++b) {
#pragma unroll
    for (int off = CPR; off < 64; off <<= 1)
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[b][e] += __shfl_xor(acc[b][e], off);
    const int cnt = e0[b] - s0[b];
#pragma unroll
    for (int e = 0; e < EPC; ++e) mean[b][e] = cnt > 0 ? acc[b][e] / (double)cnt : 0.0;
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void k_pool(PoolArgs a) {
  constexpr int EPC = DT<T>::per16;   // elements per 16-byte chunk
  constexpr int CPR = D / EPC;        // chunks per row
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

  for (int jj = w; jj < 16; jj += 4) {
    double m[1][EPC];
    pool_blocks<T, D, 1>(xh, gx * 16 + jj, 0, block, nb, N, m);
    if (lane < CPR) {
#pragma unroll
      for (int e = 0; e < EPC; ++e) stage[jj][lane * EPC + e] = m[0][e];
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
// k_select: scores, softmax and the Top-p cut (or a routing variant) for 16 query blocks of
// one head per item.  Persistent: grid = min(resident workgroups, items), at least 8.
// NWV waves (4, or 8 for more than 512 key blocks); MAXT key tiles of 16 per wave.
//   1. Scores for the 16 rows on the float64 MFMA, wave w holding key tiles w, w + NWV, ...;
//      row maxima, e = exp(s - max), fixed-point row sums Z and row minima of e across the
//      waves (two workgroup barriers).
//   2. The e values go to LDS as whole rows (RB rows at a time), and each wave then resolves
//      its rows alone: the row's values sit in registers (lane l: key blocks l + 64 t), the
//      radix passes use a histogram private to the wave, and the kept set leaves as 64-bit
//      ballots.  No workgroup barrier inside the selection.
// Outputs counts[row] and the kept-bit mask bitmask[row][nkw]; adds loads to head_load.
// ---------------------------------------------------------------------------------------
constexpr int kMaxNkw = 40;  // 1280 key blocks

// Routing variant of k_select (see fvattn_route_opts): mode, top-k count, clamp of the Top-p
// count, local window, and the block geometry the window needs.
struct SelOpts {
  int mode, topk, k_min, k_max, window, bq, bk, N;
  double *imp;   // optional [rows][nkb]: importance P of every block (SASA candidates); EXT only
};

constexpr double kFix52 = 4503599627370496.0;  // 2^52: masses as fixed point

// Kept set of one row by the wave: the shortest prefix of the (e descending, index ascending)
// order whose mass (bycnt = false: fixed-point e, target T) or count (bycnt = true, target T)
// reaches T.  ev[t] is e of key block lane + 64 t; valid below nkb.  Search range of keys (the
// float64 bit patterns of e, monotone for e >= 0): [lo0, bits(1.0)].  Each radix pass splits
// the range into 256 digit bins, walks the histogram from the largest digit down to the bin
// where the cumulative mass from the top reaches T, and narrows the range to that bin, until
// the bin holds one key or one key value (ties, resolved toward lower indices).  Returns the
// kept-bit word of key blocks 32 lane .. 32 lane + 31 (zero for lanes past the row) and sets
// `count` to the number of kept blocks.
template <int NPL>
__device__ __forceinline__ uint32_t select_row(const double (&ev)[NPL], int nkb, bool bycnt, unsigned long long T,
                                               unsigned long long lo0, bool keep_all,
                                               unsigned long long *__restrict__ hm, uint32_t *__restrict__ hc,
                                               int &count) {
  const int lane = threadIdx.x & 63;
  unsigned long long lo = lo0;
  unsigned long long width = (unsigned long long)__double_as_longlong(1.0) + 1ull - lo0;
  unsigned long long above = 0;
  int st = keep_all ? 3 : 0;   // 0 searching, 1 unique threshold key, 2 tied threshold keys, 3 all
  uint32_t ntie = 0;
  for (int pass = 0; pass < 8 && st == 0; ++pass) {
    const int sh = digit_shift(width);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      hm[4 * lane + q] = 0ull;
      hc[4 * lane + q] = 0u;
    }
    // (LDS operations of one wave take effect in issue order; the fences only keep the
    // compiler from moving them)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
    for (int t = 0; t < NPL; ++t) {
      const unsigned long long off = (unsigned long long)__double_as_longlong(ev[t]) - lo;
      if (lane + 64 * t < nkb && off < width) {
        const int dg = (int)(off >> sh);
        atomicAdd(&hc[dg], 1u);
        if (!bycnt) atomicAdd(&hm[dg], (unsigned long long)(ev[t] * kFix52));
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    unsigned long long m4[4];
    uint32_t c4[4];
    unsigned long long ms = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      c4[q] = hc[4 * lane + q];
      m4[q] = bycnt ? (unsigned long long)c4[q] : hm[4 * lane + q];
      ms += m4[q];
    }
    // mass of the digits held by higher lanes (larger keys)
    unsigned long long sm = ms;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const unsigned long long o = __shfl_down(sm, off);
      if (lane + off < 64) sm += o;
    }
    unsigned long long acc = above + (sm - ms);
    int dig = -1;
    unsigned long long nab = 0;
    uint32_t cnt = 0;
#pragma unroll
    for (int q = 3; q >= 0; --q) {
      if (m4[q] > 0 && acc < T && T <= acc + m4[q]) {
        dig = 4 * lane + q;
        nab = acc;
        cnt = c4[q];
      }
      acc += m4[q];
    }
    const unsigned long long bal = __ballot(dig >= 0);
    if (bal == 0ull) {   // unreachable: the range always holds the crossing
      st = 3;
      break;
    }
    const int L = __ffsll((long long)bal) - 1;
    dig = __shfl(dig, L);
    above = __shfl(nab, L);
    cnt = __shfl(cnt, L);
    lo += (unsigned long long)dig << sh;
    width = 1ull << sh;
    ntie = cnt;
    if (cnt == 1) st = 1;
    else if (sh == 0) st = 2;
  }
  const unsigned long long hi = lo + width;
  uint32_t need = 0;
  if (st == 2) {
    const unsigned long long rem = T - above;
    const unsigned long long mt = (unsigned long long)(__longlong_as_double((long long)lo) * kFix52);
    if (bycnt) need = (uint32_t)min((unsigned long long)ntie, rem);
    else need = mt == 0 ? ntie : (uint32_t)min((unsigned long long)ntie, (rem + mt - 1) / mt);
  }
  uint32_t cum = 0;   // ties taken so far (ascending key block)
  uint32_t word = 0;
  count = 0;
#pragma unroll
  for (int t = 0; t < NPL; ++t) {
    const bool valid = lane + 64 * t < nkb;
    const unsigned long long key = (unsigned long long)__double_as_longlong(ev[t]);
    bool keep = valid && (st == 3 || key >= hi || (st == 1 && key >= lo));
    if (st == 2) {
      const bool tie = valid && key == lo;
      const unsigned long long bt = __ballot(tie);
      const uint32_t rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(bt >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bt, 0u));
      keep = keep || (tie && cum + rank < need);
      cum += (uint32_t)__popcll(bt);
    }
    const unsigned long long mt = __ballot(keep);
    if (lane == 2 * t) word = (uint32_t)mt;
    if (lane == 2 * t + 1) word = (uint32_t)(mt >> 32);
    count += (int)__popcll(mt);
  }
  return word;
}

template <typename T, int D, int MAXT, int NWV, bool EXT>
__global__ __launch_bounds__(64 * NWV, NWV == 4 ? 2 : 1) void k_select(const void *__restrict__ qraw,
                                                const double *__restrict__ ksw, int nqb, int nkb,
                                                double scale, double p, int32_t *__restrict__ counts,
                                                uint32_t *__restrict__ bitmask, int nkw,
                                                int32_t *__restrict__ head_load, int32_t *__restrict__ bsum,
                                                int BH, SelOpts sel) {
  constexpr int KS = D / 4;               // MFMA k-steps
  constexpr int KCAP = 16 * NWV * MAXT;   // key blocks the tiles cover
  constexpr int NPL = KCAP / 64;          // values per lane in the row phase
  constexpr int RB = NWV == 4 ? 16 : 8;   // rows staged in LDS at once
  constexpr int NB = 16 / RB;
  constexpr int RPW = RB / NWV;           // rows per wave per batch
  static_assert(KCAP % 64 == 0 && RB % NWV == 0 && (RB / 4) * 4 == RB, "row phase geometry");
  constexpr int EPC = DT<T>::per16, CPR = D / EPC;
  // staged rows; before them, the item's pooled query blocks (16 D doubles)
  constexpr int ESZ = RB * KCAP > 16 * D ? RB * KCAP : 16 * D;
  __shared__ double s_eq[ESZ];
  double(*s_e)[KCAP] = reinterpret_cast<double(*)[KCAP]>(s_eq);
  __shared__ unsigned long long h_mass[NWV][256];
  __shared__ uint32_t h_cnt[NWV][256];
  __shared__ double s_part[NWV][16];
  __shared__ unsigned long long s_zpart[NWV][16];
  __shared__ double s_minpart[NWV][16];
  __shared__ int s_cnt[16];           // kept counts of the item's rows

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
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

  // ---- the item's 16 query blocks, mean-pooled straight into LDS in the float64 MFMA
  // operand order (block jj, dim c at (c / 4) 64 + jj + 16 (c % 4)); the raw Q reads of one
  // workgroup overlap the score phases of the others
  {
    const T *xh = reinterpret_cast<const T *>(qraw) + (size_t)bh * sel.N * D;
    // two blocks per wave at a time: 32 loads in flight per lane
    constexpr int NBK = NWV == 4 ? 2 : 1;
    for (int jj = w; jj < 16; jj += NBK * NWV) {
      double m[NBK][EPC];
      pool_blocks<T, D, NBK>(xh, 16 * g + jj, NWV, sel.bq, nqb, sel.N, m);
      if (lane < CPR) {
#pragma unroll
        for (int b = 0; b < NBK; ++b)
#pragma unroll
          for (int e = 0; e < EPC; ++e) {
            const int cc = lane * EPC + e;
            s_eq[(cc >> 2) * 64 + jj + b * NWV + 16 * (cc & 3)] = m[b][e];
          }
      }
    }
  }
  __syncthreads();

  // ---- scores: S[i][j] = sum_c qbar[i][c] * kbar[j][c], i = lane/16 + 4v, j = 16t + lane%16
  d4 acc[MAXT];
#pragma unroll
  for (int k = 0; k < MAXT; ++k) acc[k] = d4{0.0, 0.0, 0.0, 0.0};
  {
    const double *qa = s_eq + lane;
    // k-step outer, tiles inner: MAXT independent accumulators.  The operands of PF k-steps
    // (one of qbar, MAXT of kbar each) are in flight ahead of the MFMAs that use them, which
    // covers the L2 latency of the pooled keys.  Tiles past the last read a valid tile (their
    // key columns are >= nkb and ignored below), so the loop has no branches.
    constexpr int PF = MAXT >= 8 ? 1 : 3;
    const double *kb[MAXT];
#pragma unroll
    for (int k = 0; k < MAXT; ++k) kb[k] = ksw + ((size_t)(bh * nkt + min(w + NWV * k, nkt - 1)) * KS) * 64 + lane;
    double abuf[PF], bbuf[PF][MAXT];
#pragma unroll
    for (int s = 0; s < PF; ++s) {
      abuf[s] = qa[s * 64];
#pragma unroll
      for (int k = 0; k < MAXT; ++k) bbuf[s][k] = kb[k][s * 64];
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int slot = s % PF;
      const double a = abuf[slot];
      double b[MAXT];
#pragma unroll
      for (int k = 0; k < MAXT; ++k) b[k] = bbuf[slot][k];
      if (s + PF < KS) {
        abuf[slot] = qa[(s + PF) * 64];
#pragma unroll
        for (int k = 0; k < MAXT; ++k) bbuf[slot][k] = kb[k][(s + PF) * 64];
      }
#pragma unroll
      for (int k = 0; k < MAXT; ++k) acc[k] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b[k], acc[k], 0, 0, 0);
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

  // ---- e = exp(s - max) (in place; 0 past nkb), fixed-point masses, Z, minimum of e
  unsigned long long zs[4] = {0, 0, 0, 0};
  double mn[4] = {1.0, 1.0, 1.0, 1.0};
#pragma unroll
  for (int k = 0; k < MAXT; ++k) {
    const int j = 16 * (w + NWV * k) + jl;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const double e = (j < nkb) ? exp(acc[k][v] - mx[v]) : 0.0;
      acc[k][v] = e;
      zs[v] += (unsigned long long)(e * kFix52);
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

#pragma unroll
  for (int b = 0; b < NB; ++b) {
    // ---- stage rows [b RB, b RB + RB): lane (ig, jl) holds rows ig + 4v of its key columns
#pragma unroll
    for (int k = 0; k < MAXT; ++k) {
      const int j = 16 * (w + NWV * k) + jl;
#pragma unroll
      for (int v = b * RB / 4; v < (b + 1) * RB / 4; ++v) s_e[ig + 4 * v - b * RB][j] = acc[k][v];
    }
    __syncthreads();
    // ---- selection: wave w resolves rows b RB + rr NWV + w
    for (int rr = 0; rr < RPW; ++rr) {
      const int r = b * RB + rr * NWV + w;
      const int i = 16 * g + r;
      if (i >= nqb) {   // wave-uniform
        if (lane == 0) s_cnt[r] = 0;
        continue;
      }
      const size_t row = (size_t)bh * nqb + i;
      double ev[NPL];
#pragma unroll
      for (int t = 0; t < NPL; ++t) ev[t] = s_e[r - b * RB][lane + 64 * t];
      unsigned long long Z = 0;
      double emin = 1.0;
#pragma unroll
      for (int ww = 0; ww < NWV; ++ww) {
        Z += s_zpart[ww][r];
        emin = fmin(emin, s_minpart[ww][r]);
      }
      const unsigned long long lo0 = (unsigned long long)__double_as_longlong(emin);
      // search by mass (Top-p) or by count (top-k, or a clamped Top-p count)
      bool bycnt = false;
      unsigned long long tgt0;
      bool all;
      if (EXT && sel.mode == FVATTN_ROUTE_TOPK) {
        bycnt = true;
        tgt0 = (unsigned long long)sel.topk;
        all = sel.topk >= nkb;
      } else {
        tgt0 = (unsigned long long)ceil(p * (double)Z);
        if (tgt0 > Z) tgt0 = Z;
        if (tgt0 < 1) tgt0 = 1;
        all = p >= 1.0;
      }
      int c;
      // lane L < nkw holds kept word L (key blocks 32 L .. 32 L + 31)
      uint32_t word = select_row<NPL>(ev, nkb, bycnt, tgt0, lo0, all, h_mass[w], h_cnt[w], c);
      if (EXT && !bycnt && (sel.k_min > 1 || sel.k_max > 0)) {
        // clamp of the Top-p count: re-select by count when it lies outside [k_min, k_max]
        int tgt = max(c, sel.k_min);
        if (sel.k_max > 0) tgt = min(tgt, sel.k_max);
        tgt = min(tgt, nkb);
        if (tgt != c) word = select_row<NPL>(ev, nkb, true, (unsigned long long)tgt, lo0, tgt >= nkb, h_mass[w], h_cnt[w], c);
      }
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
      if (EXT && sel.window > 0) {
        c = __popc(word);
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) c += __shfl_xor(c, off);
      }
      if (lane < nkw) bitmask[row * nkw + lane] = word;
      if (lane == 0) {
        counts[row] = c;
        s_cnt[r] = c;
      }
      if (EXT && sel.imp != nullptr) {
        // importance of every block: the candidates' order for SASA
        const double invz = Z > 0 ? kFix52 / (double)Z : 0.0;   // 1 / Z with Z in 2^-52 units
#pragma unroll
        for (int t = 0; t < NPL; ++t)
          if (lane + 64 * t < nkb) sel.imp[row * nkb + lane + 64 * t] = ev[t] * invz;
      }
    }
    __syncthreads();   // staged rows and partial sums consumed before they are overwritten
  }
  if (w == 0) {
    // the item's load of the head and its per-64-row sums for the CSR scan (the 16 rows
    // span at most two 64-row blocks)
    const size_t row0 = (size_t)bh * nqb + 16 * g;
    const int c = lane < 16 ? s_cnt[lane] : 0;
    const bool second = lane < 16 && ((row0 + lane) >> 6) != (row0 >> 6);
    int c0 = second ? 0 : c, c1 = second ? c : 0;
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) {
      c0 += __shfl_xor(c0, off);
      c1 += __shfl_xor(c1, off);
    }
    if (lane == 0) {
      atomicAdd(&head_load[bh], c0 + c1);
      atomicAdd(&bsum[row0 >> 6], c0);
      if (c1 != 0) atomicAdd(&bsum[(row0 >> 6) + 1], c1);
    }
  }
  }
}

// ---------------------------------------------------------------------------------------
// k_csr: row_ptr (exclusive scan of counts) and ascending col_idx from the kept masks.
// grid = cdiv(rows, 16), 256 threads; wave w owns rows 16 b + 4 w .. + 3, with no workgroup
// barrier: a row's offset is the sum of the per-64-row sums before its 64-row block plus the
// counts of the rows before it inside that block (an exclusive scan across the lanes).  Lane L
// holds word L of a row's mask (the four rows' words are loaded up front), and each 64-block
// chunk of a row is one 64-bit mask from two lanes, whose set bits give every kept block its
// output slot (coalesced writes).
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_csr(const int32_t *__restrict__ counts,
                                             const uint32_t *__restrict__ bitmask,
                                             const int32_t *__restrict__ bsum, int rows, int nkw, int nkb,
                                             int32_t *__restrict__ row_ptr, int32_t *__restrict__ col_idx) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r0 = blockIdx.x * 16 + 4 * w;   // this wave's first row
  if (r0 >= rows) return;                    // wave-uniform
  uint32_t wv[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int rk = r0 + k;
    wv[k] = (rk < rows && lane < nkw) ? bitmask[(size_t)rk * nkw + lane] : 0u;
  }
  const int blk = r0 >> 6;
  const int cl = (64 * blk + lane < rows) ? counts[64 * blk + lane] : 0;
  int part = 0;
  for (int i = lane; i < blk; i += 64) part += bsum[i];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
  int incl = cl;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  const int excl = incl - cl;   // counts of the block's rows before row 64 blk + lane
  const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int nch = (nkb + 63) >> 6;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int rk = r0 + k;
    if (rk >= rows) break;
    int out = part + __shfl(excl, rk - 64 * blk);
    const int ck = __shfl(cl, rk - 64 * blk);
    if (lane == 0) {
      row_ptr[rk] = out;
      if (rk == rows - 1) row_ptr[rows] = out + ck;
    }
    for (int c = 0; c < nch; ++c) {
      const unsigned long long mask = (unsigned long long)(uint32_t)__shfl((int)wv[k], 2 * c) |
                                      ((unsigned long long)(uint32_t)__shfl((int)wv[k], 2 * c + 1) << 32);
      if ((mask >> lane) & 1ull) col_idx[out + __popcll(mask & lt)] = 64 * c + lane;
      out += __popcll(mask);
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

// Pooled K in the float64 MFMA operand order of k_select (the query blocks are pooled inside
// k_select), and the zeroing of the two counter arrays (per-64-row sums, head loads).
int launch_pool_k(const void *k, int BH, int N, int d, int dtype, int block_k, double *ksw, int32_t *zero0, int nzero0,
                  int32_t *zero1, int nzero1, hipStream_t st) {
  PoolArgs pa = {};
  pa.x[0] = k;
  pa.out[0] = ksw;
  pa.block[0] = block_k;
  pa.nb[0] = cdiv(N, block_k);
  pa.ngrp[0] = cdiv(pa.nb[0], 16);
  pa.N = N;
  pa.layout = 1;
  pa.zero[0] = zero0;
  pa.nzero[0] = nzero0;
  pa.zero[1] = zero1;
  pa.nzero[1] = nzero1;
  return launch_pool_args(pa, BH, d, dtype, st);
}

template <typename T, int D, int MT, int NWV>
static int launch_select_mt(const void *q, const double *ksw, int BH, int nqb, int nkb, double p, int32_t *counts,
                            uint32_t *bitmask, int nkw, int32_t *head_load, int32_t *bsum, const SelOpts &sel,
                            hipStream_t st) {
  auto kern = (sel.mode != FVATTN_ROUTE_TOPP || sel.k_min > 1 || sel.k_max > 0 || sel.window > 0 ||
               sel.imp != nullptr)
                  ? k_select<T, D, MT, NWV, true>
                  : k_select<T, D, MT, NWV, false>;
  int cus = 0, occ = 0;
  if (device_cus(&cus) != 0) return FVATTN_ERR_HIP;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, 64 * NWV, 0) != hipSuccess) return FVATTN_ERR_HIP;
  const int items = cdiv(nqb, 16) * BH;
  int grid = cus * (occ > 0 ? occ : 1);
  if (grid > items) grid = items;
  if (grid < 8) grid = 8;   // every XCD range needs a worker
  const double scale = 1.0 / sqrt((double)D);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * NWV), 0, st, q, ksw, nqb, nkb, scale, p, counts, bitmask, nkw,
                     head_load, bsum, BH, sel);
  FV_CHECK_LAUNCH();
  return FVATTN_OK;
}

// Key tiles (of 16 blocks) per wave: up to 512 key blocks run on 4 waves with at most 8 tiles
// each; more on 8 waves with 8 tiles each (up to 1024) or 10 (up to 1280).
template <typename T, int D>
static int launch_select_d(const void *q, const double *ksw, int BH, int nqb, int nkb, double p, int32_t *counts,
                           uint32_t *bitmask, int nkw, int32_t *head_load, int32_t *bsum, const SelOpts &sel,
                           hipStream_t st) {
  const int nkt = cdiv(nkb, 16);
#define FV_SEL(MT, NWV) \
  return launch_select_mt<T, D, MT, NWV>(q, ksw, BH, nqb, nkb, p, counts, bitmask, nkw, head_load, bsum, sel, st)
  if (nkt <= 4) FV_SEL(1, 4);
  if (nkt <= 8) FV_SEL(2, 4);
  if (nkt <= 16) FV_SEL(4, 4);
  if (nkt <= 32) FV_SEL(8, 4);
  if (nkt <= 64) FV_SEL(8, 8);
  FV_SEL(10, 8);
#undef FV_SEL
}

int launch_select(const void *q, const double *ksw, int BH, int d, int dtype, int nqb, int nkb, double p,
                  int32_t *counts, uint32_t *bitmask, int nkw, int32_t *head_load, int32_t *bsum, int mode, int topk,
                  int k_min, int k_max, int window, int bq, int bk, int N, double *imp, hipStream_t st) {
  const SelOpts sel{mode, topk, k_min, k_max, window, bq, bk, N, imp};
  if (dtype == FVATTN_BF16) {
    if (d == 128)
      return launch_select_d<uint16_t, 128>(q, ksw, BH, nqb, nkb, p, counts, bitmask, nkw, head_load, bsum, sel, st);
    return launch_select_d<uint16_t, 64>(q, ksw, BH, nqb, nkb, p, counts, bitmask, nkw, head_load, bsum, sel, st);
  }
  if (d == 128)
    return launch_select_d<float, 128>(q, ksw, BH, nqb, nkb, p, counts, bitmask, nkw, head_load, bsum, sel, st);
  return launch_select_d<float, 64>(q, ksw, BH, nqb, nkb, p, counts, bitmask, nkw, head_load, bsum, sel, st);
}

int launch_csr(const int32_t *counts, const uint32_t *bitmask, const int32_t *bsum, int rows, int nkw, int nkb,
               int32_t *row_ptr, int32_t *col_idx, hipStream_t st) {
  hipLaunchKernelGGL(k_csr, dim3(cdiv(rows, 16)), dim3(256), 0, st, counts, bitmask, bsum, rows, nkw, nkb, row_ptr,
                     col_idx);
  FV_CHECK_LAUNCH();
  return FVATTN_OK;
}

}  // namespace fv
