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
// k_pool: x [BH][N][D] -> mean of every block of `block` tokens (real tokens only).
// layout 0: plain [BH][nb][D]; layout 1: swizzled, nbp = nb rounded up to 16, padded
// blocks written as zero.  grid = (cdiv(nbp, BPW), BH), 256 threads.
// ---------------------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void k_pool(const T *__restrict__ x, int N, int block, int nb,
                                              int nbp, int layout, double *__restrict__ out,
                                              int32_t *__restrict__ zero_me, int nzero) {
  constexpr int EPC = DT<T>::per16;           // elements per 16-byte chunk
  constexpr int CPR = D / EPC;                // chunks per row
  constexpr int RPR = 256 / CPR;              // rows per load round
  constexpr int MAXR = (128 + RPR - 1) / RPR; // rounds for the largest block (128)
  __shared__ double red[RPR][D + 1];

  const int tid = threadIdx.x;
  const int bh = blockIdx.y, j = blockIdx.x;  // one block per workgroup
  const int ch = tid % CPR, r0 = tid / CPR;
  if (zero_me != nullptr && j == 0 && bh == 0)
    for (int i = tid; i < nzero; i += 256) zero_me[i] = 0;

  const T *xh = x + (size_t)bh * N * D;
  const int s0 = j * block, e0 = min(s0 + block, N);
  double acc[EPC];
#pragma unroll
  for (int t = 0; t < EPC; ++t) acc[t] = 0.0;
  if (j < nb) {
    u32x4 buf[MAXR];
#pragma unroll
    for (int k = 0; k < MAXR; ++k) {
      const int r = s0 + r0 + k * RPR;
      buf[k] = u32x4{0u, 0u, 0u, 0u};
      if (k * RPR < block && r < e0) buf[k] = *reinterpret_cast<const u32x4 *>(xh + (size_t)r * D + ch * EPC);
    }
#pragma unroll
    for (int k = 0; k < MAXR; ++k) {
      float f[EPC];
      unpack16(buf[k], f, T());
#pragma unroll
      for (int t = 0; t < EPC; ++t) acc[t] += (double)f[t];
    }
  }
#pragma unroll
  for (int t = 0; t < EPC; ++t) red[r0][ch * EPC + t] = acc[t];
  __syncthreads();
  if (tid < D) {
    double sum = 0.0;
#pragma unroll 4
    for (int r = 0; r < RPR; ++r) sum += red[r][tid];
    const double mean = (j < nb) ? sum / (double)(e0 - s0) : 0.0;
    if (layout)
      out[swz(bh, nbp / 16, D, j, tid)] = mean;
    else
      out[((size_t)bh * nb + j) * D + tid] = mean;
  }
}

// ---------------------------------------------------------------------------------------
// k_select: scores, softmax, Top-p cut for 16 query blocks of one head.
// grid = (nqbp/16, BH), 256 threads.  MAXT = key tiles (of 16) per wave.
// Outputs counts[row] and the kept-bit mask bitmask[row][nkw]; adds loads to head_load.
// ---------------------------------------------------------------------------------------
constexpr int kMaxNkw = 40;  // 1280 key blocks

// Smallest shift with (width - 1) >> shift < 256: the digit of a key in a range of `width`.
__device__ __forceinline__ int digit_shift(unsigned long long width) {
  const unsigned long long wm1 = width - 1ull;
  return wm1 < 256ull ? 0 : 64 - __clzll((long long)wm1) - 8;
}

template <int D, int MAXT>
__global__ __launch_bounds__(256, MAXT <= 8 ? 2 : 1) void k_select(const double *__restrict__ qsw,
                                                const double *__restrict__ ksw, int nqb, int nkb,
                                                double scale, double p, int32_t *__restrict__ counts,
                                                uint32_t *__restrict__ bitmask, int nkw,
                                                int32_t *__restrict__ head_load, int32_t *__restrict__ bsum) {
  constexpr int KS = D / 4;  // MFMA k-steps
  __shared__ uint32_t h_cnt[16][256];
  __shared__ unsigned long long h_mass[16][256];
  __shared__ uint32_t s_kept[16][kMaxNkw];
  __shared__ uint32_t s_ties[16][kMaxNkw];
  __shared__ double s_part[4][16];
  __shared__ unsigned long long s_zpart[4][16];
  __shared__ unsigned long long s_lo[16], s_width[16], s_above[16], s_target[16];
  __shared__ double s_minpart[4][16];
  __shared__ int s_state[16];   // 0 = searching, 1 = unique threshold found, 2 = ties, 3 = keep all
  __shared__ uint32_t s_selcnt[16];
  __shared__ int s_any;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = blockIdx.x, bh = blockIdx.y;
  const int nqg = gridDim.x;
  const int nkt = (nkb + 15) >> 4;

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
    for (int k = 0; k < MAXT; ++k) kb[k] = ksw + ((size_t)(bh * nkt + min(w + 4 * k, nkt - 1)) * KS) * 64 + lane;
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
    const int j = 16 * (w + 4 * k) + jl;
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
    mx[v] = fmax(fmax(s_part[0][r], s_part[1][r]), fmax(s_part[2][r], s_part[3][r]));
  }

  // ---- e = exp(s - max) (in place), fixed-point masses, Z
  constexpr double kFix = 4503599627370496.0;  // 2^52
  unsigned long long zs[4] = {0, 0, 0, 0};
  double mn[4] = {1.0, 1.0, 1.0, 1.0};
#pragma unroll
  for (int k = 0; k < MAXT; ++k) {
    const int j = 16 * (w + 4 * k) + jl;
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
  if (tid < 16) {
    const int r = tid;
    const unsigned long long Z = s_zpart[0][r] + s_zpart[1][r] + s_zpart[2][r] + s_zpart[3][r];
    unsigned long long T = (unsigned long long)ceil(p * (double)Z);
    if (T > Z) T = Z;
    if (T < 1) T = 1;
    s_target[r] = T;
    // search range of keys (float64 bit patterns of e, monotone for e >= 0): [e_min, 1.0]
    const double emin = fmin(fmin(s_minpart[0][r], s_minpart[1][r]), fmin(s_minpart[2][r], s_minpart[3][r]));
    const unsigned long long lo = (unsigned long long)__double_as_longlong(emin);
    s_lo[r] = lo;
    s_width[r] = (unsigned long long)__double_as_longlong(1.0) + 1ull - lo;
    s_above[r] = 0;
    s_selcnt[r] = 0;
    const bool live = (16 * g + r) < nqb;
    s_state[r] = (!live || p >= 1.0) ? 3 : 0;
  }
  __syncthreads();

  // ---- radix select over the key range [lo, lo + width): each pass splits the range into
  // 256 equal digit bins (log-linear in e), finds the bin where the cumulative mass from the
  // top crosses the target, and narrows the range to that bin.  The first range spans the
  // row's own [e_min, 1], so elements spread over the bins instead of piling into a few.
  for (int pass = 0; pass < 8; ++pass) {
    if (tid == 0) {
      int any = 0;
      for (int r = 0; r < 16; ++r) any |= (s_state[r] == 0);
      s_any = any;
    }
    for (int r = 0; r < 16; ++r) {
      h_cnt[r][tid] = 0;
      h_mass[r][tid] = 0;
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
      const int j = 16 * (w + 4 * k) + jl;
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
    for (int rr = 0; rr < 4; ++rr) {
      const int r = 4 * w + rr;
      if (s_state[r] != 0) continue;  // uniform across the wave
      unsigned long long m4[4];
      uint32_t c4[4];
      unsigned long long ms = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        m4[q] = h_mass[r][4 * lane + q];
        c4[q] = h_cnt[r][4 * lane + q];
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
  for (int i = tid; i < 16 * kMaxNkw; i += 256) {
    (&s_kept[0][0])[i] = 0;
    (&s_ties[0][0])[i] = 0;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < MAXT; ++k) {
    const int j = 16 * (w + 4 * k) + jl;
    if (j < nkb) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = ig + 4 * v;
        const int st = s_state[r];
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
    const int j = 16 * (w + 4 * k) + jl;
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
  for (int rr = 0; rr < 4; ++rr) {
    const int r = 4 * w + rr;
    if (s_state[r] != 2) continue;
    const unsigned long long rem = s_target[r] - s_above[r];
    const unsigned long long mt = s_mt[r];
    const uint32_t ntie = s_selcnt[r];
    uint32_t need = (mt == 0) ? ntie : (uint32_t)min((unsigned long long)ntie, (rem + mt - 1) / mt);
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

  // ---- write counts, masks, loads (wave w: rows 4w..4w+3)
  for (int rr = 0; rr < 4; ++rr) {
    const int r = 4 * w + rr;
    const int i = 16 * g + r;
    if (i >= nqb) continue;
    const size_t row = (size_t)bh * nqb + i;
    uint32_t word = lane < nkw ? s_kept[r][lane] : 0u;
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
template <typename T>
static int launch_pool_t(const void *x, int BH, int N, int d, int block, int nb, int nbp, int layout,
                         double *out, int32_t *zero_me, int nzero, hipStream_t st) {
  const int nlim = layout ? nbp : nb;
  dim3 grid(nlim, BH);
  if (d == 128)
    hipLaunchKernelGGL((k_pool<T, 128>), grid, dim3(256), 0, st, (const T *)x, N, block, nb, nbp, layout,
                       out, zero_me, nzero);
  else
    hipLaunchKernelGGL((k_pool<T, 64>), grid, dim3(256), 0, st, (const T *)x, N, block, nb, nbp, layout,
                       out, zero_me, nzero);
  FV_CHECK_LAUNCH();
  return FVATTN_OK;
}

int launch_pool(const void *x, int BH, int N, int d, int dtype, int block, int layout, double *out,
                int32_t *zero_me, int nzero, hipStream_t st) {
  const int nb = cdiv(N, block);
  const int nbp = cdiv(nb, 16) * 16;
  if (dtype == FVATTN_BF16)
    return launch_pool_t<uint16_t>(x, BH, N, d, block, nb, nbp, layout, out, zero_me, nzero, st);
  return launch_pool_t<float>(x, BH, N, d, block, nb, nbp, layout, out, zero_me, nzero, st);
}

template <int D>
static int launch_select_d(const double *qsw, const double *ksw, int BH, int nqb, int nkb, double p,
                           int32_t *counts, uint32_t *bitmask, int nkw, int32_t *head_load, int32_t *bsum,
                           hipStream_t st) {
  const int nkt = cdiv(nkb, 16);
  const int per_wave = cdiv(nkt, 4);
  dim3 grid(cdiv(nqb, 16), BH);
  const double scale = 1.0 / sqrt((double)D);
#define FV_SEL(MT)                                                                             \
  hipLaunchKernelGGL((k_select<D, MT>), grid, dim3(256), 0, st, qsw, ksw, nqb, nkb, scale, p, counts, \
                     bitmask, nkw, head_load, bsum)
  if (per_wave <= 1) FV_SEL(1);
  else if (per_wave <= 2) FV_SEL(2);
  else if (per_wave <= 4) FV_SEL(4);
  else if (per_wave <= 8) FV_SEL(8);
  else if (per_wave <= 12) FV_SEL(12);
  else FV_SEL(20);
#undef FV_SEL
  FV_CHECK_LAUNCH();
  return FVATTN_OK;
}

int launch_select(const double *qsw, const double *ksw, int BH, int d, int nqb, int nkb, double p,
                  int32_t *counts, uint32_t *bitmask, int nkw, int32_t *head_load, int32_t *bsum, hipStream_t st) {
  if (d == 128) return launch_select_d<128>(qsw, ksw, BH, nqb, nkb, p, counts, bitmask, nkw, head_load, bsum, st);
  return launch_select_d<64>(qsw, ksw, BH, nqb, nkb, p, counts, bitmask, nkw, head_load, bsum, st);
}

int launch_csr(const int32_t *counts, const uint32_t *bitmask, const int32_t *bsum, int rows, int nkw, int nkb,
               int32_t *row_ptr, int32_t *col_idx, hipStream_t st) {
  hipLaunchKernelGGL(k_csr, dim3(cdiv(rows, 64)), dim3(256), 0, st, counts, bitmask, bsum, rows, nkw, nkb, row_ptr,
                     col_idx);
  FV_CHECK_LAUNCH();
  return FVATTN_OK;
}

}  // namespace fv
