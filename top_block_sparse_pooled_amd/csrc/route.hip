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
//                order independent.  The descending order is never materialised: an MSB-first
//                8-bit radix select over the float64 bit pattern of e (monotone for e > 0)
//                walks the mass histogram from the largest digit down and stops at the digit
//                where the cumulative mass crosses p * Z.  That gives exactly the shortest
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
  constexpr int BPW = 4;                      // blocks per workgroup
  constexpr int MAXR = (128 + RPR - 1) / RPR; // rounds for the largest block (128)
  __shared__ double red[RPR][D + 1];

  const int tid = threadIdx.x;
  const int bh = blockIdx.y;
  const int ch = tid % CPR, r0 = tid / CPR;
  if (zero_me != nullptr && blockIdx.x == 0 && bh == 0)
    for (int i = tid; i < nzero; i += 256) zero_me[i] = 0;

  const T *xh = x + (size_t)bh * N * D;
  const int nlim = layout ? nbp : nb;
  for (int jb = 0; jb < BPW; ++jb) {
    const int j = blockIdx.x * BPW + jb;
    if (j >= nlim) break;
    const int s = j * block;
    const int e = min(s + block, N);
    double acc[EPC];
#pragma unroll
    for (int t = 0; t < EPC; ++t) acc[t] = 0.0;
    if (j < nb) {
      u32x4 buf[MAXR];
#pragma unroll
      for (int k = 0; k < MAXR; ++k) {
        const int r = s + r0 + k * RPR;
        if (k * RPR < block && r < e)
          buf[k] = *reinterpret_cast<const u32x4 *>(xh + (size_t)r * D + ch * EPC);
      }
#pragma unroll
      for (int k = 0; k < MAXR; ++k) {
        const int r = s + r0 + k * RPR;
        if (k * RPR < block && r < e) {
          float f[EPC];
          unpack16(buf[k], f, T());
#pragma unroll
          for (int t = 0; t < EPC; ++t) acc[t] += (double)f[t];
        }
      }
    }
#pragma unroll
    for (int t = 0; t < EPC; ++t) red[r0][ch * EPC + t] = acc[t];
    __syncthreads();
    if (tid < D) {
      double sum = 0.0;
#pragma unroll 4
      for (int r = 0; r < RPR; ++r) sum += red[r][tid];
      const double mean = (j < nb) ? sum / (double)(e - s) : 0.0;
      if (layout)
        out[swz(bh, nbp / 16, D, j, tid)] = mean;
      else
        out[((size_t)bh * nb + j) * D + tid] = mean;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------
// k_select: scores, softmax, Top-p cut for 16 query blocks of one head.
// grid = (nqbp/16, BH), 256 threads.  MAXT = key tiles (of 16) per wave.
// Outputs counts[row] and the kept-bit mask bitmask[row][nkw]; adds loads to head_load.
// ---------------------------------------------------------------------------------------
constexpr int kMaxNkw = 40;  // 1280 key blocks

template <int D, int MAXT>
__global__ __launch_bounds__(256) void k_select(const double *__restrict__ qsw,
                                                const double *__restrict__ ksw, int nqb, int nkb,
                                                double scale, double p, int32_t *__restrict__ counts,
                                                uint32_t *__restrict__ bitmask, int nkw,
                                                int32_t *__restrict__ head_load) {
  constexpr int KS = D / 4;  // MFMA k-steps
  __shared__ uint32_t h_cnt[16][256];
  __shared__ unsigned long long h_mass[16][256];
  __shared__ uint32_t s_kept[16][kMaxNkw];
  __shared__ uint32_t s_ties[16][kMaxNkw];
  __shared__ double s_part[4][16];
  __shared__ unsigned long long s_zpart[4][16];
  __shared__ unsigned long long s_prefix[16], s_mask[16], s_above[16], s_target[16];
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
    double a[KS];
    const double *qa = qsw + ((size_t)(bh * nqg + g) * KS) * 64 + lane;
#pragma unroll
    for (int s = 0; s < KS; ++s) a[s] = qa[s * 64];
#pragma unroll
    for (int k = 0; k < MAXT; ++k) {
      const int t = w + 4 * k;
      if (t < nkt) {
        const double *kb = ksw + ((size_t)(bh * nkt + t) * KS) * 64 + lane;
#pragma unroll
        for (int s = 0; s < KS; ++s) acc[k] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[s], kb[s * 64], acc[k], 0, 0, 0);
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
#pragma unroll
  for (int k = 0; k < MAXT; ++k) {
    const int j = 16 * (w + 4 * k) + jl;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const double e = (j < nkb) ? exp(acc[k][v] - mx[v]) : 0.0;
      acc[k][v] = e;
      zs[v] += (unsigned long long)(e * kFix);
    }
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) {
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) zs[v] += __shfl_xor(zs[v], off, 16);
    if (jl == 0) s_zpart[w][ig + 4 * v] = zs[v];
  }
  __syncthreads();
  if (tid < 16) {
    const int r = tid;
    const unsigned long long Z = s_zpart[0][r] + s_zpart[1][r] + s_zpart[2][r] + s_zpart[3][r];
    unsigned long long T = (unsigned long long)ceil(p * (double)Z);
    if (T > Z) T = Z;
    if (T < 1) T = 1;
    s_target[r] = T;
    s_prefix[r] = 0;
    s_mask[r] = 0;
    s_above[r] = 0;
    s_selcnt[r] = 0;
    const bool live = (16 * g + r) < nqb;
    s_state[r] = (!live || p >= 1.0) ? 3 : 0;
  }
  __syncthreads();

  // ---- radix select, 8 bits per pass from the most significant byte
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
    const int shift = 56 - 8 * pass;
    unsigned long long pre[4], msk[4];
    bool act[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = ig + 4 * v;
      pre[v] = s_prefix[r];
      msk[v] = s_mask[r];
      act[v] = s_state[r] == 0;
    }
#pragma unroll
    for (int k = 0; k < MAXT; ++k) {
      const int j = 16 * (w + 4 * k) + jl;
      if (j < nkb) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const unsigned long long key = (unsigned long long)__double_as_longlong(acc[k][v]);
          if (act[v] && (key & msk[v]) == pre[v]) {
            const int dg = (int)((key >> shift) & 255ull);
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
      uint32_t cs = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        m4[q] = h_mass[r][4 * lane + q];
        c4[q] = h_cnt[r][4 * lane + q];
        ms += m4[q];
        cs += c4[q];
      }
      // exclusive suffix sums over lanes (higher lanes hold larger digits)
      unsigned long long sm = ms;
      uint32_t sc = cs;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const unsigned long long om = __shfl_down(sm, off);
        const uint32_t oc = __shfl_down(sc, off);
        if (lane + off < 64) {
          sm += om;
          sc += oc;
        }
      }
      unsigned long long above_m = sm - ms;  // mass of digits held by higher lanes
      uint32_t above_c = sc - cs;
      const unsigned long long base = s_above[r];
      const unsigned long long T = s_target[r];
      for (int q = 3; q >= 0; --q) {
        const unsigned long long lo = base + above_m;
        if (m4[q] > 0 && lo < T && T <= lo + m4[q]) {
          s_above[r] = lo;
          s_prefix[r] = s_prefix[r] | ((unsigned long long)(4 * lane + q) << shift);
          s_mask[r] = s_mask[r] | (255ull << shift);
          s_selcnt[r] = c4[q];
          if (c4[q] == 1) s_state[r] = 1;
          else if (shift == 0) s_state[r] = 2;
        }
        above_m += m4[q];
        above_c += c4[q];
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
        const unsigned long long mk = key & s_mask[r];
        const uint32_t bit = 1u << (j & 31);
        if (st == 3 || mk > s_prefix[r] || (mk == s_prefix[r] && st == 1))
          atomicOr(&s_kept[r][j >> 5], bit);
        else if (mk == s_prefix[r] && st == 2)
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
    }
  }
}

// ---------------------------------------------------------------------------------------
// k_csr: row_ptr (exclusive scan of counts) and ascending col_idx from the kept masks.
// grid = cdiv(rows, 1024), 1024 threads.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_csr(const int32_t *__restrict__ counts,
                                              const uint32_t *__restrict__ bitmask, int rows, int nkw,
                                              int32_t *__restrict__ row_ptr,
                                              int32_t *__restrict__ col_idx) {
  __shared__ int s_red[16];
  __shared__ int s_scan[16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r0 = blockIdx.x * 1024;
  // sum of all counts before this workgroup's rows
  int part = 0;
  for (int i = tid; i < r0; i += 1024) part += counts[i];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
  if (lane == 0) s_red[w] = part;
  __syncthreads();
  int base = 0;
  for (int i = 0; i < 16; ++i) base += s_red[i];
  // scan of this workgroup's counts
  const int row = r0 + tid;
  const int c = row < rows ? counts[row] : 0;
  int incl = c;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) s_scan[w] = incl;
  __syncthreads();
  int wbase = base;
  for (int i = 0; i < w; ++i) wbase += s_scan[i];
  const int rp = wbase + incl - c;
  if (row < rows) row_ptr[row] = rp;
  if (row == rows - 1) row_ptr[rows] = rp + c;
  // expand kept masks: the wave walks its 64 rows
  for (int k = 0; k < 64; ++k) {
    const int rk = r0 + 64 * w + k;
    if (rk >= rows) break;
    const int start = __shfl(rp, k);
    uint32_t word = lane < nkw ? bitmask[(size_t)rk * nkw + lane] : 0u;
    const int pc = __popc(word);
    int pincl = pc;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(pincl, off);
      if (lane >= off) pincl += o;
    }
    int out = start + pincl - pc;
    while (word) {
      const int b = __ffs(word) - 1;
      col_idx[out++] = 32 * lane + b;
      word &= word - 1;
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
  dim3 grid(cdiv(nlim, 4), BH);
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
                           int32_t *counts, uint32_t *bitmask, int nkw, int32_t *head_load,
                           hipStream_t st) {
  const int nkt = cdiv(nkb, 16);
  const int per_wave = cdiv(nkt, 4);
  dim3 grid(cdiv(nqb, 16), BH);
  const double scale = 1.0 / sqrt((double)D);
#define FV_SEL(MT)                                                                             \
  hipLaunchKernelGGL((k_select<D, MT>), grid, dim3(256), 0, st, qsw, ksw, nqb, nkb, scale, p, counts, \
                     bitmask, nkw, head_load)
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
                  int32_t *counts, uint32_t *bitmask, int nkw, int32_t *head_load, hipStream_t st) {
  if (d == 128) return launch_select_d<128>(qsw, ksw, BH, nqb, nkb, p, counts, bitmask, nkw, head_load, st);
  return launch_select_d<64>(qsw, ksw, BH, nqb, nkb, p, counts, bitmask, nkw, head_load, st);
}

int launch_csr(const int32_t *counts, const uint32_t *bitmask, int rows, int nkw, int32_t *row_ptr,
               int32_t *col_idx, hipStream_t st) {
  hipLaunchKernelGGL(k_csr, dim3(cdiv(rows, 1024)), dim3(1024), 0, st, counts, bitmask, rows, nkw, row_ptr,
                     col_idx);
  FV_CHECK_LAUNCH();
  return FVATTN_OK;
}

}  // namespace fv
