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
//                persistent.  The workgroup pools the query blocks of its next item while it
//                resolves the rows of the current one (same summation order as k_pool), so
//                the raw Q reads overlap the radix passes; the first item is pooled before
//                the loop.  Scores
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
#include "routing.h"

namespace fv {

// ---------------------------------------------------------------------------------------
// Cross-lane steps without LDS traffic (DPP and the gfx950 lane swaps).  Only exact operations
// (max, min, integer sums) are regrouped, and float64 sums keep their pairs, so results are the
// same bits as with the shuffle butterflies.
// ---------------------------------------------------------------------------------------
template <int CTRL, int RM, int BM, bool BC>
__device__ __forceinline__ unsigned long long dpp64(unsigned long long x) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)x, CTRL, RM, BM, BC);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(x >> 32), CTRL, RM, BM, BC);
  return ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
}
template <int CTRL>
__device__ __forceinline__ double dppf64(double x) {
  return __longlong_as_double((long long)dpp64<CTRL, 0xf, 0xf, false>((unsigned long long)__double_as_longlong(x)));
}
// all-reduce over each row of 16 lanes: lane pairs 1 apart, 2 apart, the mirrored half-row,
// the mirrored row
__device__ __forceinline__ double row16_max(double x) {
  x = fmax(x, dppf64<0xb1>(x));
  x = fmax(x, dppf64<0x4e>(x));
  x = fmax(x, dppf64<0x141>(x));
  return fmax(x, dppf64<0x140>(x));
}
__device__ __forceinline__ double row16_min(double x) {
  x = fmin(x, dppf64<0xb1>(x));
  x = fmin(x, dppf64<0x4e>(x));
  x = fmin(x, dppf64<0x141>(x));
  return fmin(x, dppf64<0x140>(x));
}
__device__ __forceinline__ unsigned long long row16_sum(unsigned long long x) {
  x += dpp64<0xb1, 0xf, 0xf, false>(x);
  x += dpp64<0x4e, 0xf, 0xf, false>(x);
  x += dpp64<0x141, 0xf, 0xf, false>(x);
  return x + dpp64<0x140, 0xf, 0xf, false>(x);
}
// inclusive prefix sum over the 64 lanes: shifts by 1, 2, 4, 8 within rows of 16, then the
// last lane of a row into the next row (rows 1, 3) and lane 31 into rows 2, 3
__device__ __forceinline__ unsigned long long wave_scan(unsigned long long x) {
  x += dpp64<0x111, 0xf, 0xf, true>(x);
  x += dpp64<0x112, 0xf, 0xf, true>(x);
  x += dpp64<0x114, 0xf, 0xf, true>(x);
  x += dpp64<0x118, 0xf, 0xf, true>(x);
  x += dpp64<0x142, 0xa, 0xf, false>(x);
  return x + dpp64<0x143, 0xc, 0xf, false>(x);
}
__device__ __forceinline__ unsigned long long readlane64(unsigned long long x, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), l);
  return ((unsigned long long)hi << 32) | lo;
}
// the two values of the lane pair 16 or 32 apart (own and partner, in either order)
template <int OFF>
__device__ __forceinline__ void lane_pair(unsigned long long x, unsigned long long &p0, unsigned long long &p1) {
  static_assert(OFF == 16 || OFF == 32, "lane distance");
  const uint32_t lo = (uint32_t)x, hi = (uint32_t)(x >> 32);
  if constexpr (OFF == 16) {
    const auto sl = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto sh = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    p0 = ((unsigned long long)sh[0] << 32) | sl[0];
    p1 = ((unsigned long long)sh[1] << 32) | sl[1];
  } else {
    const auto sl = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    const auto sh = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    p0 = ((unsigned long long)sh[0] << 32) | sl[0];
    p1 = ((unsigned long long)sh[1] << 32) | sl[1];
  }
}
__device__ __forceinline__ double as_f64(unsigned long long x) { return __longlong_as_double((long long)x); }
__device__ __forceinline__ unsigned long long as_u64(double x) { return (unsigned long long)__double_as_longlong(x); }
// all-reduce over the 64 lanes: rows of 16, then the row pairs 16 and 32 apart
__device__ __forceinline__ double wave_max(double x) {
  unsigned long long a, b;
  x = row16_max(x);
  lane_pair<16>(as_u64(x), a, b);
  x = fmax(as_f64(a), as_f64(b));
  lane_pair<32>(as_u64(x), a, b);
  return fmax(as_f64(a), as_f64(b));
}
__device__ __forceinline__ double wave_min(double x) {
  unsigned long long a, b;
  x = row16_min(x);
  lane_pair<16>(as_u64(x), a, b);
  x = fmin(as_f64(a), as_f64(b));
  lane_pair<32>(as_u64(x), a, b);
  return fmin(as_f64(a), as_f64(b));
}
__device__ __forceinline__ unsigned long long wave_sum(unsigned long long x) {
  unsigned long long a, b;
  x = row16_sum(x);
  lane_pair<16>(x, a, b);
  x = a + b;
  lane_pair<32>(x, a, b);
  return a + b;
}
// x + (x of the lane 8, 16 or 32 apart), in the same pairs as a shuffle butterfly
template <int OFF>
__device__ __forceinline__ double add_xor(double x) {
  static_assert(OFF == 8 || OFF == 16 || OFF == 32, "lane distance");
  if constexpr (OFF == 8) {
    return x + dppf64<0x128>(x);   // row_ror:8 within a row of 16
  } else {
    const uint32_t lo = (uint32_t)__double_as_longlong(x), hi = (uint32_t)((unsigned long long)__double_as_longlong(x) >> 32);
    uint32_t a0, a1, b0, b1;
    if constexpr (OFF == 16) {
      const auto sl = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
      const auto sh = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
      a0 = sl[0], a1 = sl[1], b0 = sh[0], b1 = sh[1];
    } else {
      const auto sl = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
      const auto sh = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
      a0 = sl[0], a1 = sl[1], b0 = sh[0], b1 = sh[1];
    }
    return __longlong_as_double((long long)(((unsigned long long)b0 << 32) | a0)) +
           __longlong_as_double((long long)(((unsigned long long)b1 << 32) | a1));
  }
}

// ---------------------------------------------------------------------------------------
// k_pool: x [BH][N][D] -> mean of every block of `block` tokens (real tokens only), for one
// or two tensors (Q and K) in one launch.  Item = 16 consecutive blocks of one head of one
// tensor; grid = (groups of tensor 0 + groups of tensor 1, BH), 256 threads.  Wave w pools
// blocks w, w+4, w+8, w+12 of the group: lane l reads 16-byte chunk l % CPR of rows
// l / CPR + RPL*i (16 loads in flight per lane), accumulates in float64 and the lanes of a
// chunk are summed across lanes (DPP and lane swaps).  The 16 pooled rows are staged in LDS and
// written as one contiguous run: layout 1 is the swizzled float64 MFMA operand order of
// k_select (blocks past nb written as zero), layout 0 the plain [BH][nb][D] array.
// ---------------------------------------------------------------------------------------
struct PoolArgs {
  const void *x[2];
  double *out[2];
  int block[2], nb[2], ngrp[2];   // ngrp = ceil(nb / 16); ngrp[1] = 0 for one tensor
  int N, layout;
  int32_t *zero[3];               // zeroed by workgroup (0, 0) (may be null)
  int nzero[3];
};

// Means of the real tokens of NBK blocks j0, j0 + js, ... (block j: tokens [j block,
// min(j block + block, N))) of one head's rows xh, by one wave: lane l reads 16-byte chunk
// l % CPR of rows l / CPR + RPL i of every block (NBK x 16 loads in flight per lane),
// accumulates in float64, and the lanes of a chunk are summed by lane swaps.  Lanes
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
    for (int e = 0; e < EPC; ++e) {
      if constexpr (CPR <= 8) acc[b][e] = add_xor<8>(acc[b][e]);
      if constexpr (CPR <= 16) acc[b][e] = add_xor<16>(acc[b][e]);
      acc[b][e] = add_xor<32>(acc[b][e]);
    }
    const int cnt = e0[b] - s0[b];
#pragma unroll
    for (int e = 0; e < EPC; ++e) mean[b][e] = cnt > 0 ? acc[b][e] / (double)cnt : 0.0;
  }
}

// One block's mean split in two steps, so that its loads can be in flight while other work
// runs: pool_issue starts round `base` (rows base .. base + RPR - 1 of the block) of the same
// loads as pool_blocks, pool_take adds them to the float64 sums.  pool_keep finishes the block
// (lane swaps, division by the real-token count) and leaves lane l with dims
// (l % CPR) EPC + (l / CPR) KEEP + k, k < KEEP = D / 64: every dim exactly once over the wave.
template <typename T, int D>
struct PoolGeo {
  static constexpr int EPC = DT<T>::per16, CPR = D / EPC, RPL = 64 / CPR, NLD = 16, RPR = RPL * NLD;
  static constexpr int KEEP = D / 64;
};
template <typename T, int D>
__device__ __forceinline__ void pool_issue(const T *__restrict__ xh, int j, int block, int nb, int N, int base,
                                           u32x4 (&buf)[PoolGeo<T, D>::NLD]) {
  using P = PoolGeo<T, D>;
  const int lane = threadIdx.x & 63;
  const int c = lane % P::CPR, r = lane / P::CPR;
  const int s0 = j < nb ? j * block : 0, e0 = j < nb ? min(s0 + block, N) : 0;
#pragma unroll
  for (int i = 0; i < P::NLD; ++i) {
    const int row = s0 + base + r + P::RPL * i;
    buf[i] = u32x4{0u, 0u, 0u, 0u};
    if (row < e0) buf[i] = *reinterpret_cast<const u32x4 *>(xh + (size_t)row * D + c * P::EPC);
  }
}
template <typename T, int D>
__device__ __forceinline__ void pool_take(const u32x4 (&buf)[PoolGeo<T, D>::NLD], double (&acc)[PoolGeo<T, D>::EPC]) {
  using P = PoolGeo<T, D>;
#pragma unroll
  for (int i = 0; i < P::NLD; ++i) {
    float f[P::EPC];
    unpack16(buf[i], f, T());
#pragma unroll
    for (int e = 0; e < P::EPC; ++e) acc[e] += (double)f[e];
  }
}
template <typename T, int D>
__device__ __forceinline__ void pool_keep(int j, int block, int nb, int N, double (&acc)[PoolGeo<T, D>::EPC],
                                          double (&keep)[PoolGeo<T, D>::KEEP]) {
  using P = PoolGeo<T, D>;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int e = 0; e < P::EPC; ++e) {
    if constexpr (P::CPR <= 8) acc[e] = add_xor<8>(acc[e]);
    if constexpr (P::CPR <= 16) acc[e] = add_xor<16>(acc[e]);
    acc[e] = add_xor<32>(acc[e]);
  }
  const int s0 = j < nb ? j * block : 0, e0 = j < nb ? min(s0 + block, N) : 0;
  const int cnt = e0 - s0;
  const int sel = (lane / P::CPR) * P::KEEP;
#pragma unroll
  for (int k = 0; k < P::KEEP; ++k) {
    double x = acc[0];
#pragma unroll
    for (int e = 1; e < P::EPC; ++e) x = (sel + k == e) ? acc[e] : x;
    keep[k] = cnt > 0 ? x / (double)cnt : 0.0;
  }
}
// The whole block at once (its rounds one after the other).
template <typename T, int D>
__device__ __forceinline__ void pool_block_keep(const T *__restrict__ xh, int j, int block, int nb, int N,
                                                double (&keep)[PoolGeo<T, D>::KEEP]) {
  using P = PoolGeo<T, D>;
  double acc[P::EPC];
#pragma unroll
  for (int e = 0; e < P::EPC; ++e) acc[e] = 0.0;
  for (int base = 0; base < block; base += P::RPR) {
    u32x4 buf[P::NLD];
    pool_issue<T, D>(xh, j, block, nb, N, base, buf);
    pool_take<T, D>(buf, acc);
  }
  pool_keep<T, D>(j, block, nb, N, acc, keep);
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
    for (int z = 0; z < 3; ++z)
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
// Kept-bit words of a row: word wi (key blocks 32 wi .. 32 wi + 31) is held by lane wi % 64 in
// its register wi / 64; two registers cover 4096 key blocks.
constexpr int kRowWords = 2;

constexpr double kFix52 = 4503599627370496.0;  // 2^52: masses as fixed point

// A softmax numerator e in [0, 1] as 2^-52 fixed point, rounded to nearest: e 2^52 + 2^52 lies in
// [2^52, 2^53], where the float64 spacing is 1, so its bit pattern minus that of 2^52 is the
// rounded integer (2^53 gives 2^52).  One FMA and a 64-bit subtract.
__device__ __forceinline__ unsigned long long fix52(double e) {
  return (unsigned long long)__double_as_longlong(fma(e, kFix52, kFix52)) - 0x4330000000000000ull;
}


// Kept set of one row by the wave: the shortest prefix of the (e descending, index ascending)
// order whose mass (bycnt = false: fixed-point e, target T) or count (bycnt = true, target T)
// reaches T.  ev[t] is e of key block lane + 64 t; valid below nkb.  Search range of keys (the
// float64 bit patterns of e, monotone for e >= 0): [lo0, bits(1.0)].  Each radix pass splits
// the range into 256 digit bins, walks the histogram from the largest digit down to the bin
// where the cumulative mass from the top reaches T, and narrows the range to that bin, until
// the bin holds one key or one key value (ties, resolved toward lower indices).  Returns the
// kept-bit word of key blocks 32 lane .. 32 lane + 31 (zero for lanes past the row) and sets
// `count` to the number of kept blocks.
// A row of softmax numerators (lane l: key block l + 64 t): entries t < kRegs in registers,
// the rest in memory (the large select's scratch), read again on every pass.
template <int NPL>
struct RegRow {
  static constexpr int kRegs = NPL;
  const double (&v)[NPL];
  __device__ __forceinline__ double reg(int t) const { return v[t]; }
  __device__ __forceinline__ double mem(int) const { return 0.0; }
};
template <int R>
struct SplitRow {
  static constexpr int kRegs = R;
  const double (&v)[R];
  const double *p;
  __device__ __forceinline__ double reg(int t) const { return v[t]; }
  __device__ __forceinline__ double mem(int t) const { return p[(threadIdx.x & 63) + 64 * t]; }
};
struct MemRow {
  static constexpr int kRegs = 0;
  const double *p;
  __device__ __forceinline__ double reg(int) const { return 0.0; }
  __device__ __forceinline__ double mem(int t) const { return p[(threadIdx.x & 63) + 64 * t]; }
};
// f(t, valid, e) over the NPL entries of this lane, in order of t; e is 0 past the row (whose
// entries are never read)
template <int NPL, class Row, class F>
__device__ __forceinline__ void for_row(const Row &ev, int nkb, F &&f) {
  const int lane = threadIdx.x & 63;
  constexpr int R = Row::kRegs < NPL ? Row::kRegs : NPL;
#pragma unroll
  for (int t = 0; t < R; ++t) {
    const bool valid = lane + 64 * t < nkb;
    f(t, valid, valid ? ev.reg(t) : 0.0);
  }
#pragma unroll 4
  for (int t = R; t < NPL; ++t) {
    const bool valid = lane + 64 * t < nkb;
    f(t, valid, valid ? ev.mem(t) : 0.0);
  }
}

template <int NPL, class Row>
__device__ __forceinline__ void select_row(const Row &ev, int nkb, bool bycnt, unsigned long long T,
                                           unsigned long long lo0, bool keep_all,
                                           unsigned long long *__restrict__ hm, uint32_t *__restrict__ hc,
                                           uint32_t *__restrict__ status, uint32_t (&words)[kRowWords], int &count) {
  static_assert(NPL <= 32 * kRowWords, "row longer than the kept-word registers");
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
    for_row<NPL>(ev, nkb, [&](int, bool valid, double e) {
      const unsigned long long off = (unsigned long long)__double_as_longlong(e) - lo;
      if (valid && off < width) {
        const int dg = (int)(off >> sh);
        atomicAdd(&hc[dg], 1u);
        if (!bycnt) atomicAdd(&hm[dg], fix52(e));
      }
    });
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
    // mass of the digits held by higher lanes (larger keys): the total minus the inclusive
    // prefix over the lanes
    const unsigned long long pre = wave_scan(ms);
    unsigned long long acc = above + (readlane64(pre, 63) - pre);
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
    if (bal == 0ull) {   // not expected: the range always holds the crossing.  Flag it and keep the row whole
      if (lane == 0) atomicOr(status, (uint32_t)FVATTN_STATUS_SELECT_NOCROSS);
      st = 3;
      break;
    }
    const int L = __ffsll((long long)bal) - 1;
    dig = __builtin_amdgcn_readlane(dig, L);
    above = readlane64(nab, L);
    cnt = (uint32_t)__builtin_amdgcn_readlane((int)cnt, L);
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
    const unsigned long long mt = fix52(__longlong_as_double((long long)lo));
    if (bycnt) need = (uint32_t)min((unsigned long long)ntie, rem);
    else need = mt == 0 ? ntie : (uint32_t)min((unsigned long long)ntie, (rem + mt - 1) / mt);
  }
  uint32_t cum = 0;   // ties taken so far (ascending key block)
#pragma unroll
  for (int q = 0; q < kRowWords; ++q) words[q] = 0u;
  count = 0;
  for_row<NPL>(ev, nkb, [&](int t, bool valid, double e) {
    const unsigned long long key = (unsigned long long)__double_as_longlong(e);
    bool keep = valid && (st == 3 || key >= hi || (st == 1 && key >= lo));
    if (st == 2) {
      const bool tie = valid && key == lo;
      const unsigned long long bt = __ballot(tie);
      const uint32_t rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(bt >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bt, 0u));
      keep = keep || (tie && cum + rank < need);
      cum += (uint32_t)__popcll(bt);
    }
    const unsigned long long mt = __ballot(keep);
    // key blocks 64 t .. 64 t + 63 are words 2 t and 2 t + 1
    if (lane == (2 * t) % 64) words[(2 * t) / 64] = (uint32_t)mt;
    if (lane == (2 * t + 1) % 64) words[(2 * t + 1) / 64] = (uint32_t)(mt >> 32);
    count += (int)__popcll(mt);
  });
}

// Arguments of one select item.
struct SelArgs {
  const void *qraw;
  const double *ksw;
  int nqb, nkb, nkw;
  double scale, p;
  int32_t *counts;
  uint32_t *bitmask;
  int32_t *head_load, *bsum;
  SelOpts sel;
  uint32_t *status;
};

// The kept set of one row from its softmax numerators ev (lane l: key block l + 64 t), their
// fixed-point sum Z and minimum emin: the Top-p cut (or a routing variant), the kept-bit words
// written to bitmask, the count to counts and *cnt_out (lane 0), and for SASA the importance of
// every block.  hm / hc: the wave's radix histograms.
template <int NPL, bool EXT, class Row>
__device__ __forceinline__ void row_decide(const Row &ev, unsigned long long Z, double emin, int i,
                                           size_t row, const SelArgs &a, unsigned long long *__restrict__ hm,
                                           uint32_t *__restrict__ hc, int *cnt_out) {
  const int lane = threadIdx.x & 63;
  const int nkb = a.nkb, nkw = a.nkw;
  const unsigned long long lo0 = (unsigned long long)__double_as_longlong(emin);
  // search by mass (Top-p) or by count (top-k, or a clamped Top-p count)
  bool bycnt = false;
  unsigned long long tgt0;
  bool all;
  if (EXT && a.sel.mode == FVATTN_ROUTE_TOPK) {
    bycnt = true;
    tgt0 = (unsigned long long)a.sel.topk;
    all = a.sel.topk >= nkb;
  } else {
    tgt0 = (unsigned long long)ceil(a.p * (double)Z);
    if (tgt0 > Z) tgt0 = Z;
    if (tgt0 < 1) tgt0 = 1;
    all = a.p >= 1.0;
  }
  int c;
  uint32_t words[kRowWords];
  select_row<NPL>(ev, nkb, bycnt, tgt0, lo0, all, hm, hc, a.status, words, c);
  if (EXT && !bycnt && (a.sel.k_min > 1 || a.sel.k_max > 0)) {
    // clamp of the Top-p count: re-select by count when it lies outside [k_min, k_max]
    int tgt = max(c, a.sel.k_min);
    if (a.sel.k_max > 0) tgt = min(tgt, a.sel.k_max);
    tgt = min(tgt, nkb);
    if (tgt != c)
      select_row<NPL>(ev, nkb, true, (unsigned long long)tgt, lo0, tgt >= nkb, hm, hc, a.status,
                      words, c);
  }
  if (EXT && a.sel.window > 0) {
    // local window: key blocks within `window` of those overlapping the query block's tokens
    const int t0 = i * a.sel.bq, t1 = min(t0 + a.sel.bq, a.sel.N) - 1;
    const int ja = max(0, t0 / a.sel.bk - a.sel.window), jb = min(nkb - 1, t1 / a.sel.bk + a.sel.window);
    c = 0;
#pragma unroll
    for (int q = 0; q < kRowWords; ++q) {
      const int wi = lane + 64 * q;
      const int lo_j = max(ja, 32 * wi), hi_j = min(jb, 32 * wi + 31);
      if (wi < nkw && lo_j <= hi_j) {
        const int nbits = hi_j - lo_j + 1;
        words[q] |= (nbits == 32 ? 0xffffffffu : ((1u << nbits) - 1u)) << (lo_j - 32 * wi);
      }
      c += __popc(words[q]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) c += __shfl_xor(c, off);
  }
#pragma unroll
  for (int q = 0; q < kRowWords; ++q)
    if (lane + 64 * q < nkw) a.bitmask[row * nkw + lane + 64 * q] = words[q];
  if (lane == 0) {
    a.counts[row] = c;
    *cnt_out = c;
  }
  if (EXT && a.sel.imp != nullptr) {
    // importance of every block: the candidates' order for SASA
    const double invz = Z > 0 ? kFix52 / (double)Z : 0.0;   // 1 / Z with Z in 2^-52 units
    for_row<NPL>(ev, nkb, [&](int t, bool valid, double e) {
      if (valid) a.sel.imp[row * nkb + lane + 64 * t] = e * invz;
    });
  }
}

// LDS of a select workgroup: NWV waves, MAXT key tiles of 16 per wave.
template <typename T, int D, int MAXT, int NWV>
struct SelLds {
  static constexpr int KCAP = 16 * NWV * MAXT;   // key blocks the tiles cover
  static constexpr int RB = NWV == 4 ? 16 : 8;   // rows staged at once
  // staged rows; before them, the item's pooled query blocks (16 D doubles)
  static constexpr int ESZ = RB * KCAP > 16 * D ? RB * KCAP : 16 * D;
  double eq[ESZ];
  unsigned long long h_mass[NWV][256];
  uint32_t h_cnt[NWV][256];
  double part[NWV][16];
  unsigned long long zpart[NWV][16];
  double minpart[NWV][16];
  int cnt[16];   // kept counts of the item's rows
};

// One select item: scores, softmax and the Top-p cut (or a routing variant) for query blocks
// 16 g .. 16 g + 15 of head bh, by the whole workgroup.
//   1. The item's query blocks, pooled during the previous item's row phase (or before the
//      first item), are written from registers into LDS.
//   2. Scores for the 16 rows on the float64 MFMA, wave w holding key tiles w, w + NWV, ...;
//      row maxima, e = exp(s - max), fixed-point row sums Z and row minima of e across the
//      waves (two workgroup barriers).
//   3. The e values go to LDS as whole rows (RB rows at a time), and each wave then resolves
//      its rows alone: the row's values sit in registers (lane l: key blocks l + 64 t), the
//      radix passes use a histogram private to the wave, and the kept set leaves as 64-bit
//      ballots.  No workgroup barrier inside the selection.
// Outputs counts[row] and the kept-bit mask bitmask[row][nkw]; adds loads to head_load and bsum.
// pq holds this item's pooled query blocks (this wave's: w, w + NWV, ...) on entry and the next
// item's (head bhn, group gn) on return; bhn < 0: no next item.
template <typename T, int D, int MAXT, int NWV, bool EXT>
__device__ __forceinline__ void select_item(SelLds<T, D, MAXT, NWV> &L, const SelArgs &a, int bh, int g,
                                            double (&pq)[16 / NWV][PoolGeo<T, D>::KEEP], int bhn, int gn) {
  constexpr int KS = D / 4;               // MFMA k-steps
  constexpr int KCAP = SelLds<T, D, MAXT, NWV>::KCAP;
  constexpr int NPL = KCAP / 64;          // values per lane in the row phase
  constexpr int RB = SelLds<T, D, MAXT, NWV>::RB;
  constexpr int NB = 16 / RB;
  constexpr int RPW = RB / NWV;           // rows per wave per batch
  static_assert(KCAP % 64 == 0 && RB % NWV == 0 && (RB / 4) * 4 == RB, "row phase geometry");
  double(*s_e)[KCAP] = reinterpret_cast<double(*)[KCAP]>(L.eq);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nqb = a.nqb, nkb = a.nkb;
  const int nkt = (nkb + 15) >> 4;
  (void)tid;

  // ---- the item's 16 query blocks, pooled during the previous item's row phase (this wave:
  // blocks w, w + NWV, ...), into LDS in the float64 MFMA operand order (block jj, dim c at
  // (c / 4) 64 + jj + 16 (c % 4))
  {
    using P = PoolGeo<T, D>;
#pragma unroll
    for (int k = 0; k < 16 / NWV; ++k) {
      const int jj = w + NWV * k;
#pragma unroll
      for (int kk = 0; kk < P::KEEP; ++kk) {
        const int cc = (lane % P::CPR) * P::EPC + (lane / P::CPR) * P::KEEP + kk;
        L.eq[(cc >> 2) * 64 + jj + 16 * (cc & 3)] = pq[k][kk];
      }
    }
  }
  __syncthreads();

  // ---- scores: S[i][j] = sum_c qbar[i][c] * kbar[j][c], i = lane/16 + 4v, j = 16t + lane%16
  d4 acc[MAXT];
#pragma unroll
  for (int k = 0; k < MAXT; ++k) acc[k] = d4{0.0, 0.0, 0.0, 0.0};
  {
    const double *qa = L.eq + lane;
    // k-step outer, tiles inner: MAXT independent accumulators.  The operands of PF k-steps
    // (one of qbar, MAXT of kbar each) are in flight ahead of the MFMAs that use them, which
    // covers the L2 latency of the pooled keys.  Tiles past the last read a valid tile (their
    // key columns are >= nkb and ignored below), so the loop has no branches.
    constexpr int PF = MAXT >= 8 ? 1 : 3;
    const double *kb[MAXT];
#pragma unroll
    for (int k = 0; k < MAXT; ++k) kb[k] = a.ksw + ((size_t)(bh * nkt + min(w + NWV * k, nkt - 1)) * KS) * 64 + lane;
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
      acc[k][v] *= a.scale;
      if (j < nkb) mx[v] = fmax(mx[v], acc[k][v]);
    }
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    mx[v] = row16_max(mx[v]);
    if (jl == 0) L.part[w][ig + 4 * v] = mx[v];
  }
  __syncthreads();
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int r = ig + 4 * v;
    double m = L.part[0][r];
#pragma unroll
    for (int ww = 1; ww < NWV; ++ww) m = fmax(m, L.part[ww][r]);
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
      zs[v] += fix52(e);
      if (j < nkb) mn[v] = fmin(mn[v], e);
    }
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    zs[v] = row16_sum(zs[v]);
    mn[v] = row16_min(mn[v]);
    if (jl == 0) {
      L.zpart[w][ig + 4 * v] = zs[v];
      L.minpart[w][ig + 4 * v] = mn[v];
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
    // ---- selection: wave w resolves rows b RB + rr NWV + w; beside each row it pools one
    // of its blocks of the next item (its loads in flight during the row's radix passes)
    for (int rr = 0; rr < RPW; ++rr) {
      const int r = b * RB + rr * NWV + w;
      const int i = 16 * g + r;
      using P = PoolGeo<T, D>;
      const int jn = 16 * gn + w + NWV * (b * RPW + rr);   // next item's block (query block index)
      const T *xn = reinterpret_cast<const T *>(a.qraw) + (size_t)(bhn < 0 ? 0 : bhn) * a.sel.N * D;
      u32x4 pbuf[P::NLD];
      if (bhn >= 0) pool_issue<T, D>(xn, jn, a.sel.bq, nqb, a.sel.N, 0, pbuf);
      if (i < nqb) {   // wave-uniform
        const size_t row = (size_t)bh * nqb + i;
        double ev[NPL];
#pragma unroll
        for (int t = 0; t < NPL; ++t) ev[t] = s_e[r - b * RB][lane + 64 * t];
        unsigned long long Z = 0;
        double emin = 1.0;
#pragma unroll
        for (int ww = 0; ww < NWV; ++ww) {
          Z += L.zpart[ww][r];
          emin = fmin(emin, L.minpart[ww][r]);
        }
        row_decide<NPL, EXT>(RegRow<NPL>{ev}, Z, emin, i, row, a, L.h_mass[w], L.h_cnt[w], &L.cnt[r]);
      } else if (lane == 0) {
        L.cnt[r] = 0;
      }
      if (bhn >= 0) {
        double pacc[P::EPC];
#pragma unroll
        for (int e = 0; e < P::EPC; ++e) pacc[e] = 0.0;
        pool_take<T, D>(pbuf, pacc);
        for (int base = P::RPR; base < a.sel.bq; base += P::RPR) {   // blocks longer than one round
          pool_issue<T, D>(xn, jn, a.sel.bq, nqb, a.sel.N, base, pbuf);
          pool_take<T, D>(pbuf, pacc);
        }
        // rotate: after all of this wave's rows, pq[k] holds block w + NWV k
#pragma unroll
        for (int k = 0; k + 1 < 16 / NWV; ++k)
#pragma unroll
          for (int kk = 0; kk < P::KEEP; ++kk) pq[k][kk] = pq[k + 1][kk];
        pool_keep<T, D>(jn, a.sel.bq, nqb, a.sel.N, pacc, pq[16 / NWV - 1]);
      }
    }
    __syncthreads();   // staged rows and partial sums consumed before they are overwritten
  }
  if (w == 0) {
    // the item's load of the head and its per-64-row sums for the CSR scan (the 16 rows
    // span at most two 64-row blocks)
    const size_t row0 = (size_t)bh * nqb + 16 * g;
    const int c = lane < 16 ? L.cnt[lane] : 0;
    const bool second = lane < 16 && ((row0 + lane) >> 6) != (row0 >> 6);
    int c0 = second ? 0 : c, c1 = second ? c : 0;
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) {
      c0 += __shfl_xor(c0, off);
      c1 += __shfl_xor(c1, off);
    }
    if (lane == 0) {
      atomicAdd(&a.head_load[bh], c0 + c1);
      atomicAdd(&a.bsum[row0 >> 6], c0);
      if (c1 != 0) atomicAdd(&a.bsum[(row0 >> 6) + 1], c1);
    }
  }
}

// Persistent select over all items (head bh, group g of 16 query blocks).  Workgroup b runs on
// XCD b % 8 (round-robin dispatch); XCD x owns the x-th eighth of the items in head-major
// order, so its L2 holds the pooled keys of only a few heads.  gridDim.x >= 8.
template <typename T, int D, int MAXT, int NWV, bool EXT>
__global__ __launch_bounds__(64 * NWV, NWV == 4 ? 2 : 1) void k_select(SelArgs a, int BH) {
  __shared__ SelLds<T, D, MAXT, NWV> L;
  const int nqg = (a.nqb + 15) >> 4;
  const int items = BH * nqg;
  const int xcd = blockIdx.x & 7;
  const int nwx = ((int)gridDim.x - xcd + 7) >> 3;
  const int it_end = (int)((long long)items * (xcd + 1) / 8);
  const int it0 = (int)((long long)items * xcd / 8) + (int)(blockIdx.x >> 3);
  // the first item's query blocks, pooled here; each item pools the next one's
  double pq[16 / NWV][PoolGeo<T, D>::KEEP];
  if (it0 < it_end) {
    const int bh = it0 / nqg, g = it0 - bh * nqg;
    const T *xh = reinterpret_cast<const T *>(a.qraw) + (size_t)bh * a.sel.N * D;
    const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
#pragma unroll
    for (int k = 0; k < 16 / NWV; ++k) pool_block_keep<T, D>(xh, 16 * g + w + NWV * k, a.sel.bq, a.nqb, a.sel.N, pq[k]);
  }
  for (int it = it0; it < it_end; it += nwx) {
    const int bh = it / nqg, g = it - bh * nqg;
    const int itn = it + nwx;
    const int bhn = itn < it_end ? itn / nqg : -1, gn = itn < it_end ? itn - (itn / nqg) * nqg : 0;
    select_item<T, D, MAXT, NWV, EXT>(L, a, bh, g, pq, bhn, gn);
  }
}

// ---------------------------------------------------------------------------------------
// Select for more than 1280 key blocks (up to 4096): 8 waves; the scores of an item's 16 rows are
// computed in chunks of 1024 key blocks (8 tiles of 16 per wave, the same float64 MFMA sequence
// as the select above) and stored, scaled, to a scratch of 16 rows owned by the workgroup; each
// wave then takes whole rows: row maximum, e = exp(s - max) written back in place, fixed-point Z
// and minimum of e by wave reductions (the same values as the select above), and the radix
// selection reading the row from the scratch (L2-resident) in each pass.
// ---------------------------------------------------------------------------------------
template <typename T, int D>
struct SelLdsL {
  double eq[16 * D];   // the item's pooled query blocks (float64 MFMA operand order)
  unsigned long long h_mass[8][256];
  uint32_t h_cnt[8][256];
  int cnt[16];
};

constexpr int kLargeRegNpl = 40;     // rows of up to 2560 key blocks are resolved in registers
constexpr int kLargeSplitRegs = 32;  // longer rows keep their first 2048 entries there
template <typename T, int D, int NPL, bool EXT>
__device__ __forceinline__ void select_item_large(SelLdsL<T, D> &L, const SelArgs &a, double *__restrict__ scr,
                                                  int nkbp, int bh, int g) {
  constexpr int NWV = 8, MAXT = 8, KS = D / 4;
  constexpr int EPC = DT<T>::per16, CPR = D / EPC;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nqb = a.nqb, nkb = a.nkb;
  const int nkt = (nkb + 15) >> 4;
  {
    const T *xh = reinterpret_cast<const T *>(a.qraw) + (size_t)bh * a.sel.N * D;
    for (int jj = w; jj < 16; jj += NWV) {
      double m[1][EPC];
      pool_blocks<T, D, 1>(xh, 16 * g + jj, NWV, a.sel.bq, nqb, a.sel.N, m);
      if (lane < CPR) {
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          const int cc = lane * EPC + e;
          L.eq[(cc >> 2) * 64 + jj + 16 * (cc & 3)] = m[0][e];
        }
      }
    }
  }
  __syncthreads();
  const int jl = lane & 15, ig = lane >> 4;
  const double *qa = L.eq + lane;
  for (int c0 = 0; c0 < nkt; c0 += NWV * MAXT) {
    d4 acc[MAXT];
#pragma unroll
    for (int k = 0; k < MAXT; ++k) acc[k] = d4{0.0, 0.0, 0.0, 0.0};
    const double *kb[MAXT];
#pragma unroll
    for (int k = 0; k < MAXT; ++k)
      kb[k] = a.ksw + ((size_t)(bh * nkt + min(c0 + w + NWV * k, nkt - 1)) * KS) * 64 + lane;
    double abuf = qa[0], bbuf[MAXT];
#pragma unroll
    for (int k = 0; k < MAXT; ++k) bbuf[k] = kb[k][0];
    // k-steps in a rolled loop (an unrolled one lets the scheduler hoist the operand loads of
    // many steps and spill at d = 128)
#pragma unroll 2
    for (int s = 0; s < KS; ++s) {
      const double av = abuf;
      double b[MAXT];
#pragma unroll
      for (int k = 0; k < MAXT; ++k) b[k] = bbuf[k];
      if (s + 1 < KS) {
        abuf = qa[(s + 1) * 64];
#pragma unroll
        for (int k = 0; k < MAXT; ++k) bbuf[k] = kb[k][(s + 1) * 64];
      }
#pragma unroll
      for (int k = 0; k < MAXT; ++k) acc[k] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, b[k], acc[k], 0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < MAXT; ++k) {
      const int tile = c0 + w + NWV * k;
      if (tile < nkt) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          acc[k][v] *= a.scale;
          scr[(size_t)(ig + 4 * v) * nkbp + 16 * tile + jl] = acc[k][v];
        }
      }
    }
  }
  __syncthreads();   // every wave's scores stored and visible to the workgroup
  for (int rr = 0; rr < 16 / NWV; ++rr) {
    const int r = w + NWV * rr, i = 16 * g + r;
    if (i >= nqb) {   // wave-uniform
      if (lane == 0) L.cnt[r] = 0;
      continue;
    }
    const size_t row = (size_t)bh * nqb + i;
    double *sr = scr + (size_t)r * nkbp;   // this lane reads and writes entries lane + 64 t only
    // the first R entries per lane are read once into registers, the rest (rows longer than
    // the registers hold) stay in the scratch and are read again on every pass
    constexpr int R = NPL <= kLargeRegNpl ? NPL : kLargeSplitRegs;
    double ev[R];
#pragma unroll
    for (int t = 0; t < R; ++t) {
      const int j = lane + 64 * t;
      ev[t] = j < nkb ? sr[j] : -INFINITY;
    }
    double mx = ev[0];
#pragma unroll
    for (int t = 1; t < R; ++t) mx = fmax(mx, ev[t]);
#pragma unroll 2
    for (int t = R; t < NPL; ++t) {
      const int j = lane + 64 * t;
      if (j < nkb) mx = fmax(mx, sr[j]);
    }
    mx = wave_max(mx);
    unsigned long long Z = 0;
    double emin = 1.0;
#pragma unroll
    for (int t = 0; t < R; ++t) {
      const bool valid = lane + 64 * t < nkb;
      const double e = valid ? exp(ev[t] - mx) : 0.0;
      ev[t] = e;
      Z += fix52(e);
      if (valid) emin = fmin(emin, e);
    }
#pragma unroll 2
    for (int t = R; t < NPL; ++t) {
      const int j = lane + 64 * t;
      if (j < nkb) {
        const double e = exp(sr[j] - mx);
        sr[j] = e;
        Z += fix52(e);
        emin = fmin(emin, e);
      }
    }
    Z = wave_sum(Z);
    emin = wave_min(emin);
    if constexpr (R == NPL)
      row_decide<NPL, EXT>(RegRow<NPL>{ev}, Z, emin, i, row, a, L.h_mass[w], L.h_cnt[w], &L.cnt[r]);
    else
      row_decide<NPL, EXT>(SplitRow<R>{ev, sr}, Z, emin, i, row, a, L.h_mass[w], L.h_cnt[w], &L.cnt[r]);
  }
  __syncthreads();   // row counts in LDS; scratch rows consumed before the next item's scores
  if (w == 0) {
    const size_t row0 = (size_t)bh * nqb + 16 * g;
    const int c = lane < 16 ? L.cnt[lane] : 0;
    const bool second = lane < 16 && ((row0 + lane) >> 6) != (row0 >> 6);
    int c0 = second ? 0 : c, c1 = second ? c : 0;
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) {
      c0 += __shfl_xor(c0, off);
      c1 += __shfl_xor(c1, off);
    }
    if (lane == 0) {
      atomicAdd(&a.head_load[bh], c0 + c1);
      atomicAdd(&a.bsum[row0 >> 6], c0);
      if (c1 != 0) atomicAdd(&a.bsum[(row0 >> 6) + 1], c1);
    }
  }
}

// Persistent large select: items split into 8 XCD ranges as k_select; workgroup b owns scratch
// rows scr + 16 b nkbp (gridDim.x <= kLargeSelGrid).
template <typename T, int D, int NPL, bool EXT>
__global__ __launch_bounds__(512, 1) void k_select_large(SelArgs a, int BH, double *scr, int nkbp) {
  __shared__ SelLdsL<T, D> L;
  const int nqg = (a.nqb + 15) >> 4;
  const int items = BH * nqg;
  const int xcd = blockIdx.x & 7;
  const int nwx = ((int)gridDim.x - xcd + 7) >> 3;
  const int it_end = (int)((long long)items * (xcd + 1) / 8);
  double *my = scr + (size_t)blockIdx.x * 16 * nkbp;
  for (int it = (int)((long long)items * xcd / 8) + (int)(blockIdx.x >> 3); it < it_end; it += nwx) {
    const int bh = it / nqg, g = it - bh * nqg;
    select_item_large<T, D, NPL, EXT>(L, a, my, nkbp, bh, g);
  }
}

// ---------------------------------------------------------------------------------------
// k_csr: row_ptr (exclusive scan of counts) and ascending col_idx from the kept masks.
// grid = cdiv(rows, 16), 256 threads; wave w owns rows 16 b + 4 w .. + 3, with no workgroup
// barrier: a row's offset is the sum of the per-64-row sums before its 64-row block plus the
// counts of the rows before it inside that block (an exclusive scan across the lanes).  Lane L
// holds word L of a row's mask (the four rows' words are loaded up front), and each 64-block
// chunk of a row is one 64-bit mask from two lanes, whose set bits give every kept block its
// output slot (coalesced writes).  Rows of up to 128 words (4096 key blocks): lane L holds words
// L and L + 64.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_csr(const int32_t *__restrict__ counts,
                                             const uint32_t *__restrict__ bitmask,
                                             const int32_t *__restrict__ bsum, int rows, int nkw, int nkb,
                                             int32_t *__restrict__ row_ptr, int32_t *__restrict__ col_idx) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r0 = blockIdx.x * 16 + 4 * w;   // this wave's first row
  if (r0 >= rows) return;                    // wave-uniform
  uint32_t wv[4][kRowWords];   // row k's word lane + 64 q in wv[k][q]
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int rk = r0 + k;
#pragma unroll
    for (int q = 0; q < kRowWords; ++q)
      wv[k][q] = (rk < rows && lane + 64 * q < nkw) ? bitmask[(size_t)rk * nkw + lane + 64 * q] : 0u;
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
      // words 2 c and 2 c + 1 sit in the same register (c / 32) of lanes 2 c % 64 and 2 c % 64 + 1
      const int src = c >> 5, l0 = (2 * c) & 63;
      const uint32_t wq = src == 0 ? wv[k][0] : wv[k][kRowWords - 1];
      const unsigned long long mask = (unsigned long long)(uint32_t)__shfl((int)wq, l0) |
                                      ((unsigned long long)(uint32_t)__shfl((int)wq, l0 + 1) << 32);
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
                  int32_t *zero1, int nzero1, int32_t *zero2, int nzero2, hipStream_t st) {
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
  pa.zero[2] = zero2;
  pa.nzero[2] = nzero2;
  return launch_pool_args(pa, BH, d, dtype, st);
}

// Pooling of K (k_pool, which also zeroes the per-64-row sums, head loads and status word), then
// the persistent select over all items.
template <typename T, int D, int MT, int NWV, bool EXT>
static int launch_route_k(const RouteLaunch &r, hipStream_t st) {
  const SelArgs a{r.q, r.ksw, r.nqb, r.nkb, r.nkw, 1.0 / sqrt((double)D), r.p, r.counts, r.bitmask, r.head_load,
                  r.bsum, r.sel, r.status};
  int rc = launch_pool_k(r.k, r.BH, r.N, D, r.dtype, r.bk, r.ksw, r.bsum, r.nbsum, r.head_load, r.BH,
                         (int32_t *)r.status, 1, st);
  if (rc != FVATTN_OK) return rc;
  auto kern = k_select<T, D, MT, NWV, EXT>;
  int cus = 0, occ = 0;
  if (device_cus(&cus) != 0) return FVATTN_ERR_HIP;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, 64 * NWV, 0) != hipSuccess) return FVATTN_ERR_HIP;
  const int items = cdiv(r.nqb, 16) * r.BH;
  int grid = cus * (occ > 0 ? occ : 1);
  if (grid > items) grid = items;
  if (grid < 8) grid = 8;   // every XCD range needs a worker
  hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * NWV), 0, st, a, r.BH);
  FV_CHECK_LAUNCH();
  return FVATTN_OK;
}

template <typename T, int D, int NPL, bool EXT>
static int launch_route_large(const RouteLaunch &r, hipStream_t st) {
  const SelArgs a{r.q, r.ksw, r.nqb, r.nkb, r.nkw, 1.0 / sqrt((double)D), r.p, r.counts, r.bitmask, r.head_load,
                  r.bsum, r.sel, r.status};
  int rc = launch_pool_k(r.k, r.BH, r.N, D, r.dtype, r.bk, r.ksw, r.bsum, r.nbsum, r.head_load, r.BH,
                         (int32_t *)r.status, 1, st);
  if (rc != FVATTN_OK) return rc;
  auto kern = k_select_large<T, D, NPL, EXT>;
  int cus = 0, occ = 0;
  if (device_cus(&cus) != 0) return FVATTN_ERR_HIP;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, 512, 0) != hipSuccess) return FVATTN_ERR_HIP;
  const int items = cdiv(r.nqb, 16) * r.BH;
  int grid = cus * (occ > 0 ? occ : 1);
  grid = min(grid, items);
  grid = max(grid, 8);
  grid = min(grid, kLargeSelGrid);   // the scratch holds kLargeSelGrid workgroups' rows
  hipLaunchKernelGGL(kern, dim3(grid), dim3(512), 0, st, a, r.BH, r.scr, r.nkbp);
  FV_CHECK_LAUNCH();
  return FVATTN_OK;
}

template <typename T, int D, int MT, int NWV>
static int launch_route_mt(const RouteLaunch &r, hipStream_t st) {
  const SelOpts &sel = r.sel;
  const bool ext = sel.mode != FVATTN_ROUTE_TOPP || sel.k_min > 1 || sel.k_max > 0 || sel.window > 0 ||
                   sel.imp != nullptr;
  return ext ? launch_route_k<T, D, MT, NWV, true>(r, st) : launch_route_k<T, D, MT, NWV, false>(r, st);
}

// Key tiles (of 16 blocks) per wave: up to 512 key blocks run on 4 waves with at most 8 tiles
// each, up to 1024 on 8 waves with 8 tiles each and up to 1280 with 10 (this form spills 20-28
// bytes per lane, but measured 40% faster at 1182 key blocks than the chunked form, with every
// row exact); more on the chunked large select (scores through the scratch).
template <typename T, int D>
static int launch_route_d(const RouteLaunch &r, hipStream_t st) {
  const int nkt = cdiv(r.nkb, 16);
  if (nkt <= 4) return launch_route_mt<T, D, 1, 4>(r, st);
  if (nkt <= 8) return launch_route_mt<T, D, 2, 4>(r, st);
  if (nkt <= 16) return launch_route_mt<T, D, 4, 4>(r, st);
  if (nkt <= 32) return launch_route_mt<T, D, 8, 4>(r, st);
  if (nkt <= 64) return launch_route_mt<T, D, 8, 8>(r, st);
  if (nkt <= 80) return launch_route_mt<T, D, 10, 8>(r, st);
  const SelOpts &sel = r.sel;
  const bool ext = sel.mode != FVATTN_ROUTE_TOPP || sel.k_min > 1 || sel.k_max > 0 || sel.window > 0 ||
                   sel.imp != nullptr;
  if (r.nkb <= 2048)
    return ext ? launch_route_large<T, D, 32, true>(r, st) : launch_route_large<T, D, 32, false>(r, st);
  if (r.nkb <= 2368)   // the 720p layer with 32-token key blocks (2,363) without a long spill
    return ext ? launch_route_large<T, D, 37, true>(r, st) : launch_route_large<T, D, 37, false>(r, st);
  if (r.nkb <= 2560)
    return ext ? launch_route_large<T, D, 40, true>(r, st) : launch_route_large<T, D, 40, false>(r, st);
  return ext ? launch_route_large<T, D, 64, true>(r, st) : launch_route_large<T, D, 64, false>(r, st);
}

int launch_route(const RouteLaunch &r, hipStream_t st) {
  if (r.dtype == FVATTN_BF16) return r.d == 128 ? launch_route_d<uint16_t, 128>(r, st) : launch_route_d<uint16_t, 64>(r, st);
  return r.d == 128 ? launch_route_d<float, 128>(r, st) : launch_route_d<float, 64>(r, st);
}

int launch_csr(const int32_t *counts, const uint32_t *bitmask, const int32_t *bsum, int rows, int nkw, int nkb,
               int32_t *row_ptr, int32_t *col_idx, hipStream_t st) {
  hipLaunchKernelGGL(k_csr, dim3(cdiv(rows, 16)), dim3(256), 0, st, counts, bitmask, bsum, rows, nkw, nkb, row_ptr,
                     col_idx);
  FV_CHECK_LAUNCH();
  return FVATTN_OK;
}

}  // namespace fv
