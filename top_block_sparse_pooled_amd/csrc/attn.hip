// Block-sparse softmax attention over the kept key blocks, and the device-built work list.
//
// Method: FVAttn summary page (PaperDaily, arXiv:2607.16190): attention runs only over the
// key blocks kept by Top-p routing and is otherwise exact; its RLB section balances work by
// moving the heaviest units first.  On one GPU the balanced units are (head, query-block)
// tiles handed to persistent workgroups, heaviest first.
//
// gfx950 design of the bf16 kernel (k_attn_bf16):
//  * one workgroup = one query block of BQ rows, BQ/32 waves, each wave owns 32 query rows;
//  * per kept key block: the K tile [BK][D] and the V^T tile [D][BK] are staged through LDS
//    (the next block's global loads are issued into registers before the current block is
//    computed, so HBM/L2 latency overlaps the MFMA work);
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (K from LDS as operand A, Q held in registers as
//    operand B), so each lane owns one query column: the softmax row statistics need only
//    one cross-half exchange (v_permlane32_swap) per block;
//  * online softmax in float32 with exp2 and the 1/sqrt(d)*log2(e) scale folded into one
//    multiply; P is rounded to bf16 and fed straight from registers as operand B of
//    O^T += V^T P^T -- the key order inside each 16-key group of V^T is permuted in memory
//    (bits 2 and 3 of the key index swapped) so that the lane's P registers and its 16-byte
//    V^T read cover the same keys;
//  * persistent grid: workgroups pop tiles from a device work list through one atomic
//    counter, so long rows start first and short rows fill the tail.
#include "common.h"

namespace fv {

// ---------------------------------------------------------------------------------------
// k_vt: V [BH][N][D] bf16 -> V^T [BH][D][NKP] bf16, zero for keys >= N, keys permuted
// inside each 16-key group: key 16t + 8c + 4h + b is stored at 16t + 8h + 4c + b.
// grid = (NKP/64, D/64, BH), 256 threads.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ int vperm(int key) {
  return (key & ~15) | ((key & 4) << 1) | ((key & 8) >> 1) | (key & 3);
}

__global__ __launch_bounds__(256) void k_vt(const uint16_t *__restrict__ v, uint16_t *__restrict__ vt, int N,
                                            int D, int NKP) {
  __shared__ uint16_t tile[64][64 + 2];
  const int tid = threadIdx.x;
  const int key0 = blockIdx.x * 64, d0 = blockIdx.y * 64, bh = blockIdx.z;
  const uint16_t *vh = v + (size_t)bh * N * D;
  // read 64 keys x 64 dims: 512 chunks of 8 dims
  for (int c = tid; c < 512; c += 256) {
    const int r = c >> 3, dc = (c & 7) * 8;
    const int key = key0 + r;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (key < N) val = *reinterpret_cast<const u32x4 *>(vh + (size_t)key * D + d0 + dc);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      tile[r][dc + 2 * i] = (uint16_t)(val[i] & 0xffffu);
      tile[r][dc + 2 * i + 1] = (uint16_t)(val[i] >> 16);
    }
  }
  __syncthreads();
  // write 64 dims x 64 keys: 512 chunks of 8 (permuted) key positions
  uint16_t *vth = vt + (size_t)bh * D * NKP;
  for (int c = tid; c < 512; c += 256) {
    const int dd = c >> 3, pc = (c & 7) * 8;
    uint32_t wv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k0 = vperm(pc + 2 * i), k1 = vperm(pc + 2 * i + 1);  // physical -> logical
      wv[i] = (uint32_t)tile[k0][dd] | ((uint32_t)tile[k1][dd] << 16);
    }
    *reinterpret_cast<u32x4 *>(vth + (size_t)(d0 + dd) * NKP + key0 + pc) = u32x4{wv[0], wv[1], wv[2], wv[3]};
  }
}

// ---------------------------------------------------------------------------------------
// k_worklist: permutation of the rows in the requested order.
// single workgroup of 1024 threads (16 waves).
//   LPT:      key = nkb - count (ascending key = descending count), stable in row id.
//   HEAD_LPT: heads by load descending (ties: head id), then each head's rows as LPT.
// Stable counting sort: per-wave bin counts in LDS, bases by scan, then each wave scatters
// its rows in 64-row chunks, ranking equal keys inside a chunk with bit-sliced ballots.
// ---------------------------------------------------------------------------------------
constexpr int kWlWaves = 16;
constexpr int kWlMaxBins = 1281 + 3;

__device__ __forceinline__ int wl_key(const int32_t *row_ptr, int r, int nkb) {
  int c = row_ptr[r + 1] - row_ptr[r];
  c = c < 0 ? 0 : (c > nkb ? nkb : c);
  return nkb - c;
}

// Stable scatter of rows [lo, hi) of one wave by key, into out[] at positions given by the
// running per-key bases in bins[] (already offset).  Keys < 2048.
__device__ void wl_scatter(const int32_t *row_ptr, int lo, int hi, int nkb, int *bins, int32_t *out) {
  const int lane = threadIdx.x & 63;
  const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int c0 = lo; c0 < hi; c0 += 64) {
    const int r = c0 + lane;
    const bool act = r < hi;
    const int key = act ? wl_key(row_ptr, r, nkb) : 0;
    unsigned long long peers = __ballot(act);
#pragma unroll
    for (int b = 0; b < 11; ++b) {
      const unsigned long long bb = __ballot(act && ((key >> b) & 1));
      peers &= ((key >> b) & 1) ? bb : ~bb;
    }
    const int rank = __popcll(peers & lt);
    int base = 0;
    if (act) base = bins[key];
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    if (act) {
      out[base + rank] = r;
      if (rank == 0) bins[key] = base + __popcll(peers);
    }
    __builtin_amdgcn_wave_barrier();
  }
}

__global__ __launch_bounds__(1024) void k_worklist(const int32_t *__restrict__ row_ptr, int rows, int nqb,
                                                   int nkb, int sched, int32_t *__restrict__ wl,
                                                   int32_t *__restrict__ counter) {
  __shared__ int bins[kWlWaves][kWlMaxBins];
  __shared__ int s_scan[1024];
  __shared__ int s_hbase[1024];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (tid == 0 && counter != nullptr) {
    counter[0] = 0;  // tile ticket
    counter[1] = 0;  // workgroups that have finished
  }
  if (sched == FVATTN_SCHED_IDENTITY) {
    for (int r = tid; r < rows; r += 1024) wl[r] = r;
    return;
  }
  const int nbins = nkb + 1;
  if (sched == FVATTN_SCHED_LPT) {
    for (int i = tid; i < kWlWaves * kWlMaxBins; i += 1024) (&bins[0][0])[i] = 0;
    __syncthreads();
    const int seg = cdiv(rows, kWlWaves);
    const int lo = min(rows, w * seg), hi = min(rows, lo + seg);
    for (int r = lo + lane; r < hi; r += 64) atomicAdd(&bins[w][wl_key(row_ptr, r, nkb)], 1);
    __syncthreads();
    // totals per bin, exclusive scan over bins (two bins per thread)
    int t0 = 0, t1 = 0;
    const int b0 = 2 * tid, b1 = 2 * tid + 1;
    for (int i = 0; i < kWlWaves; ++i) {
      if (b0 < nbins) t0 += bins[i][b0];
      if (b1 < nbins) t1 += bins[i][b1];
    }
    s_scan[tid] = t0 + t1;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int o = tid >= off ? s_scan[tid - off] : 0;
      __syncthreads();
      s_scan[tid] += o;
      __syncthreads();
    }
    int run0 = s_scan[tid] - (t0 + t1);
    int run1 = run0 + t0;
    for (int i = 0; i < kWlWaves; ++i) {
      if (b0 < nbins) { const int c = bins[i][b0]; bins[i][b0] = run0; run0 += c; }
      if (b1 < nbins) { const int c = bins[i][b1]; bins[i][b1] = run1; run1 += c; }
    }
    __syncthreads();
    wl_scatter(row_ptr, lo, hi, nkb, bins[w], wl);
    return;
  }
  // HEAD_LPT
  const int nh = rows / nqb;
  // rank heads by load (desc), ties by id; bases = prefix of ranked head sizes (all nqb)
  for (int h = tid; h < nh; h += 1024) {
    const int lh = row_ptr[(h + 1) * nqb] - row_ptr[h * nqb];
    int rank = 0;
    for (int h2 = 0; h2 < nh; ++h2) {
      const int l2 = row_ptr[(h2 + 1) * nqb] - row_ptr[h2 * nqb];
      rank += (l2 > lh) || (l2 == lh && h2 < h);
    }
    s_hbase[h] = rank * nqb;
  }
  __syncthreads();
  for (int h = w; h < nh; h += kWlWaves) {
    int *bw = bins[w];
    for (int i = lane; i < nbins; i += 64) bw[i] = 0;
    __builtin_amdgcn_wave_barrier();
    const int lo = h * nqb, hi = lo + nqb;
    for (int r = lo + lane; r < hi; r += 64) atomicAdd(&bw[wl_key(row_ptr, r, nkb)], 1);
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    // exclusive scan of the bins by this wave (chunks of 64)
    int run = s_hbase[h];
    for (int c0 = 0; c0 < nbins; c0 += 64) {
      const int i = c0 + lane;
      const int c = i < nbins ? bw[i] : 0;
      int incl = c;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
      }
      if (i < nbins) bw[i] = run + incl - c;
      run += __shfl(incl, 63);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    wl_scatter(row_ptr, lo, hi, nkb, bw, wl);
  }
}

// ---------------------------------------------------------------------------------------
// bf16 MFMA attention.  Template: BQ query rows per tile (32/64/128), BK keys per block
// (32/64), D head dim (64/128).
//
// LDS holds one K tile [BK][D] and one V^T tile [D][BK], filled straight from global memory
// by global_load_lds_dwordx4 (no staging registers).  Each row of a tile is a run of 16-byte
// chunks stored in XOR-swizzled order (chunk c of row r sits at position c ^ (r mod chunks)),
// so the 16-byte operand reads of 16 consecutive rows hit distinct banks.  The two tiles are
// refilled in a split pipeline with two barriers per key block:
//    S = K_j Q^T | wait, barrier X | load K_{j+1} | softmax_j | O += V_j P | wait, barrier Y |
//    load V_{j+1}
// so K_{j+1} streams in behind the softmax and P.V of block j, and V_{j+1} behind S of j+1.
// ---------------------------------------------------------------------------------------
template <int BQ, int BK, int D>
struct AttnCfg {
  static constexpr int NW = BQ / 32;       // waves, each owns 32 query rows
  static constexpr int NT = NW * 64;       // threads (= 2 * BQ)
  static constexpr int KROW = D * 2;       // bytes per K tile row (one key)
  static constexpr int KCR = D / 8;        // 16-byte chunks per K row
  static constexpr int VROW = BK * 2;      // bytes per V^T tile row (one dim)
  static constexpr int VCR = BK / 8;       // chunks per V^T row
  static constexpr int KBYTES = BK * D * 2;
  static constexpr int VBYTES = D * BK * 2;
  static constexpr int KI = KBYTES / 1024 / NW;  // 1 KB direct-to-LDS loads per wave
  static constexpr int VI = VBYTES / 1024 / NW;
  static constexpr int NKT = BK / 32;      // 32-key tiles per block
  static constexpr int NS = D / 16;        // k-steps of S^T = K Q^T
  static constexpr int NM = D / 32;        // 32-dim tiles of O^T
  static_assert(KBYTES % (1024 * NW) == 0 && VBYTES % (1024 * NW) == 0, "tile/wave mismatch");
};

typedef __attribute__((address_space(3))) void *lds_void_ptr;

__device__ __forceinline__ void dma16(const void *src, void *lds_dst_uniform) {
  __builtin_amdgcn_global_load_lds(src, (lds_void_ptr)lds_dst_uniform, 16, 0, 0);
}

__device__ __forceinline__ uint64_t hw_id_word() {
  const uint32_t hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);    // HW_ID
  const uint32_t xcc = __builtin_amdgcn_s_getreg((31 << 11) | 20);  // XCC_ID
  return ((uint64_t)xcc << 32) | hw;
}

template <int BQ, int BK, int D>
__global__ __launch_bounds__(2 * BQ, 2) void k_attn_bf16(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ vt,
    void *__restrict__ o, int out_f32, const int32_t *__restrict__ row_ptr, const int32_t *__restrict__ col_idx,
    const int32_t *__restrict__ worklist, int32_t *__restrict__ counter, int rows, int nqb, int N, int NKP,
    float sl2, uint64_t *__restrict__ trace) {
  using C = AttnCfg<BQ, BK, D>;
  __shared__ __attribute__((aligned(1024))) uint8_t Ks[C::KBYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t Vs[C::VBYTES];
  __shared__ int s_tile;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, kept in an SGPR
  const int l32 = lane & 31, h = lane >> 5;

  // Swizzled positions.  The tile loads of one wave cover rows in groups (1 KB each);
  // per lane the row inside the group and the chunk position are fixed, so only one row
  // base and one XOR key are kept per lane and the rest is folded into constants.
  constexpr int KRPI = 1024 / C::KROW;   // K rows per 1 KB load
  constexpr int VRPI = 1024 / C::VROW;   // V^T rows per 1 KB load
  const int k_r0 = lane / (C::KROW / 16), k_pos = lane % (C::KROW / 16);
  const int v_r0 = lane / (C::VROW / 16), v_pos = lane % (C::VROW / 16);
  // operand reads: row 32kt + l32 of K, row 32m + l32 of V^T; XOR keys depend only on l32
  const int kx = l32 & (C::KCR - 1), vx = l32 & (C::VCR - 1);

  for (;;) {
    if (tid == 0) s_tile = atomicAdd(&counter[0], 1);
    __syncthreads();
    const int t = s_tile;
    __syncthreads();
    if (t >= rows) break;
    uint64_t t_start = 0;
    if (trace != nullptr) t_start = __builtin_amdgcn_s_memrealtime();

    const int row = worklist[t];
    const int bh = row / nqb, qi = row - bh * nqb;
    const int beg = row_ptr[row], cnt = row_ptr[row + 1] - beg;
    const uint16_t *kh = k + (size_t)bh * N * D;
    const uint16_t *vth = vt + (size_t)bh * D * NKP;

    auto load_k = [&](int jb) {
      const int key0 = jb * BK;
#pragma unroll
      for (int i = 0; i < C::KI; ++i) {
        const int r = (w * C::KI + i) * KRPI + k_r0;          // tile row = key offset
        const int key = min(key0 + r, N - 1);                // rows past N: any valid row, masked later
        dma16(kh + (size_t)key * D + (k_pos ^ (r & (C::KCR - 1))) * 8, Ks + (w * C::KI + i) * 1024);
      }
    };
    auto load_v = [&](int jb) {
      const uint16_t *src = vth + jb * BK;
#pragma unroll
      for (int i = 0; i < C::VI; ++i) {
        const int r = (w * C::VI + i) * VRPI + v_r0;          // tile row = head dim
        dma16(src + (size_t)r * NKP + (v_pos ^ (r & (C::VCR - 1))) * 8, Vs + (w * C::VI + i) * 1024);
      }
    };

    int jb = cnt > 0 ? col_idx[beg] : 0;
    if (cnt > 0) {
      load_k(jb);
      load_v(jb);
    }
    // Q fragments (operand B of S^T = K Q^T): query qrow, dims 16s + 8h .. +7
    const int qrow = qi * BQ + 32 * w + l32;
    bf16x8 qf[C::NS];
    {
      const uint16_t *qp = q + ((size_t)bh * N + (qrow < N ? qrow : 0)) * D + 8 * h;
#pragma unroll
      for (int s = 0; s < C::NS; ++s) {
        u32x4 raw = {0u, 0u, 0u, 0u};
        if (qrow < N) raw = *reinterpret_cast<const u32x4 *>(qp + 16 * s);
        qf[s] = __builtin_bit_cast(bf16x8, raw);
      }
    }
    f16v oacc[C::NM];
#pragma unroll
    for (int m = 0; m < C::NM; ++m)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[m][i] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;   // m_run in log2 units (scores times sl2)
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int jj = 0; jj < cnt; ++jj) {
      const int jn = (jj + 1 < cnt) ? col_idx[beg + jj + 1] : 0;
      // S^T tiles: 32 keys x 32 queries each
      f16v sacc[C::NKT];
#pragma unroll
      for (int kt = 0; kt < C::NKT; ++kt) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[kt][i] = 0.f;
#pragma unroll
        for (int s = 0; s < C::NS; ++s) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8 *>(
              Ks + (32 * kt + l32) * C::KROW + (((2 * s + h) ^ kx) << 4));
          sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[s], sacc[kt], 0, 0, 0);
        }
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();                 // X: K tile free, V_j landed
      if (jj + 1 < cnt) load_k(jn);

      // online softmax (lane: query l32 of wave w; keys 32kt + 8(v/4) + 4h + v%4)
      const int kbase = jb * BK;
      if (kbase + BK > N) {            // ragged last block: mask keys >= N
        const int lim = N - kbase - 4 * h;
#pragma unroll
        for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            if (32 * kt + 8 * (v >> 2) + (v & 3) >= lim) sacc[kt][v] = -INFINITY;
      }
      float mloc = sacc[0][0];
#pragma unroll
      for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v) mloc = fmaxf(mloc, sacc[kt][v]);
      {
        auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mloc), __float_as_uint(mloc), false, false);
        mloc = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      const float mb = mloc * sl2;
      // rescale only when some row's maximum grew (wave-uniform branch); the largest
      // weight of a row then stays exactly 1, so its bf16 copy carries no rounding error
      if (__any(mb > m_run)) {
        const float m_new = fmaxf(m_run, mb);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int m = 0; m < C::NM; ++m)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[m][i] *= alpha;
      }
      const float nm = -m_run;
      float psum = 0.f;
      bf16x8 pf[C::NKT][2];
#pragma unroll
      for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          bf16x8 pv;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float pe = __builtin_amdgcn_exp2f(fmaf(sacc[kt][8 * t2 + i], sl2, nm));
            psum += pe;
            pv[i] = (__bf16)pe;
          }
          pf[kt][t2] = pv;
        }
      l_run += psum;
      // O^T += V^T P^T
#pragma unroll
      for (int m = 0; m < C::NM; ++m)
#pragma unroll
        for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
          for (int t2 = 0; t2 < 2; ++t2) {
            const bf16x8 va = *reinterpret_cast<const bf16x8 *>(
                Vs + (32 * m + l32) * C::VROW + (((4 * kt + 2 * t2 + h) ^ vx) << 4));
            oacc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf[kt][t2], oacc[m], 0, 0, 0);
          }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();                 // Y: V tile free, K_{j+1} landed
      if (jj + 1 < cnt) load_v(jn);
      jb = jn;
    }
    // finalise: l over both halves, O / l, store (lane: query qrow, dims 32m + 8a + 4h + b)
    {
      auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
      const float ltot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      const float inv = 1.f / ltot;
      if (qrow < N && out_f32) {
        float *op = (float *)o + ((size_t)bh * N + qrow) * D + 4 * h;
#pragma unroll
        for (int m = 0; m < C::NM; ++m)
#pragma unroll
          for (int a = 0; a < 4; ++a)
            *reinterpret_cast<f4 *>(op + 32 * m + 8 * a) =
                f4{oacc[m][4 * a] * inv, oacc[m][4 * a + 1] * inv, oacc[m][4 * a + 2] * inv, oacc[m][4 * a + 3] * inv};
      } else if (qrow < N) {
        uint16_t *op = (uint16_t *)o + ((size_t)bh * N + qrow) * D + 4 * h;
#pragma unroll
        for (int m = 0; m < C::NM; ++m)
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const uint32_t w0 = pack_bf16(oacc[m][4 * a] * inv, oacc[m][4 * a + 1] * inv);
            const uint32_t w1 = pack_bf16(oacc[m][4 * a + 2] * inv, oacc[m][4 * a + 3] * inv);
            *reinterpret_cast<u32x2 *>(op + 32 * m + 8 * a) = u32x2{w0, w1};
          }
      }
    }
    if (trace != nullptr && tid == 0) {
      const uint64_t t_end = __builtin_amdgcn_s_memrealtime();
      trace[4 * (size_t)t + 0] = hw_id_word();
      trace[4 * (size_t)t + 1] = t_start;
      trace[4 * (size_t)t + 2] = t_end;
      trace[4 * (size_t)t + 3] = (uint64_t)row;
    }
  }
  // The last workgroup to leave has seen every other workgroup's final ticket: reset the
  // ticket and exit counters so the same plan can be run again.
  if (tid == 0) {
    __threadfence();
    if (atomicAdd(&counter[1], 1) == (int)gridDim.x - 1) {
      atomicExch(&counter[0], 0);
      atomicExch(&counter[1], 0);
    }
  }
}

// ---------------------------------------------------------------------------------------
// float32 attention: one thread per query row, K/V tiles through LDS, online softmax in
// float32.  grid = rows (tile t processes worklist[t]).
// ---------------------------------------------------------------------------------------
template <int BQ, int BK, int D>
__global__ __launch_bounds__(BQ) void k_attn_f32(const float *__restrict__ q, const float *__restrict__ k,
                                                 const float *__restrict__ v, float *__restrict__ o,
                                                 const int32_t *__restrict__ row_ptr,
                                                 const int32_t *__restrict__ col_idx,
                                                 const int32_t *__restrict__ worklist, int nqb, int N,
                                                 float scale, uint64_t *__restrict__ trace) {
  __shared__ float Kt[BK][D + 1];
  __shared__ float Vt[BK][D];
  const int tid = threadIdx.x;
  const int t = blockIdx.x;
  uint64_t t_start = 0;
  if (trace != nullptr) t_start = __builtin_amdgcn_s_memrealtime();
  const int row = worklist[t];
  const int bh = row / nqb, qi = row - bh * nqb;
  const int qrow = qi * BQ + tid;
  const bool live = qrow < N;
  float qv[D], acc[D];
  const float *qp = q + ((size_t)bh * N + (live ? qrow : 0)) * D;
#pragma unroll
  for (int c = 0; c < D; ++c) {
    qv[c] = live ? qp[c] * scale : 0.f;
    acc[c] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;
  const int beg = row_ptr[row], end = row_ptr[row + 1];
  const float *kh = k + (size_t)bh * N * D;
  const float *vh = v + (size_t)bh * N * D;
  for (int e = beg; e < end; ++e) {
    const int key0 = col_idx[e] * BK;
    const int nk = min(BK, N - key0);
    __syncthreads();
    for (int i = tid; i < BK * D; i += BQ) {
      const int r = i / D, c = i % D;
      Kt[r][c] = r < nk ? kh[(size_t)(key0 + r) * D + c] : 0.f;
      Vt[r][c] = r < nk ? vh[(size_t)(key0 + r) * D + c] : 0.f;
    }
    __syncthreads();
    for (int r = 0; r < nk; ++r) {
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) s = fmaf(qv[c], Kt[r][c], s);
      const float m_new = fmaxf(m_run, s);
      const float corr = expf(m_run - m_new);
      const float pexp = expf(s - m_new);
      l_run = l_run * corr + pexp;
#pragma unroll
      for (int c = 0; c < D; ++c) acc[c] = fmaf(pexp, Vt[r][c], acc[c] * corr);
      m_run = m_new;
    }
  }
  if (live) {
    float *op = o + ((size_t)bh * N + qrow) * D;
    const float inv = 1.f / l_run;
#pragma unroll
    for (int c = 0; c < D; ++c) op[c] = acc[c] * inv;
  }
  if (trace != nullptr && tid == 0) {
    const uint64_t t_end = __builtin_amdgcn_s_memrealtime();
    trace[4 * (size_t)t + 0] = hw_id_word();
    trace[4 * (size_t)t + 1] = t_start;
    trace[4 * (size_t)t + 2] = t_end;
    trace[4 * (size_t)t + 3] = (uint64_t)row;
  }
}

// ---------------------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------------------
int launch_vt(const void *v, void *vt, int BH, int N, int D, int NKP, hipStream_t st) {
  hipLaunchKernelGGL(k_vt, dim3(NKP / 64, D / 64, BH), dim3(256), 0, st, (const uint16_t *)v, (uint16_t *)vt, N,
                     D, NKP);
  FV_CHECK_LAUNCH();
  return FVATTN_OK;
}

int launch_worklist(const int32_t *row_ptr, int rows, int nqb, int nkb, int sched, int32_t *wl, int32_t *counter,
                    hipStream_t st) {
  hipLaunchKernelGGL(k_worklist, dim3(1), dim3(1024), 0, st, row_ptr, rows, nqb, nkb, sched, wl, counter);
  FV_CHECK_LAUNCH();
  return FVATTN_OK;
}

template <int BQ, int BK, int D>
static int launch_attn_bf16_t(const void *q, const void *k, const void *vt, void *o, int out_f32,
                              const int32_t *row_ptr,
                              const int32_t *col_idx, const int32_t *wl, int32_t *counter, int rows, int nqb,
                              int N, int NKP, int grid, uint64_t *trace, hipStream_t st) {
  using C = AttnCfg<BQ, BK, D>;
  auto kern = k_attn_bf16<BQ, BK, D>;
  if (grid <= 0) {
    int dev = 0, cus = 0, occ = 0;
    if (hipGetDevice(&dev) != hipSuccess) return FVATTN_ERR_HIP;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return FVATTN_ERR_HIP;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, C::NT, 0) != hipSuccess) return FVATTN_ERR_HIP;
    grid = cus * (occ > 0 ? occ : 1);
  }
  if (grid > rows) grid = rows;
  const float sl2 = (float)(1.4426950408889634 / sqrt((double)D));
  hipLaunchKernelGGL(kern, dim3(grid), dim3(C::NT), 0, st, (const uint16_t *)q, (const uint16_t *)k,
                     (const uint16_t *)vt, o, out_f32, row_ptr, col_idx, wl, counter, rows, nqb, N, NKP, sl2,
                     trace);
  FV_CHECK_LAUNCH();
  return FVATTN_OK;
}

int launch_attn_bf16(const void *q, const void *k, const void *vt, void *o, int out_f32, const int32_t *row_ptr,
                     const int32_t *col_idx, const int32_t *wl, int32_t *counter, int rows, int nqb, int N, int NKP,
                     int D, int BQ, int BK, int grid, uint64_t *trace, hipStream_t st) {
#define FV_A(bq, bk, dd)                                                                                  \
  if (BQ == bq && BK == bk && D == dd)                                                                    \
    return launch_attn_bf16_t<bq, bk, dd>(q, k, vt, o, out_f32, row_ptr, col_idx, wl, counter, rows, nqb, N, NKP, grid, \
                                          trace, st);
  FV_A(64, 64, 128) FV_A(128, 64, 128) FV_A(32, 64, 128) FV_A(64, 32, 128) FV_A(128, 32, 128) FV_A(32, 32, 128)
  FV_A(64, 64, 64) FV_A(128, 64, 64) FV_A(32, 64, 64) FV_A(64, 32, 64) FV_A(128, 32, 64) FV_A(32, 32, 64)
#undef FV_A
  return FVATTN_ERR_UNSUPPORTED;
}

template <int BQ, int BK, int D>
static int launch_attn_f32_t(const void *q, const void *k, const void *v, void *o, const int32_t *row_ptr,
                             const int32_t *col_idx, const int32_t *wl, int rows, int nqb, int N, uint64_t *trace,
                             hipStream_t st) {
  const float scale = (float)(1.0 / sqrt((double)D));
  hipLaunchKernelGGL((k_attn_f32<BQ, BK, D>), dim3(rows), dim3(BQ), 0, st, (const float *)q, (const float *)k,
                     (const float *)v, (float *)o, row_ptr, col_idx, wl, nqb, N, scale, trace);
  FV_CHECK_LAUNCH();
  return FVATTN_OK;
}

int launch_attn_f32(const void *q, const void *k, const void *v, void *o, const int32_t *row_ptr,
                    const int32_t *col_idx, const int32_t *wl, int rows, int nqb, int N, int D, int BQ, int BK,
                    uint64_t *trace, hipStream_t st) {
#define FV_F(bq, bk, dd) \
  if (BQ == bq && BK == bk && D == dd) \
    return launch_attn_f32_t<bq, bk, dd>(q, k, v, o, row_ptr, col_idx, wl, rows, nqb, N, trace, st);
  FV_F(64, 64, 128) FV_F(128, 64, 128) FV_F(32, 64, 128) FV_F(64, 32, 128) FV_F(128, 32, 128) FV_F(32, 32, 128)
  FV_F(64, 64, 64) FV_F(128, 64, 64) FV_F(32, 64, 64) FV_F(64, 32, 64) FV_F(128, 32, 64) FV_F(32, 32, 64)
#undef FV_F
  return FVATTN_ERR_UNSUPPORTED;
}

}  // namespace fv
