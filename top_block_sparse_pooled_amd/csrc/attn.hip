// Block-sparse softmax attention over the kept key blocks, and the device-built work list.
//
// Method: FVAttn summary page (PaperDaily, arXiv:2607.16190): attention runs only over the
// key blocks kept by Top-p routing and is otherwise exact; its RLB section balances work by
// moving the heaviest units first.  On one GPU the balanced units are (head, query-block)
// tiles handed to persistent workgroups, heaviest first.
//
// gfx950 design of the bf16 kernels:
//  * a work unit is 128 query rows = 128/BQ adjacent query blocks of one head; a persistent
//    grid of workgroups pops units from a device work list through an atomic ticket, so the
//    order (identity, heaviest first, ...) is the plan's choice;
//  * the unit walks the union of its query blocks' kept key blocks; each block's K and V
//    tiles go into LDS once, straight from global memory (buffer_load ... lds), and every wave
//    whose query block kept the block uses them;
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (K from LDS as operand A, Q in registers as
//    operand B), so each lane owns one query column and the softmax row statistics need one
//    cross-half exchange (v_permlane32_swap) per block;
//  * online softmax in float32 with exp2 and the 1/sqrt(d)*log2(e) scale folded into one FMA;
//    P is rounded to bf16 and fed from registers as operand B of O^T += V^T P^T;
//  * k_attn_pp: 8 waves in two groups that split the union into 64-key tiles (one 64-token
//    block or two 32-token blocks) and alternate MFMA and softmax phases; V tiles keep V's
//    layout and the V^T operand comes from transposing LDS reads.
#include <type_traits>

#include "common.h"

namespace fv {

// ---------------------------------------------------------------------------------------
// Geometry of a K or V tile of BK keys x D dims in LDS, loaded by NW waves as 1 KB pieces
// straight from global memory (buffer_load ... lds; per-head buffer resources make rows past N
// read as zero).  Rows are runs of 16-byte chunks in XOR-swizzled order (rows that share a
// 256-byte bank line get different XOR keys) so the 16-byte operand reads of 16 consecutive
// rows hit distinct banks.
// ---------------------------------------------------------------------------------------
template <int BK, int D>
struct AttnCfg {
  static constexpr int NW = 4;             // waves loading a tile (one wave group)
  static constexpr int NT = NW * 64;
  static constexpr int KROW = D * 2;       // bytes per K tile row (one key)
  static constexpr int KCR = D / 8;        // 16-byte chunks per K row
  static constexpr int KBYTES = BK * D * 2;
  static constexpr int VBYTES = D * BK * 2;
  static constexpr int KI = KBYTES / 1024 / NW;  // 1 KB direct-to-LDS loads per wave
  static constexpr int VI = VBYTES / 1024 / NW;
  static constexpr int KRP = KROW >= 256 ? 1 : 256 / KROW;   // rows sharing one 256-byte bank line
  static constexpr int KRPI = 1024 / KROW; // rows per 1 KB load
  static constexpr int KPER = (KCR * KRP) / KRPI > 0 ? (KCR * KRP) / KRPI : 1;  // loads before the
                                                                                // swizzle repeats
  static_assert(KPER * KRPI == KRP * KCR, "swizzle period");
  static constexpr bool KTAB = (KI % KPER) == 0;  // load i of every wave has swizzle phase i % KPER
  static constexpr int NKT = BK / 32;      // 32-key MFMA tiles per tile
  static constexpr int NS = D / 16;        // k-steps of S^T = K Q^T
  static constexpr int NM = D / 32;        // 32-dim tiles of O^T
  static_assert(KBYTES % (1024 * NW) == 0 && VBYTES % (1024 * NW) == 0, "tile/wave mismatch");
};

typedef __attribute__((address_space(3))) void *lds_void_ptr;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 *lds_v4i16_ptr;

// Raw buffer resource over `bytes` bytes at `base`: loads past the end return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// 16 bytes per lane from the buffer straight into LDS at lds_dst (wave-uniform) + 16 * lane,
// with an instruction offset OFF, which the hardware adds to both the buffer address and the
// LDS address: consecutive 1 KB pieces of a tile then share one LDS base (M0).
template <int OFF>
__device__ __forceinline__ void dma16_at(__amdgpu_buffer_rsrc_t r, uint32_t voff, void *lds_dst) {
  static_assert(OFF >= 0 && OFF < 4096, "12-bit instruction offset");
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_ptr)lds_dst, 16, voff, 0, OFF, 0);
}

// 16-byte chunk position of chunk c in row r of a swizzled tile (rows of `rowbytes` bytes,
// `cr` chunks per row): rows that share a 256-byte bank line get different XOR keys.
__host__ __device__ constexpr int swz_pos(int c, int r, int rowbytes, int cr) {
  return c ^ ((r / (rowbytes >= 256 ? 1 : 256 / rowbytes)) & (cr - 1));
}

__device__ __forceinline__ uint64_t hw_id_word() {
  const uint32_t hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);    // HW_ID
  const uint32_t xcc = __builtin_amdgcn_s_getreg((31 << 11) | 20);  // XCC_ID
  return ((uint64_t)xcc << 32) | hw;
}

// ---------------------------------------------------------------------------------------
// bf16 MFMA attention, two wave groups per unit (k_attn_pp).
//
// A workgroup is 8 waves in two groups of 4.  Both groups cover the same 128 query rows (one
// work unit) and split the unit's union of kept key blocks into 64-key tiles: one 64-token
// block, or two 32-token blocks (the next two union entries, rows 0-31 and 32-63 of the
// tile; the union is then ordered by the query blocks that kept each block, so both blocks of
// a tile serve the same waves).  Group g takes tiles g, g+2, g+4, ... with its own
// online-softmax state, and the two partial results (row maximum, row sum, O) are merged
// through LDS at the end of the unit.
// Each group alternates two phases separated by workgroup barriers:
//   M_i  S_i = K_i Q^T  and  O += V_{i-1} P_{i-1}            (MFMA)
//   X_i  loads of K_{i+2} and V_{i+1};  P_i = softmax step of S_i   (VALU)
// Group 1 starts one phase late, so on each SIMD one wave issues MFMAs while its partner
// (the same SIMD slot of the other group) runs the exponentials.  K tiles are fetched two
// steps ahead and V tiles one step ahead; buffers of each parity are separate LDS objects.
// ---------------------------------------------------------------------------------------
// Workgroup barrier for LDS hand-offs: the wave's own LDS operations complete, then s_barrier.
// Deliberately no fence: a fence would also wait for the direct-to-LDS tile loads still in
// flight, which the callers track themselves with wait_vmcnt.  The memory clobber keeps the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }


template <int BQ, int BK, int D>
__global__ __launch_bounds__(512, 1) void k_attn_pp(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    void *__restrict__ o, int out_f32, const int32_t *__restrict__ row_ptr, const int32_t *__restrict__ col_idx,
    const int32_t *__restrict__ worklist, int32_t *__restrict__ counter, int units, int ngroups, int nqb, int nkb,
    int N, float sl2, uint64_t *__restrict__ trace) {
  using C = AttnCfg<64, D>;        // tile geometry (64 keys); the 4 waves of a group load its tiles
  static_assert(BK == 64 || BK == 32, "64-key tiles of one or two key blocks");
  constexpr int PB = 64 / BK;     // key blocks per tile
  constexpr int G = 128 / BQ;     // query blocks per unit
  constexpr int WPQ = BQ / 32;    // waves per query block (within a group)
  constexpr int MAXW = 128;       // kept-block bitmap words (4096 key blocks)
  constexpr int NTH = 512;
  constexpr int NH = C::NM / 2;   // 32-dim output tiles finalised by each group
  __shared__ __attribute__((aligned(1024))) uint8_t K0[2][C::KBYTES];   // [group]; parity 0
  __shared__ __attribute__((aligned(1024))) uint8_t K1[2][C::KBYTES];   // parity 1
  __shared__ __attribute__((aligned(1024))) uint8_t V0[2][C::VBYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t V1[2][C::VBYTES];
  __shared__ uint32_t s_bm[G + 1][MAXW];   // kept key blocks of each query block; row G: union
  __shared__ int s_list[MAXW * 32];        // union, ascending: (key block << 4) | keeping query blocks
  __shared__ int s_cpre[PB == 2 ? (1 << G) - 1 : 1][MAXW];   // list position of each class's word
  __shared__ float s_xm[2][4][64], s_xl[2][4][64];
  __shared__ int s_n, s_tile;
  static_assert(2 * C::KBYTES >= 4 * NH * 16 * 64 * 4, "exchange area");

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = w >> 2, wg = w & 3;                       // group, wave within the group
  const int wq = wg / WPQ, wr = wg % WPQ;                   // query block of the unit, 32-row slice
  const int nkw = (N + BK * 32 - 1) / (BK * 32);
  const int l32 = lane & 31, h = lane >> 5;

  const int k_r0 = lane / C::KCR, k_pos = lane % C::KCR;
  uint32_t k_vo[C::KPER];
#pragma unroll
  for (int j = 0; j < C::KPER; ++j) {
    const int r = j * C::KRPI + k_r0;
    k_vo[j] = (uint32_t)(k_r0 * C::KROW + swz_pos(k_pos, r, C::KROW, C::KCR) * 16);
  }
  // V tiles keep V's own layout (one key per row of 2D bytes).  The 16-byte chunk c of key row
  // r sits at chunk position c ^ (vsw(r) << 2), vsw(r) = r & 3 for d = 128 and (r >> 1) & 1 for
  // d = 64: the eight key rows that one transposing read of the P.V operand touches then fall
  // on all banks twice.  Each 1 KB load covers whole rows starting at a multiple of 4 (d = 128)
  // or 8 (d = 64), so vsw depends only on the lane.
  const int v_sw = D == 128 ? (k_r0 & 3) : ((k_r0 >> 1) & 1);
  const uint32_t v_vo = (uint32_t)(k_r0 * C::KROW + ((k_pos ^ (v_sw << 2)) * 16));
  // P.V operand reads: in each 16-lane group, lane a supplies dims 4(a & 3) .. +3 (of the
  // group's 16) of key row a >> 2, and the transposing read hands every lane the 4 keys of
  // its own dim.  Read 1 covers keys 16 kk + 4 h + 0..3, read 2 the same + 8: the key order of
  // the P fragment taken from the S accumulator.  tr_off[m]: byte offset for output tile m.
  const int tra = lane & 15, trg = (lane >> 4) & 1;
  const int tr_sw = D == 128 ? (tra >> 2) : ((tra >> 3) & 1);
  uint32_t tr_off[C::NM];
#pragma unroll
  for (int m = 0; m < C::NM; ++m)
    tr_off[m] = (uint32_t)((4 * h + (tra >> 2)) * C::KROW + (4 * (m ^ tr_sw) + 2 * trg + ((tra & 3) >> 1)) * 16 +
                           8 * (tra & 1));

  {
    // consume only a plan built for this launch (same dtype, unit size and CSR shape)
    const int32_t *sg = counter + ctl::kSig;
    const bool ok = sg[0] == units && sg[1] == G && sg[2] == FVATTN_BF16 && sg[3] == nqb && sg[4] == units / ngroups &&
                    sg[5] == nkb && sg[6] == N && sg[7] == ctl::kMagic;
    if (!ok) {
      if (tid == 0) atomicOr(reinterpret_cast<uint32_t *>(counter + ctl::kStatus), (uint32_t)FVATTN_STATUS_PLAN_MISMATCH);
      return;
    }
  }
  const bool per_xcd = counter[ctl::kPerXcd] != 0;
  const int xcc = (int)(__builtin_amdgcn_s_getreg((31 << 11) | 20) & 7);   // XCC_ID
  for (;;) {
    if (tid == 0) {
      int tk = units;
      if (!per_xcd) {
        tk = atomicAdd(&counter[ctl::kTicket], 1);
      } else {
        for (int qq = 0; qq < 8; ++qq) {
          const int x = (xcc + qq) & 7;
          const int c = atomicAdd(&counter[ctl::kXcdTicket + x], 1);
          if (c < counter[ctl::kXcdStart + 1 + x]) {
            tk = c;
            break;
          }
        }
      }
      s_tile = tk;
    }
    __syncthreads();
    const int t = s_tile;
    __syncthreads();
    if (t >= units) break;
    uint64_t t_start = 0;
    if (trace != nullptr) t_start = __builtin_amdgcn_s_memrealtime();

    const int u = worklist[t];
    const int bh = u / ngroups, g = u - bh * ngroups;
    const int r0 = bh * nqb + g * G;
    const int nrow = min(G, nqb - g * G);
    const uint16_t *kh = k + (size_t)bh * N * D;
    const uint16_t *vh = v + (size_t)bh * N * D;
    const __amdgpu_buffer_rsrc_t krs = buf_rsrc(kh, (uint32_t)N * D * 2);
    const __amdgpu_buffer_rsrc_t vrs = buf_rsrc(vh, (uint32_t)N * D * 2);
    // Tile loads of this group.  A negative block index loads from far outside the buffer:
    // the range check returns zeros without touching memory, so every X phase issues the same
    // number of loads and the vmcnt waits stay static.
    constexpr uint32_t kFar = 0x7fff0000u;
    // Piece i of a wave's part is 1 KB further in both the tile and LDS, so all pieces use the
    // part's LDS base with instruction offsets 1024 i.
    static_assert(C::KRPI * C::KROW == 1024 && C::KI * 1024 <= 4096, "1 KB pieces, 12-bit offsets");
    // Wave wg loads tile rows 16 wg .. 16 wg + 15: rows 16 wg.. of the block (64-token blocks)
    // or rows 16 (wg & 1).. of block `jb` of the tile's half wg / 2 (32-token blocks).
    const uint32_t row_off = (uint32_t)(PB == 1 ? wg : (wg & 1)) * C::KI * C::KRPI * C::KROW;
    auto load_k = [&](int jb, uint8_t *kbuf) {
      const uint32_t sbase = jb < 0 ? kFar : (uint32_t)jb * BK * D * 2 + row_off;
      uint8_t *dst = kbuf + wg * C::KI * 1024;
      auto piece = [&](auto ic) {
        constexpr int i = decltype(ic)::value;
        uint32_t vo;
        if constexpr (C::KTAB) {
          vo = k_vo[i % C::KPER];
        } else {
          const int gi = wg * C::KI + i;
          vo = (uint32_t)(k_r0 * C::KROW + swz_pos(k_pos, gi * C::KRPI + k_r0, C::KROW, C::KCR) * 16);
        }
        dma16_at<i * 1024>(krs, vo + sbase, dst);
      };
      piece(std::integral_constant<int, 0>{});
      if constexpr (C::KI > 1) piece(std::integral_constant<int, 1>{});
      if constexpr (C::KI > 2) piece(std::integral_constant<int, 2>{});
      if constexpr (C::KI > 3) piece(std::integral_constant<int, 3>{});
    };
    auto load_v = [&](int jb, uint8_t *vbuf) {
      const uint32_t sbase = jb < 0 ? kFar : (uint32_t)jb * BK * D * 2 + row_off;
      uint8_t *dst = vbuf + wg * C::KI * 1024;
      dma16_at<0>(vrs, v_vo + sbase, dst);
      if constexpr (C::KI > 1) dma16_at<1024>(vrs, v_vo + sbase, dst);
      if constexpr (C::KI > 2) dma16_at<2048>(vrs, v_vo + sbase, dst);
      if constexpr (C::KI > 3) dma16_at<3072>(vrs, v_vo + sbase, dst);
    };

    // this wave's query rows; loaded first, so the
    // barriers of the list construction below retire them before the first tile load
    const int qi = g * G + wq;
    const int qrow = qi * BQ + 32 * wr + l32;
    const bool qlive = qi < nqb && qrow < N;
    bf16x8 qf[C::NS];
    {
      const uint16_t *qp = q + ((size_t)bh * N + (qlive ? qrow : 0)) * D + 8 * h;
#pragma unroll
      for (int s = 0; s < C::NS; ++s) {
        u32x4 raw = {0u, 0u, 0u, 0u};
        if (qlive) raw = *reinterpret_cast<const u32x4 *>(qp + 16 * s);
        qf[s] = __builtin_bit_cast(bf16x8, raw);
      }
    }
    // kept lists of the unit's query blocks as LDS bitmaps, then their union as a list
    for (int i = tid; i < (G + 1) * MAXW; i += NTH) (&s_bm[0][0])[i] = 0;
    // the unit's rows are consecutive CSR rows: their entries form one range, loaded in one
    // round (row gi of entry e from the row boundaries)
    int rb[G + 1];
#pragma unroll
    for (int gi = 0; gi <= G; ++gi) rb[gi] = row_ptr[r0 + min(gi, nrow)];
    __syncthreads();
    for (int e = rb[0] + tid; e < rb[G]; e += NTH) {
      const int j = col_idx[e];
      int gi = 0;
#pragma unroll
      for (int x = 1; x < G; ++x) gi += e >= rb[x];
      atomicOr(&s_bm[gi][j >> 5], 1u << (j & 31));
      atomicOr(&s_bm[G][j >> 5], 1u << (j & 31));
    }
    __syncthreads();
    // union list: word prefix counts by one wave, then every thread places the blocks of its
    // own key positions.  64-token blocks: ascending.  32-token blocks: grouped by the set of
    // query blocks that kept them (ascending within a set, sets in increasing mask order), so
    // the two blocks of a tile are kept by the same waves, which compute it whole or skip it.
    constexpr int NCLS = PB == 2 ? (1 << G) - 1 : 1;
    auto class_word = [&](int c, int x) -> uint32_t {   // blocks of word x in class c
      uint32_t cw = s_bm[G][x];
      if constexpr (PB == 2) {
#pragma unroll
        for (int gi = 0; gi < G; ++gi) cw &= (((c + 1) >> gi) & 1) ? s_bm[gi][x] : ~s_bm[gi][x];
      }
      return cw;
    };
    if (w == 0) {
      int base = 0;
      for (int c = 0; c < NCLS; ++c) {
        for (int w0 = 0; w0 < nkw; w0 += 64) {   // 64 words at a time
          const int x = w0 + lane;
          const uint32_t word = x < nkw ? class_word(c, x) : 0u;
          const int pc = __popc(word);
          int incl = pc;
#pragma unroll
          for (int off = 1; off < 64; off <<= 1) {
            const int ov = __shfl_up(incl, off);
            if (lane >= off) incl += ov;
          }
          if (x < MAXW) s_cpre[c][x] = base + incl - pc;
          base += __shfl(incl, 63);
        }
      }
      if (lane == 0) s_n = base;
    }
    __syncthreads();
    for (int j = tid; j < nkw * 32; j += NTH) {
      const uint32_t word = s_bm[G][j >> 5];
      if ((word >> (j & 31)) & 1u) {
        int msk = 0;
#pragma unroll
        for (int gi = 0; gi < G; ++gi) msk |= (int)((s_bm[gi][j >> 5] >> (j & 31)) & 1u) << gi;
        const int c = PB == 2 ? msk - 1 : 0;
        s_list[s_cpre[c][j >> 5] + __popc(class_word(c, j >> 5) & ((1u << (j & 31)) - 1u))] = (j << 4) | msk;
      }
    }
    __syncthreads();
    const int n = s_n;
    const int S = (n + 2 * PB - 1) / (2 * PB);   // steps (tiles) of either group
    // List entries of a tile's key blocks (b: second block of a 32-token pair), -1 if none.
    struct Ent {
      int a, b;
    };
    auto entry = [&](int i) -> Ent {              // this group's step i
      const int e = PB * (2 * i + grp);
      Ent r;
      r.a = e < n ? __builtin_amdgcn_readfirstlane(s_list[e]) : -1;
      r.b = (PB == 2 && e + 1 < n) ? __builtin_amdgcn_readfirstlane(s_list[e + 1]) : -1;
      return r;
    };
    // the entry whose block this wave loads (entry -1 >> 4 = -1: an empty load)
    auto own = [&](const Ent &e) -> int { return (PB == 2 && (wg >> 1)) ? e.b : e.a; };
    auto keeps = [&](int e) -> bool { return e >= 0 && ((e >> wq) & 1); };

    Ent ep = {-1, -1}, ec = entry(0), e1 = entry(1);   // entries of steps i-1, i, i+1
    // X_i needs the entries of step i+2: they are read from LDS one phase ahead, so the
    // read's latency is spent in the M phase in between
    auto entry_lds = [&](int i) -> Ent {
      const int e = PB * (2 * i + grp);
      return Ent{e < n ? s_list[e] : -1, (PB == 2 && e + 1 < n) ? s_list[e + 1] : -1};
    };
    Ent enx = entry_lds(2);
    // prologue in the order a previous X phase would use: K_0, then K_1 and V_0
    load_k(own(ec) >> 4, K0[grp]);
    load_k(own(e1) >> 4, K1[grp]);
    load_v(own(ec) >> 4, V0[grp]);

    f16v oacc[C::NM];
#pragma unroll
    for (int m = 0; m < C::NM; ++m)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[m][i] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    bf16x8 pf[C::NKT][2];
#pragma unroll
    for (int kt = 0; kt < C::NKT; ++kt) pf[kt][0] = pf[kt][1] = bf16x8{};

    if (grp == 1) lds_barrier();   // group 1 runs one phase behind group 0

    // M_i: kb holds K_i, vbp holds V_{i-1}.  X_i loads K_{i+2} into kdst (the buffer of K_i)
    // and V_{i+1} into vdst (the buffer of V_{i-1}).  The loop is rotated so that its header
    // sits before an X phase (no tile reads there).
    f16v sacc[C::NKT];
    bool dos = false;
    auto phaseM = [&](const uint8_t *kb, const uint8_t *vbp) {
      // K_i and V_{i-1} landed: only the previous X phase's loads (K_{i+1}, then V_i) may
      // still be in flight
      wait_vmcnt<C::KI + C::VI>();
      lds_barrier();
      dos = keeps(ec.a) || keeps(ec.b);
      const bool dop = keeps(ep.a) || keeps(ep.b);
      __builtin_amdgcn_s_setprio(2);   // MFMA issue ahead of the partner wave's VALU work
      // Consecutive MFMAs go to independent accumulators (the NKT chains of S, the NM chains
      // of O).  Operands come from a ring of RING fragments read from LDS RING MFMAs ahead;
      // sched_barrier keeps the compiler from sinking the reads back to their uses.
      constexpr int RING = 3;
      if (dos) {
        constexpr int NT_S = C::NS * C::NKT;   // MFMA t: k-step t / NKT, key tile t % NKT
        auto kaddr = [&](int t) {
          const int s = t / C::NKT, kt = t % C::NKT;
          return reinterpret_cast<const bf16x8 *>(kb + (32 * kt + l32) * C::KROW +
                                                  swz_pos(2 * s + h, l32, C::KROW, C::KCR) * 16);
        };
        bf16x8 fr[RING];
#pragma unroll
        for (int t = 0; t < RING; ++t) fr[t] = *kaddr(t);
#pragma unroll
        for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
          for (int i2 = 0; i2 < 16; ++i2) sacc[kt][i2] = 0.f;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < NT_S; ++t) {
          sacc[t % C::NKT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[t % RING], qf[t / C::NKT], sacc[t % C::NKT], 0, 0, 0);
          if (t + RING < NT_S) fr[t % RING] = *kaddr(t + RING);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (dop) {
        constexpr int NT_P = C::NKT * 2 * C::NM;   // MFMA t: (kt, t2) = t / NM, output tile t % NM
        auto vfrag = [&](int t) -> bf16x8 {
          const int kk = t / C::NM, m = t % C::NM;
          const uint8_t *p0 = vbp + tr_off[m] + 16 * kk * C::KROW;
          const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)p0);
          const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(p0 + 8 * C::KROW));
          return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        bf16x8 fr[RING];
#pragma unroll
        for (int t = 0; t < RING; ++t) fr[t] = vfrag(t);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < NT_P; ++t) {
          const int kk = t / C::NM;
          oacc[t % C::NM] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[t % RING], pf[kk >> 1][kk & 1], oacc[t % C::NM], 0, 0, 0);
          if (t + RING < NT_P) fr[t % RING] = vfrag(t + RING);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __builtin_amdgcn_s_setprio(0);
    };
    auto phaseX = [&](int i, uint8_t *kdst, uint8_t *vdst) {
      lds_barrier();
      // ---- X_i
      const Ent e2 = {__builtin_amdgcn_readfirstlane(enx.a), __builtin_amdgcn_readfirstlane(enx.b)};
      enx = entry_lds(i + 3);
      load_k(own(e2) >> 4, kdst);
      load_v(own(e1) >> 4, vdst);
      if (dos) {
        // online softmax (lane: query qrow; keys 32kt + 8(v/4) + 4h + v%4 of the tile)
        if constexpr (PB == 1) {
          const int kbase = (ec.a >> 4) * BK;
          if (kbase + BK > N) {
            const int lim = N - kbase - 4 * h;
#pragma unroll
            for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
              for (int v = 0; v < 16; ++v)
                if (32 * kt + 8 * (v >> 2) + (v & 3) >= lim) sacc[kt][v] = -INFINITY;
          }
        } else {
          // 32-key half kt holds block (kt ? b : a): masked whole when this wave's query block
          // did not keep it (or it is absent), and past N when it is the ragged last block
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) {
            const int e = kt ? ec.b : ec.a;
            const bool kp = keeps(e);
            const int kbase = kp ? (e >> 4) * BK : 0;
            if (!kp || kbase + BK > N) {
              const int lim = kp ? N - kbase - 4 * h : -64;
#pragma unroll
              for (int v = 0; v < 16; ++v)
                if (8 * (v >> 2) + (v & 3) >= lim) sacc[kt][v] = -INFINITY;
            }
          }
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
        // Lazy rescale (wave-uniform branch): the reference maximum m_run is raised only when
        // some row's maximum exceeds it by more than kLazy (log2 units), so weights stay
        // below 2^kLazy and O is rescaled a few times per unit instead of at most steps.  The
        // row sum adds the bf16 weights that P.V uses, so O / l is an exact weighted mean of
        // those weights and their rounding cancels in the largest ones.
        constexpr float kLazy = 8.f;
        if (__any(mb > m_run + kLazy)) {
          const float m_new = fmaxf(m_run, mb);
          if (m_run != -INFINITY) {
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int m = 0; m < C::NM; ++m)
#pragma unroll
              for (int i2 = 0; i2 < 16; ++i2) oacc[m][i2] *= alpha;
          }
          m_run = m_new;
        }
        const float nm = -m_run;
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
        float ps[2] = {0.f, 0.f};
#pragma unroll
        for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
          for (int t2 = 0; t2 < 2; ++t2) {
            bf16x8 pv;
#pragma unroll
            for (int i2 = 0; i2 < 8; ++i2) pv[i2] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sacc[kt][8 * t2 + i2], sl2, nm));
            pf[kt][t2] = pv;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const bf16x2 pr = {pv[2 * j], pv[2 * j + 1]};
              ps[t2] = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, ps[t2], false);
            }
          }
        l_run += ps[0] + ps[1];
      }
      ep = ec;
      ec = e1;
      e1 = e2;
    };
    phaseM(K0[grp], V1[grp]);                      // M_0
    for (int i = 0; i < S; i += 2) {
      phaseX(i, K0[grp], V1[grp]);
      phaseM(K1[grp], V0[grp]);                    // M_{i+1}
      if (i + 1 == S) break;
      phaseX(i + 1, K1[grp], V0[grp]);
      phaseM(K0[grp], V1[grp]);                    // M_{i+2}
    }
    // The last X phase's tile loads (empty: zeros from past the buffer end) may still be in
    // flight into the buffers the merge reuses as its exchange area.
    wait_vmcnt<0>();
    if (grp == 0) lds_barrier();   // equal barrier counts for both groups
    lds_barrier();                 // both groups are past their last phase: tile buffers free

    // ---- merge: group g finalises output tiles [g*NH, g*NH + NH) and hands the partner
    // (same rows, other group) the other tiles through LDS.  The group number is made a
    // compile-time constant so that the accumulators are indexed statically.
    auto merge = [&](auto gc) {
      constexpr int GG = decltype(gc)::value;
      {
        float *xo = reinterpret_cast<float *>(GG == 0 ? &K0[0][0] : &K1[0][0]);
#pragma unroll
        for (int mm = 0; mm < NH; ++mm)
#pragma unroll
          for (int i = 0; i < 16; ++i) xo[((wg * NH + mm) * 16 + i) * 64 + lane] = oacc[(GG ^ 1) * NH + mm][i];
        s_xm[GG][wg][lane] = m_run;
        s_xl[GG][wg][lane] = l_run;
      }
      lds_barrier();
      const float *xi = reinterpret_cast<const float *>(GG == 0 ? &K1[0][0] : &K0[0][0]);
      const float m2 = s_xm[GG ^ 1][wg][lane], l2 = s_xl[GG ^ 1][wg][lane];
      const float mx = fmaxf(m_run, m2);
      const float a1 = mx == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mx);
      const float a2 = mx == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m2 - mx);
      const float lp = a1 * l_run + a2 * l2;
      auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lp), __float_as_uint(lp), false, false);
      const float inv = 1.f / (__uint_as_float(sw[0]) + __uint_as_float(sw[1]));
      f16v res[NH];
#pragma unroll
      for (int mm = 0; mm < NH; ++mm)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          res[mm][i] = (a1 * oacc[GG * NH + mm][i] + a2 * xi[((wg * NH + mm) * 16 + i) * 64 + lane]) * inv;
      // store (lane: query qrow, dims 32m + 8a + 4h + b)
      if (qlive && out_f32) {
        float *op = (float *)o + ((size_t)bh * N + qrow) * D + 4 * h;
#pragma unroll
        for (int mm = 0; mm < NH; ++mm)
#pragma unroll
          for (int a = 0; a < 4; ++a)
            *reinterpret_cast<f4 *>(op + 32 * (GG * NH + mm) + 8 * a) =
                f4{res[mm][4 * a], res[mm][4 * a + 1], res[mm][4 * a + 2], res[mm][4 * a + 3]};
      } else if (qlive) {
        uint16_t *op = (uint16_t *)o + ((size_t)bh * N + qrow) * D + 4 * h;
#pragma unroll
        for (int mm = 0; mm < NH; ++mm)
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const uint32_t w0 = pack_bf16(res[mm][4 * a], res[mm][4 * a + 1]);
            const uint32_t w1 = pack_bf16(res[mm][4 * a + 2], res[mm][4 * a + 3]);
            *reinterpret_cast<u32x2 *>(op + 32 * (GG * NH + mm) + 8 * a) = u32x2{w0, w1};
          }
      }
    };
    if (grp == 0) merge(std::integral_constant<int, 0>{});
    else merge(std::integral_constant<int, 1>{});
    if (trace != nullptr && tid == 0) {
      const uint64_t t_end = __builtin_amdgcn_s_memrealtime();
      trace[4 * (size_t)t + 0] = hw_id_word();
      trace[4 * (size_t)t + 1] = t_start;
      trace[4 * (size_t)t + 2] = t_end;
      trace[4 * (size_t)t + 3] = (uint64_t)u;
    }
  }
  // The last workgroup to leave restores the ticket counters and the exit count.
  if (tid == 0) {
    __threadfence();
    if (atomicAdd(&counter[ctl::kExit], 1) == (int)gridDim.x - 1) {
      atomicExch(&counter[ctl::kTicket], 0);
      for (int x = 0; x < 8; ++x) atomicExch(&counter[ctl::kXcdTicket + x], counter[ctl::kXcdStart + x]);
      atomicExch(&counter[ctl::kExit], 0);
    }
  }
}

// ---------------------------------------------------------------------------------------
// float32 attention on the float32 MFMA (v_mfma_f32_32x32x2_f32).  grid = rows (workgroup t
// processes CSR row worklist[t]); BQ / 32 waves, wave w owns query rows 32 w .. 32 w + 31 of the
// block.  The row's kept key blocks are walked in tiles of 32 keys staged in LDS, rows padded
// to D + 1 floats so that the 32 key rows of an operand read fall on distinct banks:
//   S^T (32 keys x 32 queries) = sum over the D / 2 steps j of K[key][2 j + h] Q[query][2 j + h]
//   (lane l: key or query l % 32, h = l / 32); online softmax in float32, exp2 with the scale
//   folded into one FMA; O^T (D x 32 queries) += V^T P, where step s of the product pairs the
//   two keys that accumulator element s holds in the lower and upper lane halves
//   (8 (s / 4) + s % 4 and the same + 4), so P feeds the MFMA straight from the S layout.
// ---------------------------------------------------------------------------------------
template <int BQ, int BK, int D>
__global__ __launch_bounds__(BQ * 2) void k_attn_f32(const float *__restrict__ q, const float *__restrict__ k,
                                                     const float *__restrict__ v, float *__restrict__ o,
                                                     const int32_t *__restrict__ row_ptr,
                                                     const int32_t *__restrict__ col_idx,
                                                     const int32_t *__restrict__ worklist,
                                                     int32_t *__restrict__ counter, int rows, int nqb, int nkb, int N,
                                                     float scale, uint64_t *__restrict__ trace) {
  static_assert(BQ % 32 == 0 && BK % 32 == 0 && D % 32 == 0, "32-row, 32-key and 32-dim tiles");
  constexpr int NT = BQ * 2;      // threads: BQ / 32 waves
  constexpr int LD = D + 1;       // padded tile row (floats)
  constexpr int NM = D / 32;      // 32-dim output tiles
  __shared__ float Kt[32 * LD];
  __shared__ float Vt[32 * LD];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int t = blockIdx.x;
  {
    // consume only a plan built for this launch (float32, one query block per unit, same CSR shape)
    const int32_t *sg = counter + ctl::kSig;
    const bool ok = sg[0] == rows && sg[1] == 1 && sg[2] == FVATTN_F32 && sg[3] == nqb && sg[4] == rows / nqb &&
                    sg[5] == nkb && sg[6] == N && sg[7] == ctl::kMagic;
    if (!ok) {
      if (tid == 0) atomicOr(reinterpret_cast<uint32_t *>(counter + ctl::kStatus), (uint32_t)FVATTN_STATUS_PLAN_MISMATCH);
      return;
    }
  }
  uint64_t t_start = 0;
  if (trace != nullptr) t_start = __builtin_amdgcn_s_memrealtime();
  const int row = worklist[t];
  const int bh = row / nqb, qi = row - bh * nqb;
  const int qrow = qi * BQ + 32 * w + l32;
  const bool live = qrow < N;
  // this lane's Q operand: Q[qrow][2 j + h]
  float qv[D / 2];
  const float *qp = q + ((size_t)bh * N + (live ? qrow : 0)) * D;
#pragma unroll
  for (int j = 0; j < D / 2; ++j) qv[j] = live ? qp[2 * j + h] : 0.f;
  f16v oacc[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[m][i] = 0.f;
  const float sl2 = scale * 1.4426950408889634f;
  float m_run = -INFINITY, l_run = 0.f;
  const int beg = row_ptr[row], end = row_ptr[row + 1];
  const float *kh = k + (size_t)bh * N * D;
  const float *vh = v + (size_t)bh * N * D;
  for (int e = beg; e < end; ++e) {
    const int kb0 = col_idx[e] * BK;
    for (int tt = 0; tt < BK / 32; ++tt) {
      const int key0 = kb0 + 32 * tt;
      if (key0 >= N) break;   // the same for every wave
      const int nk = min(32, N - key0);
      __syncthreads();        // the previous tile is consumed
      for (int i = tid; i < 32 * D; i += NT) {
        const int r = i / D, c = i % D;
        Kt[r * LD + c] = r < nk ? kh[(size_t)(key0 + r) * D + c] : 0.f;
        Vt[r * LD + c] = r < nk ? vh[(size_t)(key0 + r) * D + c] : 0.f;
      }
      __syncthreads();
      f16v sacc = {};
#pragma unroll
      for (int j = 0; j < D / 2; ++j)
        sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(Kt[l32 * LD + 2 * j + h], qv[j], sacc, 0, 0, 0);
      if (nk < 32) {   // keys past N (the ragged last block) do not take part
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (8 * (i >> 2) + 4 * h + (i & 3) >= nk) sacc[i] = -INFINITY;
      }
      float mloc = sacc[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mloc = fmaxf(mloc, sacc[i]);
      {
        auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mloc), __float_as_uint(mloc), false, false);
        mloc = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      // the tile holds at least one key below N, so the new maximum is finite
      const float m_new = fmaxf(m_run, mloc * sl2);
      const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sacc[i] = __builtin_amdgcn_exp2f(fmaf(sacc[i], sl2, -m_new));
        ps += sacc[i];
      }
      l_run = l_run * alpha + ps;
      m_run = m_new;
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[m][i] *= alpha;
#pragma unroll
      for (int s2 = 0; s2 < 16; ++s2) {
        const int key = 8 * (s2 >> 2) + 4 * h + (s2 & 3);
#pragma unroll
        for (int m = 0; m < NM; ++m)
          oacc[m] = __builtin_amdgcn_mfma_f32_32x32x2f32(Vt[key * LD + 32 * m + l32], sacc[s2], oacc[m], 0, 0, 0);
      }
    }
  }
  // the row sum is split between the lane halves (each holds 16 of every 32 keys)
  auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
  const float inv = 1.f / (__uint_as_float(sw[0]) + __uint_as_float(sw[1]));
  if (live) {
    // lane: query qrow, dims 32 m + 8 a + 4 h + b
    float *op = o + ((size_t)bh * N + qrow) * D + 4 * h;
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        *reinterpret_cast<f4 *>(op + 32 * m + 8 * a) =
            f4{oacc[m][4 * a] * inv, oacc[m][4 * a + 1] * inv, oacc[m][4 * a + 2] * inv, oacc[m][4 * a + 3] * inv};
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
template <int BQ, int BK, int D>
static int launch_attn_bf16_t(const void *q, const void *k, const void *v, void *o, int out_f32,
                              const int32_t *row_ptr, const int32_t *col_idx, const int32_t *wl, int32_t *counter,
                              int rows, int nqb, int nkb, int N, int grid, uint64_t *trace, hipStream_t st) {
  // two wave groups per unit (k_attn_pp), V as given
  auto kern = k_attn_pp<BQ, BK, D>;
  const int nthreads = 512;
  constexpr int G = 128 / BQ;
  const int ngroups = (nqb + G - 1) / G;
  const int units = (rows / nqb) * ngroups;
  if (grid <= 0) {
    int cus = 0, occ = 0;
    if (device_cus(&cus) != 0) return FVATTN_ERR_HIP;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, nthreads, 0) != hipSuccess) return FVATTN_ERR_HIP;
    grid = cus * (occ > 0 ? occ : 1);
  }
  if (grid > units) grid = units;
  const float sl2 = (float)(1.4426950408889634 / sqrt((double)D));
  hipLaunchKernelGGL(kern, dim3(grid), dim3(nthreads), 0, st, (const uint16_t *)q, (const uint16_t *)k,
                     (const uint16_t *)v, o, out_f32, row_ptr, col_idx, wl, counter, units, ngroups,
                     nqb, nkb, N, sl2, trace);
  FV_CHECK_LAUNCH();
  return FVATTN_OK;
}

int launch_attn_bf16(const void *q, const void *k, const void *v, void *o, int out_f32,
                     const int32_t *row_ptr,
                     const int32_t *col_idx, const int32_t *wl, int32_t *counter, int rows, int nqb, int nkb, int N,
                     int D, int BQ, int BK, int grid, uint64_t *trace, hipStream_t st) {
#define FV_A(bq, bk, dd)                                                                                 \
  if (BQ == bq && BK == bk && D == dd)                                                                   \
    return launch_attn_bf16_t<bq, bk, dd>(q, k, v, o, out_f32, row_ptr, col_idx, wl, counter, rows, nqb, nkb, N, \
                                          grid, trace, st);
  FV_A(64, 64, 128) FV_A(128, 64, 128) FV_A(32, 64, 128) FV_A(64, 32, 128) FV_A(128, 32, 128) FV_A(32, 32, 128)
  FV_A(64, 64, 64) FV_A(128, 64, 64) FV_A(32, 64, 64) FV_A(64, 32, 64) FV_A(128, 32, 64) FV_A(32, 32, 64)
#undef FV_A
  return FVATTN_ERR_UNSUPPORTED;
}

template <int BQ, int BK, int D>
static int launch_attn_f32_t(const void *q, const void *k, const void *v, void *o, const int32_t *row_ptr,
                             const int32_t *col_idx, const int32_t *wl, int32_t *counter, int rows, int nqb, int nkb,
                             int N, uint64_t *trace, hipStream_t st) {
  const float scale = (float)(1.0 / sqrt((double)D));
  hipLaunchKernelGGL((k_attn_f32<BQ, BK, D>), dim3(rows), dim3(BQ * 2), 0, st, (const float *)q, (const float *)k,
                     (const float *)v, (float *)o, row_ptr, col_idx, wl, counter, rows, nqb, nkb, N, scale, trace);
  FV_CHECK_LAUNCH();
  return FVATTN_OK;
}

int launch_attn_f32(const void *q, const void *k, const void *v, void *o, const int32_t *row_ptr,
                    const int32_t *col_idx, const int32_t *wl, int32_t *counter, int rows, int nqb, int nkb, int N,
                    int D, int BQ, int BK, uint64_t *trace, hipStream_t st) {
#define FV_F(bq, bk, dd) \
  if (BQ == bq && BK == bk && D == dd) \
    return launch_attn_f32_t<bq, bk, dd>(q, k, v, o, row_ptr, col_idx, wl, counter, rows, nqb, nkb, N, trace, st);
  FV_F(64, 64, 128) FV_F(128, 64, 128) FV_F(32, 64, 128) FV_F(64, 32, 128) FV_F(128, 32, 128) FV_F(32, 32, 128)
  FV_F(64, 64, 64) FV_F(128, 64, 64) FV_F(32, 64, 64) FV_F(64, 32, 64) FV_F(128, 32, 64) FV_F(32, 32, 64)
#undef FV_F
  return FVATTN_ERR_UNSUPPORTED;
}

}  // namespace fv
