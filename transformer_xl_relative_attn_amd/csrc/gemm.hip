// Projection GEMMs of the relative-attention layer:
//   q = h W_q^T, k = h~ W_kE^T, val^T = W_v h~^T, Rk = R W_kR^T, and (full
//   layer) Linear(a), FFN.  Every product has the form C[m][n] = sum_k A(m,k) B(n,k)
//   with both operands K-contiguous; rows are fetched through RowSrc maps so
//   that h~ = [memory ring ; segment] is gathered on the fly.
//
// gemm_bf16: bf16 operands, fp32 accumulation on the gfx950 matrix cores
//   (v_mfma_f32_32x32x16_bf16).  256x256 block tile, 8 waves in a 2x4 grid
//   (two per SIMD), each wave owns a 128x64 sub-tile (4x2 MFMA tiles, 128
//   accumulator registers); groups with few tiles use 128x128 blocks of 4
//   waves, two workgroups per CU.  Operands stream through an NSTAGE-deep LDS ring of 32-wide
//   K steps filled by direct global->LDS loads (no register staging), issued
//   NSTAGE-1 K steps ahead of their use; MFMA operand reads and refill loads
//   are spread evenly between the MFMAs.  Persistent: one workgroup per CU
//   walks the tiles; in the 256x256 variant the ring refills past a tile's
//   last K step load the next tile's first K steps (elsewhere they are issued
//   before the epilogue), so they land while the current tile's epilogue
//   stages its bf16 output through a separate 32 KB LDS region.
//   Requirements (checked by the host): K % 64 == 0, every row 16-byte
//   aligned.
//
// gemm_f32: fp32 operands and arithmetic on the vector ALUs (64x64 tile),
//   used by the fp32 path.
#include <type_traits>

#include "dev_common.h"

namespace txl {

namespace {

constexpr int BK = 32;

template <int X>
using IC = std::integral_constant<int, X>;
#ifndef TXL_GEMM_NSTAGE
#define TXL_GEMM_NSTAGE 3
#endif
constexpr int CH = BK / 8;               // 16-byte chunks per tile row (4)

// Block-tile variants: WM x WN MFMA tiles of 32x32 per wave, GM x GN waves,
// square blocks (BM == BN), NSTAGE-deep LDS ring, OCC workgroups per CU.
template <int WM_, int WN_, int GM_, int GN_, int NSTAGE_, int OCC_>
struct Var {
  static constexpr int WM = WM_, WN = WN_, GM = GM_, GN = GN_;
  static constexpr int NW = GM * GN;              // waves per workgroup
  static constexpr int NTH = 64 * NW;             // threads
  static constexpr int WTM = 32 * WM, WTN = 32 * WN;   // wave tile
  static constexpr int BM = WTM * GM, BN = WTN * GN;   // block tile
  static_assert(BM == BN, "square block tiles");
  static constexpr int TILE_U = BM * CH;          // 16-byte units per operand tile
  static constexpr int STAGE_U = 2 * TILE_U;      // A tile then B tile
  static constexpr int LOADS = TILE_U / NTH;      // LDS-DMA loads per thread per operand
  static constexpr int NSTAGE = NSTAGE_;          // LDS ring depth
  static constexpr int CPR = 4 * WN;              // 16-byte chunks per staged output row
  static constexpr int EPI_U = 32 * CPR;          // 16-byte units of a wave's staging region
  static constexpr int OCC = OCC_;
};
//   V256W8: 256x256, 8 waves of 128x64 (two per SIMD: while one waits on the
//           barrier or its LDS reads the other keeps the matrix core busy),
//           one workgroup per CU (large problems).  Measured against 4 waves of
//           128x128 on the same LDS ring: 70 vs 75 us on the eval-shaped
//           projections, 118 vs 121 us at 4096^3.
//   V128:   128x128, 4 waves of 64x64, two workgroups per CU (problems with
//           few 256-tiles)
//   V128W8: 128x128, 8 waves of 32x64, one workgroup per CU (problems with no
//           more 128-tiles than compute units, which would otherwise leave
//           one wave per SIMD and nothing to cover its waits)
using V256W8 = Var<4, 2, 2, 4, TXL_GEMM_NSTAGE, 1>;
using V128 = Var<2, 2, 2, 2, 4, 2>;
using V128W8 = Var<1, 2, 4, 2, 4, 1>;

// 128 bytes of zeros: the source of every "zero row" chunk (padding rows).
__device__ __align__(16) uint32_t g_zero_chunk[32];

__device__ __forceinline__ int find_problem(const GemmGroup& g, int32_t tile, int32_t* local) {
  int idx = 0;
#pragma unroll
  for (int i = 1; i < kMaxGroup; ++i)
    if (i < g.count && tile >= g.p[i].tile_begin) idx = i;
  *local = tile - g.p[idx].tile_begin;
  return idx;
}

// Problem and (row, column) tile of a tile id: n fastest within a problem,
// except for an interleaved pair (GemmGroup::pair1).
__device__ __forceinline__ int tile_coords(const GemmGroup& g, int32_t tile, int32_t* tm,
                                           int32_t* tn) {
  int32_t local;
  int idx = find_problem(g, tile, &local);
  const int pr = g.pair1 - 1;
  if (pr >= 0 && (idx == pr || idx == pr + 1)) {
    const GemmProblem& P = g.p[pr];
    const int32_t loc = tile - P.tile_begin;
    const int32_t per = 2 * P.tiles_n;
    const int32_t panel = loc / per, r = loc - panel * per;
    if (r < P.tiles_n) {
      *tm = panel;
      *tn = r;
      return pr;
    }
    *tm = r - P.tiles_n;
    *tn = panel;
    return pr + 1;
  }
  const GemmProblem& P = g.p[idx];
  *tm = local / P.tiles_n;
  *tn = local - *tm * P.tiles_n;
  return idx;
}

// Wait until at most N LDS-DMA loads of this wave are still in flight.  The
// loads are not fenced by the compiler (a __syncthreads would wait for all of
// them), so the waits are explicit.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier after this wave's LDS reads have completed, without
// waiting on outstanding global loads.  The LDS wait is the compiler's own
// s_waitcnt, so its wait-count bookkeeping knows the reads are done.
__device__ __forceinline__ void barrier_lds() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt / expcnt untouched
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// Vectorised epilogue: four consecutive output columns per store.  FLAGS < 0
// means "read the residual / ReLU flags at run time".
template <class V, int DTYPE, int FLAGS>
__device__ __forceinline__ void epilogue_vec(const OutDst& o, const floatx16 (&acc)[V::WM][V::WN],
                                             int32_t mb, int32_t nb) {
  constexpr int WM = V::WM, WN = V::WN;
  const int flags = FLAGS < 0 ? o.flags : FLAGS;
  int64_t roff[WM];
  bool mok[WM];
#pragma unroll
  for (int i = 0; i < WM; ++i) {
    mok[i] = mb + 32 * i < o.m_valid;
    roff[i] = axis_off(o.row, mb + 32 * i);
  }
#pragma unroll
  for (int j = 0; j < WN; ++j)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int32_t n = nb + 32 * j + 8 * g;
      if (n >= o.n_valid) continue;
      const int64_t coff = col_off(o, n);
#pragma unroll
      for (int i = 0; i < WM; ++i) {
        if (!mok[i]) continue;
        const int64_t off = roff[i] + coff;
        floatx4 v = floatx4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                            acc[i][j][4 * g + 3]};
        if (flags & EPI_RESID) v += *reinterpret_cast<const floatx4*>(o.resid + off);
        if (flags & EPI_RELU) {
#pragma unroll
          for (int c = 0; c < 4; ++c) v[c] = fmaxf(v[c], 0.0f);
        }
        if (DTYPE == TXL_F32) {
          *reinterpret_cast<floatx4*>(static_cast<float*>(o.p) + off) = v;
        } else {
          typedef float floatx2_t __attribute__((ext_vector_type(2)));
          typedef bf16 bf16x2_t __attribute__((ext_vector_type(2)));
          const bf16x2_t lo = __builtin_convertvector(floatx2_t{v[0], v[1]}, bf16x2_t);
          const bf16x2_t hi = __builtin_convertvector(floatx2_t{v[2], v[3]}, bf16x2_t);
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(o.p) + off) =
              u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
        }
      }
    }
}

// bf16 output without a residual (ReLU optional): the wave's WTM x WTN
// sub-tile (rows mw.., columns nw..) passes through the wave's own LDS region
// in rounds of 32 rows, so that the global stores write whole lines (CPR
// lanes cover one output row of the sub-tile contiguously) instead of
// 16-byte pieces of 32 rows, which the L2 would receive as 32 partial-line
// writes per instruction.  The region is separate from the operand ring, so
// the next tile's first K steps can already be landing.  Staging layout: row
// r (0..31) is CPR chunks of 16 bytes, chunk c at slot c ^ (r % CPR); both the
// 8-byte writes (32 rows x 2 halves) and the 16-byte reads (CPR lanes per row)
// are then spread over all 64 banks.
template <class V, bool RELU>
__device__ __forceinline__ void epilogue_staged(const OutDst& o,
                                                const floatx16 (&acc)[V::WM][V::WN], int32_t mw,
                                                int32_t nw, int lane, u32x4* region) {
  constexpr int WM = V::WM, WN = V::WN;
  typedef float floatx2_t __attribute__((ext_vector_type(2)));
  typedef bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  constexpr int CPR = V::CPR;            // chunks (lanes) per row
  constexpr int RG = 64 / CPR;           // rows per store instruction
  constexpr int NR = 32 / RG;            // store instructions per round
  char* base = reinterpret_cast<char*>(region);
  const int lrow = lane & 31, lhalf = lane >> 5;
  // lane -> chunk c (columns nw + 8c .. +7) of rows RG*t + rsub
  const int c = lane % CPR, rsub = lane / CPR;
  const int32_t n = nw + 8 * c;
  const bool nok = n < o.n_valid;
  const int64_t coff = col_off(o, n);
  // row offsets advance incrementally: +RG rows per step, at most one wrap of
  // the row axis (div >= 8)
  int32_t m = mw + rsub;
  const int32_t q0 = axis_quot(o.row, m);
  int32_t rem = m - q0 * o.row.div;
  int64_t off = (int64_t)q0 * o.row.s1 + (int64_t)rem * o.row.s2 + coff;
  const int64_t step = RG * o.row.s2, wrap = o.row.s1 - (int64_t)o.row.div * o.row.s2;
  uint16_t* out = static_cast<uint16_t*>(o.p);
  auto act = [](float x) { return RELU ? fmaxf(x, 0.0f) : x; };
#pragma unroll
  for (int i = 0; i < WM; ++i) {
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int cc = 4 * j + q;   // columns 32j + 8q + 4*lhalf .. +3
        const bf16x2_t lo = __builtin_convertvector(
            floatx2_t{act(acc[i][j][4 * q]), act(acc[i][j][4 * q + 1])}, bf16x2_t);
        const bf16x2_t hi = __builtin_convertvector(
            floatx2_t{act(acc[i][j][4 * q + 2]), act(acc[i][j][4 * q + 3])}, bf16x2_t);
        *reinterpret_cast<u32x2*>(base + lrow * (CPR * 16) + ((cc ^ (lrow % CPR)) << 4) +
                                  8 * lhalf) =
            u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
      }
    wave_lds_fence();
    u32x4 v[NR];
#pragma unroll
    for (int t = 0; t < NR; ++t) {
      const int r = RG * t + rsub;
      v[t] = *reinterpret_cast<const u32x4*>(base + r * (CPR * 16) + ((c ^ (r % CPR)) << 4));
    }
    wave_lds_fence();   // the next round rewrites the region
#pragma unroll
    for (int t = 0; t < NR; ++t) {
      if (nok && m < o.m_valid) *reinterpret_cast<u32x4*>(out + off) = v[t];
      m += RG;
      rem += RG;
      off += step;
      if (rem >= o.row.div) {
        rem -= o.row.div;
        off += wrap;
      }
    }
  }
}

// Epilogue of one tile, straight from the accumulators.  The MFMA operands are
// swapped (B fragment first), so block (i, j) holds C^T: element 4g + r of a
// lane is C[m][n] with m = mb + 32i and n = nb + 32j + 8g + r, i.e. four
// consecutive output columns of one row per (i, j, g).
template <class V>
__device__ __forceinline__ void epilogue(const GemmProblem& P, const floatx16 (&acc)[V::WM][V::WN],
                                         int32_t m0, int32_t n0, int wm, int wn, int lane,
                                         u32x4* smem) {
  constexpr int WM = V::WM, WN = V::WN, WTM = V::WTM, WTN = V::WTN, EPI_U = V::EPI_U;
  const int lrow = lane & 31, lhalf = lane >> 5, wave = wm * V::GN + wn;
  const OutDst& o = P.out;
  const int32_t mb = m0 + wm * WTM + lrow;
  const int32_t nb = n0 + wn * WTN + 4 * lhalf;
  if (o.vec8_ok && o.flags == 0) {
    epilogue_staged<V, false>(o, acc, m0 + wm * WTM, n0 + wn * WTN, lane, smem + wave * EPI_U);
    return;
  }
  if (o.vec8_ok && o.flags == EPI_RELU) {
    epilogue_staged<V, true>(o, acc, m0 + wm * WTM, n0 + wn * WTN, lane, smem + wave * EPI_U);
    return;
  }
  if (o.vec_ok) {
    if (o.flags == 0 && o.dtype == TXL_BF16)
      epilogue_vec<V, TXL_BF16, 0>(o, acc, mb, nb);
    else if (o.flags == 0)
      epilogue_vec<V, TXL_F32, 0>(o, acc, mb, nb);
    else if (o.dtype == TXL_BF16)
      epilogue_vec<V, TXL_BF16, -1>(o, acc, mb, nb);
    else
      epilogue_vec<V, TXL_F32, -1>(o, acc, mb, nb);
    return;
  }
  // Rare layouts (unaligned or odd leading dimension): one element at a time
  // through an LDS transpose in the wave's staging region (a 32 x 32 float
  // block, row ml rotated by ml to spread the column accesses over the banks),
  // so that the accumulators are only indexed statically.
  static_assert(32 * 32 * 4 <= EPI_U * 16, "transpose block fits the staging region");
  float* stage = reinterpret_cast<float*>(smem + wave * EPI_U);
  auto at = [](int ml, int nl) { return ml * 32 + ((nl + ml) & 31); };
#pragma unroll
  for (int i = 0; i < WM; ++i) {
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const floatx16 a = acc[i][j];
#pragma unroll
      for (int e = 0; e < 16; ++e) stage[at(lrow, 8 * (e >> 2) + 4 * lhalf + (e & 3))] = a[e];
      wave_lds_fence();
      // stage[m_local][n_local] for m = mb - lrow + m_local, n = nb - 4*lhalf + 32j + n_local
      for (int t = lane; t < 32 * 32; t += 64) {
        const int ml = t >> 5, nl = t & 31;
        const int32_t m = m0 + wm * WTM + 32 * i + ml;
        const int32_t n = n0 + wn * WTN + 32 * j + nl;
        if (m < o.m_valid && n < o.n_valid)
          epi_store(o, axis_off(o.row, m) + col_off(o, n), stage[at(ml, nl)]);
      }
      wave_lds_fence();
    }
  }
}

template <class V>
__device__ __forceinline__ void gemm_bf16_body(const GemmGroup& g, int32_t padded, int32_t grid) {
  constexpr int WM = V::WM, WN = V::WN, NW = V::NW, BM = V::BM, BN = V::BN, WTM = V::WTM,
                WTN = V::WTN, TILE_U = V::TILE_U, STAGE_U = V::STAGE_U, LOADS = V::LOADS,
                NSTAGE = V::NSTAGE, EPI_U = V::EPI_U;
  // LDS ring: stage s holds A rows [0,BM) then B rows [0,BN), each row 4
  // chunks of 16 bytes; chunk c of row r is stored at slot c ^ ((r >> 2) & 3).
  // gfx950 serves a 16-byte read for 16 lanes at a time from 64 four-byte
  // banks, so rows r, r+4, r+8, r+12 (same bank group at a 64-byte pitch) must
  // use different slots: 16 consecutive rows then read one chunk conflict-free.
  // the per-wave epilogue staging follows the ring in the same LDS object
  // (a second object defeats the compiler's LDS-DMA alias tracking, which
  // then waits for every load before each LDS read)
  __shared__ u32x4 smem[NSTAGE * STAGE_U + NW * EPI_U];
  u32x4* const stage_out = smem + NSTAGE * STAGE_U;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / V::GN, wn = wave % V::GN;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);

  // LDS-DMA mapping: load i of this wave fills units [(NW*i + wave)*64, +64)
  // of a tile, i.e. row (NW*i + wave)*16 + lane/4, slot lane%4, which holds
  // global chunk (lane%4) ^ ((row >> 2) & 3) = (lane%4) ^ ((lane >> 4) & 3).
  const int gchunk = (lane & 3) ^ ((lane >> 4) & 3);
  const char* zero = reinterpret_cast<const char*>(g_zero_chunk) + gchunk * 16;

  // Persistent: this workgroup walks tiles seq = blockIdx.x, +grid, ...; the
  // XCD swizzle keeps tiles that share A rows on one XCD.
  int32_t seq = blockIdx.x;
  auto next_tile = [&](int32_t s) {   // first valid tile at or after sequence s
    while (s < padded && xcd_swizzle(s, padded) >= g.total_tiles) s += grid;
    return s;
  };
  seq = next_tile(seq);
  if (seq >= padded) return;

  // per-tile state (the problem is addressed by index: a pointer into the
  // kernel-argument block would force a private copy of it)
  int pidx = 0;
  int32_t m0 = 0, n0 = 0, nk = 0;
  const char* pa[LOADS];
  const char* pb[LOADS];
  int64_t sa[LOADS], sb[LOADS];   // per-K-step advance: BK*2 bytes, or 0 for zero rows
  auto setup = [&](int32_t tile) {
    int32_t tm, tn;
    pidx = tile_coords(g, tile, &tm, &tn);
    const GemmProblem& P = g.p[pidx];
    m0 = tm * BM;
    n0 = tn * BN;
    nk = P.K / BK;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int r = (NW * i + wave) * 16 + (lane >> 2);
      const char* a = (m0 + r < P.M) ? row_address(P.a, m0 + r, 2) : nullptr;
      const char* b = (n0 + r < P.N) ? row_address(P.b, n0 + r, 2) : nullptr;
      pa[i] = a ? a + gchunk * 16 : zero;
      pb[i] = b ? b + gchunk * 16 : zero;
      sa[i] = a ? BK * 2 : 0;
      sb[i] = b ? BK * 2 : 0;
    }
  };

  // LDS-DMA q (0..2*LOADS-1: operand q & 1, row group q >> 1) of the next K step
  // into a ring stage; the running pointer advances by one K step.  With
  // `real` false (past the end of K) the zero chunk is loaded instead, into a
  // slot that is never read again: the loop body stays the same in every
  // iteration and the wait counts stay fixed.
  auto issue_one = [&](u32x4* st, int q, bool real) {
    const int i = q >> 1;
    if (q & 1) {
      __builtin_amdgcn_global_load_lds(real ? pb[i] : zero, st + NW * i * 64 + TILE_U, 16, 0, 0);
      pb[i] += sb[i];
    } else {
      __builtin_amdgcn_global_load_lds(real ? pa[i] : zero, st + NW * i * 64, 16, 0, 0);
      pa[i] += sa[i];
    }
  };
  auto stage_ptr = [&](int slot) { return smem + slot * STAGE_U; };

  const int lrow = lane & 31, lhalf = lane >> 5;
  const int sw = (lrow >> 2) & 3;  // same for every fragment row of a lane
  int fa[WM], fb[WN];              // fragment row base (16-byte units) within a stage
#pragma unroll
  for (int i = 0; i < WM; ++i) fa[i] = (wm * WTM + i * 32 + lrow) * CH;
#pragma unroll
  for (int j = 0; j < WN; ++j) fb[j] = TILE_U + (wn * WTN + j * 32 + lrow) * CH;
  // fragment f (0..WM-1: A rows 32f.., WM..WM+WN-1: B rows 32(f-WM)..) of
  // k-step s (0 or 1) of a staged 32-wide K step
  auto read_one = [&](const u32x4* st, int s, int f, bf16x8* af, bf16x8* bfr) {
    const int c = (2 * s + lhalf) ^ sw;
    if (f < WM)
      af[f] = __builtin_bit_cast(bf16x8, st[fa[f] + c]);
    else
      bfr[f - WM] = __builtin_bit_cast(bf16x8, st[fb[f - WM] + c]);
  };
  floatx16 acc[WM][WN];
  auto mfma_one = [&](int x, const bf16x8* af, const bf16x8* bfr) {
    const int i = x / WN, j = x % WN;
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
  };

  // One K step (ring slot `slot`, 32 wide = two MFMA k-steps), in two halves
  // whose instruction order is fixed with scheduling fences:
  //   A: WM*WN MFMAs on k-step 0 (fragments F0, already in registers); the
  //      k-step 1 fragments F1 are read during the first WM+WN;
  //   wait until K step kt+1 has landed (`vm` loads may stay in flight),
  //   barrier: every wave is done with this slot;
  //   B: WM*WN MFMAs on F1, interleaved with the 2*LOADS refill loads of this
  //      slot (K step kt+NSTAGE; zero chunk if that is past the end) and, in
  //      the first half of them, the reads of K step kt+1's F0.
  // Spreading the loads and reads evenly keeps the single wave per SIMD
  // issuing MFMAs back to back.  (In the last step the F0 read is of a stale
  // slot and unused.)
  bf16x8 f0a[WM], f0b[WN], f1a[WM], f1b[WN];
  constexpr int NF = WM + WN;             // fragments per k-step
  constexpr int NQ = 2 * LOADS;           // refill loads per wave and K step
  constexpr int MPQ = WM * WN / NQ;       // MFMAs per refill load
  static_assert(MPQ * NQ == WM * WN, "MFMAs split evenly between the loads");
  auto kstep = [&](auto X, int slot, int nslot, bool refill) {
    constexpr int EXTRA = decltype(X)::value;   // stores queued behind K step kt+1
    const u32x4* st = stage_ptr(slot);
#pragma unroll
    for (int x = 0; x < WM * WN; ++x) {
      mfma_one(x, f0a, f0b);
      if (x < NF) read_one(st, 1, x, f1a, f1b);
      __builtin_amdgcn_sched_barrier(0);
    }
    // (a wave tile of fewer 32x32 blocks than fragments reads the rest here)
#pragma unroll
    for (int x = WM * WN; x < NF; ++x) read_one(st, 1, x, f1a, f1b);
    wait_vm<(NSTAGE - 2) * 2 * LOADS + EXTRA>();
    barrier_lds();
    u32x4* rs = smem + slot * STAGE_U + wave_s * 64;
    const u32x4* nst = stage_ptr(nslot);
    // F0 reads in the order the next MFMAs consume them (A0, B0..B(WN-1),
    // A1..A(WM-1)), all in the first half so that they have landed when the
    // next step starts
    constexpr int RPQ = (NF + NQ / 2 - 1) / (NQ / 2);   // reads per load
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
#pragma unroll
      for (int x = 0; x < MPQ; ++x) mfma_one(MPQ * q + x, f1a, f1b);
      issue_one(rs, q, refill);
#pragma unroll
      for (int r = 0; r < RPQ; ++r) {
        const int k = RPQ * q + r;   // k-th fragment in consumption order
        if (k < NF) read_one(nst, 0, k == 0 ? 0 : k <= WN ? WM + k - 1 : k - WN, f0a, f0b);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Stage the first NSTAGE K steps of the current tile (zero chunks past K).
  auto prologue = [&]() {
#pragma unroll
    for (int s = 0; s < NSTAGE; ++s) {
      u32x4* rs = smem + s * STAGE_U + wave_s * 64;
#pragma unroll
      for (int q = 0; q < 2 * LOADS; ++q) issue_one(rs, q, s < nk);
    }
  };

  setup(xcd_swizzle(seq, padded));
  prologue();
  int slot0 = 0;   // ring slot of the current tile's K step 0

  // A staged epilogue of a sub-tile that lies wholly inside the output issues
  // exactly EPI_STORES global stores, after the next tile's first NSTAGE
  // stages.  Vector memory operations of a wave complete in issue order, so
  // the waits for those stages may leave the stores in flight: the next
  // tile's first K steps overlap the previous tile's write-back.
  constexpr int EPI_STORES = WM * (32 / (64 / V::CPR));
  bool pend = false;
  while (true) {
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int j = 0; j < WN; ++j) acc[i][j] = floatx16{0};

    // Loads return in order and every step issues exactly one stage, so the
    // wait counts are fixed: K step 0 has landed once at most NSTAGE-1 stages
    // issued after it remain, step kt+1 once NSTAGE-2 remain (plus, while it
    // is one of the first NSTAGE stages, the previous tile's stores).
    // Epilogue stores other than the counted ones only make the waits stricter.
    const bool peel = pend && nk >= NSTAGE - 1;
    if (peel)
      wait_vm<(NSTAGE - 1) * 2 * LOADS + EPI_STORES>();
    else
      wait_vm<(NSTAGE - 1) * 2 * LOADS>();
    barrier_lds();
    {
      const u32x4* st = stage_ptr(slot0);
#pragma unroll
      for (int f = 0; f < NF; ++f) read_one(st, 0, f, f0a, f0b);
    }
    // This tile's problem and position (the epilogue's), and the next tile of
    // this workgroup.  Once the refills run past this tile's last K step they
    // load the next tile's first NSTAGE K steps instead of zero chunks: its
    // operands then land while this tile finishes and writes its epilogue.
    // The next tile's step j goes to the slot of this tile's step nk + j, so
    // its K loop starts at slot (slot0 + nk) % NSTAGE.  Tiles shorter than the
    // ring (nk < NSTAGE) keep the plain prologue after the loop.
    const int cpidx = pidx;
    const int32_t cm0 = m0, cn0 = n0, nkc = nk;
    const int32_t nseq = next_tile(seq + grid);
    const bool more = nseq < padded;
    // (the 128x128 variants, which mostly run one tile per workgroup, keep the
    // plain prologue: the set-up inside their K loop made the compiler copy
    // the kernel-argument block to scratch)
    const bool ahead = V::BM == 256 && more && nkc >= NSTAGE;
    int32_t nkn = 0;   // the next tile's K steps (known once its pointers are set up)
    auto refill = [&](int32_t tgt) {   // refill for step tgt of this tile: real load?
      if (tgt < nkc) return true;
      if (!ahead) return false;
      if (tgt == nkc) {
        setup(xcd_swizzle(nseq, padded));
        nkn = nk;
      }
      return tgt - nkc < nkn;
    };
    int slot = slot0, kt = 0;
    if (peel) {
#pragma unroll
      for (int p = 0; p < NSTAGE - 1; ++p) {
        const int cs = slot + 1 == NSTAGE ? 0 : slot + 1;
        const bool real = refill(p + NSTAGE);
        kstep(IC<EPI_STORES>{}, slot, cs, real);
        slot = cs;
      }
      kt = NSTAGE - 1;
    }
#pragma unroll 1
    for (; kt < nkc - 1; ++kt) {
      const int nslot = slot + 1 == NSTAGE ? 0 : slot + 1;
      const bool real = refill(kt + NSTAGE);
      kstep(IC<0>{}, slot, nslot, real);
      slot = nslot;
    }
    if (kt == nkc - 1) {
      // the last K step: the stage after it (the next tile's first, or zero
      // chunks) is not read by this tile, so its loads may stay in flight
      const int nslot = slot + 1 == NSTAGE ? 0 : slot + 1;
      const bool real = refill(kt + NSTAGE);
      kstep(IC<2 * LOADS>{}, slot, nslot, real);
      slot = nslot;
    }
    // Every wave is done reading the ring.  Without the look-ahead the next
    // tile's first K steps are issued now (into slots 0 .. NSTAGE-1; this
    // tile's trailing zero-chunk loads into the same slots were issued earlier
    // by the same lanes and land first); either way they land while this
    // tile's epilogue runs.
    barrier_lds();
    seq = nseq;
    if (ahead) {
      slot0 = (slot0 + nkc) % NSTAGE;
    } else if (more) {
      setup(xcd_swizzle(seq, padded));
      prologue();
      slot0 = 0;
    }
    {
      const OutDst& o = g.p[cpidx].out;
      const int wms = wave_s / V::GN, wns = wave_s % V::GN;   // wave-uniform
      pend = more && o.vec8_ok && (o.flags & ~EPI_RELU) == 0 && cm0 + wms * WTM + WTM <= o.m_valid &&
             cn0 + wns * WTN + WTN <= o.n_valid;
    }
    epilogue<V>(g.p[cpidx], acc, cm0, cn0, wm, wn, lane, stage_out);
    if (!more) break;
  }
  // no LDS-DMA may still be writing when the workgroup exits
  wait_vm<0>();
}

// 256x256 blocks of 8 waves (two per SIMD), one workgroup per CU
__global__ __launch_bounds__(V256W8::NTH, 1) void gemm_bf16_kernel(GemmGroup g, int32_t padded,
                                                                   int32_t grid) {
  gemm_bf16_body<V256W8>(g, padded, grid);
}

// 128x128 blocks, two workgroups per CU
__global__ __launch_bounds__(V128::NTH, 2) void gemm_bf16_t128_kernel(GemmGroup g,
                                                                      int32_t padded,
                                                                      int32_t grid) {
  gemm_bf16_body<V128>(g, padded, grid);
}

// 128x128 blocks of 8 waves (two per SIMD), one workgroup per CU
__global__ __launch_bounds__(V128W8::NTH, 1) void gemm_bf16_t128w8_kernel(GemmGroup g,
                                                                          int32_t padded,
                                                                          int32_t grid) {
  gemm_bf16_body<V128W8>(g, padded, grid);
}

// ------------------------------------------------------------------ fp32 GEMM
constexpr int FT = 64, FK = 16;

__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmGroup g, int32_t padded) {
  const int32_t tile = xcd_swizzle(blockIdx.x, padded);
  if (tile >= g.total_tiles) return;
  int32_t tm, tn;
  const GemmProblem& P = g.p[tile_coords(g, tile, &tm, &tn)];
  const int32_t m0 = tm * FT, n0 = tn * FT;

  __shared__ float sA[FK][FT + 1];
  __shared__ float sB[FK][FT + 1];
  const int tid = threadIdx.x;
  // loader: each thread stages 4 elements of A and 4 of B per k-step
  const int lr = tid >> 2;          // row 0..63
  const int lk = (tid & 3) * 4;     // k 0,4,8,12
  const float* ar = (m0 + lr < P.M) ? reinterpret_cast<const float*>(row_address(P.a, m0 + lr, 4))
                                    : nullptr;
  const float* br = (n0 + lr < P.N) ? reinterpret_cast<const float*>(row_address(P.b, n0 + lr, 4))
                                    : nullptr;
  const int tx = tid & 15, ty = tid >> 4;  // 16x16 threads, 4x4 outputs each
  float acc[4][4] = {};
  for (int k0 = 0; k0 < P.K; k0 += FK) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      int k = k0 + lk + e;
      sA[lk + e][lr] = (ar && k < P.K) ? ar[k] : 0.0f;
      sB[lk + e][lr] = (br && k < P.K) ? br[k] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sA[kk][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = sB[kk][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  const OutDst& o = P.out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int32_t m = m0 + ty + 16 * i;
    if (m >= o.m_valid) continue;
    const int64_t roff = axis_off(o.row, m);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int32_t n = n0 + tx + 16 * j;
      if (n < o.n_valid) epi_store(o, roff + col_off(o, n), acc[i][j]);
    }
  }
}

}  // namespace

// Compute units of the current device (cached per device id).
int32_t device_cu_count() {
  static int32_t cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

int launch_tiles(const GemmGroup& g, bool small, void* stream) {
  const int32_t padded = (g.total_tiles + 7) & ~7;
  const int cus = device_cu_count();
  // persistent workgroups, one (256x256, or 128x128 of 8 waves) or two
  // (128x128 of 4 waves) per compute unit, a multiple of 8 (the XCD count)
  const bool w8 = small && g.total_tiles <= cus;
  int32_t grid = (cus * (small && !w8 ? 2 : 1) + 7) & ~7;
  if (grid > padded) grid = padded;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (w8)
    hipLaunchKernelGGL(gemm_bf16_t128w8_kernel, dim3(grid), dim3(V128W8::NTH), 0, st, g, padded, grid);
  else if (small)
    hipLaunchKernelGGL(gemm_bf16_t128_kernel, dim3(grid), dim3(V128::NTH), 0, st, g, padded, grid);
  else
    hipLaunchKernelGGL(gemm_bf16_kernel, dim3(grid), dim3(V256W8::NTH), 0, st, g, padded, grid);
  return static_cast<int>(hipGetLastError());
}

// An interleaved pair needs matching panel counts (see GemmGroup::pair1).
static bool pair_ok(const GemmGroup& g) {
  const int pr = g.pair1 - 1;
  if (pr < 0) return true;
  if (pr + 1 >= g.count) return false;
  const GemmProblem &x = g.p[pr], &y = g.p[pr + 1];
  return x.tiles_n == y.tiles_m && x.tiles_m == y.tiles_n &&
         y.tile_begin == x.tile_begin + x.tiles_m * x.tiles_n;
}

// The group arrives tiled for 256x256 blocks.  A group with no more such
// tiles than half the compute units is re-tiled for 128x128 blocks: two
// workgroups of 4 waves per CU, or, if the 128x128 tiles do not outnumber the
// compute units, one workgroup of 8 waves per tile.
// The problems of g selected by `pick` (all if null), numbered afresh, in
// tiles of `t` x `t`.
GemmGroup regroup(const GemmGroup& g, const bool* pick, int t) {
  GemmGroup s{};
  int newidx[kMaxGroup];
  for (int i = 0; i < g.count; ++i) {
    newidx[i] = -1;
    if (pick && !pick[i]) continue;
    GemmProblem p = g.p[i];
    set_tiling(p, t);
    p.tile_begin = s.total_tiles;
    s.total_tiles += p.tiles_m * p.tiles_n;
    newidx[i] = s.count;
    s.p[s.count++] = p;
  }
  const int pr = g.pair1 - 1;
  if (pr >= 0 && newidx[pr] >= 0 && newidx[pr + 1] == newidx[pr] + 1) {
    s.pair1 = newidx[pr] + 1;
    if (!pair_ok(s)) s.pair1 = 0;
  }
  return s;
}

int launch_gemm_bf16(const GemmGroup& g, void* stream) {
  if (g.total_tiles <= 0) return 0;
  if (!pair_ok(g)) return static_cast<int>(hipErrorInvalidValue);
  const int cus = device_cu_count();
  // 128x128 tiles when the 256x256 ones fill at most half the chip, or when
  // both tilings take one round (two 128x128 workgroups per CU then share the
  // work that one 256x256 workgroup per CU would do alone)
  int64_t t128 = 0;
  for (int i = 0; i < g.count; ++i)
    t128 += (int64_t)((g.p[i].M + 127) / 128) * ((g.p[i].N + 127) / 128);
  if (2 * g.total_tiles <= cus || (g.total_tiles <= cus && t128 <= 2 * (int64_t)cus))
    return launch_tiles(regroup(g, nullptr, 128), true, stream);
  // A last round of 256x256 tiles less than a quarter full would take as long
  // as a full one: the smallest problem that covers it (else the smallest
  // ones together) moves to a 128x128 launch of its own, and the rest takes
  // one round less (16-layer stack at memory 3800: the 64-tile Rk product of
  // 568 tiles).
  const int32_t excess = g.total_tiles % cus;
  if (g.count > 1 && g.total_tiles > cus && excess > 0 && 4 * excess <= cus) {
    bool pick[kMaxGroup] = {};
    auto tiles = [&](int i) { return g.p[i].tiles_m * g.p[i].tiles_n; };
    int one = -1;
    for (int i = 0; i < g.count; ++i)
      if (tiles(i) >= excess && (one < 0 || tiles(i) < tiles(one))) one = i;
    int32_t moved = 0;
    if (one >= 0) {
      pick[one] = true;
      moved = tiles(one);
    } else {
      while (moved < excess) {
        int k = -1;
        for (int i = 0; i < g.count; ++i)
          if (!pick[i] && (k < 0 || tiles(i) < tiles(k))) k = i;
        pick[k] = true;
        moved += tiles(k);
      }
    }
    if (2 * moved <= cus && moved < g.total_tiles) {
      bool rest[kMaxGroup];
      for (int i = 0; i < g.count; ++i) rest[i] = !pick[i];
      const int e = launch_tiles(regroup(g, rest, 256), false, stream);
      if (e) return e;
      return launch_tiles(regroup(g, pick, 128), true, stream);
    }
  }
  return launch_tiles(g, false, stream);
}

int launch_gemm_f32(const GemmGroup& g, void* stream) {
  if (g.total_tiles <= 0) return 0;
  int32_t padded = (g.total_tiles + 7) & ~7;
  hipLaunchKernelGGL(gemm_f32_kernel, dim3(padded), dim3(256), 0,
                     static_cast<hipStream_t>(stream), g, padded);
  return static_cast<int>(hipGetLastError());
}

}  // namespace txl
