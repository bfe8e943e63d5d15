// Fused relative-position attention core (Dai et al., Transformer-XL, Sec. 3.3
// summary equations; App. B for the shift structure of terms (b) and (d)).
//
// For one (batch b, head h) and queries i, keys j of [memory ; segment]:
//   s_ij = c * ( (q_i+u).k_j + (q_i+v).Rk[M+i-j] ),  visible iff j <= M+i
//   out_i = sum_j softmax_j(s_ij) val_j
// (q+u).k_j carries terms (a) and (c), (q+v).Rk carries (b) and (d).
//
// bf16 kernel (d_head <= 64, padded to 64).  A workgroup owns 128 queries (4
// waves x 32) of one (b, h) and a contiguous range of 32-key blocks.  Scores are
// kept transposed, S^T[j][i], so each lane owns one query column and the
// softmax row statistics stay in-lane (plus the partner lane ii+32).
//   * Block tb's K tile, V^T tile (both 4 KB contiguous in the workspace) and
//     Rk chunk tb (32 rows) stream into LDS by direct global->LDS loads, up
//     to NST-1 blocks ahead; one barrier per block.  Rk chunks stay resident
//     for four blocks (wave w uses chunk tb-w).
//   * Term (b)+(d): per block a wave multiplies its 32 queries (q+v) by a
//     32-row chunk of Rk on the matrix cores: BDw[w][i] = (q_i+v).Rk[D-31+w],
//     D = M + i0 - j0.  The pair (i, j) needs row delta = D + i - j, i.e.
//     position 31 + i - j of the 63-row window [chunk_t ; chunk_{t-1}]; the
//     previous chunk stays in registers, so every chunk is computed once.  A
//     per-wave LDS window, skewed by query, turns App. B's per-row left shift
//     into aligned reads.  No L x (M+L) matrix is ever written.
//   * (q+u).K (terms (a), (c)) runs as a second, independent MFMA chain and the
//     shifted (b)+(d) is added to it.
//   * Online softmax in base 2 (c = scale*log2 e is folded into q+u and q+v),
//     with a lazy rescale: the reference maximum only moves when a block's
//     maximum exceeds it by more than 8, which keeps every p <= 2^8.
//   * P (bf16) times V^T on the matrix cores: bf16 pairs of P are exchanged
//     with the partner lane so that both operands list the keys in order; the
//     same P times a ones operand accumulates the softmax denominators.
//   * With several key-range splits each workgroup writes (max, sum, O) and a
//     combine kernel merges them in split order (deterministic).  (Merging in
//     the last-arriving workgroup would need device-scope fences, i.e. L2
//     write-back and invalidation, which cost far more than a second launch.)
//
// fp32 kernel: one workgroup per (b, h, i), plain loops; used by the fp32 path.
#include "dev_common.h"

namespace txl {

namespace {

constexpr int DP = 64;        // padded head width of the bf16 path
constexpr int KB = 32;        // keys per block
constexpr int NWAVE = 4;      // waves per workgroup, 32 queries each
constexpr int QG = 32 * NWAVE;
#ifndef TXL_ATTN_NST
#define TXL_ATTN_NST 4
#endif
constexpr int NST = TXL_ATTN_NST;  // K / V^T ring stages: blocks tb .. tb+NST-1 resident or in flight
constexpr int RKS = NST + 3;  // Rk chunk slots: chunks tb-3 .. tb in use, NST-1 ahead
constexpr int WP = 36;        // floats per row of a wave's (b)+(d) window
constexpr int KT_U = KB * 8;  // 16-byte units of a K tile (32 keys x 128 bytes)
constexpr int VT_U = DP * 4;  // of a V^T tile (64 rows x 64 bytes)
constexpr int RK_U = KB * 8;  // of an Rk chunk (32 rows x 128 bytes)
constexpr float kNegInf = -__builtin_inff();

struct AttnSmem {
  u32x4 kv[NST][KT_U + VT_U];   // per stage: K tile, then V^T tile
  u32x4 rk[RKS][RK_U];          // Rk chunk ring
  float bd[NWAVE][32 * WP];     // per-wave skewed (b)+(d) window
  float uv[2 * DP];             // u then v of this head, zero padded
};

// 16-byte slot of chunk c (0..7) in row r of a K tile or Rk chunk.  gfx950
// serves 16-byte LDS reads 16 lanes at a time; the fragment reads cover rows
// 0..15 (128-byte pitch, two rows per 64-bank line) at one chunk, and
// c ^ ((r >> 1) & 7) puts those 16 rows on 16 distinct bank groups.
__device__ __forceinline__ int ksw(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }
// V^T tile: row d (64 bytes) holds 4 chunks of 8 keys, chunk c at slot
// c ^ ((d >> 2) & 3); a 16-byte read of one chunk by rows 0..15 then covers all
// 64 banks.
__device__ __forceinline__ int vsw(int d, int c) { return KT_U + d * 4 + (c ^ ((d >> 2) & 3)); }

__device__ __forceinline__ bf16x8 pack8(const float* x) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = static_cast<bf16>(x[e]);
  return r;
}

// Wait until at most 3*n LDS-DMA loads of this wave are in flight (n uniform).
__device__ __forceinline__ void wait_stages(int n) {
  if (n >= 3)
    asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
  else if (n >= 2)
    asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
  else if (n >= 1)
    asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

__device__ __forceinline__ void barrier_lds() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

__global__ __launch_bounds__(256, 2) void attn_bf16_kernel(AttnArgs a, int32_t padded, int32_t nqg) {
  const int32_t total = a.B * a.H * nqg * a.n_split;
  const int32_t wid = xcd_swizzle(blockIdx.x, padded);
  if (wid >= total) return;
  const int32_t split = wid % a.n_split;
  const int32_t rest = wid / a.n_split;
  const int32_t qg = rest % nqg;
  const int32_t bh = rest / nqg;
  const int32_t b = bh / a.H, head = bh - b * a.H;
  const int32_t M = a.M, L = a.L;

  __shared__ AttnSmem sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);

  // Optional fused memory-ring update (segment step): this workgroup copies
  // segment rows wid, wid + total, ... into their ring slots.  The projections
  // that read the old memory ran before this kernel.
  if (a.upd_mem) {
    const int64_t chunks = a.upd_row_bytes / 16;
    const int32_t nrow = a.B * a.upd_rows;
    for (int32_t r = wid; r < nrow; r += total) {
      const int32_t bb = r / a.upd_rows, t = r - bb * a.upd_rows;
      const int32_t src = a.L < a.M ? t : a.L - a.M + t;
      const int32_t slot = a.L < a.M ? (a.upd_start + t) % a.M : t;
      const u32x4* sp = reinterpret_cast<const u32x4*>(
          static_cast<const char*>(a.upd_src) + ((int64_t)bb * a.L + src) * a.upd_row_bytes);
      u32x4* dp = reinterpret_cast<u32x4*>(static_cast<char*>(a.upd_mem) +
                                           ((int64_t)bb * a.M + slot) * a.upd_row_bytes);
      for (int64_t c = tid; c < chunks; c += 256) dp[c] = sp[c];
    }
  }
  const int ii = lane & 31, hf = lane >> 5;

  const int32_t i_base = qg * QG;
  const int32_t i_last = min(i_base + QG, L) - 1;
  const int32_t nb = (M + i_last + 1 + KB - 1) / KB;  // key blocks visible to the group
  const int32_t t_lo = (int32_t)((int64_t)split * nb / a.n_split);
  const int32_t t_hi = (int32_t)((int64_t)(split + 1) * nb / a.n_split);

  const int32_t i0 = i_base + 32 * wave;
  const bool wave_on = i0 < L;
  // blocks past this are fully masked for every query of the wave
  const int32_t t_wave_end = wave_on ? (M + min(i0 + 31, L - 1) + 1 + KB - 1) / KB : 0;

  // ---- u, v of this head (zero padded) and the per-wave query operands
  // (q+u)*c, (q+v)*c as bf16, d = 16s + 8hf + e
  if (tid < 2 * DP) {
    const int d = tid & (DP - 1);
    const uint16_t* src = static_cast<const uint16_t*>(tid < DP ? a.u : a.v) + (int64_t)head * a.dh;
    sm.uv[tid] = d < a.dh ? bf16_to_f32(src[d]) : 0.0f;
  }
  __syncthreads();
  bf16x8 qu[4], qv[4];
  {
    const floatx4* qrow =
        reinterpret_cast<const floatx4*>(a.q + ((int64_t)bh * a.Lp + (wave_on ? i0 + ii : 0)) * DP);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int d0 = 16 * s + 8 * hf;
      const floatx4 q0 = qrow[d0 / 4], q1 = qrow[d0 / 4 + 1];
      float xu[8], xv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float qd = e < 4 ? q0[e] : q1[e - 4];
        xu[e] = (qd + sm.uv[d0 + e]) * a.c_scale;
        xv[e] = (qd + sm.uv[DP + d0 + e]) * a.c_scale;
      }
      qu[s] = pack8(xu);
      qv[s] = pack8(xv);
    }
  }

  // ---- LDS-DMA of one block's operands.  Block tb brings K tile tb, V^T tile
  // tb and Rk chunk tb (rows M + i_base - 32 tb - 31 + r, r = 0..31; the
  // padding of the table covers rows outside [0, Pp)).  Each is 4 KB
  // contiguous, i.e. four wave-instructions of 64 lanes x 16 bytes; the 12
  // instructions of a block are dealt 3 per wave.  A lane fetches the global
  // chunk that lands in the swizzled slot, at a fixed byte offset from a
  // workgroup-uniform base.
  const int32_t nkb = a.Np / KB;
  const char* kbase = static_cast<const char*>(a.k) + (int64_t)bh * a.Np * DP * 2;
  const char* vbase = static_cast<const char*>(a.vt) + ((int64_t)b * nkb * a.H + head) * DP * KB * 2;
  const int64_t vstep = (int64_t)a.H * DP * KB * 2;
  const char* rbase = static_cast<const char*>(a.rk) +
                      ((int64_t)head * (a.Pp + 2 * kRkPad) + kRkPad + M + i_base - (KB - 1)) * DP * 2;
  auto rk_slot = [&](int32_t c) { return ((c % RKS) + RKS) % RKS; };
  auto row_off = [&](int n) {      // instruction n (0..3) of a K tile or Rk chunk
    const int r = n * 8 + (lane >> 3);
    return (uint32_t)(r * 128 + (((lane & 7) ^ ((r >> 1) & 7)) << 4));
  };
  uint32_t loff[3];
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int n = 3 * wave + j;
    if (n < 4 || n >= 8) {
      loff[j] = row_off(n & 3);
    } else {
      const int d = (n - 4) * 16 + (lane >> 2);
      loff[j] = (uint32_t)(d * 64 + (((lane & 3) ^ ((d >> 2) & 3)) << 4));
    }
  }
  auto issue_block = [&](int32_t tb) {
    u32x4* kv = sm.kv[tb % NST];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int n = 3 * wave_s + j;
      if (n < 4)
        __builtin_amdgcn_global_load_lds(kbase + (int64_t)tb * (KB * DP * 2) + loff[j],
                                         kv + n * 64, 16, 0, 0);
      else if (n < 8)
        __builtin_amdgcn_global_load_lds(vbase + tb * vstep + loff[j], kv + KT_U + (n - 4) * 64,
                                         16, 0, 0);
      else
        __builtin_amdgcn_global_load_lds(rbase - (int64_t)tb * (KB * DP * 2) + loff[j],
                                         &sm.rk[rk_slot(tb)][(n - 8) * 64], 16, 0, 0);
    }
  };

  // ---- (b)+(d) through the per-wave window.  At block tb the wave's queries
  // i0 + ii meet keys tb*32 + jj at distance delta = D + ii - jj, D = M + i0 -
  // 32 tb, i.e. at row y = 31 + ii - jj of the 64-row window
  // [Rk chunk tb-wave ; Rk chunk tb-wave-1] (rows D-31 .. D+32).  The window
  // is kept skewed per query: row ii holds W[ii][k] = window row ii + k,
  // k = 0..31, so the 16 values a lane needs (k = 31 - jj) are four aligned
  // float4 reads.  W[ii][(w - ii) & 31] takes chunk tb-wave's row w when
  // w >= ii and chunk tb-wave-1's row w otherwise; both chunks are computed
  // on the matrix cores (BDw[w][i] = (q_i+v).Rk[row w]) and each exactly once
  // (the previous one stays in registers; the loop is unrolled twice so the
  // two register sets trade roles instead of being copied).
  float* win = sm.bd[wave] + ii * WP;
  float* wptr[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) wptr[e] = win + (((8 * (e >> 2) + 4 * hf + (e & 3)) - ii) & 31);
  auto bd_chunk = [&](const u32x4* rs) {
    bf16x8 ar[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) ar[s] = __builtin_bit_cast(bf16x8, rs[ksw(ii, 2 * s + hf)]);
    floatx16 acc = floatx16{0};
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ar[s], qv[s], acc, 0, 0, 0);
    return acc;   // lane: rows w = 8g + 4hf + r (element 4g + r) of column ii
  };

  // ---- prologue: Rk chunks t_lo-4 .. t_lo-1 (one per wave), then blocks
  // t_lo .. t_lo+NST-2
  const int32_t nblk = t_hi - t_lo;
  if (nblk > 0) {
    const int32_t c = t_lo - 4 + wave_s;
#pragma unroll
    for (int n = 0; n < 4; ++n)
      __builtin_amdgcn_global_load_lds(rbase - (int64_t)c * (KB * DP * 2) + row_off(n),
                                       &sm.rk[rk_slot(c)][n * 64], 16, 0, 0);
    for (int32_t t = 0; t < NST - 1 && t < nblk; ++t) issue_block(t_lo + t);
  }
  // the four prologue chunks are the oldest loads of every wave
  wait_stages(min(NST - 1, nblk));
  barrier_lds();
  floatx16 bd_a = floatx16{0}, bd_b = floatx16{0};
  if (wave_on && t_lo < t_wave_end && nblk > 0) bd_b = bd_chunk(sm.rk[rk_slot(t_lo - wave - 1)]);
  // bf16 ones: A operand of the MFMA that sums P over keys
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = static_cast<bf16>(1.0f);
  floatx16 lacc = floatx16{0};   // every row: sum_j p_ij of column ii

  floatx16 o[2] = {floatx16{0}, floatx16{0}};
  float m_ref = kNegInf;

  // one key block: `cur` receives Rk chunk tb-wave, `prev` holds chunk tb-wave-1
  auto block = [&](int32_t tb, floatx16& cur, const floatx16& prev) {
    // block tb has landed once the loads of later blocks are all that remain
    wait_stages(min(NST - 2, t_hi - 1 - tb));
    barrier_lds();   // ... for every wave; block tb-1 is done everywhere
    const bool refill = tb + NST - 1 < t_hi;

    if (wave_on && tb < t_wave_end) {
      const u32x4* kv = sm.kv[tb % NST];
      const u32x4* rs = sm.rk[rk_slot(tb - wave)];
      // operand fragments of this block, read up front in the order the MFMAs
      // use them: K (keys x d) and Rk chunk tb-wave (rows x d), then V^T
      // (d x keys, rows d = 32e + ii, keys 16 t2 + 8 hf .. +7 in order)
      bf16x8 kf[4], rf[4];
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        kf[st] = __builtin_bit_cast(bf16x8, kv[ksw(ii, 2 * st + hf)]);
        rf[st] = __builtin_bit_cast(bf16x8, rs[ksw(ii, 2 * st + hf)]);
      }
      bf16x8 vf[2][2];
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int e = 0; e < 2; ++e) vf[t2][e] = __builtin_bit_cast(bf16x8, kv[vsw(32 * e + ii, 2 * t2 + hf)]);
      // (q+u).K (terms a, c) and BDw = (q+v).Rk (terms b, d): two independent
      // MFMA chains
      floatx16 s = floatx16{0};
      cur = floatx16{0};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[st], qu[st], s, 0, 0, 0);
        cur = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rf[st], qv[st], cur, 0, 0, 0);
      }
      // the refill of block tb-1's ring slot is issued while they run
      if (refill) issue_block(tb + NST - 1);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int w = 8 * (e >> 2) + 4 * hf + (e & 3);
        *wptr[e] = w >= ii ? cur[e] : prev[e];
      }
      wave_lds_fence();
      // add the shifted (b)+(d): key jj = 8g + 4hf + r
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const floatx4 x = *reinterpret_cast<const floatx4*>(win + 28 - 8 * g - 4 * hf);
#pragma unroll
        for (int r = 0; r < 4; ++r) s[4 * g + r] += x[3 - r];
      }
      // causal/memory mask: key j = tb*32 + jj visible iff j <= M + i0 + ii
      const int32_t j0 = tb * KB;
      if (j0 + KB - 1 > M + i0) {
        const int32_t lim = M + i0 + ii - j0;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int jj = 8 * (e >> 2) + 4 * hf + (e & 3);
          if (jj > lim) s[e] = kNegInf;
        }
      }
      float mb = s[0];
#pragma unroll
      for (int e = 1; e < 16; ++e) mb = fmaxf(mb, s[e]);
      {  // with the partner lane (ii, 1-hf): both halves of the column
        const auto mm = __builtin_amdgcn_permlane32_swap(__float_as_uint(mb), __float_as_uint(mb), false, false);
        mb = fmaxf(__uint_as_float(mm[0]), __uint_as_float(mm[1]));
      }
      const bool need = mb > m_ref + 8.0f;
      if (__ballot(need)) {
        const float alpha = need ? __builtin_amdgcn_exp2f(m_ref - mb) : 1.0f;
        if (need) m_ref = mb;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          o[0][e] *= alpha;
          o[1][e] *= alpha;
          lacc[e] *= alpha;
        }
      }
      const float m_use = (m_ref == kNegInf) ? 0.0f : m_ref;
      float p[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) p[e] = __builtin_amdgcn_exp2f(s[e] - m_use);
      // P^T (keys x queries) times V^T.  The lane holds p for keys
      // 16t2 + 4hf + {0..3} and 16t2 + 8 + 4hf + {0..3}; swapping bf16 pairs
      // with the partner lane (ii, 1-hf) gives it keys 16t2 + 8hf .. +7 in
      // order, the k-slots of the V^T fragment.  The same operand times ones
      // accumulates the row sums.
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const u32x4 pw = __builtin_bit_cast(u32x4, pack8(&p[8 * t2]));
        const auto s02 = __builtin_amdgcn_permlane32_swap(pw[0], pw[2], false, false);
        const auto s13 = __builtin_amdgcn_permlane32_swap(pw[1], pw[3], false, false);
        const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{s02[0], s13[0], s02[1], s13[1]});
#pragma unroll
        for (int e = 0; e < 2; ++e) o[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[t2][e], pb, o[e], 0, 0, 0);
        lacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones, pb, lacc, 0, 0, 0);
      }
    } else if (refill) {
      issue_block(tb + NST - 1);
    }
  };
  for (int32_t tb = t_lo; tb < t_hi; tb += 2) {
    block(tb, bd_a, bd_b);
    if (tb + 1 < t_hi) block(tb + 1, bd_b, bd_a);
  }


  const float l_sum = lacc[0];
  const int32_t i = i0 + ii;
  typedef float floatx2_t __attribute__((ext_vector_type(2)));
  typedef bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  // out[b, i, head, :] = num / den; lane holds d = 32e + 8g + 4hf + r (r = 0..3)
  auto write_out = [&](const floatx16 (&num)[2], float den) {
    if (i >= L) return;
    const float inv = 1.0f / den;
    uint16_t* out = static_cast<uint16_t*>(a.out) + (((int64_t)b * L + i) * a.H + head) * a.dh;
    const bool vec = (a.dh == DP);
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * e + 8 * g + 4 * hf;
        if (vec) {
          const bf16x2_t lo = __builtin_convertvector(
              floatx2_t{num[e][4 * g] * inv, num[e][4 * g + 1] * inv}, bf16x2_t);
          const bf16x2_t hi = __builtin_convertvector(
              floatx2_t{num[e][4 * g + 2] * inv, num[e][4 * g + 3] * inv}, bf16x2_t);
          *reinterpret_cast<u32x2*>(out + d0) =
              u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (d0 + r < a.dh) out[d0 + r] = f32_to_bf16_bits(num[e][4 * g + r] * inv);
        }
      }
  };
  if (a.n_split == 1) {
    if (wave_on) write_out(o, l_sum);
    return;
  }

  // key-range splits: (max, sum, O) of this range, merged by attn_combine_kernel
  if (!wave_on) return;
  const int64_t row = (int64_t)split * a.B * a.H * a.Lp + (int64_t)bh * a.Lp + i;
  floatx4* po = reinterpret_cast<floatx4*>(a.part_o + row * DP);
#pragma unroll
  for (int e = 0; e < 2; ++e)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      po[(32 * e + 8 * g + 4 * hf) / 4] =
          floatx4{o[e][4 * g], o[e][4 * g + 1], o[e][4 * g + 2], o[e][4 * g + 3]};
  if (hf == 0) {
    a.part_ml[row * 2 + 0] = m_ref;
    a.part_ml[row * 2 + 1] = l_sum;
  }
}

// Merge split partials in split order: out = sum_s 2^(m_s-m*) O_s / sum_s 2^(m_s-m*) l_s.
// 16 threads per output row, 4 columns each.
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);   // (b, h, i), i < L
  const int c4 = threadIdx.x & 15;
  const int64_t rows = (int64_t)a.B * a.H * a.L;
  if (row >= rows) return;
  const int32_t i = row % a.L;
  const int64_t bh = row / a.L;
  const int32_t b = bh / a.H, head = bh % a.H;
  const int64_t prow = bh * a.Lp + i;
  const int64_t stride = (int64_t)a.B * a.H * a.Lp;
  float mx = kNegInf;
  for (int s = 0; s < a.n_split; ++s) mx = fmaxf(mx, a.part_ml[(s * stride + prow) * 2]);
  floatx4 num = floatx4{0.f, 0.f, 0.f, 0.f};
  float den = 0.0f;
  for (int s = 0; s < a.n_split; ++s) {
    const int64_t pr = s * stride + prow;
    const float ms = a.part_ml[pr * 2];
    const float w = (ms == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(ms - mx);
    num += w * reinterpret_cast<const floatx4*>(a.part_o + pr * DP)[c4];
    den += w * a.part_ml[pr * 2 + 1];
  }
  const float inv = 1.0f / den;
  uint16_t* out = static_cast<uint16_t*>(a.out) + ((int64_t)b * a.L + i) * a.H * a.dh +
                  (int64_t)head * a.dh;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int d = 4 * c4 + r;
    if (d < a.dh) out[d] = f32_to_bf16_bits(num[r] * inv);
  }
}

// ------------------------------------------------------------ fp32 kernel
// One workgroup (256 threads) per (b, h, i).  Scores of all visible keys are
// kept in LDS (dynamic, Np floats).
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnArgs a) {
  extern __shared__ float dyn[];
  const int32_t i = blockIdx.x % a.L;
  const int32_t bh = blockIdx.x / a.L;
  const int32_t b = bh / a.H, head = bh % a.H;
  const int32_t dh = a.dh, M = a.M;
  const int tid = threadIdx.x;
  float* s = dyn;                     // [Np]
  float* qu = dyn + a.Np;             // [dh]
  float* qv = qu + dh;                // [dh]
  __shared__ float red[256];

  const float* q = a.q + ((int64_t)bh * a.Lp + i) * dh;
  const float* uu = static_cast<const float*>(a.u) + (int64_t)head * dh;
  const float* vv = static_cast<const float*>(a.v) + (int64_t)head * dh;
  for (int d = tid; d < dh; d += 256) {
    qu[d] = q[d] + uu[d];
    qv[d] = q[d] + vv[d];
  }
  __syncthreads();
  const float* kb = static_cast<const float*>(a.k) + (int64_t)bh * a.Np * dh;
  const float* vb = static_cast<const float*>(a.vt) + (int64_t)bh * a.Np * dh;
  const float* rb = static_cast<const float*>(a.rk) + (int64_t)head * a.Pp * dh;
  const int32_t nvis = M + i + 1;
  float mx = kNegInf;
  for (int32_t j = tid; j < nvis; j += 256) {
    const float* kr = kb + (int64_t)j * dh;
    const float* rr = rb + (int64_t)(M + i - j) * dh;
    float acc = 0.0f;
    for (int d = 0; d < dh; ++d) acc += qu[d] * kr[d] + qv[d] * rr[d];
    acc *= a.c_scale;
    s[j] = acc;
    mx = fmaxf(mx, acc);
  }
  red[tid] = mx;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) red[tid] = fmaxf(red[tid], red[tid + w]);
    __syncthreads();
  }
  mx = red[0];
  __syncthreads();
  float sum = 0.0f;
  for (int32_t j = tid; j < nvis; j += 256) {
    const float e = expf(s[j] - mx);
    s[j] = e;
    sum += e;
  }
  red[tid] = sum;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  const float inv = 1.0f / red[0];
  float* out = static_cast<float*>(a.out) + (((int64_t)b * a.L + i) * a.H + head) * dh;
  for (int d = tid; d < dh; d += 256) {
    float acc = 0.0f;
    for (int32_t j = 0; j < nvis; ++j) acc += s[j] * vb[(int64_t)j * dh + d];
    out[d] = acc * inv;
  }
}

}  // namespace

int launch_attn_bf16(const AttnArgs& a, void* stream) {
  const int32_t nqg = (a.L + QG - 1) / QG;
  const int32_t total = a.B * a.H * nqg * a.n_split;
  const int32_t padded = (total + 7) & ~7;
  hipLaunchKernelGGL(attn_bf16_kernel, dim3(padded), dim3(256), 0,
                     static_cast<hipStream_t>(stream), a, padded, nqg);
  return static_cast<int>(hipGetLastError());
}

int launch_attn_combine(const AttnArgs& a, void* stream) {
  const int64_t rows = (int64_t)a.B * a.H * a.L;
  hipLaunchKernelGGL(attn_combine_kernel, dim3((rows + 15) / 16), dim3(256), 0,
                     static_cast<hipStream_t>(stream), a);
  return static_cast<int>(hipGetLastError());
}

int launch_attn_f32(const AttnArgs& a, void* stream) {
  const size_t shmem = sizeof(float) * ((size_t)a.Np + 2 * (size_t)a.dh);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(attn_f32_kernel, dim3(a.B * a.H * a.L), dim3(256), shmem, st, a);
  return static_cast<int>(hipGetLastError());
}

}  // namespace txl
