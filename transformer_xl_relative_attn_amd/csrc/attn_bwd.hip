// Backward of the relative-position attention core (Dai et al., Transformer-XL,
// Sec. 3.3 score A^rel with its four terms; Sec. 3.2: the memory enters with a
// stop-gradient, so gradients stop at the cached states, while the keys and
// values computed from them are ordinary tensors of the segment).
//
// With s_ij = scale * A_ij, P = softmax_j(s) over visible keys j <= M + i,
// out = P val, and G = dLoss/dout:
//   dP_ij  = G_i . val_j,  D_i = G_i . out_i,  dS_ij = P_ij (dP_ij - D_i)
//   dq_i   = scale * sum_j dS_ij (k_j + Rk[M+i-j])        terms (a), (b)
//   dk_j   = scale * sum_i dS_ij (q_i + u)                terms (a), (c)
//   dval_j = sum_i P_ij G_i
//   du     = scale * sum_ij dS_ij k_j,  dv = scale * sum_ij dS_ij Rk[M+i-j]
//   dRk[delta] = scale * sum over pairs with M+i-j = delta of dS_ij (q_i + v)
//
// attn_bwd_q_kernel (a workgroup of 4 waves x 32 queries of one (b, h)): the
//   forward's K and V^T tiles and the Rk and Rk^T chunks of every 32-key block
//   are staged in LDS by direct loads two blocks ahead, one barrier per block,
//   and shared by the four waves (K^T and the val rows are the same tiles read
//   through transposing LDS reads).  For every visible block a wave recomputes
//   the scores exactly as the forward kernel does (the (b)+(d) window written
//   shifted to LDS and read back as the accumulator of (q+u).K), P from the
//   forward's log-sum-exp, dP^T = val G^T on the matrix cores, and dS.  It
//   accumulates dq's k-part (K^T times dS^T) and its Rk-part (Rk^T chunks
//   times dS written shifted, row 31 + i - j of the window holds pair (i, j),
//   the App. B shift in reverse), and writes P^T, dS^T and the shifted dS'^T
//   (row delta) as fragment tiles for the key-side products, which need sums
//   over queries.
// bmm64_kernel: batched A B^T with 64 output columns (dk, dval, dRk), the
//   masked entries of A selected away by index.
// bwd_pre_kernel / bwd_post_kernel: the small steps before the query kernel
//   (D, operand layouts, Rk^T, R^T) and after the key-side products (dRk's
//   ordered batch sum and its transpose, du, dv), one launch each.
#include <type_traits>

#include "dev_common.h"

namespace txl {

namespace {

template <int X>
using IC = std::integral_constant<int, X>;

constexpr int DP = 64;
constexpr int KB = 32;
constexpr int WP = 68;     // floats per query row of the score window (64 + pad)
constexpr int NST = 3;     // K / V^T ring stages (blocks t .. t+2)
constexpr int RKS = 8;     // Rk and Rk^T chunk slots: chunk c in slot (c + 8) & 7
constexpr int TU = 256;    // 16-byte units of a 4 KB tile
constexpr int TPW = 36;    // bf16 per query row of the P / dS transpose tiles (32 + pad)

struct BwdSmem {
  u32x4 kv[NST][2 * TU];            // per stage: K tile (32 keys x 128 B), V^T tile (64 d x 64 B)
  u32x4 rk[RKS][TU];                // Rk chunk: 32 rows x 128 B
  u32x4 rkt[RKS][TU];               // Rk^T chunk: 64 d x 32 distances (64 B)
  float win[4][33 * WP];            // per wave: shifted (b)+(d) window of the scores (+ a spill row)
  uint16_t half[4][2][32 * 32];     // per wave: two 32-row halves of dS'^T [row][query]
  uint16_t tp[4][2][32 * TPW];      // per wave: P and dS of a block, [query][key]
};
static_assert(sizeof(BwdSmem) <= 160 * 1024, "one workgroup per CU");

// 16-byte slots: chunk c of a 128-byte row r at r*8 + (c ^ ((r >> 1) & 7)),
// of a 64-byte row d at d*4 + (c ^ ((d >> 2) & 3)); a fragment read (16 rows
// at one chunk per 16 lanes) then covers all 64 banks.
__device__ __forceinline__ int sw128(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }
__device__ __forceinline__ int sw64(int d, int c) { return d * 4 + (c ^ ((d >> 2) & 3)); }

__device__ __forceinline__ int rk_slot(int32_t c) { return (c + 8) & (RKS - 1); }

// 16 bytes per lane from global address p + blk_off into LDS at dst + 16 *
// lane (dst is wave-uniform; it goes to M0).
__device__ __forceinline__ void dma16(const char* p, u32x4* dst, int64_t blk_off) {
  __builtin_amdgcn_global_load_lds(p + blk_off, dst, 16, 0, 0);
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void barrier_lds() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

__device__ __forceinline__ bf16x8 load8(const void* base, int64_t elem) {
  return *reinterpret_cast<const bf16x8*>(static_cast<const uint16_t*>(base) + elem);
}

__device__ __forceinline__ bf16x8 pack8(const float* x) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = static_cast<bf16>(x[e]);
  return r;
}

__device__ __forceinline__ uint16_t bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<bf16>(x));
}

__global__ __launch_bounds__(256, 1) void attn_bwd_q_kernel(BwdArgs a) {
  const int32_t nqg = (a.L + 127) / 128;
  const int32_t wid = blockIdx.x;
  if (wid >= a.B * a.H * nqg) return;   // the whole workgroup
  // Later query groups see more keys (the causal part grows with i): they are
  // dealt first, so that the shorter groups fill the last round of the chip.
  const int32_t nbh = a.B * a.H;
  const int32_t qg = nqg - 1 - wid / nbh;
  const int32_t rest = wid % nbh;
  const int32_t b = rest % a.B, head = rest / a.B;
  const int32_t bh = b * a.H + head;

  __shared__ BwdSmem sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ii = lane & 31, hf = lane >> 5;
  const int32_t M = a.M, L = a.L, Np = a.Np, Lp = a.Lp;
  const int32_t i_base = qg * 128;
  const int32_t i_last = min(i_base + 127, L - 1);
  const int32_t nb = (M + i_last + 1 + KB - 1) / KB;   // key blocks of the workgroup
  const int32_t i0 = i_base + 32 * wave;
  const bool wave_on = i0 < L;   // waves past L only take part in the loads and barriers
  const int32_t i = i0 + ii;
  const bool qok = i < L;
  const int32_t t_end = wave_on ? (M + min(i0 + 31, L - 1) + 1 + KB - 1) / KB : 0;
  const int32_t nkb = Np / KB;

  // ---- LDS-DMA.  Block t brings K tile t (rows 32t.., 128 B each) and the
  // forward's V^T tile t ([64 d][32 keys]) into stage t % NST, and Rk chunk t
  // (rows base0 - 32t + r of the head's table) and the Rk^T chunk of the same
  // distances ([64 d][32 distances]) into slot (t + 8) & 7.  The K^T and val
  // operands come out of the K and V^T tiles through transposing reads.  Wave
  // w uses Rk chunk t-w for block t's scores and Rk^T chunk t-w-2 for its dq;
  // each chunk is loaded once per workgroup.  Every wave loads a quarter of
  // each of the four tiles per block; past the last block the loads repeat it.
  const int32_t base0 = M + i_base - (KB - 1);   // distance of chunk 0's first row
  const int32_t rk_rows = a.Pp + 2 * kRkPad;
  const int32_t ktstep = a.H * DP * KB * 2;
  // first row / column of chunk c, clamped into the tables (chunks outside
  // them are never used)
  auto rk_row0 = [&](int32_t c) { return min(max(kRkPad + base0 - KB * c, 0), rk_rows - KB); };
  auto rkt_col0 = [&](int32_t c) { return min(max(a.rkt_pad + base0 - KB * c, 0), a.rkt_ld - KB); };
  // per-lane sources: 128-byte rows r = 8w + lane/8, 64-byte rows d = 16w +
  // lane/4; a lane fetches the global chunk that lands in its swizzled slot
  const char *pk, *pvt, *prk, *prkt;
  {
    const int r = wave * 8 + (lane >> 3);
    const int64_t lo128 = r * 128 + (((lane & 7) ^ ((r >> 1) & 7)) << 4);
    const int d = wave * 16 + (lane >> 2);
    const int gc = (lane & 3) ^ ((d >> 2) & 3);
    pk = static_cast<const char*>(a.k) + (int64_t)bh * Np * DP * 2 + lo128;
    pvt = static_cast<const char*>(a.vt) + ((int64_t)b * nkb * a.H + head) * DP * KB * 2 + d * 64 +
          gc * 16;
    prk = static_cast<const char*>(a.rk) + (int64_t)head * rk_rows * DP * 2 + lo128;
    prkt = static_cast<const char*>(a.rkt) + ((int64_t)head * DP + d) * a.rkt_ld * 2 + gc * 16;
  }
  auto issue_block = [&](int32_t tb, int st) {
    const int32_t tt = min(tb, nb - 1);
    u32x4* kvs = sm.kv[st] + wave * 64;
    dma16(pk, kvs, (int64_t)tt * (KB * DP * 2));
    dma16(pvt, kvs + TU, (int64_t)tt * ktstep);
    const int sl = rk_slot(tb);
    dma16(prk, sm.rk[sl] + wave * 64, (int64_t)rk_row0(tt) * (DP * 2));
    dma16(prkt, sm.rkt[sl] + wave * 64, (int64_t)rkt_col0(tt) * 2);
  };
  // prologue loads: chunks -4 .. -1, blocks 0 and 1
#pragma unroll
  for (int32_t c = -4; c < 0; ++c) {
    dma16(prk, sm.rk[rk_slot(c)] + wave * 64, (int64_t)rk_row0(c) * (DP * 2));
    dma16(prkt, sm.rkt[rk_slot(c)] + wave * 64, (int64_t)rkt_col0(c) * 2);
  }
  issue_block(0, 0);
  issue_block(1, 1);

  // lanes past L take lse = +inf: their p = 2^(S - inf) = 0
  const float lse = qok ? a.lse[(int64_t)bh * Lp + i] : __builtin_inff();
  const float dsum = qok ? a.dsum[(int64_t)bh * Lp + i] : 0.0f;

  // query operands (q+u)c, (q+v)c, d = 16s + 8hf + e, and G_i for dP^T
  bf16x8 qu[4], qv[4], go[4];
  {
    // q rows L .. Lp-1 are not computed: those lanes take q = 0
    const int32_t ic = qok ? i : 0;
    const float* qrow = a.q + ((int64_t)bh * Lp + ic) * DP;
    const uint16_t* up = static_cast<const uint16_t*>(a.u) + (int64_t)head * a.dh;
    const uint16_t* vp = static_cast<const uint16_t*>(a.v) + (int64_t)head * a.dh;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float xu[8], xv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = 16 * s + 8 * hf + e;
        const float qd = qok ? qrow[d] : 0.0f;
        // clamped in-bounds element, selected after the load, so the loads
        // issue together instead of one branch-and-wait each
        const int dc = min(d, a.dh - 1);
        const float ur = bf16_to_f32(up[dc]), vr = bf16_to_f32(vp[dc]);
        const float uu = d < a.dh ? ur : 0.0f;
        const float vv = d < a.dh ? vr : 0.0f;
        xu[e] = (qd + uu) * a.c_scale;
        xv[e] = (qd + vv) * a.c_scale;
      }
      qu[s] = pack8(xu);
      qv[s] = pack8(xv);
      go[s] = load8(a.dop, ((int64_t)bh * Lp + ic) * DP + 16 * s + 8 * hf);
    }
  }
  wait_vm<0>();
  barrier_lds();

  // fragment offsets: rows ii of a 128-byte-row tile at chunk 2s+hf (dims
  // 16s + 8hf ..), rows d = 32e + ii of a 64-byte-row tile at chunk 2t2+hf
  int ofs128[4], ofs64[2][2];
#pragma unroll
  for (int s = 0; s < 4; ++s) ofs128[s] = sw128(ii, 2 * s + hf);
#pragma unroll
  for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
    for (int e = 0; e < 2; ++e) ofs64[t2][e] = sw64(32 * e + ii, 2 * t2 + hf);
  auto read_rows = [&](const u32x4* base, bf16x8 (&f)[4]) {
#pragma unroll
    for (int s = 0; s < 4; ++s) f[s] = __builtin_bit_cast(bf16x8, base[ofs128[s]]);
  };
  auto bd_chunk = [&](const bf16x8 (&rf)[4]) {
    floatx16 acc = floatx16{0};
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rf[s], qv[s], acc, 0, 0, 0);
    return acc;
  };
  // Score window: the value for (query ii, key jj) is row R = 31 + ii - jj of
  // [lower chunk ; upper chunk].  Each query has a 64-wide row read at
  // positions 32 .. 63 (key jj at 32 + jj); the lane writes its lower chunk
  // row w at 63 + ii - w and its upper chunk row w at 31 + ii - w, every one
  // of them, with no choice: the rows the key range needs (lower w >= ii,
  // upper w < ii) land in 32 .. 63, the others in this row's 0 .. 31 or, past
  // 63, in the next row's 0 .. 31, which no one reads (one spare row per
  // wave).  Row pitch 68: the 16-byte reads of 16 queries hit distinct banks.
  float* win = sm.win[wave] + ii * WP + ii + 31 - 4 * hf - 27;
  auto write_win = [&](const floatx16& lower, const floatx16& upper) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int w = 8 * (e >> 2) + (e & 3);   // chunk row less 4hf
      win[59 - w] = lower[e];
      win[27 - w] = upper[e];
    }
  };
  auto read_win = [&]() {
    floatx16 c;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const floatx4 x = *reinterpret_cast<const floatx4*>(sm.win[wave] + ii * WP + 32 + 8 * g + 4 * hf);
#pragma unroll
      for (int r = 0; r < 4; ++r) c[4 * g + r] = x[r];
    }
    return c;
  };

  uint16_t* halves = sm.half[wave][0];
  // the first block's upper half starts empty
  {
    u32x4* h1 = reinterpret_cast<u32x4*>(sm.half[wave][1]);
    h1[lane] = u32x4{0u, 0u, 0u, 0u};
    h1[lane + 64] = u32x4{0u, 0u, 0u, 0u};
  }
  // A complete half (distances row0 .. +31, row0 = dsp_lo mod 32) goes out as
  // the two fragment tiles of its queries: lane l holds distance row l % 32,
  // queries 16s + 8 (l / 32) .. +7, one contiguous kilobyte per tile.
  const int64_t dsp_kt = (int64_t)a.B * Lp / 16;   // 16-query tiles per tile row
  uint16_t* const dsp_h = static_cast<uint16_t*>(a.dspt) + (int64_t)head * a.dsp_tiles * 32 * a.B * Lp;
  const int64_t dsp_k0 = ((int64_t)b * Lp + i0) / 16;
  auto flush_half = [&](const uint16_t* hsrc, int32_t row0) {
    const int64_t tb = (row0 - a.dsp_lo) / 32;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const u32x4 val = *reinterpret_cast<const u32x4*>(hsrc + (lane & 31) * 32 + 16 * s2 + 8 * (lane >> 5));
      *reinterpret_cast<u32x4*>(dsp_h + ((tb * dsp_kt + dsp_k0 + s2) * 64 + lane) * 8) = val;
    }
  };

  floatx16 dqk[2] = {floatx16{0}, floatx16{0}}, dqr[2] = {floatx16{0}, floatx16{0}};
  // dq, Rk-part, one complete half at a time: dq_i += sum over its 32
  // distances of dS'[delta][i] Rk[delta], the Rk^T chunk of those distances
  // (rows d, k = distance) times the half ([distance][query], row-major).
  // The half feeds the matrix cores through transposing LDS reads: in each
  // group of 16 lanes, lane a + 4q points at row k0 + q, queries 4a .. 4a+3,
  // and lane j receives query j of rows k0 .. k0+3; two reads give the eight
  // distances 16t2 + 8(lane / 32) .. +7 of query lane % 32.
  typedef short short4_t __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) short4_t lds_short4;
  const int tr_base = (8 * (lane >> 5) + ((lane >> 2) & 3)) * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  auto half_frags = [&](const uint16_t* hsrc, bf16x8 (&bq)[2]) {
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      const short4_t r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_short4*)(hsrc + tr_base + (16 * t2) * 32));
      const short4_t r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_short4*)(hsrc + tr_base + (16 * t2 + 4) * 32));
      bq[t2] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  auto chunk_frags = [&](int32_t c, bf16x8 (&af)[2][2]) {   // [t2][e]
    const u32x4* rt = sm.rkt[rk_slot(c)];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int e = 0; e < 2; ++e) af[t2][e] = __builtin_bit_cast(bf16x8, rt[ofs64[t2][e]]);
  };
  // val and K^T operands through the same transposing reads (lane a + 4q of
  // each 16-lane group: q = (lane >> 2) & 3, a = lane & 3):
  //   val fragment s (A of dP^T: row = key lane % 32, d = 16s + 8 (lane / 32)
  //   .. +7) from the V^T tile [64 d][32 keys], 64-byte rows with chunk c of
  //   row d at c ^ ((d >> 2) & 3): lane points at d row 16s + 8 (lane / 32) +
  //   4rd + q, keys 16 ((lane / 16) % 2) + 4a .. +3;
  //   K^T fragment (t2, e) (A of dq's k-part: row = d 32e + lane % 32, keys
  //   16t2 + 8 (lane / 32) .. +7) from the K tile [32 keys][64 d], 128-byte
  //   rows with chunk c of row r at c ^ ((r >> 1) & 7): lane points at key
  //   row 16t2 + 8 (lane / 32) + 4rd + q, d 32e + 16 ((lane / 16) % 2) + 4a .. +3.
  // The swizzle terms do not depend on s or t2, so each lane keeps one byte
  // offset per (rd) and (e, rd); s and t2 add 1 KB and 2 KB.
  int vt_off[2], kt_off[2][2];
  {
    const int q4 = (lane >> 2) & 3, a4 = lane & 3, g2 = (lane >> 4) & 1, kh = lane >> 5;
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
      const int dr = 8 * kh + 4 * rd + q4;
      vt_off[rd] = dr * 64 + (((2 * g2 + (a4 >> 1)) ^ ((2 * kh + rd) & 3)) << 4) + 8 * (a4 & 1);
#pragma unroll
      for (int e = 0; e < 2; ++e)
        kt_off[e][rd] = dr * 128 + (((4 * e + 2 * g2 + (a4 >> 1)) ^ ((4 * kh + 2 * rd + (q4 >> 1)) & 7)) << 4) +
                        8 * (a4 & 1);
    }
  }
  auto tr8 = [&](const char* p0, const char* p1) {
    const short4_t r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)p0);
    const short4_t r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)p1);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto val_frags = [&](const u32x4* vtile, bf16x8 (&f)[4]) {
    const char* base = reinterpret_cast<const char*>(vtile);
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) f[s4] = tr8(base + vt_off[0] + 1024 * s4, base + vt_off[1] + 1024 * s4);
  };
  auto kt_frags = [&](const u32x4* ktile, bf16x8 (&f)[2][2]) {   // [t2][e]
    const char* base = reinterpret_cast<const char*>(ktile);
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int e = 0; e < 2; ++e) f[t2][e] = tr8(base + kt_off[e][0] + 2048 * t2, base + kt_off[e][1] + 2048 * t2);
  };
  auto half_dqr = [&](const bf16x8 (&af)[2][2], const bf16x8 (&bq)[2]) {
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int e = 0; e < 2; ++e) dqr[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[t2][e], bq[t2], dqr[e], 0, 0, 0);
  };
  // P^T, dS^T in fragment tiles: tile (jb, kb) holds keys 32jb .. +31 and
  // queries 16kb .. +15 as 64 lanes x 16 bytes, lane key % 32 + 32 ((query %
  // 16) / 8) with queries 8 apart in order, i.e. the matrix-core operand of
  // the key-side products, read there as one contiguous kilobyte.  A block's
  // two tiles are assembled by a [query][key] transpose tile in LDS (lane
  // (ii, hf) writes four keys at a time) read back with transposing reads.
  char* const pt_bh = static_cast<char*>(a.pt) + (int64_t)bh * Np * Lp * 2;
  char* const dst_bh = static_cast<char*>(a.dst) + (int64_t)bh * Np * Lp * 2;
  uint16_t* const tpp = sm.tp[wave][0];
  uint16_t* const tpd = sm.tp[wave][1];
  const int tp_w = ii * TPW + 4 * hf;   // + 8g: keys 8g + 4hf .. +3 of query ii
  const int tp_r = (8 * (lane >> 5) + ((lane >> 2) & 3)) * TPW + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  auto tile_frags = [&](const uint16_t* src, bf16x8 (&fq)[2]) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const short4_t r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(src + tp_r + (16 * s2) * TPW));
      const short4_t r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(src + tp_r + (16 * s2 + 4) * TPW));
      fq[s2] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };

  // Chunk products of the score window: block t uses [chunk t-w ; chunk
  // t-w-1] (distances base_t .. +31, base_t + 32 .. +63, base_t = M + i0 -
  // 32t - 31).  Two registers sets alternate: block t reads chunk t-w from
  // one and writes chunk t+1-w into the other.
  floatx16 C0 = floatx16{0}, C1 = floatx16{0};
  // scores and dP^T of the current and the next block (alternating sets)
  floatx16 SA = floatx16{0}, DA = floatx16{0}, SB = floatx16{0}, DB = floatx16{0};
  if (wave_on) {
    bf16x8 rf[4], vf[4], kf[4];
    read_rows(sm.rk[rk_slot(-wave - 1)], rf);
    C0 = bd_chunk(rf);
    read_rows(sm.rk[rk_slot(-wave)], rf);
    val_frags(sm.kv[0] + TU, vf);
    read_rows(sm.kv[0], kf);
    C1 = bd_chunk(rf);
#pragma unroll
    for (int s = 0; s < 4; ++s) DA = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[s], go[s], DA, 0, 0, 0);
    write_win(C1, C0);
    wave_lds_fence();
    SA = read_win();
#pragma unroll
    for (int s = 0; s < 4; ++s) SA = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qu[s], SA, 0, 0, 0);
  }

  // Block t, with its scores and dP^T in Sc, dpc and chunk t-w in up_in.
  // Order: the LDS reads of every operand this block needs (its dq products,
  // the next block's scores), the next block's chunk and dP^T products, P
  // and dS on the vector ALUs while those run, dq's k-part; then the LDS
  // writes (the next block's score window, the shifted dS) and the P^T /
  // dS^T stores, one fence, and the products that read what was written.
  // The previous block's completed dS'^T half is written out before this
  // block's shifted dS overwrites it.
  bool pend = false;   // halves[(t) & 1] holds rows pend_row .. +31, complete
  int32_t pend_row = 0;
  auto block = [&](auto PAR, int32_t t, const floatx16& Sc, const floatx16& dpc, floatx16& Sn,
                   floatx16& dpn, const floatx16& up_in, floatx16& low_out) {
    constexpr int par = decltype(PAR)::value;   // t & 1
    const int32_t j0 = t * KB;
    const int32_t base = M + i0 - 32 * t - 31;
    const bool more = t + 1 < t_end;
    // operands: K^T tile t and the Rk^T chunk t-w-2 of the half completed by
    // block t-1 for dq; Rk chunk t+1-w, val and K tiles t+1 for the next
    // block (read whether or not it exists: every slot holds valid data)
    // (the Rk chunk first and its product issued at once: with the other
    // reads ahead of it the compiler fetched it one fragment at a time)
    bf16x8 ktf[2][2], rtf[2][2], rf[4], vf[4], kf[4];
    const u32x4* kvn = sm.kv[(t + 1) % NST];
    read_rows(sm.rk[rk_slot(t + 1 - wave)], rf);
    __builtin_amdgcn_sched_barrier(0);
    if (more) low_out = bd_chunk(rf);
    __builtin_amdgcn_sched_barrier(0);
    val_frags(kvn + TU, vf);
    kt_frags(sm.kv[t % NST], ktf);
    chunk_frags(t - wave - 2, rtf);
    read_rows(kvn, kf);
    if (more) {
      dpn = floatx16{0};
#pragma unroll
      for (int s = 0; s < 4; ++s) dpn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[s], go[s], dpn, 0, 0, 0);
    }
    // P and dS; key jj = 8g + 4hf + r (element 4g + r) visible iff j0 + jj <= M + i
    // (only blocks that reach past the wave's first query need the mask)
    float p[16], ds[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) p[e] = __builtin_amdgcn_exp2f(Sc[e] - lse);
    if (j0 + KB - 1 > M + i0) {
      const int32_t lim = M + i - j0 - 4 * hf;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int kk = 8 * (e >> 2) + (e & 3);
        if (kk > lim) p[e] = 0.0f;
      }
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) ds[e] = p[e] * (dpc[e] - dsum);
    // bf16 pairs: keys (8g + 4hf + r, r+1) for e = 4g + r, r even
    typedef float floatx2_t __attribute__((ext_vector_type(2)));
    typedef bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    uint32_t pw[8], dw2[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      pw[m] = __builtin_bit_cast(uint32_t, __builtin_convertvector(floatx2_t{p[2 * m], p[2 * m + 1]}, bf16x2_t));
      dw2[m] = __builtin_bit_cast(uint32_t, __builtin_convertvector(floatx2_t{ds[2 * m], ds[2 * m + 1]}, bf16x2_t));
    }
    // dq, k-part: K^T tile times dS^T (bf16 pairs exchanged with the partner
    // lane so that the operand lists keys 16t2 + 8hf .. +7 in order)
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      const auto s02 = __builtin_amdgcn_permlane32_swap(dw2[4 * t2 + 0], dw2[4 * t2 + 2], false, false);
      const auto s13 = __builtin_amdgcn_permlane32_swap(dw2[4 * t2 + 1], dw2[4 * t2 + 3], false, false);
      const bf16x8 dsb = __builtin_bit_cast(bf16x8, u32x4{s02[0], s13[0], s02[1], s13[1]});
#pragma unroll
      for (int e = 0; e < 2; ++e)
        dqk[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ktf[t2][e], dsb, dqk[e], 0, 0, 0);
    }
    if (more) write_win(low_out, up_in);
    // the half completed by block t-1 (distances base + 64 .. +95): dq's
    // Rk-part and the write-out, before this block's lower half reuses it
    if (pend) {
      bf16x8 bq[2];
      half_frags(halves + par * (32 * 32), bq);
      flush_half(halves + par * (32 * 32), pend_row);
      half_dqr(rtf, bq);
    }
    // dS shifted by distance: window position r = 31 + ii - jj, rows base + r.
    // The two halves form a ring of 64 rows: block t's lower half (r < 32)
    // is half t & 1 and its upper half the other, i.e. ring row r for even
    // t and r ^ 32 for odd t.  Block t writes entries r >= ii of its lower
    // half and r < ii of its upper half (block t-1's lower half), so the two
    // halves it touches are whole once it is done; only the last block's
    // lower half keeps stale entries (r < ii), cleared after the loop.
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int jj = 8 * (e >> 2) + 4 * hf + (e & 3);
      const int r = 31 + ii - jj;
      const uint16_t x = (uint16_t)(dw2[e >> 1] >> (16 * (e & 1)));
      halves[(par ? r ^ 32 : r) * 32 + ii] = x;
    }
    // P and dS of block t into the transpose tiles (keys 8g + 4hf .. +3 of
    // query ii: the bf16 pairs 2g, 2g+1)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      *reinterpret_cast<uint2*>(tpp + tp_w + 8 * g) = uint2{pw[2 * g], pw[2 * g + 1]};
      *reinterpret_cast<uint2*>(tpd + tp_w + 8 * g) = uint2{dw2[2 * g], dw2[2 * g + 1]};
    }
    wave_lds_fence();
    if (more) {
      Sn = read_win();
#pragma unroll
      for (int s = 0; s < 4; ++s) Sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qu[s], Sn, 0, 0, 0);
    }
    // P^T and dS^T tiles (t, i0/16 + s2): one contiguous kilobyte each
    {
      bf16x8 fp[2], fd[2];
      tile_frags(tpp, fp);
      tile_frags(tpd, fd);
      const int64_t tile0 = (int64_t)t * (Lp / 16) + i0 / 16;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int64_t off = ((tile0 + s2) * 64 + lane) * 16;
        *reinterpret_cast<bf16x8*>(pt_bh + off) = fp[s2];
        *reinterpret_cast<bf16x8*>(dst_bh + off) = fd[s2];
      }
    }
    // rows base + 32 .. +63 are complete (keys of blocks t-1 and t): written
    // out at the start of the next block
    pend = true;
    pend_row = base + 32;
  };

  // one loop step: DMA block t+1 (issued one block ago) and this wave's
  // stores of the previous block have landed; the stage of block t-1 takes
  // DMA block t+2
  auto step = [&](auto PAR, int32_t t, const floatx16& Sc, const floatx16& dpc, floatx16& Sn,
                  floatx16& dpn, const floatx16& up_in, floatx16& low_out) {
    if (t > 0) {
      wait_vm<0>();
      barrier_lds();
    }
    issue_block(t + 2, (t + 2) % NST);
    if (t < t_end) block(PAR, t, Sc, dpc, Sn, dpn, up_in, low_out);
  };
  // unrolled twice so that the two register sets trade roles without copies
  // and the ring parity of the dS halves is a constant
  for (int32_t t = 0; t < nb; t += 2) {
    step(IC<0>{}, t, SA, DA, SB, DB, C1, C0);
    if (t + 1 < nb) step(IC<1>{}, t + 1, SB, DB, SA, DA, C0, C1);
  }
  wait_vm<0>();   // the repeated loads past the last block
  if (wave_on) {
    bf16x8 af[2][2], bq[2];
    if (pend) {   // block t_end-1's upper half: distances base + 32 .. +63 of that block
      const uint16_t* hp = halves + (t_end & 1) * (32 * 32);
      chunk_frags(t_end - wave - 2, af);
      half_frags(hp, bq);
      flush_half(hp, pend_row);
      half_dqr(af, bq);
    }
    // entries r < ii of the last lower half belong to keys past the last
    // block (not visible): zero
    uint16_t* lo = halves + ((t_end - 1) & 1) * (32 * 32);
    for (int r = 0; r < ii; ++r) lo[r * 32 + ii] = 0;
    wave_lds_fence();
    chunk_frags(t_end - 1 - wave, af);
    half_frags(lo, bq);
    flush_half(lo, M + i0 - 32 * (t_end - 1) - 31);
    half_dqr(af, bq);
  }
  if (!wave_on) return;

  // dq = scale (k-part + Rk-part); lane holds d = 32e + 8g + 4hf + r of query i
  if (qok) {
    float* dqrow = a.dq + (((int64_t)b * L + i) * a.H + head) * a.dh;
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int d = 32 * e + 8 * g + 4 * hf + r;
          if (d < a.dh) dqrow[d] = a.scale * (dqk[e][4 * g + r] + dqr[e][4 * g + r]);
        }
  }
  // per-32-query sums of both parts (-> du, dv); padded queries hold zeros
  const int32_t nch = Lp / 32;
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    float* dst = a.duv_part + ((((int64_t)which * a.B + b) * a.H + head) * nch + i0 / 32) * DP;
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        float val = which == 0 ? dqk[e][x] : dqr[e][x];
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) val += __shfl_xor(val, o);
        if (ii == 0) dst[32 * e + 8 * (x >> 2) + 4 * hf + (x & 3)] = a.scale * val;
      }
  }
}

// ------------------------------------------------------------------ bmm64
// One wave per 64 rows of A (two 32-row tiles) and both 32-column halves of
// the output: four matrix-core products per 16-wide k-step.  A fragments come
// straight from global memory (rows are K-contiguous; each lane streams its
// row), loaded a group of G k-steps ahead.  B (64 rows, shared by the whole
// workgroup) is staged in LDS once per 512-wide K chunk by direct
// global->LDS loads and read from there: fetched per wave from global memory
// it cost as much as A.  A(m, k) counts iff m - moff <= k < min(K, klim): a
// step whose 32 x 16 fragment lies inside that band (decided per wave, so on
// the scalar unit) runs unmasked; only the band's edge pays for masking.
constexpr int BMM_RM = 2;                   // 32-row tiles per wave
constexpr int BMM_ROWS = 4 * 32 * BMM_RM;   // rows per workgroup
constexpr int BMM_KC = 512;                 // K chunk staged in LDS

// zero the elements e of a row fragment outside [lo, hi), all if !ok
__device__ __forceinline__ bf16x8 band_mask(bf16x8 f, int32_t lo, int32_t hi, bool ok) {
  const int32_t l = min(max(lo, 0), 8), h = min(max(hi, 0), 8);
  const uint32_t bits = ok && h > l ? ((1u << h) - 1u) & ~((1u << l) - 1u) : 0u;
  u32x4 w = __builtin_bit_cast(u32x4, f);
#pragma unroll
  for (int p = 0; p < 4; ++p)
    w[p] &= ((bits >> (2 * p)) & 1u ? 0x0000ffffu : 0u) | ((bits >> (2 * p + 1)) & 1u ? 0xffff0000u : 0u);
  return __builtin_bit_cast(bf16x8, w);
}

// Up to three products in one launch (blockIdx.z): their workgroups share the
// chip instead of each product's last partial round running alone.
struct BmmBatch {
  BmmArgs p[3];
  int32_t kind[3];      // layout of A (see launch_bmm64)
  int32_t row_off[3];   // output row of A row m: m + row_off
  int32_t kper[3];      // kind 2: K spans K / kper batch rows of kper queries each
                        // (klim applies within each), 0 = one
};

__global__ __launch_bounds__(256, 2) void bmm64_kernel(BmmBatch bt) {
  const int z = blockIdx.z;
  const BmmArgs a = z == 0 ? bt.p[0] : z == 1 ? bt.p[1] : bt.p[2];
  if ((int32_t)blockIdx.x * BMM_ROWS >= a.M || (int32_t)blockIdx.y >= a.batch) return;
  // B chunk: row n (1 KB) holds 16-byte chunk c at slot c ^ (n & 15), so the
  // 16 rows a fragment read serves at once sit on distinct bank groups
  __shared__ u32x4 bsm[64 * (BMM_KC / 8)];
  const int32_t bi = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ii = lane & 31, hf = lane >> 5;
  const int32_t mwg = blockIdx.x * BMM_ROWS;
  const int32_t m0 = mwg + 32 * BMM_RM * wave;
  const bool wave_on = m0 < a.M;   // idle waves still take part in the staging
  const uint16_t* A = static_cast<const uint16_t*>(a.A) + axis_offset(a.a_batch, bi);
  const uint16_t* Bm = static_cast<const uint16_t*>(a.Bm) + axis_offset(a.b_batch, bi);
  // rows past M read row m0 (valid memory, masked); B rows past n_valid read
  // row 0: a B row only reaches its own, unstored, output column
  const uint16_t* arow[BMM_RM];
  bool mok[BMM_RM];
  int32_t lo_row[BMM_RM];   // first k of the lane's row in each tile
#pragma unroll
  for (int r = 0; r < BMM_RM; ++r) {
    const int32_t m = m0 + 32 * r + ii;
    mok[r] = m < a.M;
    arow[r] = A + (int64_t)(mok[r] ? m : (wave_on ? m0 : 0)) * a.lda;
    lo_row[r] = m - a.moff;
  }
  floatx16 acc[BMM_RM][2];
#pragma unroll
  for (int r = 0; r < BMM_RM; ++r) acc[r][0] = acc[r][1] = floatx16{0};
  // Fragment tiles (kind 1, 2): the lane's 16 bytes of k-step 0 in each of
  // its row tiles (clamped into the rows that hold data; rows past M are not
  // stored).  Tiles no wave of the query kernel wrote hold no data and are
  // skipped; a tile (row tile, k-step) belongs to the wave of queries 32w ..
  // +31, w = k-step / 2.  Key-row tiles (kind 1, P^T and dS^T): written iff
  // that wave visited the key block, i.e. row tile < t_end(w).
  //   Distance-row tiles (kind 2, dS'^T): that wave flushed the halves of
  // distances M + 32w + 1 - 32u, u = 0 .. t_end(w), i.e. tile rows
  // top(w) - t_end(w) .. top(w) counted from row_off.
  const int kind = z == 0 ? bt.kind[0] : z == 1 ? bt.kind[1] : bt.kind[2];
  const int32_t row_off = z == 0 ? bt.row_off[0] : z == 1 ? bt.row_off[1] : bt.row_off[2];
  const int32_t kper = z == 0 ? bt.kper[0] : z == 1 ? bt.kper[1] : bt.kper[2];
  const bool frag = kind != 0;
  if (frag) {   // lda: the tile row's length in elements (16 per tile)
#pragma unroll
    for (int r = 0; r < BMM_RM; ++r) {
      const int32_t jb = min(m0 / 32 + r, (a.M + 31) / 32 - 1);
      arow[r] = A + ((int64_t)jb * (a.lda / 16) * 64 + lane) * 8;
    }
  }
  auto tile_written = [&](int r, int32_t kk) {
    // query of the step within its batch row (kind 2 may span several)
    const int32_t kq = kper > 0 ? kk % kper : kk;
    if (kq >= a.klim) return false;
    const int32_t w = kq >> 5;   // query tile of 32
    const int32_t t_end = (a.moff + min(32 * w + 31, a.klim - 1) + 32) / 32;
    const int32_t tr = m0 / 32 + r;
    if (kind == 1) return tr < t_end;
    const int32_t top = (a.moff + 32 * w + 1 - row_off) / 32;
    return tr <= top && tr >= top - t_end;
  };
  // rows need k >= m - moff and none at or past kend
  const int32_t kend = kper > 0 ? a.K : min(a.K, a.klim);
  const int32_t kfirst_wg = kind == 2 ? 0 : max(0, mwg - a.moff) & ~(BMM_KC - 1);
  const int32_t kfirst = kind == 2 ? 0 : max(0, m0 - a.moff) & ~15;
  int bofs[2];   // this lane's B row base (16-byte units) and swizzle
#pragma unroll
  for (int e = 0; e < 2; ++e) bofs[e] = (32 * e + ii) * (BMM_KC / 8);
  const int bsw = ii & 15;
  constexpr int G = 4;
  struct Frag {
    bf16x8 a[BMM_RM];
    int32_t kk;   // first k of the step (wave-uniform)
  };
  // the K loop, instantiated once per layout of A (registers are allocated
  // per instantiation)
  auto run = [&](auto FR) {
  constexpr bool fr = decltype(FR)::value;
  for (int32_t kc = kfirst_wg; kc < kend; kc += BMM_KC) {
    const int32_t kc_end = min(kend, kc + BMM_KC);
    // stage B[:, kc .. kc + 512): wave w fills rows 16w .. 16w+15, one 1 KB
    // row per instruction (columns past K are never read as data)
    __syncthreads();   // every wave is done with the previous chunk
#pragma unroll 4
    for (int t = 0; t < 16; ++t) {
      const int n = 16 * wave + t;
      const int nr = n < a.n_valid ? n : 0;
      const int c = lane ^ (n & 15);   // chunk that lands in slot `lane`
      const int32_t k = min(kc + 8 * c, a.K - 8);
      __builtin_amdgcn_global_load_lds(Bm + (int64_t)nr * a.ldb + k, bsm + n * (BMM_KC / 8), 16, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): this wave's rows have landed
    __syncthreads();
    const int32_t k_lo = max(kfirst, kc);
    const int32_t nsteps = wave_on && kc_end > k_lo ? (kc_end - k_lo + 15) / 16 : 0;
    auto load = [&](int32_t st, Frag& f) {
      f.kk = k_lo + 16 * st;
      const int32_t k = f.kk + 8 * hf;
      const int32_t off = fr ? (f.kk >> 4) * 512 : k;
#pragma unroll
      for (int r = 0; r < BMM_RM; ++r) f.a[r] = *reinterpret_cast<const bf16x8*>(arow[r] + off);
    };
    auto use = [&](Frag& f) {
      const int c = (f.kk - kc) / 8 + hf;
      bf16x8 b[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) b[e] = __builtin_bit_cast(bf16x8, bsm[bofs[e] + (c ^ bsw)]);
#pragma unroll
      for (int r = 0; r < BMM_RM; ++r) {
        if (fr) {
          if (!tile_written(r, f.kk)) continue;
        } else {
          const int32_t mlast = m0 + 32 * r + 31;
          const bool inside = mlast < a.M && mlast - a.moff <= f.kk && f.kk + 16 <= kend;
          if (!inside) {
            const int32_t k8 = f.kk + 8 * hf;
            f.a[r] = band_mask(f.a[r], lo_row[r] - k8, kend - k8, mok[r]);
          }
        }
#pragma unroll
        for (int e = 0; e < 2; ++e)
          acc[r][e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[r], b[e], acc[r][e], 0, 0, 0);
      }
    };
    Frag fa[G], fb[G];
    // Loads are unconditional (steps past the end re-read the last one) so
    // that the waits before each group count only the loads issued after it.
    auto load_group = [&](int32_t g0, Frag (&f)[G]) {
#pragma unroll
      for (int x = 0; x < G; ++x) load(min(g0 + x, nsteps - 1), f[x]);
    };
    auto use_group = [&](int32_t g0, Frag (&f)[G]) {
#pragma unroll
      for (int x = 0; x < G; ++x)
        if (g0 + x < nsteps) use(f[x]);
    };
    if (nsteps > 0) load_group(0, fa);
    for (int32_t g0 = 0; g0 < nsteps; g0 += 2 * G) {
      load_group(g0 + G, fb);
      use_group(g0, fa);
      load_group(g0 + 2 * G, fa);
      use_group(g0 + G, fb);
    }
  }
  };
  if (frag)
    run(IC<1>{});
  else
    run(IC<0>{});
  if (!wave_on) return;
  // lane holds column n = 32e + ii, rows m0 + 32r + 8g + 4hf + q (element 4g + q)
  float* C = a.C + axis_offset(a.c_batch, bi);
  float* C2 = a.C2 ? a.C2 + axis_offset(a.c2_batch, bi) : nullptr;
#pragma unroll
  for (int r = 0; r < BMM_RM; ++r)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int n = 32 * e + ii;
      if (n >= a.n_valid) continue;
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const int32_t row = m0 + 32 * r + 8 * (x >> 2) + 4 * hf + (x & 3) + row_off;
        if (row < 0 || row >= a.m_valid) continue;
        const float val = a.alpha * acc[r][e][x];
        C[(int64_t)row * a.ldc + n] = val;
        if (C2) C2[(int64_t)row * a.c2_m + (int64_t)n * a.c2_n] = val;
      }
    }
}

// ------------------------------------------------------------------ helpers
// One workgroup per (b, h) and 64 queries: D_i = G_i . out_i, G repacked
// [bh][i][64] and, through an LDS tile, transposed [bh][64][i]; (q+u)^T
// [bh][64][i] and (q+v)^T [h][64][b*Lp + i].  Rows i >= L and columns d >= dh
// are zeros.
__device__ __forceinline__ void bwd_prep_block(const BwdPrepArgs& a, int32_t blk) {
  __shared__ __align__(16) uint16_t tg[64][72];   // [i][d], 144-byte rows
  __shared__ __align__(16) uint16_t tu[64][72];
  __shared__ __align__(16) uint16_t tv[64][72];
  __shared__ float red[64][4];
  const int32_t nch = a.Lp / 64 + (a.Lp % 64 ? 1 : 0);
  const int32_t bh = blk / nch, i_base = (blk % nch) * 64;
  const int32_t b = bh / a.H, head = bh % a.H;
  const int tid = threadIdx.x;
  {
    // thread -> row r = tid / 4, columns 16 * (tid % 4) .. +15
    const int r = tid >> 2, c0 = 16 * (tid & 3);
    const int32_t i = i_base + r;
    const bool ok = i < a.L;
    const int64_t src = (((int64_t)b * a.L + (ok ? i : 0)) * a.H + head) * a.dh;
    const uint16_t* g = static_cast<const uint16_t*>(a.dout) + src;
    const uint16_t* o = static_cast<const uint16_t*>(a.out) + src;
    const float* q = a.q + ((int64_t)bh * a.Lp + (i < a.Lp ? i : 0)) * DP;
    const uint16_t* up = static_cast<const uint16_t*>(a.u) + (int64_t)head * a.dh;
    const uint16_t* vp = static_cast<const uint16_t*>(a.v) + (int64_t)head * a.dh;
    float dsum = 0.0f;
    if (ok && a.dh == DP) {
      // whole rows: 16-byte loads
      uint16_t gv[16], ov[16], uv[16], vv[16];
      float qv[16];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const u32x4 gx = *reinterpret_cast<const u32x4*>(g + c0 + 8 * h2);
        const u32x4 ox = *reinterpret_cast<const u32x4*>(o + c0 + 8 * h2);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          gv[8 * h2 + 2 * w] = gx[w] & 0xffff;
          gv[8 * h2 + 2 * w + 1] = gx[w] >> 16;
          ov[8 * h2 + 2 * w] = ox[w] & 0xffff;
          ov[8 * h2 + 2 * w + 1] = ox[w] >> 16;
        }
      }
      // u, v carry no alignment guarantee: element loads (cached, tiny)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        uv[e] = up[c0 + e];
        vv[e] = vp[c0 + e];
      }
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const floatx4 x = *reinterpret_cast<const floatx4*>(q + c0 + 4 * f);
#pragma unroll
        for (int w = 0; w < 4; ++w) qv[4 * f + w] = x[w];
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int d = c0 + e;
        const float gd = bf16_to_f32(gv[e]);
        dsum += gd * bf16_to_f32(ov[e]);
        tg[r][d] = gv[e];
        tu[r][d] = bf16_bits(qv[e] + bf16_to_f32(uv[e]));
        tv[r][d] = bf16_bits(qv[e] + bf16_to_f32(vv[e]));
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int d = c0 + e;
        const bool dok = ok && d < a.dh;
        const float gd = dok ? bf16_to_f32(g[d]) : 0.0f;
        const float od = dok ? bf16_to_f32(o[d]) : 0.0f;
        dsum += gd * od;
        tg[r][d] = bf16_bits(gd);
        const float qd = dok ? q[d] : 0.0f;
        tu[r][d] = dok ? bf16_bits(qd + bf16_to_f32(up[d])) : uint16_t(0);
        tv[r][d] = dok ? bf16_bits(qd + bf16_to_f32(vp[d])) : uint16_t(0);
      }
    }
    red[r][tid & 3] = dsum;
    if (i < a.Lp) {
      uint16_t* dop = static_cast<uint16_t*>(a.dop) + ((int64_t)bh * a.Lp + i) * DP + c0;
      *reinterpret_cast<u32x4*>(dop) = *reinterpret_cast<const u32x4*>(&tg[r][c0]);
      *reinterpret_cast<u32x4*>(dop + 8) = *reinterpret_cast<const u32x4*>(&tg[r][c0 + 8]);
    }
  }
  __syncthreads();
  if (tid < 64 && i_base + tid < a.Lp)
    a.dsum[(int64_t)bh * a.Lp + i_base + tid] =
        (red[tid][0] + red[tid][1]) + (red[tid][2] + red[tid][3]);
  // transposed: thread -> column d = tid / 4, queries 16 * (tid % 4) .. +15
  {
    const int d = tid >> 2, r0 = 16 * (tid & 3);
    const int32_t i = i_base + r0;
    if (i < a.Lp) {
      u32x4 xg[2], xu[2], xv[2];   // 16 bf16 each, packed in pairs
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        xg[e >> 3][(e & 7) >> 1] = (uint32_t)tg[r0 + e][d] | ((uint32_t)tg[r0 + e + 1][d] << 16);
        xu[e >> 3][(e & 7) >> 1] = (uint32_t)tu[r0 + e][d] | ((uint32_t)tu[r0 + e + 1][d] << 16);
        xv[e >> 3][(e & 7) >> 1] = (uint32_t)tv[r0 + e][d] | ((uint32_t)tv[r0 + e + 1][d] << 16);
      }
      const int64_t qv_ld = (int64_t)a.B * a.Lp;
      uint16_t* dot = static_cast<uint16_t*>(a.dot) + ((int64_t)bh * DP + d) * a.Lp + i;
      uint16_t* qut = static_cast<uint16_t*>(a.qut) + ((int64_t)bh * DP + d) * a.Lp + i;
      uint16_t* qvt = static_cast<uint16_t*>(a.qvt) + ((int64_t)head * DP + d) * qv_ld +
                      (int64_t)b * a.Lp + i;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        *reinterpret_cast<u32x4*>(dot + 8 * h2) = xg[h2];
        *reinterpret_cast<u32x4*>(qut + 8 * h2) = xu[h2];
        *reinterpret_cast<u32x4*>(qvt + 8 * h2) = xv[h2];
      }
    }
  }
}

// Rk^T [h][d][c] = Rk[h][pad_ws + c - pad_t][d] for 0 <= c - pad_t < Pp, else 0
// (ld a multiple of 8).  One workgroup per (64 columns c, head): the 64 Rk
// rows (128 bytes each) are read whole into an LDS tile, and each output row
// segment is written as 16-byte chunks.
__device__ __forceinline__ void rk_transpose_block(const uint16_t* rk, uint16_t* rkt, int32_t Pp,
                                                   int32_t pad_ws, int32_t ld, int32_t pad_t,
                                                   int32_t bx, int32_t h) {
  __shared__ uint16_t tile[64][DP + 2];   // [c][d]
  const int32_t c0 = bx * 64;
  const int tid = threadIdx.x;
  const uint16_t* src = rk + ((int64_t)h * (Pp + 2 * pad_ws) + pad_ws) * DP;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int cl = 32 * pass + (tid >> 3), d0 = 8 * (tid & 7);
    const int32_t delta = c0 + cl - pad_t;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (delta >= 0 && delta < Pp) x = *reinterpret_cast<const u32x4*>(src + (int64_t)delta * DP + d0);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      tile[cl][d0 + 2 * w] = x[w] & 0xffff;
      tile[cl][d0 + 2 * w + 1] = x[w] >> 16;
    }
  }
  __syncthreads();
  const int d = tid >> 2;
  uint16_t* dst = rkt + ((int64_t)h * DP + d) * ld;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int cl = 16 * (tid & 3) + 8 * q;
    if (c0 + cl >= ld) continue;
    u32x4 v;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      v[w] = (uint32_t)tile[cl + 2 * w][d] | ((uint32_t)tile[cl + 2 * w + 1][d] << 16);
    *reinterpret_cast<u32x4*>(dst + c0 + cl) = v;
  }
}

// dst[c][r] = bf16(src[r][c]) for r < rows, zero for rows <= r < ld (src in
// `dtype`, [rows][cols]; dst [cols][ld], ld a multiple of 16).  One workgroup
// per 16 rows x 64 columns: each thread reads four elements of src along c
// (consecutive threads, consecutive columns; all four in flight) into LDS, and
// each row of dst gets two 16-byte chunks.
__device__ __forceinline__ void transpose_block(const void* src, int32_t rows, int32_t cols,
                                                int32_t dtype, int32_t ld, uint16_t* dst,
                                                int32_t bx, int32_t by) {
  __shared__ uint16_t tile[16][66];   // [r][c]
  const int32_t r0 = bx * 16, c0 = by * 64;
  const int tid = threadIdx.x;
  {
    const int cl = tid & 63;
    const int32_t c = c0 + cl;
    float x[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int32_t r = r0 + (tid >> 6) + 4 * k;
      x[k] = (r < rows && c < cols) ? load_as_f32(src, (int64_t)r * cols + c, dtype) : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) tile[(tid >> 6) + 4 * k][cl] = bf16_bits(x[k]);
  }
  __syncthreads();
  if (tid >= 128) return;
  const int cl = tid >> 1, rl = 8 * (tid & 1);
  if (c0 + cl >= cols) return;
  u32x4 v;
#pragma unroll
  for (int w = 0; w < 4; ++w)
    v[w] = (uint32_t)tile[rl + 2 * w][cl] | ((uint32_t)tile[rl + 2 * w + 1][cl] << 16);
  *reinterpret_cast<u32x4*>(dst + (int64_t)(c0 + cl) * ld + r0 + rl) = v;
}

// du[h][d], dv[h][d] = sums over batch rows and 32-query chunks.  One
// workgroup per (which, h, 8 columns): 32 strided partial sums per column,
// then a fixed-order tree.
__device__ __forceinline__ void duv_reduce_block(const float* part, int32_t B, int32_t H,
                                                 int32_t nchunk, int32_t dh, float* du, float* dv,
                                                 int32_t blk) {
  __shared__ float red[32][8];
  const int32_t nblk = (dh + 7) / 8;
  const int32_t which = blk / (H * nblk);
  const int32_t rest = blk % (H * nblk);
  const int32_t h = rest / nblk, d0 = 8 * (rest % nblk);
  const int tid = threadIdx.x, dd = tid & 7, grp = tid >> 3;
  const int32_t n = B * nchunk;
  float s = 0.0f;
  // partial p = grp, grp + 32, ... added in that order; eight loads in flight
  for (int32_t p0 = grp; p0 < n; p0 += 8 * 32) {
    float x[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int32_t p = p0 + 32 * k;
      const int32_t bb = p / nchunk, c = p % nchunk;
      x[k] = p < n ? part[((((int64_t)which * B + bb) * H + h) * nchunk + c) * DP + d0 + dd] : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (p0 + 32 * k < n) s += x[k];
  }
  red[grp][dd] = s;
  __syncthreads();
  for (int w = 16; w > 0; w >>= 1) {
    if (grp < w) red[grp][dd] += red[grp + w][dd];
    __syncthreads();
  }
  if (tid < 8 && d0 + tid < dh) (which == 0 ? du : dv)[(int64_t)h * dh + d0 + tid] = red[0][tid];
}

// dst[x] = sum_r src[r][x] over n_rows rows of length row_len, in row order
// (eight rows' loads in flight at a time).
__global__ void sum_rows_kernel(const float* src, int32_t n_rows, int64_t row_len, float* dst) {
  const int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (x >= row_len) return;
  float s = 0.0f;
  for (int32_t r0 = 0; r0 < n_rows; r0 += 8) {
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = r0 + k < n_rows ? src[(int64_t)(r0 + k) * row_len + x] : 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (r0 + k < n_rows) s += v[k];
  }
  dst[x] = s;
}

// dRk[delta][x] = sum_r part[r][delta][x] in row order for a tile of 16
// distances x 64 columns (four elements per thread, eight rows' loads in
// flight), and, when drkt is set, the tile's bf16 transpose into
// drkt[x][delta] (distances P .. r_ld-1 zero) as 16-byte chunks.
__device__ __forceinline__ void drk_sum_block(const BwdPostArgs& a, int32_t bx, int32_t by) {
  __shared__ uint16_t tile[16][66];   // [delta][x]
  const int32_t d0 = bx * 16, x0 = by * 64;
  const int tid = threadIdx.x;
  const int xl = tid & 63;
  const int32_t x = x0 + xl;
  const int64_t plane = (int64_t)a.P * a.HD;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int dl = (tid >> 6) + 4 * k;
    const int32_t delta = d0 + dl;
    const bool ok = delta < a.P && x < a.HD;
    float s = 0.0f;
    if (ok) {
      const float* src = a.drk_part + (int64_t)delta * a.HD + x;
      for (int32_t b0 = 0; b0 < a.drk_rows; b0 += 8) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = b0 + j < a.drk_rows ? src[(b0 + j) * plane] : 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (b0 + j < a.drk_rows) s += v[j];
      }
      a.d_rk[(int64_t)delta * a.HD + x] = s;
    }
    tile[dl][xl] = bf16_bits(s);   // zero past P
  }
  if (!a.drkt) return;
  __syncthreads();
  if (tid >= 128) return;
  const int cl = tid >> 1, rl = 8 * (tid & 1);
  if (x0 + cl >= a.HD) return;
  u32x4 v;
#pragma unroll
  for (int w = 0; w < 4; ++w)
    v[w] = (uint32_t)tile[rl + 2 * w][cl] | ((uint32_t)tile[rl + 2 * w + 1][cl] << 16);
  *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.drkt) + (int64_t)(x0 + cl) * a.r_ld + d0 + rl) = v;
}

// Grid of the pre step: prep blocks, then Rk^T tiles (64 columns x head),
// then R^T tiles (16 rows x 64 columns).
struct PreGrid {
  int32_t n_prep, rk_nx, n_rk, r_nx, n_r;
};
__host__ __device__ inline PreGrid pre_grid(const BwdPreArgs& a) {
  PreGrid g;
  g.n_prep = a.prep.B * a.prep.H * ((a.prep.Lp + 63) / 64);
  g.rk_nx = (a.rkt_ld + 63) / 64;
  g.n_rk = g.rk_nx * a.prep.H;
  g.r_nx = a.r ? a.r_ld / 16 : 0;
  g.n_r = a.r ? g.r_nx * ((a.d_pos + 63) / 64) : 0;
  return g;
}

__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdPreArgs a) {
  const PreGrid g = pre_grid(a);
  int32_t blk = blockIdx.x;
  if (blk < g.n_prep) {
    bwd_prep_block(a.prep, blk);
    return;
  }
  blk -= g.n_prep;
  if (blk < g.n_rk) {
    rk_transpose_block(static_cast<const uint16_t*>(a.rk_ws), static_cast<uint16_t*>(a.rkt), a.Pp,
                       a.pad_ws, a.rkt_ld, a.pad_t, blk % g.rk_nx, blk / g.rk_nx);
    return;
  }
  blk -= g.n_rk;
  transpose_block(a.r, a.P, a.d_pos, a.r_dtype, a.r_ld, static_cast<uint16_t*>(a.rt), blk % g.r_nx,
                  blk / g.r_nx);
}

// Grid of the post step: dRk tiles (16 distances x 64 columns, over r_ld
// distances when the transpose is written), then du/dv blocks.
struct PostGrid {
  int32_t sum_nx, n_sum;
};
__host__ __device__ inline PostGrid post_grid(const BwdPostArgs& a) {
  PostGrid g;
  g.sum_nx = ((a.drkt ? a.r_ld : a.P) + 15) / 16;
  g.n_sum = g.sum_nx * ((a.HD + 63) / 64);
  return g;
}

__global__ __launch_bounds__(256) void bwd_post_kernel(BwdPostArgs a) {
  const PostGrid g = post_grid(a);
  const int32_t blk = blockIdx.x;
  if (blk < g.n_sum) {
    drk_sum_block(a, blk % g.sum_nx, blk / g.sum_nx);
    return;
  }
  duv_reduce_block(a.duv_part, a.B, a.H, a.nchunk, a.dh, a.d_u, a.d_v, blk - g.n_sum);
}

dim3 grid_for(int64_t n) { return dim3((unsigned)((n + 255) / 256)); }

}  // namespace

int launch_attn_bwd_q(const BwdArgs& a, void* stream) {
  const int32_t nqg = (a.L + 127) / 128;
  hipLaunchKernelGGL(attn_bwd_q_kernel, dim3(a.B * a.H * nqg), dim3(256), 0,
                     static_cast<hipStream_t>(stream), a);
  return static_cast<int>(hipGetLastError());
}

int launch_bmm64(const BmmArgs* a, int n, const int32_t* kind, const int32_t* row_off,
                 const int32_t* kper, void* stream) {
  if (n < 1 || n > 3) return static_cast<int>(hipErrorInvalidValue);
  BmmBatch bt{};
  for (int i = 0; i < n; ++i) {
    bt.kind[i] = kind[i];
    bt.row_off[i] = row_off[i];
    bt.kper[i] = kper ? kper[i] : 0;
    if (bt.kper[i] != 0 && (kind[i] != 2 || bt.kper[i] % 32 != 0 || a[i].K % bt.kper[i] != 0))
      return static_cast<int>(hipErrorInvalidValue);
  }
  int32_t gx = 1, gy = 1;
  for (int i = 0; i < n; ++i) {
    if (a[i].K % 16 != 0) return static_cast<int>(hipErrorInvalidValue);
    bt.p[i] = a[i];
    gx = std::max(gx, (a[i].M + BMM_ROWS - 1) / BMM_ROWS);
    gy = std::max(gy, a[i].batch);
  }
  hipLaunchKernelGGL(bmm64_kernel, dim3(gx, gy, n), dim3(256), 0,
                     static_cast<hipStream_t>(stream), bt);
  return static_cast<int>(hipGetLastError());
}

int launch_bwd_pre(const BwdPreArgs& a, void* stream) {
  if (a.rkt_ld % 8 != 0 || (a.r && (a.r_ld % 16 != 0 || a.P > a.r_ld)))
    return static_cast<int>(hipErrorInvalidValue);
  const PreGrid g = pre_grid(a);
  hipLaunchKernelGGL(bwd_pre_kernel, dim3(g.n_prep + g.n_rk + g.n_r), dim3(256), 0,
                     static_cast<hipStream_t>(stream), a);
  return static_cast<int>(hipGetLastError());
}

int launch_bwd_post(const BwdPostArgs& a, void* stream) {
  if (a.drkt && (a.r_ld % 16 != 0 || a.P > a.r_ld)) return static_cast<int>(hipErrorInvalidValue);
  const PostGrid g = post_grid(a);
  const int32_t n_duv = 2 * a.H * ((a.dh + 7) / 8);
  hipLaunchKernelGGL(bwd_post_kernel, dim3(g.n_sum + n_duv), dim3(256), 0,
                     static_cast<hipStream_t>(stream), a);
  return static_cast<int>(hipGetLastError());
}

int launch_sum_rows(const float* src, int32_t n_rows, int64_t row_len, float* dst, void* stream) {
  hipLaunchKernelGGL(sum_rows_kernel, grid_for(row_len), dim3(256), 0,
                     static_cast<hipStream_t>(stream), src, n_rows, row_len, dst);
  return static_cast<int>(hipGetLastError());
}

}  // namespace txl
