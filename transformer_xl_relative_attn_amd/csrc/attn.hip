// Fused relative-position attention core (Dai et al., Transformer-XL, Sec. 3.3
// summary equations; App. B for the shift structure of terms (b) and (d)).
//
// For one (batch b, head h) and queries i, keys j of [memory ; segment]:
//   s_ij = c * ( (q_i+u).k_j + (q_i+v).Rk[M+i-j] ),  visible iff j <= M+i
//   out_i = sum_j softmax_j(s_ij) val_j
// (q+u).k_j carries terms (a) and (c), (q+v).Rk carries (b) and (d).
//
// bf16 kernel (d_head <= 64, padded to 64).  A workgroup owns 128 queries (4
// waves x 32) of one (b, h) and a contiguous range of 32-key blocks (key-range
// splits fill the chip when B*H is small).  Scores are kept transposed,
// S^T[j][i], so a lane owns one query column and the softmax statistics stay
// in the lane and its partner (ii, 1-hf).
//   * LDS-DMA ring: block t's K tile and V^T tile (4 KB each, contiguous in the
//     workspace) and Rk chunk t+1 (32 rows, one block ahead) are loaded by
//     direct buffer->LDS loads three blocks ahead, one block per barrier;
//     every wave issues exactly three loads per block (a quarter of each), so
//     the vmcnt waits are constants.  Wave w uses Rk chunk t+2-w at block t.
//   * Term (b)+(d): for block t+2 a wave multiplies its 32 queries (q+v) by the
//     32-row Rk chunk that starts at distance D-31, D = M + i0 - 32(t+2), on the
//     matrix cores.  Pair (i, j) needs distance D + i - j: row 31 + i - j of the
//     window [this chunk ; previous chunk], and the previous chunk's product is
//     still in registers, so every chunk is multiplied once.  Each lane writes
//     its query's window row to LDS already shifted (App. B's left shift done as
//     an address computation), and the shifted row becomes the initial
//     accumulator of the (q+u).K product: summing the four terms costs no
//     vector instruction.
//   * Online softmax in base 2: c = scale * log2(e) is folded into q+u and q+v.
//     The reference maximum moves only when a block's maximum exceeds it by
//     more than 8 (p <= 2^8); it starts at -FLT_MAX, so the first block with a
//     visible key sets it.
//   * Software pipeline, two blocks deep: block t issues the (b)+(d) product
//     for block t+2 and the (q+u).K product of block t+1 on the matrix cores,
//     passes the block's barrier and runs block t's softmax on the vector ALUs
//     while they execute, then P.V of block t; block t+2's window is written
//     and block t+1's operands are read from LDS at the end of block t.
//   * P (bf16) times V^T on the matrix cores: bf16 pairs of P are exchanged
//     with the partner lane so that both operands list the keys in order.  The
//     softmax denominators are per-lane sums of the same bf16 p (half of a
//     column's keys each, two per dot instruction), joined with the partner
//     lane at the end.
//   * With several key-range splits each workgroup writes (max, sum, O) and
//     attn_combine_kernel merges them in split order (deterministic).  The
//     segment step's memory-ring update rides on that launch (or on the tail of
//     this kernel when there is one split).
//
// fp32 kernel: one workgroup per (b, h, i), plain loops; used by the fp32 path.
#include <type_traits>

#include "dev_common.h"

namespace txl {

namespace {

constexpr int DP = 64;        // padded head width of the bf16 path
constexpr int KB = 32;        // keys per block
constexpr int NWAVE = 4;      // waves per workgroup, 32 queries each
constexpr int QG = 32 * NWAVE;
constexpr int NST = 4;        // K / V^T ring stages (blocks t .. t+3 resident or in flight)
constexpr int RKS = 7;        // Rk chunk slots (the prologue holds chunks t_lo-3 .. t_lo+3)
constexpr int WP = 36;        // floats per query row of a wave's shifted (b)+(d) window
constexpr int KT_U = KB * 8;  // 16-byte units of a K tile (32 keys x 128 bytes)
constexpr int VT_U = DP * 4;  // of a V^T tile (64 rows x 64 bytes)
constexpr int RK_U = KB * 8;  // of an Rk chunk (32 rows x 128 bytes)
constexpr int LOADS_PER_BLOCK = 3;   // LDS-DMA instructions per wave per block
constexpr float kNegInf = -__builtin_inff();
constexpr float kNoMax = -3.40282347e38f;   // -FLT_MAX
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));

struct AttnSmem {
  u32x4 kv[NST][KT_U + VT_U];   // per stage: K tile, then V^T tile
  u32x4 rk[RKS][RK_U];          // Rk chunk ring
  float win[NWAVE][32 * WP];    // per-wave shifted (b)+(d) window
  float uv[2 * DP];             // u then v of this head, zero padded
};
static_assert(sizeof(AttnSmem) <= 80 * 1024, "two workgroups per CU");
static_assert(32 * WP * 4 >= RK_U * 16, "a window region holds one Rk chunk (prologue)");

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

// Wait until at most N loads of this wave are in flight (loads and LDS-DMA
// complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Raw buffer resource over `bytes` bytes at `base` (word 3: 32-bit data
// format, the value gfx9 untyped loads expect).  Offsets at or past `bytes`
// read zero instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// 16 bytes per lane from buffer offset lane_off + blk_off into LDS at dst +
// 16 * lane (dst is wave-uniform; it goes to M0).
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t rs, u32x4* dst,
                                                  uint32_t lane_off, int32_t blk_off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rs, (__attribute__((address_space(3))) void*)dst, 16, (int)lane_off, blk_off, 0, 0);
}

__device__ __forceinline__ void barrier_lds() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

__device__ __forceinline__ void compiler_fence() { __asm__ volatile("" ::: "memory"); }

// Copy min(L, M) segment rows into their memory-ring slots (the segment step's
// update, Sec. 3.2): row r of the flattened [B][rows] range goes to slot
// (start + t) mod M, or to slot t with the last M rows when L >= M.  Rows are
// dealt to `nworkers` workers of 256 threads, in words of W bytes.
template <class W>
__device__ __forceinline__ void ring_copy_words(const AttnArgs& a, int32_t worker,
                                                int32_t nworkers, int tid) {
  // the (row, word) pairs of all copied rows, 256 consecutive ones per
  // workgroup and pass, so that every thread copies one word per pass
  const int64_t words = a.upd_row_bytes / (int64_t)sizeof(W);
  const int64_t n = (int64_t)a.B * a.upd_rows * words;
  for (int64_t g = (int64_t)worker * 256 + tid; g < n; g += (int64_t)nworkers * 256) {
    const int32_t r = (int32_t)(g / words);
    const int64_t c = g - (int64_t)r * words;
    const int32_t bb = r / a.upd_rows, t = r - bb * a.upd_rows;
    const int32_t src = a.L < a.M ? t : a.L - a.M + t;
    const int32_t slot = a.L < a.M ? (a.upd_start + t) % a.M : t;
    const W* sp = reinterpret_cast<const W*>(static_cast<const char*>(a.upd_src) +
                                             ((int64_t)bb * a.L + src) * a.upd_row_bytes);
    W* dp = reinterpret_cast<W*>(static_cast<char*>(a.upd_mem) +
                                 ((int64_t)bb * a.M + slot) * a.upd_row_bytes);
    dp[c] = sp[c];
  }
}

__device__ __forceinline__ void ring_copy(const AttnArgs& a, int32_t worker, int32_t nworkers,
                                          int tid) {
  if (a.upd_unit == 16)
    ring_copy_words<u32x4>(a, worker, nworkers, tid);
  else
    ring_copy_words<uint32_t>(a, worker, nworkers, tid);
}

template <int V>
using IC = std::integral_constant<int, V>;

__device__ __forceinline__ float max3(float a, float b, float c) {
  return __builtin_fmaxf(__builtin_fmaxf(a, b), c);
}
__device__ __forceinline__ float max2(float a, float b) { return __builtin_fmaxf(a, b); }

__global__ __launch_bounds__(256, 2) void attn_bf16_kernel(AttnArgs a, int32_t padded, int32_t nqg) {
  const int32_t total = a.B * a.H * nqg * a.n_split;
  const int32_t wid = xcd_swizzle(blockIdx.x, padded);
  if (wid >= total) return;
  // work order: split fastest, then batch, query group, head, so that the
  // work items dealt to one XCD share a head's position keys in its L2
  const int32_t split = wid % a.n_split;
  int32_t rest = wid / a.n_split;
  const int32_t b = rest % a.B;
  rest /= a.B;
  // within a head, later query groups (more visible keys) come first, so the
  // shorter ones fill the last round of each XCD
  const int32_t qg = nqg - 1 - rest % nqg;
  const int32_t head = rest / nqg;
  const int32_t bh = b * a.H + head;
  const int32_t M = a.M, L = a.L;

  __shared__ AttnSmem sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ii = lane & 31, hf = lane >> 5;

  const int32_t i_base = qg * QG;
  const int32_t i_last = min(i_base + QG, L) - 1;
  const int32_t nb = (M + i_last + 1 + KB - 1) / KB;  // key blocks visible to the group
  const int32_t t_lo = (int32_t)((int64_t)split * nb / a.n_split);
  const int32_t t_hi = (int32_t)((int64_t)(split + 1) * nb / a.n_split);

  const int32_t i0 = i_base + 32 * wave;
  const bool wave_on = i0 < L;
  // blocks [t_lo, t_end) hold a visible key for some query of this wave
  const int32_t t_end =
      wave_on ? max(t_lo, min(t_hi, (M + min(i0 + 31, L - 1) + 1 + KB - 1) / KB)) : t_lo;

  // ---- LDS-DMA.  Block t brings K tile t, V^T tile t and Rk chunk t (rows
  // M + i_base - 31 - 32 t + r, r = 0..31; the table's padding covers rows
  // outside [0, Pp)).  Each is 4 KB contiguous; wave w loads quarter w of all
  // three (one wave-instruction of 64 lanes x 16 bytes each), so every wave
  // issues three loads per block.  A lane fetches the global chunk that lands
  // in its swizzled slot.  Block t uses K/V stage (t - t_lo) % NST and chunk c
  // slot (c - t_lo + 4) % RKS.  The loads go through buffer resources: the
  // lane offset is a constant register and the block offset a scalar, so a
  // block's three loads cost no vector instruction.
  const int32_t nkb = a.Np / KB;
  const char* kbase = static_cast<const char*>(a.k) + (int64_t)bh * a.Np * DP * 2;
  const char* vbase = static_cast<const char*>(a.vt) + ((int64_t)b * nkb * a.H + head) * DP * KB * 2;
  const int32_t vstep = a.H * DP * KB * 2;
  const char* rbase = static_cast<const char*>(a.rk) +
                      ((int64_t)head * (a.Pp + 2 * kRkPad) + kRkPad + M + i_base - (KB - 1)) * DP * 2;
  auto row_off = [&](int n) {      // instruction n (0..3) of a K tile or Rk chunk
    const int r = n * 8 + (lane >> 3);
    return (uint32_t)(r * 128 + (((lane & 7) ^ ((r >> 1) & 7)) << 4));
  };
  // buffers: this (b, h)'s K tiles, its V^T tiles (stride vstep), and the Rk
  // chunks t_lo - 4 .. t_hi addressed from chunk t_hi upwards
  constexpr int32_t kTileBytes = KB * DP * 2;
  const __amdgpu_buffer_rsrc_t rs_k = make_rsrc(kbase, a.Np * DP * 2);
  const __amdgpu_buffer_rsrc_t rs_v = make_rsrc(vbase, (nkb - 1) * vstep + kTileBytes);
  const __amdgpu_buffer_rsrc_t rs_r =
      make_rsrc(rbase - (int64_t)t_hi * kTileBytes, (t_hi - t_lo + 5) * kTileBytes);
  auto rk_off = [&](int32_t c) { return (t_hi - c) * kTileBytes; };   // chunk c, t_lo-4 <= c <= t_hi
  const uint32_t lo_k = row_off(wave), lo_r = lo_k;
  const uint32_t lo_v = [&] {
    const int d = wave * 16 + (lane >> 2);
    return (uint32_t)(d * 64 + (((lane & 3) ^ ((d >> 2) & 3)) << 4));
  }();
  // DMA block tb: this wave's three loads, K tile and V^T tile tb into K/V
  // stage `kv` and Rk chunk tb+1 (one block ahead of the keys) into slot `rs`.
  // Past the split's last block the loads repeat that block (valid memory)
  // into the free slots, so every wave always issues three per block.  K/V
  // tiles are addressed through the ring rotation (block t at tile
  // (t + kv_tile0) mod nkb; kv_tile0 = 0 outside the ring).
  auto issue_block = [&](int32_t tb, u32x4* kv, u32x4* rs) {
    const int32_t tl = min(tb, t_hi - 1);
    int32_t tk = tl + a.kv_tile0;
    tk -= tk >= nkb ? nkb : 0;
    const int32_t q = wave * 64;
    buffer_load_lds16(rs_k, kv + q, lo_k, tk * kTileBytes);
    buffer_load_lds16(rs_v, kv + KT_U + q, lo_v, tk * vstep);
    buffer_load_lds16(rs_r, rs + q, lo_r, rk_off(tl + 1));
  };
  auto rk_slot = [&](int32_t c) { return (c - t_lo + 4) % RKS; };   // c >= t_lo - 4

  // ---- prologue.  Rk chunks t_lo-4 .. t_lo (wave w loads chunk t_lo-4+w
  // whole, and quarter w of chunk t_lo; chunk t_lo-4, which only wave 3 needs,
  // goes to wave 3's window region, still unused), DMA blocks t_lo .. t_lo+2
  // (Rk chunks t_lo+1 .. t_lo+3), and this head's u, v and the wave's q rows.
  {
    const int32_t c = t_lo - 4 + wave;
    u32x4* dst = wave == 0 ? reinterpret_cast<u32x4*>(sm.win[3]) : sm.rk[rk_slot(c)];
#pragma unroll
    for (int n = 0; n < 4; ++n) buffer_load_lds16(rs_r, dst + n * 64, row_off(n), rk_off(c));
    buffer_load_lds16(rs_r, sm.rk[rk_slot(t_lo)] + wave * 64, lo_r, rk_off(t_lo));
    issue_block(t_lo, sm.kv[0], sm.rk[rk_slot(t_lo + 1)]);
    issue_block(t_lo + 1, sm.kv[1], sm.rk[rk_slot(t_lo + 2)]);
  }
  float uvv = 0.0f;
  if (tid < 2 * DP) {
    const int d = tid & (DP - 1);
    const uint16_t* src = static_cast<const uint16_t*>(tid < DP ? a.u : a.v) + (int64_t)head * a.dh;
    if (d < a.dh) uvv = bf16_to_f32(src[d]);
  }
  floatx4 qraw[8];
  {
    // rows L .. Lp-1 of q are not computed: those lanes take q = 0 (their
    // outputs are never stored)
    const bool q_ok = i0 + ii < L;
    const floatx4* qrow =
        reinterpret_cast<const floatx4*>(a.q + ((int64_t)bh * a.Lp + (q_ok ? i0 + ii : 0)) * DP);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      qraw[2 * s] = qrow[(16 * s + 8 * hf) / 4];
      qraw[2 * s + 1] = qrow[(16 * s + 8 * hf) / 4 + 1];
    }
#pragma unroll
    for (int x = 0; x < 8; ++x)
      if (!q_ok) qraw[x] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  compiler_fence();   // the q loads go out before the third block's DMA
  issue_block(t_lo + 2, sm.kv[2], sm.rk[rk_slot(t_lo + 3)]);
  // everything but DMA block t_lo+2 has landed
  wait_vm<LOADS_PER_BLOCK>();
  if (tid < 2 * DP) sm.uv[tid] = uvv;
  barrier_lds();

  // per-wave query operands (q+u)*c, (q+v)*c as bf16, d = 16s + 8hf + e
  bf16x8 qu[4], qv[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int d0 = 16 * s + 8 * hf;
    float xu[8], xv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float qd = qraw[2 * s + (e >> 2)][e & 3];
      xu[e] = (qd + sm.uv[d0 + e]) * a.c_scale;
      xv[e] = (qd + sm.uv[DP + d0 + e]) * a.c_scale;
    }
    qu[s] = pack8(xu);
    qv[s] = pack8(xv);
  }

  // ---- fragment reads (lane-constant unit offsets within a tile) and products
  int kofs[4], vofs[2][2];
#pragma unroll
  for (int s = 0; s < 4; ++s) kofs[s] = ksw(ii, 2 * s + hf);
#pragma unroll
  for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
    for (int e = 0; e < 2; ++e) vofs[t2][e] = vsw(32 * e + ii, 2 * t2 + hf);
  auto read_rows = [&](const u32x4* base, bf16x8 (&f)[4]) {   // K tile or Rk chunk, row ii
#pragma unroll
    for (int s = 0; s < 4; ++s) f[s] = __builtin_bit_cast(bf16x8, base[kofs[s]]);
  };
  auto read_vt = [&](const u32x4* kv, bf16x8 (&vf)[2][2]) {   // V^T rows d = 32e + ii
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int e = 0; e < 2; ++e) vf[t2][e] = __builtin_bit_cast(bf16x8, kv[vofs[t2][e]]);
  };
  // BD[w][i] = (q_i+v).Rk[chunk row w]: lane holds rows w = 8g + 4hf + r
  // (element 4g + r) of column ii
  auto bd_chunk = [&](const bf16x8 (&rf)[4]) {
    floatx16 acc = floatx16{0};
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rf[s], qv[s], acc, 0, 0, 0);
    return acc;
  };
  // Shifted window of block t' = [chunk t'-w ; chunk t'-w-1]: the value for
  // (query ii, key jj) is window row 31 + ii - jj, stored at position jj of row
  // ii, i.e. row w of the current chunk (w >= ii) or of the previous (w < ii)
  // lands at position (31 + ii - w) mod 32.
  float* win = sm.win[wave] + ii * WP;
  auto write_win = [&](const floatx16& cur, const floatx16& prev) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int w = 8 * (e >> 2) + 4 * hf + (e & 3);
      win[(31 + ii - w) & 31] = w >= ii ? cur[e] : prev[e];
    }
  };
  auto read_win = [&]() {   // initial accumulator: element 4g + r is key 8g + 4hf + r
    floatx16 c;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const floatx4 x = *reinterpret_cast<const floatx4*>(win + 8 * g + 4 * hf);
#pragma unroll
      for (int r = 0; r < 4; ++r) c[4 * g + r] = x[r];
    }
    return c;
  };
  auto qk = [&](const bf16x8 (&kf)[4], floatx16 c) {
#pragma unroll
    for (int s = 0; s < 4; ++s) c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qu[s], c, 0, 0, 0);
    return c;
  };

  // ---- prologue compute: (b)+(d) products of chunks t_lo-1-w, t_lo-w and
  // t_lo+1-w, the scores of block t_lo on its window, and block t_lo+1's
  // window left in LDS
  floatx16 SA, SB = floatx16{0}, bdA = floatx16{0}, bdB;
  bf16x8 kf[4], rf[4], vf[2][2];
  floatx16 W;
  {
    const u32x4* pc = wave == 3 ? reinterpret_cast<const u32x4*>(sm.win[3])
                                : sm.rk[rk_slot(t_lo - wave - 1)];
    bf16x8 pf[4], cf[4], nf[4];
    read_rows(pc, pf);
    read_rows(sm.rk[rk_slot(t_lo - wave)], cf);
    read_rows(sm.rk[rk_slot(t_lo + 1 - wave)], nf);
    read_rows(sm.kv[0], kf);
    const floatx16 bp = bd_chunk(pf);
    const floatx16 bc = bd_chunk(cf);
    bdB = bd_chunk(nf);
    compiler_fence();   // (wave 3) the chunk reads precede the window writes in LDS order
    write_win(bc, bp);
    compiler_fence();
    SA = qk(kf, read_win());
    write_win(bdB, bc);
    compiler_fence();
    // operands of block t_lo's products: window t_lo+1, K tile t_lo+1, Rk
    // chunk t_lo+2-w
    W = read_win();
    read_rows(sm.kv[1], kf);
    read_rows(sm.rk[rk_slot(t_lo + 2 - wave)], rf);
  }

  float lpart = 0.0f;             // sum of this lane's p (half of column ii's keys)
  floatx16 o[2] = {floatx16{0}, floatx16{0}};
  // Running reference maximum (lazy) and the threshold m_ref + 8 that moves it.
  // Before the first visible key it is -FLT_MAX: every finite block maximum
  // then moves it, the rescale factor 2^(m_ref - mb) is 0 (the accumulators
  // are still zero), and p = 2^(-inf - m_ref) = 0 for masked keys.
  float m_ref = kNoMax, m_thr = kNoMax;

  // Rk slots of chunk t+3-w (read at the end of block t) and of the next
  // chunk to load, advanced once per block (wave-uniform scalars).
  int32_t rd_slot = rk_slot(t_lo + 3 - wave);
  int32_t is_slot = rk_slot(t_lo + 4);
  auto next_slot = [](int32_t sl) { return sl == RKS - 1 ? 0 : sl + 1; };

  // One block t (K/V stage U = (t - t_lo) % NST).  On entry the registers hold
  // the scores S of block t, block t+1's window W, K fragments kf of tile t+1,
  // Rk fragments rf of chunk t+2-w, and `prev`, the (b)+(d) product of chunk
  // t+1-w.  The block issues the (b)+(d) product of chunk t+2-w and block
  // t+1's (q+u).K on the matrix cores first, runs block t's softmax on the
  // vector ALUs while they execute, then P.V of block t, writes block t+2's
  // window and reads the operands of block t+1's products.  The
  // loop is unrolled NST times so that stages are static and the register
  // sets trade roles instead of being copied.
  auto block = [&](auto U, int32_t t, floatx16& S, floatx16& Snext, floatx16& cur,
                   floatx16& prev) {
    constexpr int u = decltype(U)::value;
    constexpr int u2 = (u + 2) % NST, u3 = (u + 3) % NST;
    const bool cur_on = t < t_end;
    const bool n1_on = t + 1 < t_end;
    const bool n2_on = t + 2 < t_end;
    if (n2_on) cur = bd_chunk(rf);   // chunk t+2-w
    if (n1_on) Snext = qk(kf, W);    // block t+1
    // A barrier per block, passed while those products execute: DMA block t+2
    // (issued one block ago) has landed and is visible to every wave; the
    // stage of block t-1 (its K tile read in block t-3, its V^T tile in block
    // t-1) takes DMA block t+3.
    wait_vm<0>();
    barrier_lds();
    issue_block(t + 3, sm.kv[u3], sm.rk[is_slot]);
    is_slot = next_slot(is_slot);
    if (cur_on) read_vt(sm.kv[u], vf);   // V^T tile t, used after the softmax
    bf16x8 pb[2];
    if (cur_on) {
      // causal/memory mask: key j = 32t + jj visible iff k_lo <= j <= M + i0 + ii
      const int32_t j0 = t * KB;
      if (j0 + KB - 1 > M + i0 || j0 < a.k_lo) {
        const int32_t lim = M + i0 + ii - j0 - 4 * hf;   // key jj = 8g + 4hf + r
        const int32_t lo = a.k_lo - j0 - 4 * hf;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int kk = 8 * (e >> 2) + (e & 3);
          if (kk > lim || kk < lo) S[e] = kNegInf;
        }
      }
      float mb = max3(S[0], S[1], S[2]);
#pragma unroll
      for (int e = 3; e < 15; e += 2) mb = max3(mb, S[e], S[e + 1]);
      mb = max2(mb, S[15]);
      {  // with the partner lane (ii, 1-hf): both halves of the column
        const auto mm = __builtin_amdgcn_permlane32_swap(__float_as_uint(mb), __float_as_uint(mb), false, false);
        mb = max2(__uint_as_float(mm[0]), __uint_as_float(mm[1]));
      }
      const bool need = mb > m_thr;
      if (__builtin_expect(__ballot(need) != 0, 0)) {
        // move the reference up to mb and rescale the accumulators (by 0 before
        // the first visible key: 2^(-FLT_MAX - mb) = 0)
        const float alpha = need ? __builtin_amdgcn_exp2f(m_ref - mb) : 1.0f;
        if (need) {
          m_ref = mb;
          m_thr = mb + 8.0f;
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          o[0][e] *= alpha;
          o[1][e] *= alpha;
        }
        lpart *= alpha;
      }
      float p[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) p[e] = __builtin_amdgcn_exp2f(S[e] - m_ref);
      // The lane holds p for keys 16t2 + 4hf + {0..3} and 16t2 + 8 + 4hf +
      // {0..3}; swapping bf16 pairs with the partner lane gives it keys
      // 16t2 + 8hf .. +7 in order, the k-slots of the V^T fragment.  The
      // denominator sums the same bf16 values the P.V product uses, two per
      // dot instruction.
      const bf16x8 pk[2] = {pack8(&p[0]), pack8(&p[8])};
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          lpart = __builtin_amdgcn_fdot2_f32_bf16(
              bf16x2{pk[t2][2 * e], pk[t2][2 * e + 1]}, bf16x2{(bf16)1.0f, (bf16)1.0f}, lpart, false);
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const u32x4 pw = __builtin_bit_cast(u32x4, pk[t2]);
        const auto s02 = __builtin_amdgcn_permlane32_swap(pw[0], pw[2], false, false);
        const auto s13 = __builtin_amdgcn_permlane32_swap(pw[1], pw[3], false, false);
        pb[t2] = __builtin_bit_cast(bf16x8, u32x4{s02[0], s13[0], s02[1], s13[1]});
      }
    }
    if (cur_on) {
      // P^T (keys x queries) times V^T
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
#pragma unroll
        for (int e = 0; e < 2; ++e)
          o[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[t2][e], pb[t2], o[e], 0, 0, 0);
      }
    }
    if (n2_on) write_win(cur, prev);   // window of block t+2
    compiler_fence();
    // operands of block t+1's products (landed before this block's barrier)
    if (n2_on) {
      W = read_win();
      read_rows(sm.kv[u2], kf);
      read_rows(sm.rk[rd_slot], rf);   // chunk t+3-w
    }
    rd_slot = next_slot(rd_slot);
  };
  for (int32_t t = t_lo; t < t_hi; t += NST) {
    block(IC<0>{}, t, SA, SB, bdA, bdB);
    if (t + 1 < t_hi) block(IC<1>{}, t + 1, SB, SA, bdB, bdA);
    if (t + 2 < t_hi) block(IC<2>{}, t + 2, SA, SB, bdA, bdB);
    if (t + 3 < t_hi) block(IC<3>{}, t + 3, SB, SA, bdB, bdA);
  }
  static_assert(NST == 4, "the block loop is unrolled NST times");
  // the repeated loads past the split's last block must land before exit
  wait_vm<0>();

  float l_sum;   // both halves of the column's keys
  {
    const auto ll = __builtin_amdgcn_permlane32_swap(__float_as_uint(lpart), __float_as_uint(lpart), false, false);
    l_sum = __uint_as_float(ll[0]) + __uint_as_float(ll[1]);
  }
  const int32_t i = i0 + ii;
  typedef float floatx2_t __attribute__((ext_vector_type(2)));
  typedef bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  if (a.n_split == 1) {
    // out[b, i, head, :] = num / den; lane holds d = 32e + 8g + 4hf + r (r = 0..3)
    if (wave_on && i < L) {
      const float inv = 1.0f / l_sum;
      if (a.lse && hf == 0) a.lse[(int64_t)bh * a.Lp + i] = m_ref + log2f(l_sum);
      uint16_t* out = static_cast<uint16_t*>(a.out) + (((int64_t)b * L + i) * a.H + head) * a.dh;
      const bool vec = (a.dh == DP);
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = 32 * e + 8 * g + 4 * hf;
          if (vec) {
            const bf16x2_t lo =
                __builtin_convertvector(floatx2_t{o[e][4 * g] * inv, o[e][4 * g + 1] * inv}, bf16x2_t);
            const bf16x2_t hi =
                __builtin_convertvector(floatx2_t{o[e][4 * g + 2] * inv, o[e][4 * g + 3] * inv}, bf16x2_t);
            *reinterpret_cast<u32x2*>(out + d0) =
                u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (d0 + r < a.dh) out[d0 + r] = f32_to_bf16_bits(o[e][4 * g + r] * inv);
          }
        }
    }
    if (a.upd_mem) ring_copy(a, wid, total, tid);
    return;
  }

  // key-range splits: (max, sum) of this range and its normalised output O/sum
  // in bf16, merged by attn_combine_kernel
  if (!wave_on) return;
  const int64_t row = (int64_t)split * a.B * a.H * a.Lp + (int64_t)bh * a.Lp + i;
  uint16_t* po = static_cast<uint16_t*>(a.part_o) + row * DP;
  const float inv = l_sum > 0.0f ? 1.0f / l_sum : 0.0f;
#pragma unroll
  for (int e = 0; e < 2; ++e)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const bf16x2_t lo =
          __builtin_convertvector(floatx2_t{o[e][4 * g] * inv, o[e][4 * g + 1] * inv}, bf16x2_t);
      const bf16x2_t hi =
          __builtin_convertvector(floatx2_t{o[e][4 * g + 2] * inv, o[e][4 * g + 3] * inv}, bf16x2_t);
      *reinterpret_cast<u32x2*>(po + 32 * e + 8 * g + 4 * hf) =
          u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
    }
  if (hf == 0) {
    // a range with no visible key for this query reports max -inf, sum 0
    a.part_ml[row * 2 + 0] = m_ref == kNoMax ? kNegInf : m_ref;
    a.part_ml[row * 2 + 1] = l_sum;
  }
}

// Merge split partials in split order: with w_s = 2^(m_s-m*) l_s,
// out = sum_s w_s (O_s / l_s) / sum_s w_s.  8 threads per output row, 8
// columns (16 bytes) each; the partials of all splits are loaded before any
// is used.  The workgroups past the output rows copy the segment into the
// memory ring when the step asks for it.
template <int S>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a, int32_t out_blocks) {
  if ((int32_t)blockIdx.x >= out_blocks) {
    ring_copy(a, blockIdx.x - out_blocks, gridDim.x - out_blocks, threadIdx.x);
    return;
  }
  const int64_t row = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);   // (b, h, i), i < L
  const int c8 = threadIdx.x & 7;
  const int64_t rows = (int64_t)a.B * a.H * a.L;
  if (row >= rows) return;
  const int32_t i = row % a.L;
  const int64_t bh = row / a.L;
  const int32_t b = bh / a.H, head = bh % a.H;
  const int64_t prow = bh * a.Lp + i;
  const int64_t stride = (int64_t)a.B * a.H * a.Lp;
  const int ns = S > 0 ? S : a.n_split;
  constexpr int CAP = S > 0 ? S : 16;
  float ms[CAP], ls[CAP];
  u32x4 os[CAP];   // eight bf16 of O/sum
#pragma unroll
  for (int s = 0; s < CAP; ++s) {
    if (s < ns) {
      const int64_t pr = s * stride + prow;
      const float2 ml = reinterpret_cast<const float2*>(a.part_ml)[pr];
      ms[s] = ml.x;
      ls[s] = ml.y;
      os[s] = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.part_o) + pr * DP)[c8];
    }
  }
  float mx = kNegInf;
#pragma unroll
  for (int s = 0; s < CAP; ++s)
    if (s < ns) mx = fmaxf(mx, ms[s]);
  float num[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float den = 0.0f;
#pragma unroll
  for (int s = 0; s < CAP; ++s) {
    if (s < ns) {
      const float w = (ms[s] == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(ms[s] - mx) * ls[s];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        num[2 * e] += w * __uint_as_float(os[s][e] << 16);
        num[2 * e + 1] += w * __uint_as_float(os[s][e] & 0xffff0000u);
      }
      den += w;
    }
  }
  const float inv = 1.0f / den;
  if (a.lse && c8 == 0) a.lse[prow] = mx + log2f(den);
  uint16_t* out = static_cast<uint16_t*>(a.out) + ((int64_t)b * a.L + i) * a.H * a.dh +
                  (int64_t)head * a.dh;
  if (a.dh == DP) {
    typedef float floatx2_t __attribute__((ext_vector_type(2)));
    typedef bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    u32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      v[e] = __builtin_bit_cast(
          uint32_t, __builtin_convertvector(floatx2_t{num[2 * e] * inv, num[2 * e + 1] * inv}, bf16x2_t));
    *reinterpret_cast<u32x4*>(out + 8 * c8) = v;
  } else {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int d = 8 * c8 + r;
      if (d < a.dh) out[d] = f32_to_bf16_bits(num[r] * inv);
    }
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
  const int32_t out_blocks = (int32_t)((rows + 31) / 32);
  // the memory-ring copy (segment step) gets one workgroup per 256 words
  // (of 16 bytes: two rows of d_model 1024 in bf16)
  const int32_t copy_blocks =
      a.upd_mem ? (int32_t)(((int64_t)a.B * a.upd_rows * (a.upd_row_bytes / a.upd_unit) + 255) / 256)
                : 0;
  const dim3 grid(out_blocks + copy_blocks);
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (a.n_split) {
    case 2: hipLaunchKernelGGL(attn_combine_kernel<2>, grid, dim3(256), 0, st, a, out_blocks); break;
    case 3: hipLaunchKernelGGL(attn_combine_kernel<3>, grid, dim3(256), 0, st, a, out_blocks); break;
    case 4: hipLaunchKernelGGL(attn_combine_kernel<4>, grid, dim3(256), 0, st, a, out_blocks); break;
    default: hipLaunchKernelGGL(attn_combine_kernel<0>, grid, dim3(256), 0, st, a, out_blocks); break;
  }
  return static_cast<int>(hipGetLastError());
}

int launch_attn_f32(const AttnArgs& a, void* stream) {
  const size_t shmem = sizeof(float) * ((size_t)a.Np + 2 * (size_t)a.dh);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(attn_f32_kernel, dim3(a.B * a.H * a.L), dim3(256), shmem, st, a);
  return static_cast<int>(hipGetLastError());
}

}  // namespace txl
