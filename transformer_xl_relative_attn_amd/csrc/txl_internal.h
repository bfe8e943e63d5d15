// Internal declarations shared by the libtxl translation units (not part of the ABI).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "txl.h"

namespace txl {

// ---------------------------------------------------------------------------
// Operand row maps.  A GEMM operand is a set of K-contiguous rows; the kernel
// asks a RowSrc for the address of virtual row `v` (or NULL = a row of zeros).
//   ROW_PLAIN   v < rows ? p0 + v*ld : zero
//   ROW_HEADPAD v = head*dp + c;  c < dh ? p0 + (head*dh + c)*ld : zero
//               (weight rows of one head padded from dh to dp columns)
//   ROW_HTILDE  v = b*np + lead + r;  r < 0   -> zero
//                                     r < M   -> memory ring row (start + r) mod M of batch b
//                                     r < M+L -> segment row r - M of batch b
//                                     else    -> zero
//               (the extended context [memory ; segment] of Sec. 3.2, gathered in
//               place: never materialised)
// ---------------------------------------------------------------------------
enum RowMapKind : int32_t { ROW_PLAIN = 0, ROW_HEADPAD = 1, ROW_HTILDE = 2 };

struct RowSrc {
  int32_t kind;
  int32_t rows;    // PLAIN: valid rows
  int32_t dh, dp;  // HEADPAD
  int32_t np, M, L, start;  // HTILDE
  int32_t lead;             // HTILDE: zero rows before the memory rows
  uint32_t qmul;   // floor(v / dp) (HEADPAD) or floor(v / np) (HTILDE) as
  int32_t qshift;  //   (v * qmul) >> qshift, set up by the host
  int64_t ld;      // elements between consecutive source rows
  const void* p0;  // PLAIN/HEADPAD base, HTILDE memory base
  const void* p1;  // HTILDE segment base
};

#if defined(__HIPCC__)
#define TXL_HD __host__ __device__
#else
#define TXL_HD
#endif

// Output address of element (m, n) = rowoff(m) + coloff(n) + col2off(n), with
//   off(x) = (x / div) * s1 + (x % div) * s2.
// Covers row-major stores, head-split stores [b][head][r][c] and transposed
// head-split stores [b][head][c][r]; the second column term adds a per-batch
// jump (K/V ring tiles, whose batch stride is not a multiple of the tokens
// written).  The quotient uses a precomputed
// multiply-shift (exact for 0 <= x < 2^31); div == kLinearDiv means q = 0.
struct AxisMap {
  int32_t div;
  uint32_t mul;
  int32_t shift;
  int64_t s1, s2;
};

constexpr int32_t kLinearDiv = 0x7fffffff;

// Multiplier and shift with floor(x / d) == (x * mul) >> shift for all
// 0 <= x < 2^31 and 1 <= d < 2^31 (round-up reciprocal with
// l = ceil(log2 d) extra bits).  A divisor below 1 (no rows) gives quotient 0.
inline void div_magic(int32_t d, uint32_t* mul, int32_t* shift) {
  if (d < 1) {
    *mul = 0u;
    *shift = 0;
    return;
  }
  int l = 0;
  while ((1ull << l) < (uint64_t)d) ++l;
  *mul = (uint32_t)(((1ull << (31 + l)) / (uint64_t)d) + 1);
  *shift = 31 + l;
}

TXL_HD inline int32_t magic_quot(int32_t x, uint32_t mul, int32_t shift) {
  return (int32_t)(((uint64_t)(uint32_t)x * mul) >> shift);
}

inline AxisMap make_axis(int32_t div, int64_t s1, int64_t s2) {
  AxisMap a{div, 0u, 0, s1, s2};
  if (div == kLinearDiv) return a;
  div_magic(div, &a.mul, &a.shift);
  return a;
}

TXL_HD inline int32_t axis_quot(const AxisMap& a, int32_t x) { return magic_quot(x, a.mul, a.shift); }

TXL_HD inline int64_t axis_offset(const AxisMap& a, int32_t x) {
  const int32_t q = axis_quot(a, x);
  return (int64_t)q * a.s1 + (int64_t)(x - q * a.div) * a.s2;
}

// K/V ring placement.  A ring of C slots (C a multiple of 32) holds K as
// [B][H][C][DP] and, right after it, V^T in 32-slot tiles [B][C/32][H][DP][32].
// The GEMM problems that project n tokens per batch (token index b*n + r) to
// slots slot0 + r (n, slot0 multiples of 32, slot0 + n <= C) store through
// these maps; offsets are in elements, relative to the start of K (k_*) and of
// V^T (v_*).  K rows are tokens and columns head*DP + d; V^T rows are
// head*DP + d and columns tokens.
struct RingMaps {
  int64_t k_base, v_base;
  AxisMap k_row, k_col, v_row, v_col, v_col2;
};

inline RingMaps ring_maps(int32_t H, int32_t DP, int32_t C, int32_t n, int32_t slot0) {
  const int64_t T = (int64_t)H * DP * 32;   // one 32-slot V^T tile of all heads
  RingMaps m;
  m.k_base = (int64_t)slot0 * DP;
  m.k_row = make_axis(n, (int64_t)H * C * DP, DP);
  m.k_col = make_axis(DP, (int64_t)C * DP, 1);
  // token b*n + r -> tile b*C/32 + (slot0 + r)/32, lane (slot0 + r) % 32:
  // (token/32)*T + token%32 plus a jump of (C - n)/32 tiles per batch
  m.v_base = (int64_t)(slot0 / 32) * T;
  m.v_row = make_axis(kLinearDiv, 0, 32);
  m.v_col = make_axis(32, T, 1);
  m.v_col2 = make_axis(n, (int64_t)(C / 32 - n / 32) * T, 0);
  return m;
}

// The segment's L rows go to slots (base + p) mod C, base = (start + Mk) mod C:
// n1 rows from `base`, then (if they wrap) L - n1 rows from slot 0.
inline int32_t ring_first_piece(int32_t start, int32_t Mk, int32_t L, int32_t C) {
  const int32_t base = (start + Mk) % C;
  return L < C - base ? L : C - base;
}

enum EpiFlags : int32_t { EPI_RELU = 1, EPI_RESID = 2 };

struct OutDst {
  void* p;
  int32_t dtype;         // TXL_F32 / TXL_BF16
  int32_t flags;         // EpiFlags
  int32_t vec_ok;        // groups of 4 columns (n % 4 == 0) are contiguous and
                         // 16-byte (f32) / 8-byte (bf16) aligned
  int32_t vec8_ok;       // bf16: groups of 8 columns are contiguous and 16-byte
                         // aligned, and the row map has div >= 4
  int32_t m_valid, n_valid;  // store only m < m_valid, n < n_valid
  AxisMap row, col, col2;
  const float* resid;    // EPI_RESID: out += resid[rowoff + coloff] (same map)
};

struct GemmProblem {
  // C[m][n] = sum_k A(m,k) * B(n,k),  m < M, n < N
  int32_t M, N, K;
  int32_t tiles_m, tiles_n;
  int32_t tile_begin;    // first tile id of this problem in a grouped launch
  RowSrc a, b;
  OutDst out;
};

// Tile counts of a problem for square tiles of `tile` rows.
inline void set_tiling(GemmProblem& p, int32_t tile) {
  p.tiles_m = (p.M + tile - 1) / tile;
  p.tiles_n = (p.N + tile - 1) / tile;
}

constexpr int kMaxGroup = 8;

struct GemmGroup {
  int32_t count;
  int32_t total_tiles;
  // 1 + index i of an interleaved pair (0 = none): problems i and i+1 share
  // an operand, as A of i and B of i+1 (the keys and the values^T both read
  // the rows of h~), with p[i].tiles_n == p[i+1].tiles_m and p[i].tiles_m ==
  // p[i+1].tiles_n.  Their tiles are dealt panel by panel: the tiles_n tiles
  // of row panel x of problem i, then the tiles_m tiles of column panel x of
  // problem i+1, so that tiles reading the same rows are consecutive and run
  // on one XCD.
  int32_t pair1;
  GemmProblem p[kMaxGroup];
};

// Attention kernel arguments (device workspace layouts, see api.cpp).
// bf16 path: the position-key table in the workspace carries kRkPad rows of
// padding before and after each head's Pp rows, so that the attention kernel
// can fetch 32-row chunks without clamping (padding rows only ever meet
// masked query/key pairs, so their contents do not matter).
constexpr int32_t kRkPad = 192;

struct AttnArgs {
  int32_t B, H, L, M, dh;
  int32_t Lp, Np, Pp;      // padded query rows, key rows, position rows
  int32_t n_split;         // key-range splits per query group (>= 1)
  int32_t k_lo;            // keys j < k_lo are masked (ghost keys of the K/V ring)
  int32_t kv_tile0;        // key block t is stored at 32-key tile (t + kv_tile0) mod (Np / 32)
  float c_scale;           // scale * log2(e) (bf16 path) or scale (fp32 path)
  const float* q;          // [B][H][Lp][DP] fp32
  const void* k;           // bf16 [B][H][Np][DP]   | f32 [B][H][Np][dh]
  const void* vt;          // bf16 [B][Np/32][H][DP][32] (transposed 32-key tiles) | f32 [B][H][Np][dh]
                           // (K/V ring: Np = ring slots, block t at tile (t + kv_tile0) mod (Np/32))
  const void* rk;          // bf16 [H][kRkPad + Pp + kRkPad][DP] | f32 [H][Pp][dh]
  const void* u;           // [H][dh] in the call dtype
  const void* v;
  void* out;               // [B][L][H][dh] in the call dtype
  void* part_o;            // split partials: bf16 O/sum [n_split][B*H*Lp][DP]
  float* part_ml;          // [n_split][B*H*Lp][2] (running max, sum)
  float* lse;              // optional [B*H*Lp]: log2 of each row's softmax denominator,
                           // in the base-2 units of the bf16 kernel (rows i < L)
  int32_t dtype;
  // optional fused ring update (bf16 kernel): copy min(L, M) rows of upd_src
  // [B][L][*] into upd_mem [B][M][*] in words of upd_unit bytes (16 or 4; a
  // divisor of row_bytes and of both base addresses' alignment); NULL = none
  const void* upd_src;
  void* upd_mem;
  int32_t upd_start, upd_rows;
  int64_t upd_row_bytes;
  int32_t upd_unit;
};

// Compute units of the current device (cached per device id).
int32_t device_cu_count();

// Record `msg` as the calling thread's last error and return st.
txl_status_t set_error(txl_status_t st, const char* msg);

// While set on the calling thread, the timing diagnostics record no events.
void suppress_timing(bool on);

// Backward of the bf16 attention core (attn_bwd.hip).  Gradients are taken
// with respect to the score s = scale * A (dS), then scaled by `scale`.
struct BwdArgs {
  int32_t B, H, L, M, dh, Lp, Np, Pp;
  float c_scale;           // scale * log2(e), the forward kernel's score units
  float scale;
  const float* q;          // fp32 [B][H][Lp][DP]
  const void* k;           // bf16 K [B][H][Np][DP]
  const void* vt;          // bf16 val^T in 32-key tiles [B][Np/32][H][DP][32] (the forward's V^T)
  const void* rk;          // bf16 [H][kRkPad + Pp + kRkPad][DP]
  const void* rkt;         // bf16 Rk^T [H][DP][rkt_ld], distance delta at column rkt_pad + delta
  int32_t rkt_ld, rkt_pad;
  const void* u;           // bf16 [H][dh]
  const void* v;
  const void* dop;         // bf16 dLoss/dout [B][H][Lp][DP] (zero padded)
  const float* lse;        // [B*H*Lp] log2 softmax denominators (base-2 score units)
  const float* dsum;       // [B*H*Lp] D_i = dout_i . out_i
  void* pt;                // bf16 P^T  [B][H], fragment tiles: keys 32jb.., queries 16kb..
                           //   at ((jb * Lp/16 + kb) * 64 + lane) * 8, lane = key % 32 +
                           //   32 ((query % 16) / 8), eight consecutive queries per lane
  void* dst;               // bf16 dS^T [B][H], the same tiles
  void* dspt;              // bf16 dS'^T per head: row delta, column b*Lp + i holds dS[i][M+i-delta],
                           //   in fragment tiles of 32 rows from delta dsp_lo and 16 columns
                           //   ([dsp_tiles][B*Lp/16] tiles per head, tiles no wave flushed unwritten)
  int32_t dsp_lo, dsp_tiles;
  float* dq;               // fp32 [B][L][H][dh]
  float* duv_part;         // fp32 [2][B][H][Lp/32][DP]: per 32 queries, the sums of the
                           //   k-part and the Rk-part of dq (-> du, dv)
};

// Batched "A times B^T" with 64 output columns, fp32 result:
//   C[bi][m][n] = alpha * sum_k A[bi][m][k] B[bi][n][k],  n < n_valid <= 64,
// A and B bf16 with rows K-contiguous (K a multiple of 16).  A(m, k) counts
// only where min(K, klim) > k >= m - moff (the other entries are never read
// as data: they may hold anything).  Batch bi starts at a_batch(bi), b_batch(bi),
// c_batch(bi) elements; C2 (optional) receives the same values at
// c2_batch(bi) + m*c2_m + n*c2_n.
struct BmmArgs {
  const void* A;
  const void* Bm;
  int64_t lda, ldb;
  AxisMap a_batch, b_batch;
  int32_t M, K, batch, n_valid, m_valid;
  int32_t moff, klim;
  float alpha;
  float* C;
  int64_t ldc;
  AxisMap c_batch;
  float* C2;
  int64_t c2_m, c2_n;
  AxisMap c2_batch;
};

struct BwdPrepArgs {
  int32_t B, H, L, dh, Lp;
  const void* dout;        // bf16 [B][L][H][dh]
  const void* out;         // bf16 [B][L][H][dh] (forward output)
  const float* q;          // fp32 [B][H][Lp][DP]
  const void* u;
  const void* v;
  void* dop;               // bf16 [B][H][Lp][DP]
  void* dot;               // bf16 [B][H][DP][Lp]   dout^T
  void* qut;               // bf16 [B][H][DP][Lp]   (q+u)^T
  void* qvt;               // bf16 [H][DP][B*Lp]    (q+v)^T
  float* dsum;             // [B*H*Lp]
};

// Launch wrappers (return a hipError_t as int).
int launch_gemm_bf16(const GemmGroup& g, void* stream);
int launch_gemm_f32(const GemmGroup& g, void* stream);
int launch_attn_bf16(const AttnArgs& a, void* stream);
int launch_attn_combine(const AttnArgs& a, void* stream);
int launch_attn_f32(const AttnArgs& a, void* stream);
int launch_sinusoid(void* R, int32_t n_pos, int32_t d_pos, int32_t dtype, void* stream);
int launch_mfma_probe(const void* operands, int32_t n_wg, int32_t iters, uint64_t* clocks,
                      void* stream);
int launch_mem_update(void* mem, int32_t start, const void* h, int32_t B, int32_t M, int32_t L,
                      int32_t d, int32_t dtype, void* stream);
int launch_pack_rows(void* dst, int64_t ld_dst, const void* src, int64_t ld_src, int64_t rows,
                     int32_t cols, int32_t dtype, void* stream);

// Several bf16 row packs in one launch: job j copies rows x cols elements from
// src (row pitch ld_src) into dst (row pitch ld_dst), zero-filling columns
// cols .. ld_dst-1.
constexpr int kMaxPackJobs = 8;
struct PackJob {
  void* dst;
  const void* src;
  int64_t ld_dst, ld_src, rows;
  int32_t cols;
};
struct PackGroup {
  int32_t n;
  int64_t row_begin[kMaxPackJobs + 1];   // first global row of each job; [n] = total rows
  PackJob job[kMaxPackJobs];
  int32_t words4;        // every row start and length is a multiple of 4 bytes
  // optional memory-ring update carried by job ring_job (the pack of the
  // ring [B][M][cols] itself): after a thread has read its columns of ring
  // row (b, slot) it overwrites them with segment row t of ring_h [B][L][cols],
  // where slot = (start + t) mod M for t < L (L < M), or t = L - M + slot (L >= M)
  int32_t ring_job;      // -1 = none
  const void* ring_h;
  int32_t ring_L, ring_M, ring_start;
};
int launch_pack_group(const PackGroup& g, void* stream);
int launch_layernorm(const float* resid, const float* parts, int32_t n_parts, int64_t part_stride,
                     float* y_f32, void* y_lo, int32_t rows, int32_t d, int32_t lo_dtype, float eps,
                     void* stream);
int launch_cast_f32(const void* src, float* dst, int64_t n, int32_t dtype, void* stream);
int launch_attn_bwd_q(const BwdArgs& a, void* stream);
// n <= 3 products in one launch.  kind[z]: 0 = A in rows; 1 = A in the query
// kernel's key-row fragment tiles (P^T, dS^T); 2 = A in its distance-row
// fragment tiles (dS'^T).  Output row of A row m: m + row_off[z].  kper[z]
// (kind 2 only; NULL = all 0): K covers K / kper consecutive batch rows of
// kper (a multiple of 32) padded queries each, klim applying within each.
int launch_bmm64(const BmmArgs* a, int n, const int32_t* kind, const int32_t* row_off,
                 const int32_t* kper, void* stream);
// The backward's small steps before the query kernel, one grid: the prep
// (BwdPrepArgs), the Rk^T table and, for dW_kR, the bf16 transpose of R.
struct BwdPreArgs {
  BwdPrepArgs prep;
  const void* rk_ws;       // bf16 [H][pad_ws + Pp + pad_ws][64] (the attention's table)
  void* rkt;               // bf16 [H][64][rkt_ld]: distance delta at column pad_t + delta,
                           // zeros elsewhere (rkt_ld a multiple of 8)
  int32_t Pp, pad_ws, rkt_ld, pad_t;
  const void* r;           // optional [P][d_pos] in r_dtype -> rt bf16 [d_pos][r_ld],
  void* rt;                // zero columns P .. r_ld-1 (r_ld a multiple of 16)
  int32_t P, d_pos, r_dtype, r_ld;
};
// ... and after the key-side products, one grid: dRk = the batch rows' partials
// summed in row order (with, for dW_kR, its bf16 transpose), and du, dv.
struct BwdPostArgs {
  const float* drk_part;   // [drk_rows][P][HD]
  float* d_rk;             // [P][HD]
  void* drkt;              // optional bf16 [HD][r_ld], zero columns P .. r_ld-1
  int32_t drk_rows, B, P, HD, r_ld;
  const float* duv_part;   // [2][B][H][nchunk][64] (per 32-query chunk)
  float* d_u;              // [H][dh]
  float* d_v;
  int32_t H, nchunk, dh;
};
int launch_bwd_pre(const BwdPreArgs& a, void* stream);
int launch_bwd_post(const BwdPostArgs& a, void* stream);
int launch_sum_rows(const float* src, int32_t n_rows, int64_t row_len, float* dst, void* stream);
int launch_repack_rk(const void* rk_pub, void* rk_ws, int32_t P, int32_t Pp, int32_t pad, int32_t H,
                     int32_t dh, int32_t dp, int32_t dtype, void* stream);

}  // namespace txl
