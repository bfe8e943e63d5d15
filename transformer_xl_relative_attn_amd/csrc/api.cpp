// libtxl C-ABI: argument validation, workspace planning and kernel dispatch.
// Every check runs before anything is enqueued; on an error nothing is launched
// and in/out arguments keep their values.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "txl_internal.h"

namespace txl {
namespace {

thread_local std::string g_last_error;

txl_status_t fail(txl_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

txl_status_t hip_status(int err, const char* where) {
  if (err == 0) return TXL_OK;
  return fail(TXL_ERR_HIP, "%s: %s", where, hipGetErrorString(static_cast<hipError_t>(err)));
}

#define TXL_TRY(expr)                                  \
  do {                                                 \
    txl_status_t _st = (expr);                         \
    if (_st != TXL_OK) return _st;                     \
  } while (0)

#define TXL_HIP(expr, where)                           \
  do {                                                 \
    int _e = (expr);                                   \
    if (_e != 0) return hip_status(_e, where);         \
  } while (0)

constexpr int64_t kMaxDim = 1 << 20;
constexpr int kBf16Dp = 64;   // padded head width of the bf16 path
constexpr int kBf16Dmax = 64;

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
inline int esize(int dtype) { return dtype == TXL_F32 ? 4 : 2; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

bool debug_sync() {
  static const bool on = [] {
    const char* e = getenv("TXL_DEBUG_SYNC");
    return e && *e && *e != '0';
  }();
  return on;
}

txl_status_t after_launch(int err, const char* what, void* stream) {
  if (err) return hip_status(err, what);
  if (debug_sync()) {
    int e = static_cast<int>(hipStreamSynchronize(static_cast<hipStream_t>(stream)));
    if (e) return hip_status(e, what);
  }
  return TXL_OK;
}

// ------------------------------------------------------------ kernel timing
// Optional diagnostics: when enabled, every kernel launch is bracketed by two
// HIP events (created without the system-scope fence) recorded on the launch
// stream; txl_timing_read() waits for them.
enum Kind : int {
  K_PROJ_GEMM, K_ATTN, K_ATTN_COMBINE, K_MEM_UPDATE, K_REL_PROJ, K_WO_GEMM, K_FFN1_GEMM,
  K_FFN2_GEMM, K_LAYERNORM, K_PACK, K_SINUSOID, K_CAST, K_REPACK_RK, K_BWD_Q, K_BWD_BMM,
  K_BWD_AUX, K_NKINDS
};
const char* const kKindNames[K_NKINDS] = {
    "proj_gemm", "rel_attn", "attn_combine", "mem_update", "rel_proj_gemm", "wo_gemm",
    "ffn1_gemm", "ffn2_gemm", "layernorm", "pack_rows", "sinusoid", "cast_f32", "repack_rk",
    "attn_bwd_q", "bwd_bmm64", "bwd_aux"};

struct TimingState {
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> pool;
  struct Rec { int kind; hipEvent_t a, b; };
  std::vector<Rec> pending;
  double ms[K_NKINDS] = {};
  int64_t count[K_NKINDS] = {};
};
TimingState& timing() {
  static TimingState t;
  return t;
}

hipEvent_t take_event(TimingState& t) {
  if (!t.pool.empty()) {
    hipEvent_t e = t.pool.back();
    t.pool.pop_back();
    return e;
  }
  // timing-only events: no system-scope fence (cache writeback) when they
  // are recorded, so the bracket measures the kernel rather than the fence
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

// Set while a call must not create events (the no-allocation entry point).
thread_local bool g_timing_suppressed = false;

// Run a launch function, bracketed by timing events when timing is on.
template <class F>
int timed(int kind, void* stream, F&& launch) {
  TimingState& t = timing();
  hipEvent_t a = nullptr, b = nullptr;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (!g_timing_suppressed) {
    std::lock_guard<std::mutex> lk(t.mu);
    if (t.on) {
      a = take_event(t);
      b = take_event(t);
    }
  }
  if (a && b) (void)hipEventRecord(a, st);
  int err = launch();
  if (a && b) {
    (void)hipEventRecord(b, st);
    std::lock_guard<std::mutex> lk(t.mu);
    t.pending.push_back({kind, a, b});
  }
  return err;
}

// ---------------------------------------------------------------- planning
struct Region {
  size_t off = 0, bytes = 0;
};

// What a plan is for: the plain layer (K, V^T of [memory ; segment] in the
// workspace), a step over a carried K/V ring (only the segment's K, V^T are
// projected, into the ring), or the ring's initial projection of a memory.
enum PlanKind { PLAN_STD = 0, PLAN_RING = 1, PLAN_RING_INIT = 2 };

struct AttnPlan {
  int kind;
  int B, L, M, d, H, dh, dpos, dtype;
  float scale;
  int DP, Lp, Np, Pp, P;
  int Mk, G;               // keys before the segment as the kernel sees them
                           // (ring: M rounded up to 32, G = Mk - M ghost keys)
  int rk_pad;              // padding rows before / after each head's Rk rows
  int n_split, nqg;
  bool pack_d, pack_pos;   // bf16 operands repacked to a K multiple of 64
  int Kd, Kpos;            // reduction lengths seen by the GEMMs
  Region q, k, v, rk, po, pml, ph, pmem, pwq, pwk, pwv, pwr, pr;
  size_t total;
};

txl_status_t check_shape(const txl_attn_shape_t* s) {
  if (!s) return fail(TXL_ERR_NULL_ARG, "shape is NULL");
  if (s->dtype != TXL_F32 && s->dtype != TXL_BF16)
    return fail(TXL_ERR_BAD_DTYPE, "dtype %d is not TXL_F32 or TXL_BF16", s->dtype);
  if (s->batch < 1 || s->seg_len < 1 || s->mem_len < 0 || s->d_model < 1 || s->n_heads < 1 ||
      s->d_head < 1 || s->d_pos < 1)
    return fail(TXL_ERR_BAD_SHAPE,
                "sizes out of range (batch=%d seg_len=%d mem_len=%d d_model=%d n_heads=%d "
                "d_head=%d d_pos=%d)",
                s->batch, s->seg_len, s->mem_len, s->d_model, s->n_heads, s->d_head, s->d_pos);
  if (s->batch > kMaxDim || s->seg_len > kMaxDim || s->mem_len > kMaxDim ||
      s->d_model > kMaxDim || s->n_heads > 4096 || s->d_head > 4096 || s->d_pos > kMaxDim)
    return fail(TXL_ERR_BAD_SHAPE, "a size exceeds the supported range");
  if (std::isnan(s->scale) || std::isinf(s->scale))
    return fail(TXL_ERR_BAD_SHAPE, "scale is not finite");
  if ((int64_t)s->mem_len + s->seg_len > INT32_MAX / 2)
    return fail(TXL_ERR_BAD_SHAPE, "mem_len + seg_len too large");
  if (s->dtype == TXL_BF16 && s->d_head > kBf16Dmax)
    return fail(TXL_ERR_UNSUPPORTED, "bf16 path supports d_head <= %d (got %d)", kBf16Dmax,
                s->d_head);
  if (s->dtype == TXL_F32) {
    // fp32 kernel keeps one query's scores in LDS
    const int64_t lds = 4 * ((int64_t)s->mem_len + s->seg_len + 2 * s->d_head);
    if (lds > 60 * 1024)
      return fail(TXL_ERR_UNSUPPORTED, "fp32 path supports mem_len + seg_len <= ~15000");
  }
  return TXL_OK;
}

// The K/V ring path: bf16, and segments of whole 32-key tiles.
txl_status_t check_ring_shape(const txl_attn_shape_t* s) {
  TXL_TRY(check_shape(s));
  if (s->dtype != TXL_BF16) return fail(TXL_ERR_UNSUPPORTED, "the K/V ring is bf16 only");
  if (s->seg_len % 32 != 0)
    return fail(TXL_ERR_UNSUPPORTED, "the K/V ring needs seg_len %% 32 == 0 (got %d)",
                s->seg_len);
  return TXL_OK;
}

AttnPlan make_plan(const txl_attn_shape_t* s, bool compute_rk, int kind = PLAN_STD) {
  AttnPlan p{};
  p.kind = kind;
  p.B = s->batch;
  p.L = s->seg_len;
  p.M = s->mem_len;
  p.d = s->d_model;
  p.H = s->n_heads;
  p.dh = s->d_head;
  p.dpos = s->d_pos;
  p.dtype = s->dtype;
  p.scale = s->scale > 0 ? s->scale : 1.0f / std::sqrt((float)s->d_head);
  p.P = p.M + p.L;
  const bool bf = p.dtype == TXL_BF16;
  p.DP = bf ? kBf16Dp : p.dh;
  p.Lp = bf ? (int)round_up(p.L, 32) : p.L;
  p.Np = bf ? (int)round_up(p.P, 32) : p.P;
  p.Pp = p.Np;
  p.Mk = p.M;
  p.G = 0;
  if (kind != PLAN_STD) {
    // ring of Mk + L slots: ghost keys, memory, segment; 32-key tiles
    p.Mk = (int)round_up(p.M, 32);
    p.G = p.Mk - p.M;
    p.Np = p.Mk + p.L;
  }
  p.rk_pad = bf ? kRkPad : 0;
  p.nqg = (p.L + 127) / 128;
  p.n_split = 1;
  if (bf) {
    // Key-range splits fill the workgroup slots (two per compute unit) in one
    // round: S = floor(slots / work items), so a split never adds a partial
    // round (measured on 256 CUs: d_head 41, L = M = 150, 320 items: 1 split
    // 23 us, 2 splits 25 us plus the combine).  Every split keeps >= 4 key
    // blocks.
    const int64_t wgs = (int64_t)p.B * p.H * p.nqg;
    const int64_t slots = 2 * (int64_t)device_cu_count();
    const int nb_min = (p.Mk + std::min(p.L, 128) + 31) / 32;
    int want = (int)std::min<int64_t>(slots / wgs, 16);
    want = std::min(want, std::max(1, nb_min / 4));
    p.n_split = std::max(1, want);
  }
  p.pack_d = bf && (p.d % 64 != 0);
  p.pack_pos = bf && compute_rk && (p.dpos % 64 != 0);
  p.Kd = p.pack_d ? (int)round_up(p.d, 64) : p.d;
  p.Kpos = p.pack_pos ? (int)round_up(p.dpos, 64) : p.dpos;
  const size_t es = esize(p.dtype);
  size_t off = 0;
  auto take = [&](Region& r, size_t bytes) {
    r.off = off;
    r.bytes = bytes;
    off = align256(off + bytes);
  };
  const size_t BH = (size_t)p.B * p.H;
  if (kind != PLAN_RING_INIT) take(p.q, BH * p.Lp * p.DP * 4);
  if (kind == PLAN_STD) {
    take(p.k, BH * p.Np * p.DP * es);
    take(p.v, BH * p.Np * p.DP * es);
  }
  if (kind != PLAN_RING_INIT) take(p.rk, (size_t)p.H * (p.Pp + 2 * p.rk_pad) * p.DP * es);
  if (kind != PLAN_RING_INIT && p.n_split > 1) {
    take(p.po, (size_t)p.n_split * BH * p.Lp * p.DP * 2);
    take(p.pml, (size_t)p.n_split * BH * p.Lp * 2 * 4);
  }
  const size_t Hd = (size_t)p.H * p.dh;
  if (p.pack_d) {
    if (kind != PLAN_RING_INIT) take(p.ph, (size_t)p.B * p.L * p.Kd * 2);
    if (kind != PLAN_RING) take(p.pmem, (size_t)p.B * p.M * p.Kd * 2);
    if (kind != PLAN_RING_INIT) take(p.pwq, Hd * p.Kd * 2);
    take(p.pwk, Hd * p.Kd * 2);
    take(p.pwv, Hd * p.Kd * 2);
  }
  if (p.pack_pos && kind != PLAN_RING_INIT) {
    take(p.pwr, Hd * p.Kpos * 2);
    take(p.pr, (size_t)p.P * p.Kpos * 2);
  }
  p.total = off;
  return p;
}

// Output maps ------------------------------------------------------------
AxisMap axis(int32_t div, int64_t s1, int64_t s2) { return make_axis(div, s1, s2); }
AxisMap axis_linear(int64_t s) { return make_axis(kLinearDiv, 0, s); }

RowSrc src_plain(const void* p, int64_t ld, int32_t rows) {
  RowSrc r{};
  r.kind = ROW_PLAIN;
  r.p0 = p;
  r.ld = ld;
  r.rows = rows;
  return r;
}
RowSrc src_headpad(const void* w, int64_t ld, int32_t dh, int32_t dp) {
  RowSrc r{};
  r.kind = ROW_HEADPAD;
  r.p0 = w;
  r.ld = ld;
  r.dh = dh;
  r.dp = dp;
  div_magic(dp, &r.qmul, &r.qshift);
  return r;
}
RowSrc src_htilde(const void* mem, const void* h, int64_t ld, int32_t np, int32_t M, int32_t L,
                  int32_t start, int32_t lead = 0) {
  RowSrc r{};
  r.lead = lead;
  r.kind = ROW_HTILDE;
  r.p0 = mem;
  r.p1 = h;
  r.ld = ld;
  r.np = np;
  r.M = M;
  r.L = L;
  r.start = start;
  div_magic(np, &r.qmul, &r.qshift);
  return r;
}

void add_problem(GemmGroup& g, int32_t M, int32_t N, int32_t K, const RowSrc& a, const RowSrc& b,
                 const OutDst& o, int tile) {
  GemmProblem& p = g.p[g.count++];
  p.M = M;
  p.N = N;
  p.K = K;
  set_tiling(p, tile);
  p.tile_begin = g.total_tiles;
  p.a = a;
  p.b = b;
  p.out = o;
  g.total_tiles += p.tiles_m * p.tiles_n;
}

const AxisMap kNoAxis = make_axis(kLinearDiv, 0, 0);

OutDst out_map(void* ptr, int dtype, int32_t mv, int32_t nv, AxisMap row, AxisMap col,
               int flags = 0, const float* resid = nullptr, AxisMap col2 = kNoAxis) {
  OutDst o{};
  o.p = ptr;
  o.dtype = dtype;
  o.flags = flags;
  o.m_valid = mv;
  o.n_valid = nv;
  o.row = row;
  o.col = col;
  o.col2 = col2;
  o.resid = resid;
  // vectorised epilogue: 4 consecutive columns (n % 4 == 0) map to 4
  // consecutive, aligned elements for every row
  // (the second column term must be constant over those groups)
  const auto col2_ok = [&](int g) {
    return col2.s2 == 0 && col2.s1 % g == 0 && (col2.div == kLinearDiv || col2.div % g == 0);
  };
  const bool col_ok = col.s2 == 1 && col.s1 % 4 == 0 &&
                      (col.div == kLinearDiv || col.div % 4 == 0) && col2_ok(4);
  const bool row_ok = row.s1 % 4 == 0 && row.s2 % 4 == 0;
  const bool ptr_ok = (reinterpret_cast<uintptr_t>(ptr) % 16) == 0 &&
                      (!resid || (reinterpret_cast<uintptr_t>(resid) % 16) == 0);
  o.vec_ok = col_ok && row_ok && ptr_ok && nv % 4 == 0;
  // staged bf16 epilogue: 8 consecutive columns per 16-byte store, and rows
  // advanced up to 8 at a time with at most one wrap of the row axis per step
  const bool col8 = col.s2 == 1 && col.s1 % 8 == 0 &&
                    (col.div == kLinearDiv || col.div % 8 == 0) && col2_ok(8);
  const bool row8 = row.s1 % 8 == 0 && row.s2 % 8 == 0 && row.div >= 8;
  o.vec8_ok = dtype == TXL_BF16 && col8 && row8 && ptr_ok && nv % 8 == 0;
  return o;
}

int launch_gemm(const GemmGroup& g, int dtype, void* stream) {
  return dtype == TXL_BF16 ? launch_gemm_bf16(g, stream) : launch_gemm_f32(g, stream);
}
int gemm_tile(int dtype) { return dtype == TXL_BF16 ? 256 : 64; }

// ----------------------------------------------------------- rel_attn core
struct AttnPtrs {
  const void *h, *mem, *W_q, *W_kE, *W_kR, *W_v, *u, *v, *R, *Rk;
  int32_t mem_start;
  void* out;
};

txl_status_t check_attn_ptrs(const txl_attn_shape_t* s, const AttnPtrs& a, bool need_ws,
                             const void* ws, bool need_mem = true) {
  if (!a.h || !a.W_q || !a.W_kE || !a.W_v || !a.u || !a.v || !a.out)
    return fail(TXL_ERR_NULL_ARG, "h, W_q, W_kE, W_v, u, v and out are required");
  if (need_mem && s->mem_len > 0 && !a.mem)
    return fail(TXL_ERR_NULL_ARG, "mem is NULL but mem_len > 0");
  if (!a.Rk && (!a.W_kR || !a.R))
    return fail(TXL_ERR_NULL_ARG, "either Rk or both W_kR and R are required");
  if (need_ws && !ws) return fail(TXL_ERR_NULL_ARG, "workspace is NULL");
  if (need_mem &&
      (s->mem_len > 0 ? (a.mem_start < 0 || a.mem_start >= s->mem_len) : a.mem_start != 0))
    return fail(TXL_ERR_BAD_SHAPE, "mem_start %d outside [0, mem_len=%d)", a.mem_start,
                s->mem_len);
  if (s->dtype == TXL_BF16) {
    const void* ptrs[] = {a.h, a.mem, a.W_q, a.W_kE, a.W_kR, a.W_v, a.R, a.Rk, a.out};
    for (const void* q : ptrs)
      if (q && !aligned16(q))
        return fail(TXL_ERR_UNSUPPORTED, "bf16 path needs 16-byte aligned tensor pointers");
  }
  return TXL_OK;
}

// Operands as the GEMMs read them: the caller's tensors, or bf16 copies whose
// rows are padded to a multiple of 64 elements.
struct Operands {
  const void *h, *mem, *Wq, *WkE, *Wv, *WkR, *R;
  int64_t ld_d, ld_pos;
};

// If `ring_upd` is set (and is the memory being packed) the pack of the
// memory also applies the ring update with h, and *ring_upd is cleared.
txl_status_t pack_operands(const AttnPlan& p, const AttnPtrs& a, char* ws, void* stream,
                           Operands& o, void** ring_upd = nullptr) {
  const int dt = p.dtype;
  const int32_t Hd = p.H * p.dh;
  o = Operands{a.h, a.mem, a.W_q, a.W_kE, a.W_v, a.W_kR, a.R, p.d, p.dpos};
  const bool seg = p.kind != PLAN_RING_INIT;    // the segment h and W_q are read
  const bool mem = p.kind != PLAN_RING && p.M > 0;
  // every repack of the call goes into one grouped launch
  PackGroup pg{};
  pg.ring_job = -1;
  auto pack = [&](const Region& r, const void* src, int64_t rows, int64_t ld_dst, int64_t cols,
                  const void*& dst) {
    PackJob& J = pg.job[pg.n];
    J.dst = ws + r.off;
    J.src = src;
    J.ld_dst = ld_dst;
    J.ld_src = cols;
    J.rows = rows;
    J.cols = (int32_t)cols;
    pg.row_begin[pg.n + 1] = pg.row_begin[pg.n] + rows;
    ++pg.n;
    dst = ws + r.off;
  };
  (void)dt;
  if (p.pack_d) {
    if (seg) pack(p.ph, a.h, (int64_t)p.B * p.L, p.Kd, p.d, o.h);
    if (mem) {
      if (ring_upd && *ring_upd == a.mem) {
        // the GEMMs read the packed copy, so the ring itself may take the
        // segment now (the attention reads only the projections)
        pg.ring_job = pg.n;
        pg.ring_h = a.h;
        pg.ring_L = p.L;
        pg.ring_M = p.M;
        pg.ring_start = a.mem_start;
        *ring_upd = nullptr;
      }
      pack(p.pmem, a.mem, (int64_t)p.B * p.M, p.Kd, p.d, o.mem);
    }
    if (seg) pack(p.pwq, a.W_q, Hd, p.Kd, p.d, o.Wq);
    pack(p.pwk, a.W_kE, Hd, p.Kd, p.d, o.WkE);
    pack(p.pwv, a.W_v, Hd, p.Kd, p.d, o.Wv);
    o.ld_d = p.Kd;
  }
  if (seg && !a.Rk && p.pack_pos) {
    pack(p.pwr, a.W_kR, Hd, p.Kpos, p.dpos, o.WkR);
    pack(p.pr, a.R, p.P, p.Kpos, p.dpos, o.R);
    o.ld_pos = p.Kpos;
  }
  if (pg.n > 0) {
    bool w4 = true;
    for (int i = 0; i < pg.n; ++i) {
      const PackJob& J = pg.job[i];
      w4 = w4 && J.cols % 2 == 0 && J.ld_src % 2 == 0 && J.ld_dst % 2 == 0 &&
           (reinterpret_cast<uintptr_t>(J.src) & 3) == 0 && (reinterpret_cast<uintptr_t>(J.dst) & 3) == 0;
    }
    if (pg.ring_job >= 0) w4 = w4 && (reinterpret_cast<uintptr_t>(pg.ring_h) & 3) == 0;
    pg.words4 = w4 ? 1 : 0;
    TXL_HIP(timed(K_PACK, stream, [&] { return launch_pack_group(pg, stream); }), "operand packs");
  }
  return TXL_OK;
}

// q = h W_q^T -> fp32 [B][H][Lp][DP], rows i < L only (the attention kernels
// read the padding rows L .. Lp-1 as zeros without loading them)
void add_q_problem(GemmGroup& g, const AttnPlan& p, const Operands& o, char* ws) {
  const int64_t DP = p.DP;
  add_problem(g, p.B * p.L, p.H * p.DP, p.Kd,
              src_htilde(nullptr, o.h, o.ld_d, p.L, 0, p.L, 0), src_headpad(o.Wq, o.ld_d, p.dh, p.DP),
              out_map(ws + p.q.off, TXL_F32, p.B * p.L, p.H * p.DP,
                      axis(p.L, (int64_t)p.H * p.Lp * DP, DP), axis(p.DP, (int64_t)p.Lp * DP, 1)),
              gemm_tile(p.dtype));
}

// Position keys: computed into the workspace table [H][pad + Pp + pad][DP] as
// one more problem of the group (rows of the padding not written), or the
// caller's Rk repacked into it.
txl_status_t add_rk(GemmGroup& g, const AttnPlan& p, const AttnPtrs& a, const Operands& o,
                    char* ws, void* stream) {
  const int dt = p.dtype;
  const int64_t DP = p.DP;
  char* rk = ws + p.rk.off;
  const int64_t rk_rows = p.Pp + 2 * p.rk_pad;   // per head, padding included
  if (!a.Rk) {
    add_problem(g, p.Pp, p.H * p.DP, p.Kpos, src_plain(o.R, o.ld_pos, p.P),
                src_headpad(o.WkR, o.ld_pos, p.dh, p.DP),
                out_map(rk + (size_t)p.rk_pad * DP * esize(dt), dt, p.Pp, p.H * p.DP,
                        axis_linear(DP), axis(p.DP, rk_rows * DP, 1)),
                gemm_tile(dt));
    return TXL_OK;
  }
  TXL_HIP(timed(K_REPACK_RK, stream, [&] { return launch_repack_rk(a.Rk, rk, p.P, p.Pp, p.rk_pad, p.H, p.dh, p.DP, dt, stream); }), "repack Rk");
  return TXL_OK;
}

// Enqueue the fused attention (and the split combine) over K, V^T already in
// place.  `mem_upd` (optional) is the hidden-state ring to update with h.
txl_status_t run_attention(const AttnPlan& p, const AttnPtrs& a, char* ws, void* stream,
                           const void* k, const void* vt, int32_t kv_tile0, void* mem_upd,
                           int32_t* new_start, float* lse = nullptr) {
  const bool bf = p.dtype == TXL_BF16;
  const int dt = p.dtype;
  // The ring update rides on the bf16 attention launch (the split combine, or
  // the attention kernel's tail with one split) when rows are multiples of 4
  // bytes (copied in 16-byte words when they are multiples of 16); otherwise
  // it is a kernel of its own.  (Not when the output overlaps h: other
  // workgroups may still be copying it.)
  const char* h_lo = static_cast<const char*>(a.h);
  const char* h_hi = h_lo + (size_t)p.B * p.L * p.d * esize(dt);
  const char* o_lo = static_cast<const char*>(a.out);
  const char* o_hi = o_lo + (size_t)p.B * p.L * p.H * p.dh * esize(dt);
  const bool overlap = o_lo < h_hi && h_lo < o_hi;
  const int upd_unit = (p.d * 2) % 16 == 0 ? 16 : (p.d * 2) % 4 == 0 ? 4 : 0;
  const bool fuse_upd = mem_upd && bf && p.M > 0 && upd_unit > 0 && !overlap;
  if (mem_upd) {
    if (!fuse_upd)
      TXL_TRY(after_launch(timed(K_MEM_UPDATE, stream, [&] { return launch_mem_update(mem_upd, a.mem_start, a.h, p.B, p.M, p.L, p.d, dt,
                                             stream); }),
                           "memory update", stream));
    *new_start = (p.M == 0) ? 0 : (p.L < p.M ? (a.mem_start + p.L) % p.M : 0);
  }

  AttnArgs aa{};
  aa.B = p.B;
  aa.H = p.H;
  aa.L = p.L;
  aa.M = p.Mk;
  aa.dh = p.dh;
  aa.Lp = p.Lp;
  aa.Np = p.Np;
  aa.Pp = p.Pp;
  aa.n_split = p.n_split;
  aa.k_lo = p.G;
  aa.kv_tile0 = kv_tile0;
  aa.c_scale = bf ? p.scale * 1.4426950408889634f : p.scale;
  aa.q = reinterpret_cast<const float*>(ws + p.q.off);
  aa.k = k;
  aa.vt = vt;
  aa.rk = ws + p.rk.off;
  aa.u = a.u;
  aa.v = a.v;
  aa.out = a.out;
  aa.part_o = p.n_split > 1 ? ws + p.po.off : nullptr;
  aa.part_ml = p.n_split > 1 ? reinterpret_cast<float*>(ws + p.pml.off) : nullptr;
  aa.dtype = dt;
  aa.lse = lse;
  if (fuse_upd) {
    aa.upd_src = a.h;
    aa.upd_mem = mem_upd;
    aa.upd_start = a.mem_start;
    aa.upd_rows = p.L < p.M ? p.L : p.M;
    aa.upd_row_bytes = (int64_t)p.d * 2;
    aa.upd_unit = upd_unit;
  }
  TXL_TRY(after_launch(timed(K_ATTN, stream,
                             [&] {
                               return bf ? launch_attn_bf16(aa, stream)
                                         : launch_attn_f32(aa, stream);
                             }),
                       "attention kernel", stream));
  if (bf && p.n_split > 1)
    TXL_TRY(after_launch(timed(K_ATTN_COMBINE, stream, [&] { return launch_attn_combine(aa, stream); }),
                         "attention combine", stream));
  return TXL_OK;
}

// Enqueue the projections and the fused attention of one layer.  If mem_update
// is set the ring update (reading `h`) is enqueued between them.
txl_status_t run_rel_attn(const AttnPlan& p, const AttnPtrs& a, char* ws, void* stream,
                          void* mem_upd, int32_t* new_start) {
  const bool bf = p.dtype == TXL_BF16;
  const int dt = p.dtype;
  char* k = ws + p.k.off;
  char* v = ws + p.v.off;
  Operands o;
  const int32_t start0 = a.mem_start;
  void* upd = mem_upd;
  TXL_TRY(pack_operands(p, a, ws, stream, o, &upd));
  if (mem_upd && !upd)   // the pack carried the ring update
    *new_start = (p.M == 0) ? 0 : (p.L < p.M ? (start0 + p.L) % p.M : 0);

  const int tile = gemm_tile(dt);
  const int64_t DP = p.DP;
  GemmGroup g{};
  add_q_problem(g, p, o, ws);
  // k = h~ W_kE^T -> [B][H][Np][DP]
  const RowSrc ht = src_htilde(o.mem, o.h, o.ld_d, p.Np, p.M, p.L, a.mem_start);
  const int k_idx = g.count;
  add_problem(g, p.B * p.Np, p.H * p.DP, p.Kd, ht, src_headpad(o.WkE, o.ld_d, p.dh, p.DP),
              out_map(k, dt, p.B * p.Np, p.H * p.DP, axis(p.Np, (int64_t)p.H * p.Np * DP, DP),
                      axis(p.DP, (int64_t)p.Np * DP, 1)),
              tile);
  if (bf) {
    // val^T = W_v h~^T in 32-key tiles -> [B][Np/32][H][DP][32]: row (head, d)
    // at (head*DP + d)*32, token b*Np + key at (token/32)*(H*DP*32) + key%32
    // (Np is a multiple of 32)
    add_problem(g, p.H * p.DP, p.B * p.Np, p.Kd, src_headpad(o.Wv, o.ld_d, p.dh, p.DP), ht,
                out_map(v, dt, p.H * p.DP, p.B * p.Np, axis_linear(32),
                        axis(32, (int64_t)p.H * DP * 32, 1)),
                tile);
    // K and V^T read the same rows of h~: their tiles are dealt panel by panel
    g.pair1 = k_idx + 1;
  } else {
    add_problem(g, p.B * p.Np, p.H * p.DP, p.Kd, ht, src_headpad(o.Wv, o.ld_d, p.dh, p.DP),
                out_map(v, dt, p.B * p.Np, p.H * p.DP, axis(p.Np, (int64_t)p.H * p.Np * DP, DP),
                        axis(p.DP, (int64_t)p.Np * DP, 1)),
                tile);
  }
  TXL_TRY(add_rk(g, p, a, o, ws, stream));
  TXL_TRY(after_launch(timed(K_PROJ_GEMM, stream, [&] { return launch_gemm(g, dt, stream); }),
                       "projection GEMMs", stream));
  return run_attention(p, a, ws, stream, k, v, 0, upd, new_start);
}

// ------------------------------------------------------------- K/V ring
// A layer's carried keys and values: C = Mk + L slots of K [B][H][C][DP]
// followed by V^T in 32-slot tiles [B][C/32][H][DP][32] (bf16).  At a step
// whose ring start is s (a multiple of 32), key j' of the kernel's sequence
// [G ghost keys ; M memory rows ; L segment rows] sits at slot (s + j') mod C:
// the ghost keys are masked, and the segment's rows are projected straight
// into slots (s + Mk + p) mod C, i.e. over the oldest rows, which the next
// step no longer sees.  The next step starts at (s + L) mod C.
size_t ring_k_bytes(const AttnPlan& p) { return (size_t)p.B * p.H * p.Np * p.DP * 2; }
size_t ring_bytes(const AttnPlan& p) { return 2 * ring_k_bytes(p); }

// Append the K and V^T problems that project rows [p0, p0 + n) of every
// batch's segment (or of the extended context, for the initial projection)
// to ring slots slot0 + r (n, slot0 multiples of 32, no wrap inside).
void add_ring_kv(GemmGroup& g, const AttnPlan& p, const RowSrc& src, int32_t n, int32_t slot0,
                 const Operands& o, void* ring) {
  const RingMaps m = ring_maps(p.H, p.DP, p.Np, n, slot0);
  uint16_t* kr = static_cast<uint16_t*>(ring);
  uint16_t* vr = kr + ring_k_bytes(p) / 2;
  const int tile = gemm_tile(p.dtype);
  add_problem(g, p.B * n, p.H * p.DP, p.Kd, src, src_headpad(o.WkE, o.ld_d, p.dh, p.DP),
              out_map(kr + m.k_base, TXL_BF16, p.B * n, p.H * p.DP, m.k_row, m.k_col), tile);
  add_problem(g, p.H * p.DP, p.B * n, p.Kd, src_headpad(o.Wv, o.ld_d, p.dh, p.DP), src,
              out_map(vr + m.v_base, TXL_BF16, p.H * p.DP, p.B * n, m.v_row, m.v_col, 0, nullptr,
                      m.v_col2),
              tile);
}

txl_status_t run_rel_attn_ring(const AttnPlan& p, const AttnPtrs& a, void* ring, int32_t start,
                               char* ws, void* stream) {
  Operands o;
  TXL_TRY(pack_operands(p, a, ws, stream, o));
  GemmGroup g{};
  add_q_problem(g, p, o, ws);
  // the segment's rows go to slots base .. base + L - 1 (mod C): at most two
  // contiguous pieces
  const int32_t base = (start + p.Mk) % p.Np;
  const int32_t n1 = ring_first_piece(start, p.Mk, p.L, p.Np);
  add_ring_kv(g, p, src_htilde(nullptr, o.h, o.ld_d, n1, 0, p.L, 0), n1, base, o, ring);
  if (n1 < p.L) {
    const char* h2 = static_cast<const char*>(o.h) + (size_t)n1 * o.ld_d * 2;
    add_ring_kv(g, p, src_htilde(nullptr, h2, o.ld_d, p.L - n1, 0, p.L, 0), p.L - n1, 0, o, ring);
  }
  TXL_TRY(add_rk(g, p, a, o, ws, stream));
  TXL_TRY(after_launch(timed(K_PROJ_GEMM, stream, [&] { return launch_gemm(g, p.dtype, stream); }),
                       "projection GEMMs", stream));
  const char* kr = static_cast<const char*>(ring);
  return run_attention(p, a, ws, stream, kr, kr + ring_k_bytes(p), start / 32, nullptr, nullptr);
}

// ------------------------------------------------------------- backward
// Workspace of the backward: the forward plan's regions (projections, split
// partials, packing), then the extra operand layouts and the intermediate
// P^T, dS^T, dS'^T of the key-side products.
struct BwdPlan {
  AttnPlan p;
  Region o, lse, dop, dot, qut, qvt, dsum, pt, dst, dspt, duv, rkt, rt, drkt, drkp;
  int32_t rkt_ld, rkt_pad, dsp_lo, dsp_tiles;
  size_t total;
};

BwdPlan make_bwd_plan(const txl_attn_shape_t* s, bool compute_rk, bool want_wkr) {
  BwdPlan bp{};
  bp.p = make_plan(s, compute_rk);
  const AttnPlan& p = bp.p;
  size_t off = align256(p.total);
  auto take = [&](Region& r, size_t bytes) {
    r.off = off;
    r.bytes = bytes;
    off = align256(off + bytes);
  };
  const size_t BH = (size_t)p.B * p.H;
  take(bp.o, (size_t)p.B * p.L * p.H * p.dh * 2);
  take(bp.lse, BH * p.Lp * 4);
  take(bp.dop, BH * p.Lp * p.DP * 2);
  take(bp.dot, BH * p.Lp * p.DP * 2);
  take(bp.qut, BH * p.Lp * p.DP * 2);
  take(bp.qvt, BH * p.Lp * p.DP * 2);
  take(bp.dsum, BH * p.Lp * 4);
  take(bp.pt, BH * p.Np * p.Lp * 2);
  take(bp.dst, BH * p.Np * p.Lp * 2);
  // dS'^T tiles of 32 distances from the lowest half the query kernel
  // flushes (its halves start at distances = M + 1 mod 32) to the highest
  // (queries 32w.. of the last wave: M + 32w + 1 .. +31)
  {
    const int32_t mu = (p.M + 1) % 32;
    bp.dsp_lo = mu <= 1 ? mu - 32 : mu - 64;
    bp.dsp_tiles = (p.M + p.Lp + 1 - bp.dsp_lo) / 32;
  }
  take(bp.dspt, (size_t)p.H * bp.dsp_tiles * 32 * p.B * p.Lp * 2);
  take(bp.duv, 2 * BH * (p.Lp / 32) * p.DP * 4);
  take(bp.drkp, (size_t)p.B * p.P * p.H * p.dh * 4);
  // Rk^T columns: distance delta at rkt_pad + delta; rkt_pad = 31 - M (mod 8)
  // keeps every window the kernel reads 16-byte aligned
  bp.rkt_pad = 64 + (((31 - p.M) % 8) + 8) % 8;
  bp.rkt_ld = (int32_t)round_up(bp.rkt_pad + p.Pp + 64, 8);
  take(bp.rkt, (size_t)p.H * p.DP * bp.rkt_ld * 2);
  if (want_wkr) {
    // bf16 transposes for dW_kR, distances padded to a multiple of 64
    const size_t Pk = round_up(p.P, 64);
    take(bp.rt, (size_t)p.dpos * Pk * 2);
    take(bp.drkt, (size_t)p.H * p.dh * Pk * 2);
  }
  bp.total = off;
  return bp;
}

struct BwdOut {
  const void* d_out;
  float *d_q, *d_k, *d_val, *d_u, *d_v, *d_Rk, *d_W_kR;
};

// Forward of the backward's plan: the projections (q, K, V^T, Rk) and the
// attention with each row's log-sum-exp, all left in the workspace, the output
// written to `out`.
txl_status_t run_bwd_forward(const BwdPlan& bp, const AttnPtrs& a, void* out, char* ws,
                             void* stream) {
  const AttnPlan& p = bp.p;
  const int dt = p.dtype;
  const int64_t DP = p.DP;
  char* k = ws + p.k.off;
  char* v = ws + p.v.off;
  Operands o;
  TXL_TRY(pack_operands(p, a, ws, stream, o));
  // projections: the forward's q, K, V^T, Rk (the backward reads K^T and the
  // val rows out of the K and V^T tiles)
  const int tile = gemm_tile(dt);
  GemmGroup gg{};
  add_q_problem(gg, p, o, ws);
  const RowSrc ht = src_htilde(o.mem, o.h, o.ld_d, p.Np, p.M, p.L, a.mem_start);
  const int k_idx = gg.count;
  add_problem(gg, p.B * p.Np, p.H * p.DP, p.Kd, ht, src_headpad(o.WkE, o.ld_d, p.dh, p.DP),
              out_map(k, dt, p.B * p.Np, p.H * p.DP, axis(p.Np, (int64_t)p.H * p.Np * DP, DP),
                      axis(p.DP, (int64_t)p.Np * DP, 1)),
              tile);
  add_problem(gg, p.H * p.DP, p.B * p.Np, p.Kd, src_headpad(o.Wv, o.ld_d, p.dh, p.DP), ht,
              out_map(v, dt, p.H * p.DP, p.B * p.Np, axis_linear(32),
                      axis(32, (int64_t)p.H * DP * 32, 1)),
              tile);
  gg.pair1 = k_idx + 1;   // K and V^T read the same rows of h~
  TXL_TRY(add_rk(gg, p, a, o, ws, stream));
  TXL_TRY(after_launch(timed(K_PROJ_GEMM, stream, [&] { return launch_gemm(gg, dt, stream); }),
                       "backward projection GEMMs", stream));
  // the forward's output and the rows' log-sum-exp
  AttnPtrs fa = a;
  fa.out = out;
  float* lse = reinterpret_cast<float*>(ws + bp.lse.off);
  return run_attention(p, fa, ws, stream, k, v, 0, nullptr, nullptr, lse);
}

// Backward from the state run_bwd_forward left in the workspace and its
// output `out` (a.u, a.v and, for dW_kR, a.R are read again).
txl_status_t run_bwd_from_state(const BwdPlan& bp, const AttnPtrs& a, const void* out,
                                const BwdOut& g, char* ws, void* stream) {
  const AttnPlan& p = bp.p;
  const int dt = p.dtype;
  const int64_t DP = p.DP;
  char* k = ws + p.k.off;
  float* lse = reinterpret_cast<float*>(ws + bp.lse.off);
  BwdPrepArgs pa{};
  pa.B = p.B; pa.H = p.H; pa.L = p.L; pa.dh = p.dh; pa.Lp = p.Lp;
  pa.dout = g.d_out;
  pa.out = out;
  pa.q = reinterpret_cast<const float*>(ws + p.q.off);
  pa.u = a.u;
  pa.v = a.v;
  pa.dop = ws + bp.dop.off;
  pa.dot = ws + bp.dot.off;
  pa.qut = ws + bp.qut.off;
  pa.qvt = ws + bp.qvt.off;
  pa.dsum = reinterpret_cast<float*>(ws + bp.dsum.off);
  // one launch: the prep, the Rk^T table and (for dW_kR) R^T in bf16 with the
  // distances padded to a multiple of 64
  const int32_t Pk = (int32_t)round_up(p.P, 64);
  BwdPreArgs pre{};
  pre.prep = pa;
  pre.rk_ws = ws + p.rk.off;
  pre.rkt = ws + bp.rkt.off;
  pre.Pp = p.Pp;
  pre.pad_ws = p.rk_pad;
  pre.rkt_ld = bp.rkt_ld;
  pre.pad_t = bp.rkt_pad;
  if (g.d_W_kR) {
    pre.r = a.R;
    pre.rt = ws + bp.rt.off;
    pre.P = p.P;
    pre.d_pos = p.dpos;
    pre.r_dtype = dt;
    pre.r_ld = Pk;
  }
  TXL_TRY(after_launch(timed(K_BWD_AUX, stream, [&] { return launch_bwd_pre(pre, stream); }),
                       "backward prep, Rk^T and R^T", stream));

  BwdArgs ba{};
  ba.B = p.B; ba.H = p.H; ba.L = p.L; ba.M = p.M; ba.dh = p.dh;
  ba.Lp = p.Lp; ba.Np = p.Np; ba.Pp = p.Pp;
  ba.c_scale = p.scale * 1.4426950408889634f;
  ba.scale = p.scale;
  ba.q = pa.q;
  ba.k = k;
  ba.vt = ws + p.v.off;
  ba.rk = ws + p.rk.off;
  ba.rkt = ws + bp.rkt.off;
  ba.rkt_ld = bp.rkt_ld;
  ba.rkt_pad = bp.rkt_pad;
  ba.u = a.u;
  ba.v = a.v;
  ba.dop = pa.dop;
  ba.lse = lse;
  ba.dsum = pa.dsum;
  ba.pt = ws + bp.pt.off;
  ba.dst = ws + bp.dst.off;
  ba.dspt = ws + bp.dspt.off;
  ba.dsp_lo = bp.dsp_lo;
  ba.dsp_tiles = bp.dsp_tiles;
  ba.dq = g.d_q;
  ba.duv_part = reinterpret_cast<float*>(ws + bp.duv.off);
  TXL_TRY(after_launch(timed(K_BWD_Q, stream, [&] { return launch_attn_bwd_q(ba, stream); }),
                       "backward query kernel", stream));

  // key side: dk = scale dS^T (q+u), dval = P^T G (per batch row and head),
  // dRk = scale dS'^T (q+v) (per head, summed over batch rows)
  const int64_t HD = (int64_t)p.H * p.dh;
  auto bmm = [&](const void* A, int64_t lda, AxisMap ab, const void* Bm, int64_t ldb, AxisMap bb,
                 int32_t batch, int32_t K, float alpha, float* C, AxisMap cb) {
    BmmArgs m{};
    m.A = A; m.Bm = Bm; m.lda = lda; m.ldb = ldb; m.a_batch = ab; m.b_batch = bb;
    m.M = p.P; m.K = K; m.batch = batch; m.n_valid = p.dh; m.m_valid = p.P;
    m.moff = p.M; m.klim = p.L; m.alpha = alpha;
    m.C = C; m.ldc = HD; m.c_batch = cb;
    m.C2 = nullptr; m.c2_batch = kNoAxis;
    return m;
  };
  const int32_t BHn = p.B * p.H;
  const AxisMap per_bh_c = make_axis(p.H, (int64_t)p.P * HD, p.dh);   // [B][P][H][dh]
  // dRk per (head, pair of batch rows) into partials [B/2][P][H][dh] (one
  // batch row per partial when B is odd), then summed over the partials in
  // order (one product per head would leave the chip idle)
  const int64_t BL = (int64_t)p.B * p.Lp;
  const int32_t rc = p.B % 2 == 0 ? 2 : 1;   // batch rows per dRk partial
  const int32_t nrc = p.B / rc;
  float* drk_part = reinterpret_cast<float*>(ws + bp.drkp.off);
  BmmArgs prods[3] = {
      bmm(ws + bp.dspt.off, BL,
          make_axis(nrc, (int64_t)bp.dsp_tiles * 32 * BL, 32 * (int64_t)rc * p.Lp), ws + bp.qvt.off,
          BL, make_axis(nrc, DP * BL, (int64_t)rc * p.Lp), p.H * nrc, rc * p.Lp, p.scale, drk_part,
          make_axis(nrc, p.dh, (int64_t)p.P * HD)),
      bmm(ws + bp.dst.off, p.Lp, axis_linear((int64_t)p.Np * p.Lp), ws + bp.qut.off, p.Lp,
          axis_linear(DP * p.Lp), BHn, p.Lp, p.scale, g.d_k, per_bh_c),
      bmm(ws + bp.pt.off, p.Lp, axis_linear((int64_t)p.Np * p.Lp), ws + bp.dot.off, p.Lp,
          axis_linear(DP * p.Lp), BHn, p.Lp, 1.0f, g.d_val, per_bh_c)};
  // all three read A from the query kernel's fragment tiles; dS'^T rows are
  // distances from dsp_lo.  The dRk product's workgroups (the longest, with
  // K over rc batch rows) are dealt first.
  prods[0].M = bp.dsp_tiles * 32;
  const int32_t kinds[3] = {2, 1, 1}, row_offs[3] = {bp.dsp_lo, 0, 0}, kpers[3] = {p.Lp, 0, 0};
  TXL_TRY(after_launch(timed(K_BWD_BMM, stream, [&] {
                         return launch_bmm64(prods, 3, kinds, row_offs, kpers, stream);
                       }),
                       "dk, dval, dRk products", stream));
  // one launch: dRk (the partials summed in order) with its bf16
  // transpose for dW_kR, and du, dv
  BwdPostArgs post{};
  post.drk_part = drk_part;
  post.d_rk = g.d_Rk;
  post.drkt = g.d_W_kR ? ws + bp.drkt.off : nullptr;
  post.drk_rows = nrc;
  post.B = p.B;
  post.P = p.P;
  post.HD = (int32_t)HD;
  post.r_ld = Pk;
  post.duv_part = ba.duv_part;
  post.d_u = g.d_u;
  post.d_v = g.d_v;
  post.H = p.H;
  post.nchunk = p.Lp / 32;
  post.dh = p.dh;
  TXL_TRY(after_launch(timed(K_BWD_AUX, stream, [&] { return launch_bwd_post(post, stream); }),
                       "dRk batch sum, du, dv", stream));
  if (g.d_W_kR) {
    // dW_kR = sum_delta dRk[delta] (x) R_delta on the matrix cores: rows
    // h*dh + c, K = distances (the bf16 transposes, padded with zero
    // distances, written by the pre and post launches)
    char* rt = ws + bp.rt.off;
    char* drkt = ws + bp.drkt.off;
    // Split K (the distances) S ways into fp32 partials, summed in order by
    // a second launch: the product alone has too few 128x128 tiles to fill
    // the chip (d_model 512: 16).  The partials reuse the dRk partial buffer,
    // whose sum has already been taken.
    const int64_t tiles = (int64_t)((HD + 127) / 128) * ((p.dpos + 127) / 128);
    int S = 1;
    while (2 * S <= 8 && Pk % (64 * 2 * S) == 0 && Pk / (2 * S) >= 128 &&
           tiles * 2 * S <= device_cu_count() && (int64_t)2 * S * p.dpos <= (int64_t)p.B * p.P)
      S *= 2;
    const int32_t Ks = Pk / S;
    float* wparts = S > 1 ? drk_part : g.d_W_kR;
    GemmGroup gw{};
    for (int sk = 0; sk < S; ++sk)
      add_problem(gw, (int32_t)HD, p.dpos, Ks, src_plain(drkt + (size_t)sk * Ks * 2, Pk, (int32_t)HD),
                  src_plain(rt + (size_t)sk * Ks * 2, Pk, p.dpos),
                  out_map(wparts + (int64_t)sk * HD * p.dpos, TXL_F32, (int32_t)HD, p.dpos,
                          axis_linear(p.dpos), axis_linear(1)),
                  gemm_tile(TXL_BF16));
    TXL_TRY(after_launch(timed(K_BWD_AUX, stream, [&] { return launch_gemm_bf16(gw, stream); }),
                         "dW_kR GEMM", stream));
    if (S > 1)
      TXL_TRY(after_launch(timed(K_BWD_AUX, stream, [&] {
                             return launch_sum_rows(wparts, S, HD * p.dpos, g.d_W_kR, stream);
                           }),
                           "dW_kR split sum", stream));
  }
  return TXL_OK;
}

// Forward recompute (output into the workspace) then the backward.
txl_status_t run_rel_attn_bwd(const BwdPlan& bp, const AttnPtrs& a, const BwdOut& g, char* ws,
                              void* stream) {
  char* o = ws + bp.o.off;
  TXL_TRY(run_bwd_forward(bp, a, o, ws, stream));
  return run_bwd_from_state(bp, a, o, g, ws, stream);
}

// --------------------------------------------------------- segment planning
// Split-K factor (a power of two <= kMaxGroup) for a rows x N product of
// reduction length K whose fp32 result feeds a LayerNorm: grow it while the
// 128x128 tiles of all splits still fit the compute units once and every split
// keeps at least 256 of K (K / S a multiple of 64).
int split_k(int32_t rows, int32_t N, int32_t K) {
  const int64_t t = (int64_t)((rows + 127) / 128) * ((N + 127) / 128);
  const int64_t cus = device_cu_count();
  int S = 1;
  while (2 * S <= kMaxGroup && t * 2 * S <= cus && K % (64 * 2 * S) == 0 && K / (2 * S) >= 256)
    S *= 2;
  return S;
}

struct SegPlan {
  AttnPlan attn;
  bool any_full;
  Region a, x32a, x32b, xlo_a, xlo_b, parts, o32, olo, hid;
  size_t total;
};

SegPlan make_seg_plan(const txl_attn_shape_t* s, int32_t d_inner, bool any_full,
                      int kind = PLAN_STD) {
  SegPlan sp{};
  sp.attn = make_plan(s, true, kind);
  sp.any_full = any_full;
  size_t off = align256(sp.attn.total);
  auto take = [&](Region& r, size_t bytes) {
    r.off = off;
    r.bytes = bytes;
    off = align256(off + bytes);
  };
  const size_t rows = (size_t)s->batch * s->seg_len;
  const size_t es = esize(s->dtype);
  const size_t Hd = (size_t)s->n_heads * s->d_head;
  take(sp.a, rows * Hd * es);
  take(sp.xlo_a, rows * std::max<size_t>(Hd, s->d_model) * es);
  take(sp.xlo_b, rows * std::max<size_t>(Hd, s->d_model) * es);
  if (any_full) {
    take(sp.x32a, rows * s->d_model * 4);
    take(sp.x32b, rows * s->d_model * 4);
    take(sp.parts, kMaxGroup * rows * s->d_model * 4);
    take(sp.o32, rows * s->d_model * 4);
    take(sp.olo, rows * s->d_model * es);
    take(sp.hid, rows * (size_t)std::max(d_inner, 1) * es);
  }
  sp.total = off;
  return sp;
}

// Segment step over n_layers layers; with `rings` (one K/V ring per layer)
// the layers attend through their rings and ly.mem is not used.
txl_status_t segment_step(const txl_attn_shape_t* shape, int32_t n_layers, int32_t d_inner,
                          const txl_layer_t* layers, void* const* rings, size_t ring_nbytes,
                          const void* R, const void* h_in, void* h_out, int32_t* mem_start,
                          void* workspace, size_t workspace_bytes, void* stream) {
  const bool kv = rings != nullptr;
  const int kind = kv ? PLAN_RING : PLAN_STD;
  TXL_TRY(check_shape(shape));
  if (n_layers < 1 || n_layers > 4096) return fail(TXL_ERR_BAD_SHAPE, "n_layers=%d", n_layers);
  if (!layers || !h_in || !h_out || !mem_start || !workspace)
    return fail(TXL_ERR_NULL_ARG, "layers, h_in, h_out, mem_start and workspace are required");
  const int32_t start = *mem_start;
  const int32_t d = shape->d_model, Hd = shape->n_heads * shape->d_head;
  bool any_full = false;
  for (int n = 0; n < n_layers; ++n) {
    const txl_layer_t& ly = layers[n];
    AttnPtrs a{h_in, kv ? nullptr : ly.mem, ly.W_q, ly.W_kE, ly.W_kR, ly.W_v, ly.u, ly.v, R,
               ly.Rk, kv ? 0 : start, h_out};
    txl_status_t st = check_attn_ptrs(shape, a, false, workspace, !kv);
    if (st == TXL_OK && kv) {
      const AttnPlan rp = make_plan(shape, true, PLAN_RING);
      if (!rings[n])
        st = fail(TXL_ERR_NULL_ARG, "ring is NULL");
      else if (!aligned16(rings[n]))
        st = fail(TXL_ERR_UNSUPPORTED, "bf16 path needs 16-byte aligned tensor pointers");
      else if (ring_nbytes < ring_bytes(rp))
        st = fail(TXL_ERR_BAD_SHAPE, "ring %zu < %zu bytes", ring_nbytes, ring_bytes(rp));
      else if (start < 0 || start >= rp.Np || start % 32 != 0)
        st = fail(TXL_ERR_BAD_SHAPE, "ring_start %d is not a multiple of 32 in [0, %d)", start,
                  rp.Np);
    }
    if (st != TXL_OK) {
      g_last_error = "layer " + std::to_string(n) + ": " + g_last_error;
      return st;
    }
    if (ly.W_o) {
      any_full = true;
      if (!ly.W_ff1 || !ly.W_ff2)
        return fail(TXL_ERR_NULL_ARG, "layer %d: W_ff1 and W_ff2 are required with W_o", n);
      if (d_inner < 1 || d_inner > kMaxDim)
        return fail(TXL_ERR_BAD_SHAPE, "d_inner=%d out of range", d_inner);
      if (shape->dtype == TXL_BF16 &&
          (!aligned16(ly.W_o) || !aligned16(ly.W_ff1) || !aligned16(ly.W_ff2)))
        return fail(TXL_ERR_UNSUPPORTED, "bf16 path needs 16-byte aligned tensor pointers");
      if (shape->dtype == TXL_BF16 && (Hd % 64 != 0 || d % 64 != 0 || d_inner % 64 != 0))
        return fail(TXL_ERR_UNSUPPORTED,
                    "bf16 full layers need H*d_head, d_model and d_inner multiples of 64");
    } else if (n + 1 < n_layers && Hd != d) {
      return fail(TXL_ERR_BAD_SHAPE,
                  "layer %d has no W_o: H*d_head (%d) must equal d_model (%d) to feed layer %d",
                  n, Hd, d, n + 1);
    }
  }
  const SegPlan sp = make_seg_plan(shape, d_inner, any_full, kind);
  if (workspace_bytes < sp.total)
    return fail(TXL_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes,
                sp.total);

  char* ws = static_cast<char*>(workspace);
  const int dt = shape->dtype;
  const int32_t rows = shape->batch * shape->seg_len;
  const int tile = gemm_tile(dt);
  const void* x_lo = h_in;        // current layer input (storage dtype)
  float* x32 = nullptr;           // fp32 residual copy of x_lo (full layers)
  char* lo_buf[2] = {ws + sp.xlo_a.off, ws + sp.xlo_b.off};
  float* f32_buf[2] = {reinterpret_cast<float*>(ws + sp.x32a.off),
                       reinterpret_cast<float*>(ws + sp.x32b.off)};
  int pp = 0;
  int32_t new_start = start;
  for (int n = 0; n < n_layers; ++n) {
    const txl_layer_t& ly = layers[n];
    const bool last = n + 1 == n_layers;
    const bool full = ly.W_o != nullptr;
    if (full && !x32) {
      x32 = f32_buf[pp];
      TXL_HIP(timed(K_CAST, stream, [&] { return launch_cast_f32(x_lo, x32, (int64_t)rows * d, dt, stream); }), "cast residual");
    }
    void* a_out = (!full && last) ? h_out : (full ? ws + sp.a.off : lo_buf[pp ^ 1]);
    AttnPtrs a{x_lo, ly.mem, ly.W_q, ly.W_kE, ly.W_kR, ly.W_v, ly.u, ly.v, R, ly.Rk, start, a_out};
    const AttnPlan p = make_plan(shape, ly.Rk == nullptr, kind);
    if (kv) {
      a.mem = nullptr;
      TXL_TRY(run_rel_attn_ring(p, a, rings[n], start, ws, stream));
      new_start = (start + p.L) % p.Np;
    } else {
      TXL_TRY(run_rel_attn(p, a, ws, stream, ly.mem, &new_start));
    }
    if (!full) {
      x_lo = a_out;
      x32 = nullptr;
      pp ^= 1;
      continue;
    }
    float* parts = reinterpret_cast<float*>(ws + sp.parts.off);
    const int64_t pstride = (int64_t)rows * d;
    float* o32 = reinterpret_cast<float*>(ws + sp.o32.off);
    void* olo = ws + sp.olo.off;
    void* hid = ws + sp.hid.off;
    // parts[s] = A[:, Ks*s ..) W[:, Ks*s ..)^T (fp32), K split S ways; the
    // LayerNorm that follows adds the residual and the S partial products
    auto split_gemm = [&](const void* A, const void* Wt, int32_t K, int kind,
                          const char* what, int* S_out) -> txl_status_t {
      const int S = dt == TXL_BF16 ? split_k(rows, d, K) : 1;
      const int32_t Ks = K / S;
      GemmGroup g{};
      for (int sk = 0; sk < S; ++sk)
        add_problem(g, rows, d, Ks,
                    src_plain(static_cast<const char*>(A) + (size_t)sk * Ks * esize(dt), K, rows),
                    src_plain(static_cast<const char*>(Wt) + (size_t)sk * Ks * esize(dt), K, d),
                    out_map(parts + sk * pstride, TXL_F32, rows, d, axis_linear(d), axis_linear(1)),
                    tile);
      *S_out = S;
      return after_launch(timed(kind, stream, [&] { return launch_gemm(g, dt, stream); }), what,
                          stream);
    };
    // o = LN(a W_o^T + x)
    int S = 1;
    TXL_TRY(split_gemm(ws + sp.a.off, ly.W_o, Hd, K_WO_GEMM, "W_o GEMM", &S));
    TXL_TRY(after_launch(timed(K_LAYERNORM, stream, [&] { return launch_layernorm(x32, parts, S, pstride, o32, olo, rows, d, dt, 1e-5f, stream); }), "LN1",
                         stream));
    {
      GemmGroup g{};
      add_problem(g, rows, d_inner, d, src_plain(olo, d, rows), src_plain(ly.W_ff1, d, d_inner),
                  out_map(hid, dt, rows, d_inner, axis_linear(d_inner), axis_linear(1), EPI_RELU),
                  tile);
      TXL_TRY(after_launch(timed(K_FFN1_GEMM, stream, [&] { return launch_gemm(g, dt, stream); }), "FFN1 GEMM",
                           stream));
    }
    // h' = LN(o + ReLU(o W_ff1^T) W_ff2^T)
    TXL_TRY(split_gemm(hid, ly.W_ff2, d_inner, K_FFN2_GEMM, "FFN2 GEMM", &S));
    float* y32 = f32_buf[pp ^ 1];
    void* ylo = last ? h_out : lo_buf[pp ^ 1];
    TXL_TRY(after_launch(timed(K_LAYERNORM, stream, [&] { return launch_layernorm(o32, parts, S, pstride, y32, ylo, rows, d, dt, 1e-5f, stream); }), "LN2",
                         stream));
    x_lo = ylo;
    x32 = y32;
    pp ^= 1;
  }
  *mem_start = new_start;
  return TXL_OK;
}

}  // namespace

txl_status_t set_error(txl_status_t st, const char* msg) { return fail(st, "%s", msg); }

void suppress_timing(bool on) { g_timing_suppressed = on; }

}  // namespace txl

using namespace txl;

extern "C" {

int txl_abi_version(void) { return TXL_ABI_VERSION; }

const char* txl_status_str(txl_status_t st) {
  switch (st) {
    case TXL_OK: return "ok";
    case TXL_ERR_NULL_ARG: return "null argument";
    case TXL_ERR_BAD_SHAPE: return "bad shape";
    case TXL_ERR_BAD_DTYPE: return "bad dtype";
    case TXL_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case TXL_ERR_UNSUPPORTED: return "unsupported";
    case TXL_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* txl_last_error(void) { return g_last_error.c_str(); }

txl_status_t txl_probe_mfma(const void* operands, int32_t n_wg, int32_t iters, uint64_t* clocks,
                            void* stream) {
  if (!operands || !clocks) return fail(TXL_ERR_NULL_ARG, "operands and clocks are required");
  if (n_wg < 1 || n_wg > 65536 || iters < 2 || iters % 2 != 0)
    return fail(TXL_ERR_BAD_SHAPE, "n_wg=%d iters=%d (need 1 <= n_wg <= 65536, even iters >= 2)", n_wg,
                iters);
  if (!aligned16(operands)) return fail(TXL_ERR_UNSUPPORTED, "operands must be 16-byte aligned");
  return after_launch(launch_mfma_probe(operands, n_wg, iters, clocks, stream), "mfma probe", stream);
}

txl_status_t txl_sinusoid_pos(void* R, int32_t n_pos, int32_t d_pos, int32_t dtype, void* stream) {
  if (!R) return fail(TXL_ERR_NULL_ARG, "R is NULL");
  if (dtype != TXL_F32 && dtype != TXL_BF16) return fail(TXL_ERR_BAD_DTYPE, "bad dtype %d", dtype);
  if (n_pos < 1 || d_pos < 1 || n_pos > kMaxDim || d_pos > kMaxDim)
    return fail(TXL_ERR_BAD_SHAPE, "n_pos=%d d_pos=%d out of range", n_pos, d_pos);
  return after_launch(timed(K_SINUSOID, stream, [&] { return launch_sinusoid(R, n_pos, d_pos, dtype, stream); }), "sinusoid", stream);
}

size_t txl_rel_proj_workspace_bytes(int32_t n_pos, int32_t d_pos, int32_t n_heads, int32_t d_head,
                                    int32_t dtype) {
  if (dtype != TXL_BF16 || d_pos % 64 == 0 || n_pos < 1 || d_pos < 1 || n_heads < 1 || d_head < 1)
    return 0;
  const int64_t Kp = round_up(d_pos, 64);
  return align256((size_t)n_pos * Kp * 2) + align256((size_t)n_heads * d_head * Kp * 2);
}

txl_status_t txl_rel_proj(const void* R, const void* W_kR, void* Rk, int32_t n_pos, int32_t d_pos,
                          int32_t n_heads, int32_t d_head, int32_t dtype, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (!R || !W_kR || !Rk) return fail(TXL_ERR_NULL_ARG, "R, W_kR and Rk are required");
  if (dtype != TXL_F32 && dtype != TXL_BF16) return fail(TXL_ERR_BAD_DTYPE, "bad dtype %d", dtype);
  if (n_pos < 1 || d_pos < 1 || n_heads < 1 || d_head < 1 || n_pos > kMaxDim || d_pos > kMaxDim ||
      (int64_t)n_heads * d_head > kMaxDim)
    return fail(TXL_ERR_BAD_SHAPE, "sizes out of range");
  const size_t need = txl_rel_proj_workspace_bytes(n_pos, d_pos, n_heads, d_head, dtype);
  if (need && !workspace) return fail(TXL_ERR_NULL_ARG, "workspace is NULL");
  if (workspace_bytes < need)
    return fail(TXL_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, need);
  if (dtype == TXL_BF16 && (!aligned16(R) || !aligned16(W_kR) || !aligned16(Rk)))
    return fail(TXL_ERR_UNSUPPORTED, "bf16 path needs 16-byte aligned tensor pointers");
  const int32_t Hd = n_heads * d_head;
  const void* Rs = R;
  const void* Ws = W_kR;
  int64_t ld = d_pos;
  if (need) {
    const int64_t Kp = round_up(d_pos, 64);
    char* ws = static_cast<char*>(workspace);
    char* pr = ws;
    char* pw = ws + align256((size_t)n_pos * Kp * 2);
    TXL_HIP(timed(K_PACK, stream, [&] { return launch_pack_rows(pr, Kp, R, d_pos, n_pos, d_pos, dtype, stream); }), "pack R");
    TXL_HIP(timed(K_PACK, stream, [&] { return launch_pack_rows(pw, Kp, W_kR, d_pos, Hd, d_pos, dtype, stream); }), "pack W_kR");
    Rs = pr;
    Ws = pw;
    ld = Kp;
  }
  GemmGroup g{};
  add_problem(g, n_pos, Hd, (int32_t)ld, src_plain(Rs, ld, n_pos), src_plain(Ws, ld, Hd),
              out_map(Rk, dtype, n_pos, Hd, axis_linear(Hd), axis_linear(1)), gemm_tile(dtype));
  return after_launch(timed(K_REL_PROJ, stream, [&] { return launch_gemm(g, dtype, stream); }),
                      "rel_proj GEMM", stream);
}

size_t txl_rel_attn_workspace_bytes(const txl_attn_shape_t* shape) {
  if (check_shape(shape) != TXL_OK) return 0;
  return make_plan(shape, true).total;
}

txl_status_t txl_rel_attn_fwd(const txl_attn_shape_t* shape, const void* h, const void* mem,
                              int32_t mem_start, const void* W_q, const void* W_kE,
                              const void* W_kR, const void* W_v, const void* u, const void* v,
                              const void* R, const void* Rk, void* out, void* workspace,
                              size_t workspace_bytes, void* stream) {
  TXL_TRY(check_shape(shape));
  AttnPtrs a{h, mem, W_q, W_kE, W_kR, W_v, u, v, R, Rk, mem_start, out};
  TXL_TRY(check_attn_ptrs(shape, a, true, workspace));
  const AttnPlan p = make_plan(shape, Rk == nullptr);
  const size_t need = make_plan(shape, true).total;
  if (workspace_bytes < need)
    return fail(TXL_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, need);
  return run_rel_attn(p, a, static_cast<char*>(workspace), stream, nullptr, nullptr);
}

size_t txl_rel_attn_bwd_workspace_bytes(const txl_attn_shape_t* shape) {
  if (check_shape(shape) != TXL_OK || shape->dtype != TXL_BF16) return 0;
  return make_bwd_plan(shape, true, true).total;
}

txl_status_t txl_rel_attn_bwd(const txl_attn_shape_t* shape, const void* h, const void* mem,
                              int32_t mem_start, const void* W_q, const void* W_kE,
                              const void* W_kR, const void* W_v, const void* u, const void* v,
                              const void* R, const void* Rk, const void* d_out, float* d_q,
                              float* d_k, float* d_val, float* d_u, float* d_v, float* d_Rk,
                              float* d_W_kR, void* workspace, size_t workspace_bytes,
                              void* stream) {
  TXL_TRY(check_shape(shape));
  if (shape->dtype != TXL_BF16) return fail(TXL_ERR_UNSUPPORTED, "the backward is bf16 only");
  AttnPtrs a{h, mem, W_q, W_kE, W_kR, W_v, u, v, R, Rk, mem_start, const_cast<void*>(d_out)};
  TXL_TRY(check_attn_ptrs(shape, a, true, workspace));
  if (!d_q || !d_k || !d_val || !d_u || !d_v || !d_Rk)
    return fail(TXL_ERR_NULL_ARG, "d_q, d_k, d_val, d_u, d_v and d_Rk are required");
  if (d_W_kR && Rk)
    return fail(TXL_ERR_BAD_SHAPE, "d_W_kR needs Rk computed from W_kR and R (Rk must be NULL)");
  const BwdPlan bp = make_bwd_plan(shape, Rk == nullptr, d_W_kR != nullptr);
  const size_t need = txl_rel_attn_bwd_workspace_bytes(shape);
  if (workspace_bytes < need)
    return fail(TXL_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, need);
  const BwdOut g{d_out, d_q, d_k, d_val, d_u, d_v, d_Rk, d_W_kR};
  return run_rel_attn_bwd(bp, a, g, static_cast<char*>(workspace), stream);
}

txl_status_t txl_rel_attn_fwd_train(const txl_attn_shape_t* shape, const void* h, const void* mem,
                                    int32_t mem_start, const void* W_q, const void* W_kE,
                                    const void* W_kR, const void* W_v, const void* u,
                                    const void* v, const void* R, const void* Rk, void* out,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  TXL_TRY(check_shape(shape));
  if (shape->dtype != TXL_BF16) return fail(TXL_ERR_UNSUPPORTED, "training calls are bf16 only");
  AttnPtrs a{h, mem, W_q, W_kE, W_kR, W_v, u, v, R, Rk, mem_start, out};
  TXL_TRY(check_attn_ptrs(shape, a, true, workspace));
  const size_t need = txl_rel_attn_bwd_workspace_bytes(shape);
  if (workspace_bytes < need)
    return fail(TXL_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, need);
  const BwdPlan bp = make_bwd_plan(shape, Rk == nullptr, true);
  return run_bwd_forward(bp, a, out, static_cast<char*>(workspace), stream);
}

txl_status_t txl_rel_attn_bwd_saved(const txl_attn_shape_t* shape, const void* u, const void* v,
                                    const void* R, int32_t rk_given, const void* out,
                                    const void* d_out, float* d_q, float* d_k, float* d_val,
                                    float* d_u, float* d_v, float* d_Rk, float* d_W_kR,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  TXL_TRY(check_shape(shape));
  if (shape->dtype != TXL_BF16) return fail(TXL_ERR_UNSUPPORTED, "the backward is bf16 only");
  if (!u || !v || !out || !d_out || !workspace)
    return fail(TXL_ERR_NULL_ARG, "u, v, out, d_out and workspace are required");
  if (!d_q || !d_k || !d_val || !d_u || !d_v || !d_Rk)
    return fail(TXL_ERR_NULL_ARG, "d_q, d_k, d_val, d_u, d_v and d_Rk are required");
  if (d_W_kR && (rk_given || !R))
    return fail(TXL_ERR_BAD_SHAPE, "d_W_kR needs Rk computed from W_kR and R (rk_given 0, R set)");
  for (const void* q : {out, d_out, static_cast<const void*>(workspace), R})
    if (q && !aligned16(q))
      return fail(TXL_ERR_UNSUPPORTED, "bf16 path needs 16-byte aligned tensor pointers");
  const size_t need = txl_rel_attn_bwd_workspace_bytes(shape);
  if (workspace_bytes < need)
    return fail(TXL_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, need);
  const BwdPlan bp = make_bwd_plan(shape, !rk_given, true);
  AttnPtrs a{};
  a.u = u;
  a.v = v;
  a.R = R;
  const BwdOut g{d_out, d_q, d_k, d_val, d_u, d_v, d_Rk, d_W_kR};
  return run_bwd_from_state(bp, a, out, g, static_cast<char*>(workspace), stream);
}

int32_t txl_kv_ring_slots(const txl_attn_shape_t* shape) {
  if (check_ring_shape(shape) != TXL_OK) return 0;
  return make_plan(shape, true, PLAN_RING).Np;
}

size_t txl_kv_ring_bytes(const txl_attn_shape_t* shape) {
  if (check_ring_shape(shape) != TXL_OK) return 0;
  return ring_bytes(make_plan(shape, true, PLAN_RING));
}

size_t txl_kv_ring_workspace_bytes(const txl_attn_shape_t* shape) {
  if (check_ring_shape(shape) != TXL_OK) return 0;
  return std::max(make_plan(shape, true, PLAN_RING).total,
                  make_plan(shape, true, PLAN_RING_INIT).total);
}

txl_status_t txl_kv_ring_init(const txl_attn_shape_t* shape, const void* mem, int32_t mem_start,
                              const void* W_kE, const void* W_v, void* ring, size_t ring_nbytes,
                              int32_t* ring_start, void* workspace, size_t workspace_bytes,
                              void* stream) {
  TXL_TRY(check_ring_shape(shape));
  if (!W_kE || !W_v || !ring || !ring_start || !workspace)
    return fail(TXL_ERR_NULL_ARG, "W_kE, W_v, ring, ring_start and workspace are required");
  if (shape->mem_len > 0 && !mem) return fail(TXL_ERR_NULL_ARG, "mem is NULL but mem_len > 0");
  if (shape->mem_len > 0 ? (mem_start < 0 || mem_start >= shape->mem_len) : mem_start != 0)
    return fail(TXL_ERR_BAD_SHAPE, "mem_start %d outside [0, mem_len=%d)", mem_start,
                shape->mem_len);
  for (const void* q : {mem, W_kE, W_v, (const void*)ring})
    if (q && !aligned16(q))
      return fail(TXL_ERR_UNSUPPORTED, "bf16 path needs 16-byte aligned tensor pointers");
  const AttnPlan p = make_plan(shape, true, PLAN_RING_INIT);
  if (ring_nbytes < ring_bytes(p))
    return fail(TXL_ERR_BAD_SHAPE, "ring %zu < %zu bytes", ring_nbytes, ring_bytes(p));
  const size_t need = txl_kv_ring_workspace_bytes(shape);
  if (workspace_bytes < need)
    return fail(TXL_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, need);
  if (p.M > 0) {
    AttnPtrs a{nullptr, mem, nullptr, W_kE, nullptr, W_v, nullptr, nullptr, nullptr, nullptr,
               mem_start, nullptr};
    char* ws = static_cast<char*>(workspace);
    Operands o;
    TXL_TRY(pack_operands(p, a, ws, stream, o));
    // slots 0 .. Mk-1: G zero rows, then the memory in logical order
    GemmGroup g{};
    add_ring_kv(g, p, src_htilde(o.mem, nullptr, o.ld_d, p.Mk, p.M, 0, mem_start, p.G), p.Mk, 0,
                o, ring);
    TXL_TRY(after_launch(timed(K_PROJ_GEMM, stream, [&] { return launch_gemm(g, p.dtype, stream); }),
                         "ring projection GEMMs", stream));
  }
  *ring_start = 0;
  return TXL_OK;
}

txl_status_t txl_rel_attn_fwd_kv(const txl_attn_shape_t* shape, const void* h, const void* W_q,
                                 const void* W_kE, const void* W_kR, const void* W_v,
                                 const void* u, const void* v, const void* R, const void* Rk,
                                 void* ring, size_t ring_nbytes, int32_t* ring_start, void* out,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  TXL_TRY(check_ring_shape(shape));
  AttnPtrs a{h, nullptr, W_q, W_kE, W_kR, W_v, u, v, R, Rk, 0, out};
  TXL_TRY(check_attn_ptrs(shape, a, true, workspace, false));
  if (!ring || !ring_start) return fail(TXL_ERR_NULL_ARG, "ring and ring_start are required");
  if (!aligned16(ring))
    return fail(TXL_ERR_UNSUPPORTED, "bf16 path needs 16-byte aligned tensor pointers");
  const AttnPlan p = make_plan(shape, Rk == nullptr, PLAN_RING);
  if (ring_nbytes < ring_bytes(p))
    return fail(TXL_ERR_BAD_SHAPE, "ring %zu < %zu bytes", ring_nbytes, ring_bytes(p));
  const int32_t start = *ring_start;
  if (start < 0 || start >= p.Np || start % 32 != 0)
    return fail(TXL_ERR_BAD_SHAPE, "ring_start %d is not a multiple of 32 in [0, %d)", start,
                p.Np);
  const size_t need = txl_kv_ring_workspace_bytes(shape);
  if (workspace_bytes < need)
    return fail(TXL_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, need);
  TXL_TRY(run_rel_attn_ring(p, a, ring, start, static_cast<char*>(workspace), stream));
  *ring_start = (start + p.L) % p.Np;
  return TXL_OK;
}

txl_status_t txl_mem_update(void* mem, int32_t* mem_start, const void* h, int32_t batch,
                            int32_t mem_len, int32_t seg_len, int32_t d_model, int32_t dtype,
                            void* stream) {
  if (!mem_start || !h || (mem_len > 0 && !mem))
    return fail(TXL_ERR_NULL_ARG, "mem, mem_start and h are required");
  if (dtype != TXL_F32 && dtype != TXL_BF16) return fail(TXL_ERR_BAD_DTYPE, "bad dtype %d", dtype);
  if (batch < 1 || mem_len < 0 || seg_len < 1 || d_model < 1 || batch > kMaxDim ||
      mem_len > kMaxDim || seg_len > kMaxDim || d_model > kMaxDim)
    return fail(TXL_ERR_BAD_SHAPE, "sizes out of range");
  const int32_t st = *mem_start;
  if (mem_len > 0 ? (st < 0 || st >= mem_len) : st != 0)
    return fail(TXL_ERR_BAD_SHAPE, "mem_start %d outside [0, mem_len=%d)", st, mem_len);
  if (mem_len == 0) return TXL_OK;
  TXL_TRY(after_launch(timed(K_MEM_UPDATE, stream, [&] { return launch_mem_update(mem, st, h, batch, mem_len, seg_len, d_model, dtype,
                                         stream); }),
                       "memory update", stream));
  *mem_start = seg_len < mem_len ? (st + seg_len) % mem_len : 0;
  return TXL_OK;
}

size_t txl_segment_workspace_bytes(const txl_attn_shape_t* shape, int32_t n_layers,
                                   int32_t d_inner) {
  if (check_shape(shape) != TXL_OK || n_layers < 1) return 0;
  return make_seg_plan(shape, d_inner, d_inner > 0).total;
}

txl_status_t txl_segment_step(const txl_attn_shape_t* shape, int32_t n_layers, int32_t d_inner,
                              const txl_layer_t* layers, const void* R, const void* h_in,
                              void* h_out, int32_t* mem_start, void* workspace,
                              size_t workspace_bytes, void* stream) {
  return segment_step(shape, n_layers, d_inner, layers, nullptr, 0, R, h_in, h_out, mem_start,
                      workspace, workspace_bytes, stream);
}

size_t txl_segment_kv_workspace_bytes(const txl_attn_shape_t* shape, int32_t n_layers,
                                      int32_t d_inner) {
  if (check_ring_shape(shape) != TXL_OK || n_layers < 1) return 0;
  return std::max(make_seg_plan(shape, d_inner, d_inner > 0, PLAN_RING).total,
                  make_plan(shape, true, PLAN_RING_INIT).total);
}

txl_status_t txl_segment_step_kv(const txl_attn_shape_t* shape, int32_t n_layers,
                                 int32_t d_inner, const txl_layer_t* layers,
                                 void* const* rings, size_t ring_bytes, const void* R,
                                 const void* h_in, void* h_out, int32_t* ring_start,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  TXL_TRY(check_ring_shape(shape));
  if (!rings) return fail(TXL_ERR_NULL_ARG, "rings is NULL");
  return segment_step(shape, n_layers, d_inner, layers, rings, ring_bytes, R, h_in, h_out,
                      ring_start, workspace, workspace_bytes, stream);
}

txl_status_t txl_timing_enable(int32_t on) {
  TimingState& t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  t.on = on != 0;
  return TXL_OK;
}

void txl_timing_reset(void) {
  TimingState& t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  for (auto& r : t.pending) {
    (void)hipEventSynchronize(r.b);
    t.pool.push_back(r.a);
    t.pool.push_back(r.b);
  }
  t.pending.clear();
  for (int k = 0; k < K_NKINDS; ++k) {
    t.ms[k] = 0.0;
    t.count[k] = 0;
  }
}

int32_t txl_timing_read(int32_t capacity, const char** names, int64_t* counts, double* total_ms) {
  TimingState& t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  for (auto& r : t.pending) {
    float ms = 0.0f;
    if (hipEventSynchronize(r.b) == hipSuccess && hipEventElapsedTime(&ms, r.a, r.b) == hipSuccess) {
      t.ms[r.kind] += ms;
      t.count[r.kind] += 1;
    }
    t.pool.push_back(r.a);
    t.pool.push_back(r.b);
  }
  t.pending.clear();
  const int n = capacity < K_NKINDS ? capacity : K_NKINDS;
  for (int k = 0; k < n; ++k) {
    if (names) names[k] = kKindNames[k];
    if (counts) counts[k] = t.count[k];
    if (total_ms) total_ms[k] = t.ms[k];
  }
  return K_NKINDS;
}

}  // extern "C"
