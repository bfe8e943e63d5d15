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
// softmax row statistics stay in-lane.
//   * K (32 keys x 64) and V^T (64 x 32 keys) tiles and 32-row chunks of Rk are
//     staged in LDS once per block and shared by the 4 waves.
//   * Term (b)+(d): per block a wave multiplies its 32 queries (q+v) by a
//     32-row chunk of Rk on the matrix cores: BDw[w][i] = (q_i+v).Rk[D-31+w],
//     D = M + i0 - j0.  The pair (i, j) needs row delta = D + i - j, i.e.
//     position 31 + i - j of the 63-row window [chunk_t ; chunk_{t-1}] — the
//     previous block's chunk is the upper half of this block's window, so every
//     chunk is computed once.  The window lives in a per-wave LDS ring (row i =
//     one query); reading position 31+i-j per lane performs App. B's per-row
//     left shift by index arithmetic.  No L x (M+L) matrix is ever written.
//   * The shifted (b)+(d) values initialise the accumulator of the
//     (q+u).K MFMA, so the sum of the four terms costs no vector instruction.
//   * Online softmax in base 2 (c = scale*log2 e is folded into q+u and q+v),
//     with a lazy rescale: the reference maximum only moves when a block's
//     maximum exceeds it by more than 8, which keeps every p <= 2^8.
//   * P (bf16) times V^T on the matrix cores; the key order inside an MFMA is
//     permuted identically in both operands to match the accumulator layout.
//   * With several key-range splits each workgroup writes (max, sum, O) and a
//     combine kernel merges them in a fixed order (deterministic).
//
// fp32 kernel: one workgroup per (b, h, i), plain loops; used by the fp32 path.
#include "dev_common.h"

namespace txl {

namespace {

constexpr int DP = 64;        // padded head width of the bf16 path
constexpr int KB = 32;        // keys per block
constexpr int NWAVE = 4;      // waves per workgroup, 32 queries each
constexpr int QG = 32 * NWAVE;
constexpr int RK_SLOTS = 5;   // Rk chunks resident in LDS
constexpr int VST = 36;       // bf16 per V^T tile row (32 keys + pad)
constexpr int BDS = 100;      // floats per row of the per-wave shift window
constexpr float kNegInf = -__builtin_inff();

struct AttnSmem {
  u32x4 k[KB * 8];                    // K tile, 16-byte chunks XOR-swizzled
  uint16_t vt[DP * VST];              // V^T tile [d][key]
  u32x4 rk[RK_SLOTS][KB * 8];         // Rk chunk ring, swizzled like K
  float bd[NWAVE][32 * BDS];          // per-wave shifted (b)+(d) window
  float uv[2 * DP];                   // u then v of this head, zero padded
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * 8 + (chunk ^ (row & 7)); }

__device__ __forceinline__ bf16x8 pack8(const float* x) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = static_cast<bf16>(x[e]);
  return r;
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

  const uint16_t* kg = static_cast<const uint16_t*>(a.k) + (int64_t)bh * a.Np * DP;
  const uint16_t* vg = static_cast<const uint16_t*>(a.vt) + (int64_t)bh * DP * a.Np;
  const uint16_t* rg = static_cast<const uint16_t*>(a.rk) + (int64_t)head * a.Pp * DP;

  // ---- cooperative staging: one 16-byte chunk of K, V^T and Rk per thread
  const int kr = tid >> 3, kc = tid & 7;     // K / Rk: row, chunk
  const int vd = tid >> 2, vc = tid & 3;     // V^T: row d, 8-key chunk
  auto rk_row = [&](int32_t chunk_id) {      // first row of a chunk, clamped later
    return M + i_base - KB * chunk_id - (KB - 1);
  };
  auto load_k = [&](int32_t tb) {
    return *reinterpret_cast<const u32x4*>(kg + (int64_t)(tb * KB + kr) * DP + kc * 8);
  };
  auto load_v = [&](int32_t tb) {
    return *reinterpret_cast<const u32x4*>(vg + (int64_t)vd * a.Np + tb * KB + vc * 8);
  };
  auto load_r = [&](int32_t chunk_id) {
    int32_t d = rk_row(chunk_id) + kr;
    d = max(0, min(d, a.Pp - 1));
    return *reinterpret_cast<const u32x4*>(rg + (int64_t)d * DP + kc * 8);
  };
  auto put_k = [&](u32x4 x) { sm.k[swz(kr, kc)] = x; };
  auto put_v = [&](u32x4 x) {
    u32x2* dst = reinterpret_cast<u32x2*>(&sm.vt[vd * VST + vc * 8]);
    dst[0] = u32x2{x[0], x[1]};
    dst[1] = u32x2{x[2], x[3]};
  };
  auto put_r = [&](int32_t chunk_id, u32x4 x) {
    int slot = ((chunk_id % RK_SLOTS) + RK_SLOTS) % RK_SLOTS;
    sm.rk[slot][swz(kr, kc)] = x;
  };

  // ---- per-wave query operands: (q+u)*c and (q+v)*c as bf16, d = 16s + 8hf + e.
  // u and v of this head are staged once in LDS, zero-padded to 64 columns.
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

  float* bdw = sm.bd[wave];
  // BDw^T chunk for `chunk_id` (rows w = delta - first row) -> window slot X.
  auto bd_chunk = [&](int32_t chunk_id, int X, bool mirror) {
    const int slot = ((chunk_id % RK_SLOTS) + RK_SLOTS) % RK_SLOTS;
    floatx16 acc = floatx16{0};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 ar = __builtin_bit_cast(bf16x8, sm.rk[slot][swz(ii, 2 * s + hf)]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ar, qv[s], acc, 0, 0, 0);
    }
    // lane holds rows w = 8g + 4hf + r of column ii
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      floatx4 v4 = floatx4{acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
      *reinterpret_cast<floatx4*>(&bdw[ii * BDS + X + 8 * g + 4 * hf]) = v4;
      if (mirror) *reinterpret_cast<floatx4*>(&bdw[ii * BDS + X + 64 + 8 * g + 4 * hf]) = v4;
    }
  };

  // ---- prologue: Rk chunks t_lo-4 .. t_lo, K/V tile t_lo
  if (t_lo < t_hi) {
#pragma unroll
    for (int c = 0; c < RK_SLOTS; ++c) put_r(t_lo - 4 + c, load_r(t_lo - 4 + c));
    put_k(load_k(t_lo));
    put_v(load_v(t_lo));
  }
  __syncthreads();
  if (wave_on && t_lo < t_wave_end && t_lo < t_hi) bd_chunk(t_lo - wave - 1, 32, false);

  floatx16 o[2] = {floatx16{0}, floatx16{0}};
  float m_ref = kNegInf, l_sum = 0.0f;

  for (int32_t tb = t_lo; tb < t_hi; ++tb) {
    const bool more = tb + 1 < t_hi;
    u32x4 nk, nv, nr;
    if (more) {
      nk = load_k(tb + 1);
      nv = load_v(tb + 1);
      nr = load_r(tb + 1);
    }
    if (wave_on && tb < t_wave_end) {
      const int tl = tb - t_lo;
      const int X = (tl & 1) ? 32 : 0;
      bd_chunk(tb - wave, X, (tl & 1) == 0);
      wave_lds_fence();
      // shifted (b)+(d): key jj = 8g + 4hf + r reads position X + 31 + ii - jj
      floatx16 s;
      const float* rbase = &bdw[ii * BDS + X + 4 + ii - 4 * hf];
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r) s[4 * g + r] = rbase[8 * (3 - g) + (3 - r)];
      // (q+u).K on top
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        bf16x8 ak = __builtin_bit_cast(bf16x8, sm.k[swz(ii, 2 * st + hf)]);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qu[st], s, 0, 0, 0);
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
      mb = fmaxf(mb, __shfl_xor(mb, 32));
      const bool need = mb > m_ref + 8.0f;
      if (__ballot(need)) {
        const float alpha = need ? __builtin_amdgcn_exp2f(m_ref - mb) : 1.0f;
        if (need) m_ref = mb;
        l_sum *= alpha;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          o[0][e] *= alpha;
          o[1][e] *= alpha;
        }
      }
      const float m_use = (m_ref == kNegInf) ? 0.0f : m_ref;
      float p[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        p[e] = __builtin_amdgcn_exp2f(s[e] - m_use);
        l_sum += p[e];
      }
      // P^T (keys x queries) times V^T: k-slot order (16t2 + 4hf + r, 16t2 + 8 + 4hf + r)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const bf16x8 pb = pack8(&p[8 * t2]);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int d = 32 * e + ii;
          const u32x2 lo = *reinterpret_cast<const u32x2*>(&sm.vt[d * VST + 16 * t2 + 4 * hf]);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(&sm.vt[d * VST + 16 * t2 + 8 + 4 * hf]);
          const bf16x8 av = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
          o[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb, o[e], 0, 0, 0);
        }
      }
    }
    __syncthreads();
    if (more) {
      put_k(nk);
      put_v(nv);
      put_r(tb + 1, nr);
    }
    __syncthreads();
  }

  if (!wave_on) return;
  l_sum += __shfl_xor(l_sum, 32);
  const int32_t i = i0 + ii;
  // lane holds d = 32e + 8g + 4hf + r (r = 0..3): four consecutive columns per (e, g)
  if (a.n_split == 1) {
    if (i >= L) return;
    const float inv = 1.0f / l_sum;
    uint16_t* out = static_cast<uint16_t*>(a.out) + (((int64_t)b * L + i) * a.H + head) * a.dh;
    const bool vec = (a.dh == DP);
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * e + 8 * g + 4 * hf;
        if (vec) {
          typedef float floatx2_t __attribute__((ext_vector_type(2)));
          typedef bf16 bf16x2_t __attribute__((ext_vector_type(2)));
          const bf16x2_t lo = __builtin_convertvector(
              floatx2_t{o[e][4 * g] * inv, o[e][4 * g + 1] * inv}, bf16x2_t);
          const bf16x2_t hi = __builtin_convertvector(
              floatx2_t{o[e][4 * g + 2] * inv, o[e][4 * g + 3] * inv}, bf16x2_t);
          *reinterpret_cast<u32x2*>(out + d0) =
              u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (d0 + r < a.dh) out[d0 + r] = f32_to_bf16_bits(o[e][4 * g + r] * inv);
        }
      }
  } else {
    const int64_t row = (int64_t)split * a.B * a.H * a.Lp + (int64_t)bh * a.Lp + i;
    floatx4* po = reinterpret_cast<floatx4*>(a.part_o + row * DP);
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        po[(32 * e + 8 * g + 4 * hf) / 4] =
            floatx4{o[e][4 * g], o[e][4 * g + 1], o[e][4 * g + 2], o[e][4 * g + 3]};
    if (hf == 0) a.part_ml[row * 2 + 0] = m_ref;
    if (hf == 0) a.part_ml[row * 2 + 1] = l_sum;
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
