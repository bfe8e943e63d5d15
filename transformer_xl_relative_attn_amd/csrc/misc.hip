// Memory-bound helpers of the segment step: the sinusoid table R, the memory
// ring update, operand packing, LayerNorm and small casts.
#include "dev_common.h"

namespace txl {

namespace {

// R[delta][2k] = sin(delta / 10000^(2k/d)), R[delta][2k+1] = cos(same):
// Transformer-XL Sec. 3.3 takes R to be Vaswani et al.'s sinusoid matrix.
// Evaluated in fp64, rounded once to the storage dtype: fp32 directly; bf16
// through fp32 rounded to odd (truncate, then set the last bit if inexact),
// whose 24 bits keep the information the final round-to-nearest-even needs,
// so the result is the correctly rounded bf16 of the fp64 value.
__global__ void sinusoid_kernel(void* R, int32_t n_pos, int32_t d, int32_t dtype) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)n_pos * d) return;
  const int32_t pos = idx / d, c = idx % d;
  const int32_t k2 = c & ~1;
  const double inv = pow(10000.0, -(double)k2 / (double)d);
  const double ang = (double)pos * inv;
  const double val = (c & 1) ? cos(ang) : sin(ang);
  if (dtype == TXL_F32) {
    static_cast<float*>(R)[idx] = (float)val;
    return;
  }
  float f = __double2float_rz(val);
  if ((double)f != val) f = __uint_as_float(__float_as_uint(f) | 1u);
  static_cast<uint16_t*>(R)[idx] = f32_to_bf16_bits(f);
}

// Ring update (Transformer-XL Sec. 3.2, memory of the M most recent states):
// slot (start + t) mod M <- h row t for t < L (case L < M), or slot p <- h row
// L - M + p (case L >= M, start then 0).  Copies 16-byte words when aligned.
__global__ void mem_update_kernel(char* mem, int32_t start, const char* h, int32_t B, int32_t M,
                                  int32_t L, int64_t row_bytes, int32_t vec) {
  const int32_t n_rows = min(L, M);
  const int64_t words = row_bytes / vec;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)B * n_rows * words) return;
  const int64_t w = idx % words;
  const int64_t rt = idx / words;
  const int32_t t = rt % n_rows;
  const int32_t b = rt / n_rows;
  int32_t slot, src;
  if (L < M) {
    slot = (start + t) % M;
    src = t;
  } else {
    slot = t;
    src = L - M + t;
  }
  char* dst = mem + ((int64_t)b * M + slot) * row_bytes + w * vec;
  const char* s = h + ((int64_t)b * L + src) * row_bytes + w * vec;
  if (vec == 16)
    *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(s);
  else if (vec == 4)
    *reinterpret_cast<uint32_t*>(dst) = *reinterpret_cast<const uint32_t*>(s);
  else
    *reinterpret_cast<uint16_t*>(dst) = *reinterpret_cast<const uint16_t*>(s);
}

// dst[r][c] = src[r][c] for c < cols, 0 for cols <= c < ld_dst.
__global__ void pack_rows_kernel(uint16_t* dst, int64_t ld_dst, const uint16_t* src, int64_t ld_src,
                                 int64_t rows, int32_t cols) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= rows * ld_dst) return;
  const int64_t r = idx / ld_dst, c = idx % ld_dst;
  dst[idx] = c < cols ? src[r * ld_src + c] : uint16_t(0);
}

// Grouped packs: wave w of workgroup b copies global row 4b + w (of the job
// whose row range holds it), one word (2 or 4 bytes) per lane and pass.  The
// job that packs the memory ring may also carry the ring update (Sec. 3.2):
// each lane overwrites exactly the words of the ring row it has just read.
constexpr int kPackRowsPerBlock = 4;
template <class T>
__device__ __forceinline__ void pack_row(const PackGroup& g, int j, int64_t row, int lane) {
  constexpr int E = sizeof(T) / 2;   // bf16 elements per word
  const PackJob& J = g.job[j];
  T* src = reinterpret_cast<T*>(const_cast<void*>(J.src)) + row * (J.ld_src / E);
  T* dst = static_cast<T*>(J.dst) + row * (J.ld_dst / E);
  const int64_t wd = J.ld_dst / E, ws = J.cols / E;
  const T* hrow = nullptr;
  if (j == g.ring_job) {
    const int32_t M = g.ring_M, L = g.ring_L;
    const int32_t b = (int32_t)(row / M), slot = (int32_t)(row - (int64_t)b * M);
    int32_t t;
    if (L < M) {
      t = slot - g.ring_start;
      if (t < 0) t += M;
    } else {
      t = L - M + slot;
    }
    if (t < L) hrow = static_cast<const T*>(g.ring_h) + ((int64_t)b * L + t) * ws;
  }
  // four words per lane and pass, all loads of a pass issued before its stores
  for (int64_t c0 = lane; c0 < wd; c0 += 256) {
    T x[4], y[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t c = c0 + 64 * u;
      x[u] = c < ws ? src[c] : T(0);
      y[u] = (hrow && c < ws) ? hrow[c] : T(0);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t c = c0 + 64 * u;
      if (c < wd) dst[c] = x[u];
      if (hrow && c < ws) src[c] = y[u];
    }
  }
}

__global__ __launch_bounds__(256) void pack_group_kernel(PackGroup g) {
  const int64_t r = (int64_t)blockIdx.x * kPackRowsPerBlock + (threadIdx.x >> 6);
  if (r >= g.row_begin[g.n]) return;
  int j = 0;
#pragma unroll
  for (int i = 1; i < kMaxPackJobs; ++i)
    if (i < g.n && r >= g.row_begin[i]) j = i;
  const int64_t row = r - g.row_begin[j];
  if (g.words4)
    pack_row<uint32_t>(g, j, row, threadIdx.x & 63);
  else
    pack_row<uint16_t>(g, j, row, threadIdx.x & 63);
}

// Sum over the 256 threads of a workgroup (fixed order: deterministic).
__device__ __forceinline__ float block_sum256(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  __syncthreads();   // red may still be read from the previous sum
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// LayerNorm (no affine parameters, fp32 statistics) of x = resid + sum of
// n_parts split-K partial products (each [rows][d], part_stride floats apart),
// one workgroup per row.  Writes fp32 y and, if y_lo is set, a copy in
// lo_dtype.  VPT > 0 keeps the row in registers (d <= 256 * VPT); VPT == 0
// uses y as the staging buffer (y must not overlap the inputs).
template <int VPT>
__global__ __launch_bounds__(256) void layernorm_kernel(const float* resid, const float* parts,
                                                        int32_t n_parts, int64_t part_stride,
                                                        float* y, void* y_lo, int32_t d,
                                                        int32_t lo_dtype, float eps) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  auto load_x = [&](int c) {
    float v = resid[row * d + c];
    for (int s = 0; s < n_parts; ++s) v += parts[s * part_stride + row * d + c];
    return v;
  };
  if constexpr (VPT > 0) {
    float x[VPT];
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int c = tid + 256 * k;
      x[k] = c < d ? load_x(c) : 0.0f;
      s += x[k];
    }
    const float mean = block_sum256(s, red) / d;
    float s2 = 0.0f;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int c = tid + 256 * k;
      const float dv = c < d ? x[k] - mean : 0.0f;
      s2 += dv * dv;
    }
    const float rstd = rsqrtf(block_sum256(s2, red) / d + eps);
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int c = tid + 256 * k;
      if (c < d) {
        const float v = (x[k] - mean) * rstd;
        y[row * d + c] = v;
        if (y_lo) store_from_f32(y_lo, row * d + c, v, lo_dtype);
      }
    }
  } else {
    float* yr = y + row * d;
    float s = 0.0f;
    for (int c = tid; c < d; c += 256) {
      const float v = load_x(c);
      yr[c] = v;
      s += v;
    }
    const float mean = block_sum256(s, red) / d;
    float s2 = 0.0f;
    for (int c = tid; c < d; c += 256) {
      const float dv = yr[c] - mean;
      s2 += dv * dv;
    }
    const float rstd = rsqrtf(block_sum256(s2, red) / d + eps);
    for (int c = tid; c < d; c += 256) {
      const float v = (yr[c] - mean) * rstd;
      yr[c] = v;
      if (y_lo) store_from_f32(y_lo, row * d + c, v, lo_dtype);
    }
  }
}

// The same LayerNorm for rows of d <= 4096 floats with d % 4 == 0 and 16-byte
// aligned operands: each thread owns the float4 chunks tid + 256k of its row
// and issues the residual load and all NP partial loads of a chunk before it
// adds them (residual first, then part 0, 1, ..., as layernorm_kernel), so
// every load of a row is in flight at once instead of one after another.
template <int NP>
__global__ __launch_bounds__(256) void layernorm_vec_kernel(const float* resid, const float* parts,
                                                            int64_t part_stride, float* y,
                                                            void* y_lo, int32_t d,
                                                            int32_t lo_dtype, float eps) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int n4 = d >> 2;
  floatx4 x[4];
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int c4 = tid + 256 * k;
    x[k] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    if (c4 < n4) {
      const int64_t off = row * d + 4 * c4;
      floatx4 ld[NP + 1];
      ld[0] = *reinterpret_cast<const floatx4*>(resid + off);
#pragma unroll
      for (int p = 0; p < NP; ++p) ld[p + 1] = *reinterpret_cast<const floatx4*>(parts + p * part_stride + off);
      floatx4 v = ld[0];
#pragma unroll
      for (int p = 0; p < NP; ++p) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] += ld[p + 1][e];
      }
      x[k] = v;
      s += (v[0] + v[1]) + (v[2] + v[3]);
    }
  }
  const float mean = block_sum256(s, red) / d;
  float s2 = 0.0f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (tid + 256 * k < n4) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float dv = x[k][e] - mean;
        s2 += dv * dv;
      }
    }
  }
  const float rstd = rsqrtf(block_sum256(s2, red) / d + eps);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int c4 = tid + 256 * k;
    if (c4 < n4) {
      const int64_t off = row * d + 4 * c4;
      floatx4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (x[k][e] - mean) * rstd;
      *reinterpret_cast<floatx4*>(y + off) = v;
      if (y_lo) {
        if (lo_dtype == TXL_F32) {
          *reinterpret_cast<floatx4*>(static_cast<float*>(y_lo) + off) = v;
        } else {
          const uint32_t lo = f32_to_bf16_bits(v[0]) | (uint32_t)f32_to_bf16_bits(v[1]) << 16;
          const uint32_t hi = f32_to_bf16_bits(v[2]) | (uint32_t)f32_to_bf16_bits(v[3]) << 16;
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(y_lo) + off) = make_uint2(lo, hi);
        }
      }
    }
  }
}

__global__ void cast_f32_kernel(const void* src, float* dst, int64_t n, int32_t dtype) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx < n) dst[idx] = load_as_f32(src, idx, dtype);
}

// Public Rk layout [P][H][dh] -> workspace layout [H][Pp][dp] (zero padded).
// Caller's Rk [P][H][dh] -> workspace [H][pad + Pp + pad][dp] (rows p >= P and
// columns c >= dh zero; the padding rows are left as they are).
__global__ void repack_rk_kernel(const void* src, void* dst, int32_t P, int32_t Pp, int32_t pad,
                                 int32_t H, int32_t dh, int32_t dp, int32_t dtype) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)H * Pp * dp) return;
  const int32_t c = idx % dp;
  const int64_t t = idx / dp;
  const int32_t p = t % Pp;
  const int32_t h = t / Pp;
  float x = 0.0f;
  if (p < P && c < dh) x = load_as_f32(src, ((int64_t)p * H + h) * dh + c, dtype);
  store_from_f32(dst, ((int64_t)h * (Pp + 2 * pad) + pad + p) * dp + c, x, dtype);
}

// bf16 with dh == dp: one 16-byte chunk (8 columns) per thread, 32-bit index
// arithmetic (the element-wise kernel's 64-bit divisions dominated its time)
__global__ void repack_rk_vec_kernel(const uint16_t* src, uint16_t* dst, int32_t P, int32_t Pp,
                                     int32_t pad, int32_t H, int32_t dp) {
  const int32_t cpr = dp / 8;
  const int32_t idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= H * Pp * cpr) return;
  const int32_t c = idx % cpr, t = idx / cpr;
  const int32_t p = t % Pp, h = t / Pp;
  u32x4 x = u32x4{0u, 0u, 0u, 0u};
  if (p < P) x = *reinterpret_cast<const u32x4*>(src + ((int64_t)p * H + h) * dp + 8 * c);
  *reinterpret_cast<u32x4*>(dst + ((int64_t)h * (Pp + 2 * pad) + pad + p) * dp + 8 * c) = x;
}

inline dim3 grid1d(int64_t n) { return dim3((unsigned)((n + 255) / 256)); }

// Matrix-core probe: each wave loads 24 bf16 operand fragments (16 bytes per
// lane each) and issues `iters` rounds of 16 independent 32x32x16 products
// on them (operands rotate between rounds; iters is even).  Wave 0 of each
// workgroup records the shader-clock cycles and 100 MHz reference ticks its
// loop took (it may finish before the other wave of its SIMD), so the caller
// can read the clock the matrix cores ran at.
__global__ __launch_bounds__(512, 1) void mfma_probe_kernel(const u32x4* operands, int32_t iters,
                                                            uint64_t* clocks) {
  const int tid = threadIdx.x;
  const u32x4* src = operands + ((int64_t)blockIdx.x * 512 + tid) * 24;
  bf16x8 f[24];
#pragma unroll
  for (int i = 0; i < 24; ++i) f[i] = __builtin_bit_cast(bf16x8, src[i]);
  floatx16 acc[8];
#pragma unroll
  for (int x = 0; x < 8; ++x) acc[x] = floatx16{0};
  __syncthreads();
  const uint64_t c0 = __builtin_amdgcn_s_memtime(), t0 = __builtin_amdgcn_s_memrealtime();
  for (int32_t it = 0; it < iters; it += 2) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int x = 0; x < 16; ++x)
        acc[x & 7] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[(3 * x + 7 * h) % 24],
                                                             f[(5 * x + 11 + h) % 24], acc[x & 7], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int x = 0; x < 8; ++x) s += acc[x][0];
  const uint64_t c1 = __builtin_amdgcn_s_memtime(), t1 = __builtin_amdgcn_s_memrealtime();
  if (tid == 0) {
    clocks[2 * blockIdx.x] = c1 - c0;
    clocks[2 * blockIdx.x + 1] = t1 - t0;
  }
  // keeps the products live (entry 2 * n_wg is a sink nobody reads)
  if (s == 12345.0f) clocks[2 * gridDim.x] = 1;
}

}  // namespace

int launch_mfma_probe(const void* operands, int32_t n_wg, int32_t iters, uint64_t* clocks,
                      void* stream) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(n_wg), dim3(512), 0, (hipStream_t)stream,
                     static_cast<const u32x4*>(operands), iters, clocks);
  return (int)hipGetLastError();
}

int launch_sinusoid(void* R, int32_t n_pos, int32_t d_pos, int32_t dtype, void* stream) {
  const int64_t n = (int64_t)n_pos * d_pos;
  hipLaunchKernelGGL(sinusoid_kernel, grid1d(n), dim3(256), 0, static_cast<hipStream_t>(stream),
                     R, n_pos, d_pos, dtype);
  return static_cast<int>(hipGetLastError());
}

int launch_mem_update(void* mem, int32_t start, const void* h, int32_t B, int32_t M, int32_t L,
                      int32_t d, int32_t dtype, void* stream) {
  if (M == 0) return 0;
  const int esize = dtype == TXL_F32 ? 4 : 2;
  const int64_t row_bytes = (int64_t)d * esize;
  const uintptr_t align = reinterpret_cast<uintptr_t>(mem) | reinterpret_cast<uintptr_t>(h) |
                          static_cast<uintptr_t>(row_bytes);
  const int vec = (align % 16 == 0) ? 16 : (align % 4 == 0) ? 4 : 2;
  const int64_t n = (int64_t)B * (L < M ? L : M) * (row_bytes / vec);
  hipLaunchKernelGGL(mem_update_kernel, grid1d(n), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<char*>(mem), start, static_cast<const char*>(h), B, M, L,
                     row_bytes, vec);
  return static_cast<int>(hipGetLastError());
}

int launch_pack_rows(void* dst, int64_t ld_dst, const void* src, int64_t ld_src, int64_t rows,
                     int32_t cols, int32_t dtype, void* stream) {
  (void)dtype;  // bf16 only
  const int64_t n = rows * ld_dst;
  if (n == 0) return 0;
  hipLaunchKernelGGL(pack_rows_kernel, grid1d(n), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<uint16_t*>(dst), ld_dst, static_cast<const uint16_t*>(src),
                     ld_src, rows, cols);
  return static_cast<int>(hipGetLastError());
}

int launch_pack_group(const PackGroup& g, void* stream) {
  const int64_t rows = g.row_begin[g.n];
  if (rows == 0) return 0;
  const int64_t blocks = (rows + kPackRowsPerBlock - 1) / kPackRowsPerBlock;
  hipLaunchKernelGGL(pack_group_kernel, dim3((uint32_t)blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), g);
  return static_cast<int>(hipGetLastError());
}

int launch_layernorm(const float* resid, const float* parts, int32_t n_parts, int64_t part_stride,
                     float* y_f32, void* y_lo, int32_t rows, int32_t d, int32_t lo_dtype, float eps,
                     void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  const bool vec = d % 4 == 0 && d <= 4096 && n_parts >= 0 && n_parts <= 8 && al16(resid) &&
                   (n_parts == 0 || (al16(parts) && part_stride % 4 == 0)) && al16(y_f32) &&
                   (y_lo == nullptr || al16(y_lo));
  if (vec) {
#define TXL_LN_VEC(NP)                                                                          \
  case NP:                                                                                     \
    hipLaunchKernelGGL(layernorm_vec_kernel<NP>, dim3(rows), dim3(256), 0, st, resid, parts,   \
                       part_stride, y_f32, y_lo, d, lo_dtype, eps);                            \
    break;
    switch (n_parts) {
      TXL_LN_VEC(0) TXL_LN_VEC(1) TXL_LN_VEC(2) TXL_LN_VEC(3) TXL_LN_VEC(4)
      TXL_LN_VEC(5) TXL_LN_VEC(6) TXL_LN_VEC(7) TXL_LN_VEC(8)
    }
#undef TXL_LN_VEC
  } else if (d <= 1024)
    hipLaunchKernelGGL(layernorm_kernel<4>, dim3(rows), dim3(256), 0, st, resid, parts, n_parts,
                       part_stride, y_f32, y_lo, d, lo_dtype, eps);
  else if (d <= 4096)
    hipLaunchKernelGGL(layernorm_kernel<16>, dim3(rows), dim3(256), 0, st, resid, parts, n_parts,
                       part_stride, y_f32, y_lo, d, lo_dtype, eps);
  else
    hipLaunchKernelGGL(layernorm_kernel<0>, dim3(rows), dim3(256), 0, st, resid, parts, n_parts,
                       part_stride, y_f32, y_lo, d, lo_dtype, eps);
  return static_cast<int>(hipGetLastError());
}

int launch_cast_f32(const void* src, float* dst, int64_t n, int32_t dtype, void* stream) {
  hipLaunchKernelGGL(cast_f32_kernel, grid1d(n), dim3(256), 0, static_cast<hipStream_t>(stream),
                     src, dst, n, dtype);
  return static_cast<int>(hipGetLastError());
}

int launch_repack_rk(const void* rk_pub, void* rk_ws, int32_t P, int32_t Pp, int32_t pad, int32_t H,
                     int32_t dh, int32_t dp, int32_t dtype, void* stream) {
  const int64_t n = (int64_t)H * Pp * dp;
  const bool vec = dtype == TXL_BF16 && dh == dp && dp % 8 == 0 && n / 8 < INT32_MAX &&
                   (reinterpret_cast<uintptr_t>(rk_pub) | reinterpret_cast<uintptr_t>(rk_ws)) % 16 == 0;
  if (vec)
    hipLaunchKernelGGL(repack_rk_vec_kernel, grid1d(n / 8), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint16_t*>(rk_pub),
                       static_cast<uint16_t*>(rk_ws), P, Pp, pad, H, dp);
  else
    hipLaunchKernelGGL(repack_rk_kernel, grid1d(n), dim3(256), 0, static_cast<hipStream_t>(stream),
                       rk_pub, rk_ws, P, Pp, pad, H, dh, dp, dtype);
  return static_cast<int>(hipGetLastError());
}

}  // namespace txl
