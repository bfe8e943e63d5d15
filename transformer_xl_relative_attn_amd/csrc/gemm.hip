// Projection GEMMs of the relative-attention layer:
//   q = h W_q^T, k = h~ W_kE^T, val^T = W_v h~^T, Rk = R W_kR^T, and (full
//   layer) Linear(a), FFN.  Every product has the form C[m][n] = sum_k A(m,k) B(n,k)
//   with both operands K-contiguous; rows are fetched through RowSrc maps so
//   that h~ = [memory ring ; segment] is gathered on the fly.
//
// gemm_bf16: bf16 operands, fp32 accumulation on the gfx950 matrix cores
//   (v_mfma_f32_32x32x16_bf16).  256x256x64 block tile, 4 waves in a 2x2
//   grid, each wave owns a 128x128 sub-tile (4x4 MFMA tiles, 256 accumulator
//   registers).  Operand tiles are double-buffered in LDS; each 16-byte chunk
//   of a 128-byte LDS row is XOR-swizzled by (row & 7) so the MFMA operand
//   reads (8 consecutive rows, same chunk) hit distinct banks.  Requirements
//   (checked by the host): K % 64 == 0, every row 16-byte aligned.
//
// gemm_f32: fp32 operands and arithmetic on the vector ALUs (64x64 tile),
//   used by the fp32 path.
#include "dev_common.h"

namespace txl {

namespace {

constexpr int BM = 256, BN = 256, BK = 64, NT = 256;
constexpr int CHUNKS = BK / 8;           // 16-byte chunks per tile row (8)
constexpr int LOADS = BM * CHUNKS / NT;  // chunks per thread per operand (8)

__device__ __forceinline__ const GemmProblem* find_problem(const GemmGroup& g, int32_t tile,
                                                           int32_t* local) {
  int idx = 0;
#pragma unroll
  for (int i = 1; i < kMaxGroup; ++i)
    if (i < g.count && tile >= g.p[i].tile_begin) idx = i;
  *local = tile - g.p[idx].tile_begin;
  return &g.p[idx];
}

__global__ __launch_bounds__(NT, 1) void gemm_bf16_kernel(GemmGroup g, int32_t padded) {
  const int32_t tile = xcd_swizzle(blockIdx.x, padded);
  if (tile >= g.total_tiles) return;
  int32_t local;
  const GemmProblem& P = *find_problem(g, tile, &local);
  // consecutive tiles share the A rows (tm), sweeping n fastest
  const int32_t tm = local / P.tiles_n, tn = local - tm * P.tiles_n;
  const int32_t m0 = tm * BM, n0 = tn * BN;

  __shared__ u32x4 smA[2][BM * CHUNKS];
  __shared__ u32x4 smB[2][BN * CHUNKS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // Rows this thread stages: row = tid/8 + 32*i, chunk = tid%8.
  const int chunk = tid & 7;
  const char* pa[LOADS];
  const char* pb[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    int r = (tid >> 3) + 32 * i;
    pa[i] = (m0 + r < P.M) ? row_address(P.a, m0 + r, 2) : nullptr;
    pb[i] = (n0 + r < P.N) ? row_address(P.b, n0 + r, 2) : nullptr;
    if (pa[i]) pa[i] += chunk * 16;
    if (pb[i]) pb[i] += chunk * 16;
  }

  u32x4 ra[LOADS], rb[LOADS];
  auto gload = [&](int kt) {
    const int64_t koff = (int64_t)kt * BK * 2;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      ra[i] = pa[i] ? *reinterpret_cast<const u32x4*>(pa[i] + koff) : u32x4{0, 0, 0, 0};
      rb[i] = pb[i] ? *reinterpret_cast<const u32x4*>(pb[i] + koff) : u32x4{0, 0, 0, 0};
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      int r = (tid >> 3) + 32 * i;
      int pos = r * CHUNKS + (chunk ^ (r & 7));
      smA[buf][pos] = ra[i];
      smB[buf][pos] = rb[i];
    }
  };

  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx16{0};

  const int nk = P.K / BK;
  gload(0);
  lstore(0);
  __syncthreads();

  const int lrow = lane & 31, lhalf = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      bf16x8 af[4], bfr[4];
      const int c = 2 * s + lhalf;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int ra_ = wm * 128 + i * 32 + lrow;
        int rb_ = wn * 128 + i * 32 + lrow;
        af[i] = __builtin_bit_cast(bf16x8, smA[buf][ra_ * CHUNKS + (c ^ (ra_ & 7))]);
        bfr[i] = __builtin_bit_cast(bf16x8, smB[buf][rb_ * CHUNKS + (c ^ (rb_ & 7))]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) {
      lstore(buf ^ 1);
      __syncthreads();
    }
  }

  // Epilogue: acc[i][j] element e -> row m = 8*(e/4) + 4*lhalf + e%4, col n = lrow.
  const OutDst& o = P.out;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int32_t n = n0 + wn * 128 + j * 32 + lrow;
    if (n >= o.n_valid) continue;
    const int64_t coff = axis_off(o.col, n);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int32_t m = m0 + wm * 128 + i * 32 + 8 * (e >> 2) + 4 * lhalf + (e & 3);
        if (m < o.m_valid) epi_store(o, axis_off(o.row, m) + coff, acc[i][j][e]);
      }
    }
  }
}

// ------------------------------------------------------------------ fp32 GEMM
constexpr int FT = 64, FK = 16;

__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmGroup g, int32_t padded) {
  const int32_t tile = xcd_swizzle(blockIdx.x, padded);
  if (tile >= g.total_tiles) return;
  int32_t local;
  const GemmProblem& P = *find_problem(g, tile, &local);
  const int32_t tm = local / P.tiles_n, tn = local - tm * P.tiles_n;
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
      if (n < o.n_valid) epi_store(o, roff + axis_off(o.col, n), acc[i][j]);
    }
  }
}

}  // namespace

int launch_gemm_bf16(const GemmGroup& g, void* stream) {
  if (g.total_tiles <= 0) return 0;
  int32_t padded = (g.total_tiles + 7) & ~7;
  hipLaunchKernelGGL(gemm_bf16_kernel, dim3(padded), dim3(NT), 0,
                     static_cast<hipStream_t>(stream), g, padded);
  return static_cast<int>(hipGetLastError());
}

int launch_gemm_f32(const GemmGroup& g, void* stream) {
  if (g.total_tiles <= 0) return 0;
  int32_t padded = (g.total_tiles + 7) & ~7;
  hipLaunchKernelGGL(gemm_f32_kernel, dim3(padded), dim3(256), 0,
                     static_cast<hipStream_t>(stream), g, padded);
  return static_cast<int>(hipGetLastError());
}

}  // namespace txl
