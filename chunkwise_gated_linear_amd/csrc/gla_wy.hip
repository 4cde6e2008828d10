// WY-representation forward of the gated delta rule on the chunk skeleton of
// this library (page "fla/ops/gated_delta_rule/backends/triton_ascend/
// wy_fast.py", recompute_w_u_fwd_kernel_npu and recompute_w_u_fwd_npu).
//
// For chunk c (64 tokens, restarting at each packed sequence) and value head
// hv, with A[i][j] the chunk's 64 x 64 matrix (row i stored with token i):
//
//   u[i] = sum_j A[i][j] beta_j v_j                 (V columns)
//   w[i] = sum_j A[i][j] beta_j 2^{g_j} k_j         (K columns; k of key head hv / G;
//                                                    the factor 2^g only when g is given)
//
// Rows past the chunk's tokens are zero operands, so A's columns past them add
// nothing, and their output rows are not stored.
//
// gla_wy_fwd: one workgroup of 4 waves per (chunk slot, value head), slots
// numbered as the segments of one chunk of the forward (gla_segment_plan with
// R = 1 for packed inputs).  A and one 64-column block of the scaled operand
// are staged in LDS, so several workgroups share a compute unit and hide each
// other's loads.  Products are taken transposed (rows: operand columns,
// columns: tokens) so that each lane holds four consecutive output columns of
// one token and stores them at once: v_mfma_f32_16x16x4f32 for fp32 inputs,
// v_mfma_f32_16x16x32_bf16 with a hi/lo split of the scaled operand for bf16.
#include <hip/hip_runtime.h>

#include "gla_device.h"

namespace gla {
namespace {

using namespace dev;

__device__ __forceinline__ f32x4_t zero4() { return f32x4_t{0.f, 0.f, 0.f, 0.f}; }

// [64][64] fp32 tile, 16-byte groups of a row XOR-swizzled by the row's low 4
// bits (float4 reads of 16 rows, and scalar reads of 4 rows 4 apart x 16
// columns, each touch 64 banks).
__device__ __forceinline__ int swz64(int row, int col) {
  return row * 64 + ((((col >> 2) ^ (row & 15))) << 2 | (col & 3));
}
__device__ __forceinline__ f32x4_t lds4(const float *a, int row, int col) {
  return *reinterpret_cast<const f32x4_t *>(a + row * 64 + (((col >> 2) ^ (row & 15)) << 2));
}
__device__ __forceinline__ void lds4_st(float *a, int row, int col, f32x4_t x) {
  *reinterpret_cast<f32x4_t *>(a + row * 64 + (((col >> 2) ^ (row & 15)) << 2)) = x;
}

template <bool BF>
__device__ __forceinline__ f32x4_t ld4(const void *base, int64_t i) {  // i a multiple of 4
  if constexpr (BF) {
    const u32x2_t w = *reinterpret_cast<const u32x2_t *>(reinterpret_cast<const uint16_t *>(base) + i);
    return f32x4_t{bf_lo(w[0]), bf_hi(w[0]), bf_lo(w[1]), bf_hi(w[1])};
  } else {
    return *reinterpret_cast<const f32x4_t *>(reinterpret_cast<const float *>(base) + i);
  }
}
template <bool BF>
__device__ __forceinline__ void st4(void *base, int64_t i, f32x4_t x) {  // i a multiple of 4
  if constexpr (BF) {
    u32x2_t wv;
    wv[0] = pack_bf16(x[0], x[1]);
    wv[1] = pack_bf16(x[2], x[3]);
    *reinterpret_cast<u32x2_t *>(reinterpret_cast<uint16_t *>(base) + i) = wv;
  } else {
    *reinterpret_cast<f32x4_t *>(reinterpret_cast<float *>(base) + i) = x;
  }
}

template <bool BF>
__global__ __launch_bounds__(256) void gla_wy_fwd_kernel(WyParams wp) {
  const WalkParams &p = wp.w;
  __shared__ __attribute__((aligned(16))) float sA[64 * 64];  // A[i][j] of the chunk
  __shared__ __attribute__((aligned(16))) float sX[64 * 64];  // scaled operand rows [j][col]
  __shared__ float sS[2][64];                                 // beta_j, beta_j 2^{g_j}

  const int hv = (int)(blockIdx.x % (unsigned)p.HV);
  const int slot = (int)(blockIdx.x / (unsigned)p.HV);
  SegInfo si;
  if (!locate(p, slot, si)) return;
  const int nch = (si.len + kChunk - 1) / kChunk;
  if (si.s >= nch) return;
  const int L = min(kChunk, si.len - kChunk * si.s);
  const int64_t row0 = si.bos + (int64_t)kChunk * si.s;
  const int h = hv / p.G;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l16 = lane & 15, lg = lane >> 4;

  // A rows (4 quads per thread) and the row scales
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int e = threadIdx.x + 256 * t, i = e >> 4, c4 = (e & 15) * 4;
    f32x4_t x = zero4();
    if (i < L) x = ld4<BF>(wp.A, ((row0 + i) * p.HV + hv) * kChunk + c4);
    lds4_st(sA, i, c4, x);
  }
  if (threadIdx.x < 64) {
    const int j = threadIdx.x;
    const float b = j < L ? wp.beta[(row0 + j) * p.HV + hv] : 0.f;
    sS[0][j] = b;
    sS[1][j] = (wp.g != nullptr && j < L) ? b * exp2f(wp.g[(row0 + j) * p.HV + hv]) : b;
  }

  // one output at a time (u over V columns, then w over K columns), in blocks of 64 columns
  for (int which = 0; which < 2; ++which) {
    const int W = which == 0 ? p.V : p.K;
    const void *src = which == 0 ? p.v : p.k;
    void *dst = which == 0 ? wp.u : wp.wout;
    const int64_t srow = which == 0 ? (int64_t)p.HV * p.V : (int64_t)p.H * p.K;  // source row stride
    const int64_t soff = which == 0 ? (int64_t)hv * p.V : (int64_t)h * p.K;      // source head offset
    for (int c0 = 0; c0 < W; c0 += 64) {
      __syncthreads();  // sS / sA ready (first block); sX free (later blocks)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int e = threadIdx.x + 256 * t, j = e >> 4, c4 = (e & 15) * 4;
        f32x4_t x = zero4();
        if (j < L && c0 + c4 < W) {
          x = ld4<BF>(src, (row0 + j) * srow + soff + c0 + c4);
          x *= sS[which][j];
        }
        lds4_st(sX, j, c4, x);
      }
      __syncthreads();
      // D[c][i] = sum_j X[j][c] A[i][j]: wave w takes columns c0 + 16 w .. + 15, all 64 tokens
      f32x4_t acc[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll 4
      for (int j0 = 0; j0 < 64; j0 += 16) {
        float xa[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) xa[r] = sX[swz64(j0 + 4 * lg + r, wave * 16 + l16)];
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) {
          const f32x4_t a4 = lds4(sA, ib * 16 + l16, j0 + 4 * lg);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[ib] = mfma_f32(xa[r], a4[r], acc[ib]);
        }
      }
      const int col = c0 + wave * 16 + 4 * lg;
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) {
        const int i = ib * 16 + l16;
        if (i < L && col < W) st4<BF>(dst, ((row0 + i) * p.HV + hv) * W + col, acc[ib]);
      }
    }
  }
}

// bf16 inputs: v_mfma_f32_16x16x32_bf16.  A is exact in bf16 and is the
// product's right operand as stored; the scaled rows beta v and beta 2^g k
// are fp32 products, split into bf16 hi + lo (hi = the nearest bf16, lo = the
// nearest bf16 of the remainder) so that hi*A + lo*A carries them to fp32
// accuracy.  Both planes are staged transposed, X^T[c][j], so that a lane
// reads its 8 consecutive tokens j with one 16-byte load.  bf16 tiles of
// [64][64] use 16-byte groups XOR-swizzled by 2 ((row >> 2) & 3): the 16-byte
// reads of 16 consecutive rows then fall on distinct banks for each 32 lanes.
__device__ __forceinline__ int bswz(int row, int col) {
  return row * 64 + ((((col >> 3) ^ (2 * ((row >> 2) & 3)))) << 3) + (col & 7);
}

__global__ __launch_bounds__(256) void gla_wy_fwd_kernel_bf16(WyParams wp) {
  const WalkParams &p = wp.w;
  __shared__ __attribute__((aligned(16))) uint16_t sA[64 * 64];   // A[i][j], bf16
  __shared__ __attribute__((aligned(16))) uint16_t sXh[64 * 64];  // X^T[c][j], hi
  __shared__ __attribute__((aligned(16))) uint16_t sXl[64 * 64];  // X^T[c][j], lo
  __shared__ float sS[2][64];                                     // beta_j, beta_j 2^{g_j}

  const int hv = (int)(blockIdx.x % (unsigned)p.HV);
  const int slot = (int)(blockIdx.x / (unsigned)p.HV);
  SegInfo si;
  if (!locate(p, slot, si)) return;
  const int nch = (si.len + kChunk - 1) / kChunk;
  if (si.s >= nch) return;
  const int L = min(kChunk, si.len - kChunk * si.s);
  const int64_t row0 = si.bos + (int64_t)kChunk * si.s;
  const int h = hv / p.G;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l16 = lane & 15, lg = lane >> 4;

  // A rows as stored (2 groups of 8 per thread) and the row scales
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int e = threadIdx.x + 256 * t, i = e >> 3, c8 = (e & 7) * 8;
    u32x4_t x = {0u, 0u, 0u, 0u};
    if (i < L)
      x = *reinterpret_cast<const u32x4_t *>(reinterpret_cast<const uint16_t *>(wp.A) +
                                            ((row0 + i) * p.HV + hv) * kChunk + c8);
    *reinterpret_cast<u32x4_t *>(sA + bswz(i, c8)) = x;
  }
  if (threadIdx.x < 64) {
    const int j = threadIdx.x;
    const float b = j < L ? wp.beta[(row0 + j) * p.HV + hv] : 0.f;
    sS[0][j] = b;
    sS[1][j] = (wp.g != nullptr && j < L) ? b * exp2f(wp.g[(row0 + j) * p.HV + hv]) : b;
  }

  // blocks of 64 output columns: u's first (from v), then w's (from k); the
  // rows of block b + 1 are loaded while block b is formed and stored
  const int nbu = (p.V + 63) / 64, nb = nbu + (p.K + 63) / 64;
  auto block = [&](int b, int &which, int &c0, int &W) {
    which = b < nbu ? 0 : 1;
    c0 = (b < nbu ? b : b - nbu) * 64;
    W = which == 0 ? p.V : p.K;
  };
  auto load_rows = [&](int b, u32x2_t (&xr)[4]) {
    int which, c0, W;
    block(b, which, c0, W);
    const void *src = which == 0 ? p.v : p.k;
    const int64_t srow = which == 0 ? (int64_t)p.HV * p.V : (int64_t)p.H * p.K;  // source row stride
    const int64_t soff = which == 0 ? (int64_t)hv * p.V : (int64_t)h * p.K;      // source head offset
    // thread: tokens 2 m + t % 2 + 32 (t / 2) (m = threadIdx.x / 16), columns
    // c4 .. c4 + 3, so that its two tokens of a pair are staged as one word
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int j = 2 * (threadIdx.x >> 4) + (t & 1) + 32 * (t >> 1), c4 = (threadIdx.x & 15) * 4;
      xr[t] = u32x2_t{0u, 0u};
      if (j < L && c0 + c4 < W)
        xr[t] = *reinterpret_cast<const u32x2_t *>(reinterpret_cast<const uint16_t *>(src) +
                                                  (row0 + j) * srow + soff + c0 + c4);
    }
  };
  u32x2_t xr[4];
  load_rows(0, xr);
  for (int b = 0; b < nb; ++b) {
    int which, c0, W;
    block(b, which, c0, W);
    __syncthreads();  // sS / sA ready (first block); sX free (later blocks)
#pragma unroll
    for (int q = 0; q < 2; ++q) {  // the token pair j, j + 1 (j even: one 4-byte word of X^T)
      const int j = 2 * (threadIdx.x >> 4) + 32 * q, c4 = (threadIdx.x & 15) * 4;
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const u32x2_t xw = xr[2 * q + u];
        const float sc = sS[which][j + u];
        const float x[4] = {bf_lo(xw[0]) * sc, bf_hi(xw[0]) * sc, bf_lo(xw[1]) * sc, bf_hi(xw[1]) * sc};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const __bf16 hi = (__bf16)x[r];
          const __bf16 lo = (__bf16)(x[r] - (float)hi);
          const uint32_t h16 = __builtin_bit_cast(uint16_t, hi), l16w = __builtin_bit_cast(uint16_t, lo);
          hw[r] = u == 0 ? h16 : hw[r] | h16 << 16;
          lw[r] = u == 0 ? l16w : lw[r] | l16w << 16;
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        *reinterpret_cast<uint32_t *>(sXh + bswz(c4 + r, j)) = hw[r];
        *reinterpret_cast<uint32_t *>(sXl + bswz(c4 + r, j)) = lw[r];
      }
    }
    if (b + 1 < nb) load_rows(b + 1, xr);
    __syncthreads();
    // D[c][i] = sum_j X[j][c] A[i][j]: wave w takes columns c0 + 16 w .. + 15, all 64 tokens
    f32x4_t acc[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
    for (int j0 = 0; j0 < 64; j0 += 32) {
      const u32x4_t xh = *reinterpret_cast<const u32x4_t *>(sXh + bswz(wave * 16 + l16, j0 + 8 * lg));
      const u32x4_t xl = *reinterpret_cast<const u32x4_t *>(sXl + bswz(wave * 16 + l16, j0 + 8 * lg));
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) {
        const u32x4_t a8 = *reinterpret_cast<const u32x4_t *>(sA + bswz(ib * 16 + l16, j0 + 8 * lg));
        acc[ib] = mfma_bf(xl, a8, acc[ib]);
        acc[ib] = mfma_bf(xh, a8, acc[ib]);
      }
    }
    void *dst = which == 0 ? wp.u : wp.wout;
    const int col = c0 + wave * 16 + 4 * lg;
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
      const int i = ib * 16 + l16;
      if (i < L && col < W) st4<true>(dst, ((row0 + i) * p.HV + hv) * W + col, acc[ib]);
    }
  }
}

}  // namespace

hipError_t launch_wy_fwd(bool bf16, const WyParams &wp, hipStream_t s) {
  const long long blocks = (long long)wp.w.seg_slots * wp.w.HV;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (bf16) hipLaunchKernelGGL(gla_wy_fwd_kernel_bf16, dim3((unsigned)blocks), dim3(256), 0, s, wp);
  else hipLaunchKernelGGL(gla_wy_fwd_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s, wp);
  return hipGetLastError();
}

}  // namespace gla
