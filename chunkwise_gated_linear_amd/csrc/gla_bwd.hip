// Backward of the chunkwise gated linear attention: the gradients of q, k, v,
// g and h0 for given gradients of o and of the final state ht.
//
// What is computed (page "fla/ops/gla/fused_chunk.py": FusedChunkGLAFunction
// .backward, fused_chunk_gla_bwd_kernel for the inter-chunk terms and the
// reverse walk of the state gradient, bwd_inner_chunk for the in-chunk terms,
// and the reverse cumulative sum that turns per-token terms into the gate
// gradient).  Per sequence and value head, with S_t the state after token t
// (S_0 = h0) and U_t the gradient of the loss with respect to S_t:
//
//   U_t = scale q_t do_t^T + diag(exp(g_{t+1})) U_{t+1},   U_T = scale q_T do_T^T + dht
//   dq_t = scale S_t do_t     dk_t = U_t v_t     dv_t = U_t^T k_t
//   dg_t = sum_{s >= t} (q_s . dq_s - k_s . dk_s) + rowsum(dht . S_T)
//   dh0  = diag(exp(g_1)) U_1
//
// (. is the elementwise product; the dg form is the derivative through the
// cumulative log decay, which the page's backward also sums in reverse.)
//
// Chunk c (64 tokens, G the inclusive in-chunk cumsum of g, a = e^{G_last},
// S_c the state before the chunk, E_c the gradient reaching the state after
// the chunk from later tokens and dht):
//
//   A   = scale tril((q e^G)(k e^-G)^T)        dA' = scale tril(do v^T)
//   dq  = e^G . (scale do S_c^T + dA' (k e^-G))
//   dk  = e^-G . (dA'^T (q e^G)) + e^{G_last - G} . (v E_c^T)
//   dv  = A^T do + (k e^{G_last - G}) E_c
//   dg  = in-chunk reverse cumsum of (q . dq - k . dk) + rowsum(E_c . S_{c+1}),
//         rowsum(E_c . S_{c+1}) = a . rowsum(E_c . S_c) + sum_j k_j . e^{G_last - G_j} . (E_c v_j)
//   E_{c-1} = scale (q e^G)^T do + diag(a) E_c,   E_last = dht,   dh0 = E_{-1}
//
// Kernels (launched by the host in this order, after the forward kernels have
// produced the state after every chunk):
//   gla_bwd_dlocal      per (chunk, value head): scale (q e^G)^T do and a
//   gla_bwd_dscan       per state element, chunks in reverse: E_c in place, dh0
//   gla_bwd_chunk       per (chunk, value head): dq, dk, dv, dg on fp32 MFMA
//   gla_bwd_chunk_exact per (chunk, value head) whose decay leaves the fp32 range
//                       of the factors e^-G (some key below e^-80 within the
//                       chunk): the same gradients token by token
//   gla_bwd_group_sum   with several value heads per key head: dq, dk summed
#include <hip/hip_runtime.h>

#include "gla_device.h"

namespace gla {
namespace {

using namespace dev;

// ---------------------------------------------------------------- LDS tiles
// fp32 tiles [rows][W] (W = 64 or 128 floats per row) with the 16-byte column
// groups of each row XOR-swizzled by the row's low 4 bits: reading a float4
// from 16 consecutive rows, or one float from each of 4 rows 4 apart and 16
// consecutive columns, touches 64 different banks.
template <int W>
__device__ __forceinline__ int swz(int row, int col) {
  return row * W + ((((col >> 2) ^ (row & 15))) << 2 | (col & 3));
}
template <int W>
__device__ __forceinline__ f32x4_t lds4(const float *a, int row, int col) {  // col a multiple of 4
  return *reinterpret_cast<const f32x4_t *>(a + row * W + (((col >> 2) ^ (row & 15)) << 2));
}
template <int W>
__device__ __forceinline__ void lds4_st(float *a, int row, int col, f32x4_t x) {
  *reinterpret_cast<f32x4_t *>(a + row * W + (((col >> 2) ^ (row & 15)) << 2)) = x;
}

// ---------------------------------------------------------------- global access
template <bool BF>
__device__ __forceinline__ float ld_el(const void *base, int64_t i) {
  if constexpr (BF) return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(base)[i] << 16);
  else return reinterpret_cast<const float *>(base)[i];
}
template <bool BF>
__device__ __forceinline__ f32x4_t ld_el4(const void *base, int64_t i) {  // i a multiple of 4
  if constexpr (BF) {
    const u32x2_t w = *reinterpret_cast<const u32x2_t *>(reinterpret_cast<const uint16_t *>(base) + i);
    return f32x4_t{bf_lo(w[0]), bf_hi(w[0]), bf_lo(w[1]), bf_hi(w[1])};
  } else {
    return *reinterpret_cast<const f32x4_t *>(reinterpret_cast<const float *>(base) + i);
  }
}
template <bool BF>
__device__ __forceinline__ void st_el(void *base, int64_t i, float x) {
  if constexpr (BF) reinterpret_cast<__bf16 *>(base)[i] = (__bf16)x;
  else reinterpret_cast<float *>(base)[i] = x;
}

__device__ __forceinline__ f32x4_t zero4() { return f32x4_t{0.f, 0.f, 0.f, 0.f}; }

// Lower-triangular 16x16 tiles of a 64x64 score matrix, idx 0..9 -> (ib, jb).
__device__ __forceinline__ void tri_tile(int idx, int &ib, int &jb) {
  ib = idx >= 6 ? 3 : (idx >= 3 ? 2 : (idx >= 1 ? 1 : 0));
  jb = idx - ib * (ib + 1) / 2;
}

// Where a chunk lives: sequence, chunk index, valid rows, first token row.
struct ChunkAt {
  SegInfo si;
  int c, L;
  int64_t row0;
};
// One chunk per segment slot (the backward plans its state tables that way).
__device__ __forceinline__ bool chunk_at(const WalkParams &p, int slot, ChunkAt &ca) {
  if (!locate(p, slot, ca.si)) return false;
  const int nch = (ca.si.len + kChunk - 1) / kChunk;
  if (ca.si.s >= nch) return false;
  ca.c = ca.si.s;
  ca.L = min(kChunk, ca.si.len - kChunk * ca.c);
  ca.row0 = ca.si.bos + (int64_t)kChunk * ca.c;
  return true;
}

// Inclusive cumsum of the chunk's log decays for value head hv.  Thread t owns
// key t % KD and rows [part * RP, part * RP + RP), part = t / KD, and returns
// G at those rows in G[]; rows past L and keys past K count as zero decay.
// Part totals go through tot[256]; the function ends with a barrier after
// which tot may be reused.  Every kernel that decides whether a chunk fits the
// factorised form calls this same function, so they decide alike.
template <int KD, bool GH>
__device__ __forceinline__ void chunk_cumsum(const WalkParams &p, int64_t row0, int L, int hv,
                                             float (&G)[64 * KD / 256], float *tot) {
  constexpr int PARTS = 256 / KD, RP = 64 / PARTS;
  const int kk = threadIdx.x % KD, part = threadIdx.x / KD;
  float x = 0.f;
#pragma unroll
  for (int r = 0; r < RP; ++r) {
    const int i = part * RP + r;
    float gi = 0.f;
    if (i < L && kk < p.K)
      gi = GH ? p.g[(row0 + i) * p.HV + hv] : p.g[((row0 + i) * p.HV + hv) * p.K + kk];
    x += gi;
    G[r] = x;
  }
  tot[threadIdx.x] = x;
  __syncthreads();
  float off = 0.f;
  for (int q = 0; q < part; ++q) off += tot[q * KD + kk];
#pragma unroll
  for (int r = 0; r < RP; ++r) G[r] += off;
  __syncthreads();
}

// ---------------------------------------------------------------- gla_bwd_dlocal
// Chunk summary of the state gradient: dstate[slot][hv] = scale (q e^G)^T do
// (K x V) and ddecay[slot][hv] = e^{G_last} (K).  One workgroup per
// (chunk slot, value head); fp32 MFMA over the chunk's 64 tokens.
template <bool BF, int KD, int VD, bool GH>
__global__ __launch_bounds__(256, 1) void gla_bwd_dlocal(BwdParams bp) {
  const WalkParams &p = bp.w;
  constexpr int PARTS = 256 / KD, RP = 64 / PARTS;
  constexpr int NKB = KD / 64, NVB = VD / 16;
  __shared__ __attribute__((aligned(16))) float sQ[64 * KD];
  __shared__ __attribute__((aligned(16))) float sO[64 * VD];
  __shared__ float tot[256];
  const int hv = (int)(blockIdx.x % (unsigned)p.HV);
  const int slot = (int)(blockIdx.x / (unsigned)p.HV);
  ChunkAt ca;
  if (!chunk_at(p, slot, ca)) return;
  const int h = hv / p.G;
  float G[RP];
  chunk_cumsum<KD, GH>(p, ca.row0, ca.L, hv, G, tot);
  const int kk = threadIdx.x % KD, part = threadIdx.x / KD;
#pragma unroll
  for (int r = 0; r < RP; ++r) {
    const int i = part * RP + r;
    const float qv = (i < ca.L && kk < p.K) ? ld_el<BF>(p.q, (ca.row0 + i) * p.H * p.K + h * p.K + kk) : 0.f;
    sQ[swz<KD>(i, kk)] = qv * __expf(G[r]);
  }
  if (part == PARTS - 1 && kk < p.K) bp.ddecay[((int64_t)slot * p.HV + hv) * p.K + kk] = __expf(G[RP - 1]);
  for (int e = threadIdx.x; e < 64 * VD / 4; e += 256) {
    const int i = e / (VD / 4), c4 = (e % (VD / 4)) * 4;
    f32x4_t x = zero4();
    if (i < ca.L && c4 < p.V) x = ld_el4<BF>(bp.dout, ((ca.row0 + i) * p.HV + hv) * p.V + c4);
    lds4_st<VD>(sO, i, c4, x);
  }
  __syncthreads();

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l16 = lane & 15, lg = lane >> 4;
  f32x4_t acc[NKB][NVB];
#pragma unroll
  for (int a = 0; a < NKB; ++a)
#pragma unroll
    for (int b = 0; b < NVB; ++b) acc[a][b] = zero4();
#pragma unroll
  for (int ib = 0; ib < 4; ++ib) {
    float qa[NKB][4], ob[NVB][4];
#pragma unroll
    for (int a = 0; a < NKB; ++a)
#pragma unroll
      for (int r = 0; r < 4; ++r) qa[a][r] = sQ[swz<KD>(ib * 16 + 4 * lg + r, (wave * NKB + a) * 16 + l16)];
#pragma unroll
    for (int b = 0; b < NVB; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) ob[b][r] = sO[swz<VD>(ib * 16 + 4 * lg + r, b * 16 + l16)];
#pragma unroll
    for (int a = 0; a < NKB; ++a)
#pragma unroll
      for (int b = 0; b < NVB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[a][b] = mfma_f32(qa[a][r], ob[b][r], acc[a][b]);
  }
  float *dst = bp.dstate + ((int64_t)slot * p.HV + hv) * p.K * p.V;
#pragma unroll
  for (int a = 0; a < NKB; ++a)
#pragma unroll
    for (int b = 0; b < NVB; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int krow = (wave * NKB + a) * 16 + 4 * lg + r, col = b * 16 + l16;
        if (krow < p.K && col < p.V) dst[(int64_t)krow * p.V + col] = p.scale * acc[a][b][r];
      }
}

// ---------------------------------------------------------------- gla_bwd_dscan
// Reverse walk of the state gradient over each sequence's chunks, per float4
// of the K x V state: the carry starts at dht (or 0); chunk c's slot receives
// the carry E_c, then carry = summary_c + a_c . carry.  The final carry is
// dh0.  Loads of a batch of chunks are issued before its serial updates.
__global__ __launch_bounds__(256) void gla_bwd_dscan(BwdParams bp, int per_state) {
  const WalkParams &p = bp.w;
  const long long pair = blockIdx.x / per_state;
  const int eb = (int)(blockIdx.x - pair * per_state);
  const int n = (int)(pair / p.HV), hv = (int)(pair - (long long)n * p.HV);
  const int e4 = eb * 256 + threadIdx.x;
  const int KV4 = p.K * p.V / 4;
  if (n >= p.N || e4 >= KV4) return;
  int first, nseg, len;
  if (p.seg_base == nullptr) {
    first = n * p.P;
    nseg = p.P;
    len = p.T;
  } else {
    first = p.seg_base[n];
    nseg = p.seg_base[n + 1] - first;
    int bos;
    seq_extent(p.cu, n, p.T, bos, len);
  }
  const int nc = min((len + kChunk - 1) / kChunk, nseg);
  const int krow = (4 * e4) / p.V, col = 4 * e4 - krow * p.V;
  f32x4_t e = zero4();
  if (bp.dht) e = *reinterpret_cast<const f32x4_t *>(bp.dht + (((int64_t)n * p.HV + hv) * p.K + krow) * p.V + col);
  constexpr int BATCH = 8;
  for (int c1 = nc; c1 > 0; c1 -= BATCH) {
    const int nb = min(BATCH, c1);
    f32x4_t d[BATCH];
    float a[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      if (b < nb) {
        const int64_t slot = (int64_t)(first + c1 - 1 - b) * p.HV + hv;
        d[b] = reinterpret_cast<const f32x4_t *>(bp.dstate + slot * p.K * p.V)[e4];
        a[b] = bp.ddecay[slot * p.K + krow];
      }
    }
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      if (b < nb) {
        const int64_t slot = (int64_t)(first + c1 - 1 - b) * p.HV + hv;
        reinterpret_cast<f32x4_t *>(bp.dstate + slot * p.K * p.V)[e4] = e;
        e = d[b] + a[b] * e;
      }
    }
  }
  if (bp.dh0) *reinterpret_cast<f32x4_t *>(bp.dh0 + (((int64_t)n * p.HV + hv) * p.K + krow) * p.V + col) = e;
}

// ---------------------------------------------------------------- dq / dk stores
// dq and dk belong to key heads.  With one value head per key head they are
// stored in the input dtype; with G > 1 each value head stores its fp32 share
// to dq_part / dk_part [B,T,HV,K] and gla_bwd_group_sum adds the G shares.
template <bool BF>
__device__ __forceinline__ void store_dqk(const BwdParams &bp, int64_t row, int hv, int k, float dqv, float dkv) {
  const WalkParams &p = bp.w;
  if (p.G == 1) {
    const int64_t off = (row * p.H + hv) * p.K + k;
    st_el<BF>(bp.dq, off, dqv);
    st_el<BF>(bp.dk, off, dkv);
  } else {
    const int64_t off = (row * p.HV + hv) * p.K + k;
    bp.dq_part[off] = dqv;
    bp.dk_part[off] = dkv;
  }
}

// ---------------------------------------------------------------- gla_bwd_chunk
// The gradients of one chunk of one value head on fp32 MFMA
// (v_mfma_f32_16x16x4f32).  4 waves; wave w owns key blocks [w NKB, w NKB +
// NKB) and value blocks [w NVB, w NVB + NVB) of 16; score tiles are shared
// through LDS.  A chunk with a key whose decay over the chunk is below e^-80
// sets its flag and leaves its outputs to gla_bwd_chunk_exact.
template <bool BF, int KD, int VD, bool GH>
__global__ __launch_bounds__(256, 1) void gla_bwd_chunk(BwdParams bp) {
  const WalkParams &p = bp.w;
  constexpr int WV = KD > VD ? KD : VD;
  constexpr int PARTS = 256 / KD, RP = 64 / PARTS;
  constexpr int NKB = KD / 64, NVB = VD / 64;
  __shared__ __attribute__((aligned(16))) float sQ[64 * KD];  // q e^G
  __shared__ __attribute__((aligned(16))) float sK[64 * KD];  // k e^-G
  __shared__ __attribute__((aligned(16))) float sO[64 * VD];  // do
  __shared__ __attribute__((aligned(16))) float sV[64 * WV];  // v, then G as [64][KD]
  __shared__ __attribute__((aligned(16))) float sX[64 * 64];  // A, then dA'
  __shared__ __attribute__((aligned(16))) float sEl[KD];      // e^{G_last}
  __shared__ float sGl[KD];                                   // G_last
  __shared__ float tot[256];
  __shared__ float sRow[64];                                  // per-row dg sums (per-head gate)

  const int hv = (int)(blockIdx.x % (unsigned)p.HV);
  const int slot = (int)(blockIdx.x / (unsigned)p.HV);
  ChunkAt ca;
  if (!chunk_at(p, slot, ca)) return;
  const int h = hv / p.G;
  const int L = ca.L;
  const int64_t row0 = ca.row0;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l16 = lane & 15, lg = lane >> 4;
  const int kk = threadIdx.x % KD, part = threadIdx.x / KD;
  bool low;
  {
    float G[RP];
    chunk_cumsum<KD, GH>(p, row0, L, hv, G, tot);
    low = part == PARTS - 1 && kk < p.K && !(G[RP - 1] >= kMinChunkLogDecay);
#pragma unroll
    for (int r = 0; r < RP; ++r) {
      const int i = part * RP + r;
      const bool in = i < L && kk < p.K;
      const int64_t off = (row0 + i) * p.H * p.K + h * p.K + kk;
      const float qv = in ? ld_el<BF>(p.q, off) : 0.f;
      const float kv = in ? ld_el<BF>(p.k, off) : 0.f;
      sQ[swz<KD>(i, kk)] = qv * __expf(G[r]);
      sK[swz<KD>(i, kk)] = kv * __expf(-G[r]);
    }
    if (part == PARTS - 1) {
      sGl[kk] = G[RP - 1];
      sEl[kk] = __expf(G[RP - 1]);
    }
  }
  for (int e = threadIdx.x; e < 64 * VD / 4; e += 256) {
    const int i = e / (VD / 4), c4 = (e % (VD / 4)) * 4;
    f32x4_t xo = zero4(), xv = zero4();
    if (i < L && c4 < p.V) {
      const int64_t off = ((row0 + i) * p.HV + hv) * p.V + c4;
      xo = ld_el4<BF>(bp.dout, off);
      xv = ld_el4<BF>(p.v, off);
    }
    lds4_st<VD>(sO, i, c4, xo);
    lds4_st<VD>(sV, i, c4, xv);
  }
  if (GH && threadIdx.x < 64) sRow[threadIdx.x] = 0.f;
  const bool exact = __syncthreads_or(low);
  if (threadIdx.x == 0) bp.flags[(int64_t)slot * p.HV + hv] = exact ? 1 : 0;
  if (exact) return;

  // ---- scores: A -> sX, dA' kept in registers until A has been used
  f32x4_t dAr[3];
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    const int idx = wave + 4 * t;
    dAr[t] = zero4();
    if (idx >= 10) continue;
    int ib, jb;
    tri_tile(idx, ib, jb);
    f32x4_t a = zero4(), d = zero4();
#pragma unroll 4
    for (int k0 = 0; k0 < KD; k0 += 16) {
      const f32x4_t q4 = lds4<KD>(sQ, ib * 16 + l16, k0 + 4 * lg);
      const f32x4_t k4 = lds4<KD>(sK, jb * 16 + l16, k0 + 4 * lg);
#pragma unroll
      for (int r = 0; r < 4; ++r) a = mfma_f32(q4[r], k4[r], a);
    }
#pragma unroll 4
    for (int v0 = 0; v0 < VD; v0 += 16) {
      const f32x4_t o4 = lds4<VD>(sO, ib * 16 + l16, v0 + 4 * lg);
      const f32x4_t w4 = lds4<VD>(sV, jb * 16 + l16, v0 + 4 * lg);
#pragma unroll
      for (int r = 0; r < 4; ++r) d = mfma_f32(o4[r], w4[r], d);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool keep = ib > jb || l16 <= 4 * lg + r;  // column j <= row i
      sX[swz<64>(ib * 16 + 4 * lg + r, jb * 16 + l16)] = keep ? p.scale * a[r] : 0.f;
      dAr[t][r] = keep ? p.scale * d[r] : 0.f;
    }
  }
  __syncthreads();

  // ---- dv = A^T do (this wave's value blocks, all row blocks)
  f32x4_t dv[NVB][4];
#pragma unroll
  for (int b = 0; b < NVB; ++b)
#pragma unroll
    for (int j = 0; j < 4; ++j) dv[b][j] = zero4();
#pragma unroll
  for (int ib = 0; ib < 4; ++ib) {
    float ov[NVB][4];
#pragma unroll
    for (int b = 0; b < NVB; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) ov[b][r] = sO[swz<VD>(ib * 16 + 4 * lg + r, (wave * NVB + b) * 16 + l16)];
#pragma unroll
    for (int jb = 0; jb <= ib; ++jb) {
      float av[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) av[r] = sX[swz<64>(ib * 16 + 4 * lg + r, jb * 16 + l16)];
#pragma unroll
      for (int b = 0; b < NVB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) dv[b][jb] = mfma_f32(av[r], ov[b][r], dv[b][jb]);
    }
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    const int idx = wave + 4 * t;
    if (idx >= 10) continue;
    int ib, jb;
    tri_tile(idx, ib, jb);
#pragma unroll
    for (int r = 0; r < 4; ++r) sX[swz<64>(ib * 16 + 4 * lg + r, jb * 16 + l16)] = dAr[t][r];
  }

  // ---- inter-chunk terms: dq = do S_c^T, dkI = v E_c^T, rs = rowsum(S_c . E_c)
  const float *Sc = nullptr;
  if (ca.c > 0) Sc = bp.fstate + ((int64_t)(ca.si.first + ca.c - 1) * p.HV + hv) * p.K * p.V;
  else if (p.h0) Sc = p.h0 + ((int64_t)ca.si.n * p.HV + hv) * p.K * p.V;
  const float *Ec = bp.dstate + ((int64_t)(ca.si.first + ca.c) * p.HV + hv) * p.K * p.V;
  f32x4_t dq[NKB][4], dkI[NKB][4];
  float rs[NKB];
#pragma unroll
  for (int a = 0; a < NKB; ++a) {
    rs[a] = 0.f;
#pragma unroll
    for (int b = 0; b < 4; ++b) dq[a][b] = dkI[a][b] = zero4();
  }
#pragma unroll 2
  for (int v0 = 0; v0 < VD; v0 += 16) {
    f32x4_t s4[NKB], e4[NKB];
#pragma unroll
    for (int a = 0; a < NKB; ++a) {
      const int krow = (wave * NKB + a) * 16 + l16, col = v0 + 4 * lg;
      const bool in = krow < p.K && col < p.V;
      const int64_t off = (int64_t)krow * p.V + col;
      s4[a] = (in && Sc) ? *reinterpret_cast<const f32x4_t *>(Sc + off) : zero4();
      e4[a] = in ? *reinterpret_cast<const f32x4_t *>(Ec + off) : zero4();
      rs[a] += s4[a][0] * e4[a][0] + s4[a][1] * e4[a][1] + s4[a][2] * e4[a][2] + s4[a][3] * e4[a][3];
    }
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
      const f32x4_t o4 = lds4<VD>(sO, ib * 16 + l16, v0 + 4 * lg);
      const f32x4_t w4 = lds4<VD>(sV, ib * 16 + l16, v0 + 4 * lg);
#pragma unroll
      for (int a = 0; a < NKB; ++a)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          dq[a][ib] = mfma_f32(o4[r], s4[a][r], dq[a][ib]);
          dkI[a][ib] = mfma_f32(w4[r], e4[a][r], dkI[a][ib]);
        }
    }
  }
  __syncthreads();  // v consumed, dA' visible
  {
    float G[RP];  // the same cumsum again (cheaper than holding it in registers)
    chunk_cumsum<KD, GH>(p, row0, L, hv, G, tot);
#pragma unroll
    for (int r = 0; r < RP; ++r) sV[swz<KD>(part * RP + r, kk)] = G[r];
  }
  __syncthreads();
  const float *sG = sV;

  // ---- dv += (k e^{G_last - G}) E_c, store dv
#pragma unroll 2
  for (int k0 = 0; k0 < KD; k0 += 16) {
    const f32x4_t el4 = *reinterpret_cast<const f32x4_t *>(sEl + k0 + 4 * lg);
    float ev[NVB][4];
#pragma unroll
    for (int b = 0; b < NVB; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int krow = k0 + 4 * lg + r, col = (wave * NVB + b) * 16 + l16;
        ev[b][r] = (krow < p.K && col < p.V) ? Ec[(int64_t)krow * p.V + col] : 0.f;
      }
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      const f32x4_t k4 = lds4<KD>(sK, jb * 16 + l16, k0 + 4 * lg) * el4;
#pragma unroll
      for (int b = 0; b < NVB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) dv[b][jb] = mfma_f32(k4[r], ev[b][r], dv[b][jb]);
    }
  }
#pragma unroll
  for (int b = 0; b < NVB; ++b)
#pragma unroll
    for (int jb = 0; jb < 4; ++jb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = jb * 16 + 4 * lg + r, col = (wave * NVB + b) * 16 + l16;
        if (j < L && col < p.V) st_el<BF>(bp.dv, ((row0 + j) * p.HV + hv) * p.V + col, dv[b][jb][r]);
      }

  // ---- dq = scale (do S_c^T) + dA' (k e^-G)
#pragma unroll
  for (int a = 0; a < NKB; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) dq[a][b] *= p.scale;
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) {
    float kv[NKB][4];
#pragma unroll
    for (int a = 0; a < NKB; ++a)
#pragma unroll
      for (int r = 0; r < 4; ++r) kv[a][r] = sK[swz<KD>(jb * 16 + 4 * lg + r, (wave * NKB + a) * 16 + l16)];
#pragma unroll
    for (int ib = jb; ib < 4; ++ib) {
      const f32x4_t a4 = lds4<64>(sX, ib * 16 + l16, jb * 16 + 4 * lg);
#pragma unroll
      for (int a = 0; a < NKB; ++a)
#pragma unroll
        for (int r = 0; r < 4; ++r) dq[a][ib] = mfma_f32(a4[r], kv[a][r], dq[a][ib]);
    }
  }
  // ---- dkA = dA'^T (q e^G)
  f32x4_t dkA[NKB][4];
#pragma unroll
  for (int a = 0; a < NKB; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) dkA[a][b] = zero4();
#pragma unroll
  for (int ib = 0; ib < 4; ++ib) {
    float qv[NKB][4];
#pragma unroll
    for (int a = 0; a < NKB; ++a)
#pragma unroll
      for (int r = 0; r < 4; ++r) qv[a][r] = sQ[swz<KD>(ib * 16 + 4 * lg + r, (wave * NKB + a) * 16 + l16)];
#pragma unroll
    for (int jb = 0; jb <= ib; ++jb) {
      float av[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) av[r] = sX[swz<64>(ib * 16 + 4 * lg + r, jb * 16 + l16)];
#pragma unroll
      for (int a = 0; a < NKB; ++a)
#pragma unroll
        for (int r = 0; r < 4; ++r) dkA[a][jb] = mfma_f32(av[r], qv[a][r], dkA[a][jb]);
    }
  }

  // ---- gradients in key space, and dg by a reverse cumsum down each key column
#pragma unroll
  for (int a = 0; a < NKB; ++a) {
    const int k = (wave * NKB + a) * 16 + l16;
    const float gl = sGl[k], el = sEl[k];
    float t[4][4];
    float colk = 0.f;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = b * 16 + 4 * lg + r;
        const float Gv = sG[swz<KD>(i, k)], qg = sQ[swz<KD>(i, k)], kg = sK[swz<KD>(i, k)];
        const float kdkI = kg * el * dkI[a][b][r];
        const float dqv = __expf(Gv) * dq[a][b][r];
        const float dkv = __expf(-Gv) * dkA[a][b][r] + __expf(gl - Gv) * dkI[a][b][r];
        if (i < L && k < p.K) store_dqk<BF>(bp, row0 + i, hv, k, dqv, dkv);
        t[b][r] = qg * dq[a][b][r] - (kg * dkA[a][b][r] + kdkI);
        colk += kdkI;
      }
    float rsa = rs[a];
    rsa += __shfl_xor(rsa, 16);
    rsa += __shfl_xor(rsa, 32);
    colk += __shfl_xor(colk, 16);
    colk += __shfl_xor(colk, 32);
    float carry = el * rsa + colk;  // dg of the first token after the chunk
#pragma unroll
    for (int b = 3; b >= 0; --b) {
      const float sb = t[b][0] + t[b][1] + t[b][2] + t[b][3];
      float after = 0.f, total = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float sq = __shfl(sb, q * 16 + l16);
        total += sq;
        if (q > lg) after += sq;
      }
      float run = carry + after;
#pragma unroll
      for (int r = 3; r >= 0; --r) {
        run += t[b][r];
        const int i = b * 16 + 4 * lg + r;
        if (i < L && k < p.K) {
          if (GH) atomicAdd(&sRow[i], run);
          else bp.dg[((row0 + i) * p.HV + hv) * p.K + k] = run;
        }
      }
      carry += total;
    }
  }
  if (GH) {
    __syncthreads();
    if (threadIdx.x < L) bp.dg[(row0 + threadIdx.x) * p.HV + hv] = sRow[threadIdx.x];
  }
}

// ---------------------------------------------------------------- gla_bwd_chunk_exact
// The gradients of a flagged chunk of one value head, token by token, with
// only decays (never their inverses) applied, so any finite gate is exact.
// Thread t owns key t / PARTS and NC = VD / PARTS consecutive columns of the
// K x V state (PARTS = 256 / KD adjacent lanes share a key).
//   forward over the chunk: S <- diag(e^{g_i}) S + k_i v_i^T, dq_i = scale S do_i
//   reverse: U = scale q_i do_i^T + Ubar, dk_i = U v_i, dv_i = U^T k_i,
//            dg_i = e^{g_i} rowsum(U . S_{i-1}),  Ubar <- diag(e^{g_i}) U,
//   starting from Ubar = E_c.  dg takes its definition here rather than the
//   reverse cumsum of q . dq - k . dk: under decays this strong that sum
//   cancels to a small fraction of its terms.  S_{i-1} is rebuilt from the
//   staged rows, S_{i-1} = sum_{j<i} w_j k_j v_j^T + w_{-1} S_c with w the
//   products of the decays in between (O(64^2) per chunk: this kernel only
//   runs for chunks whose decay is beyond the fast kernel's range).
template <bool BF, int KD, int VD, bool GH>
__global__ __launch_bounds__(256, 1) void gla_bwd_chunk_exact(BwdParams bp) {
  const WalkParams &p = bp.w;
  constexpr int PARTS = 256 / KD, NC = VD / PARTS;
  __shared__ __attribute__((aligned(16))) float sV[64 * VD];  // v rows
  __shared__ float sK[64 * KD];    // k rows
  __shared__ float sA[64 * KD];    // e^{g} per token and key
  __shared__ float sDq[64 * KD];   // dq
  __shared__ float sRed[4 * VD];   // per-wave partial dv of one token
  __shared__ float sRow[64];

  const int hv = (int)(blockIdx.x % (unsigned)p.HV);
  const int slot = (int)(blockIdx.x / (unsigned)p.HV);
  ChunkAt ca;
  if (!chunk_at(p, slot, ca)) return;
  if (bp.flags[(int64_t)slot * p.HV + hv] == 0) return;
  const int h = hv / p.G;
  const int L = ca.L;
  const int64_t row0 = ca.row0;
  const int key = threadIdx.x / PARTS, cp = threadIdx.x % PARTS;
  const int col0 = cp * NC;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const bool kin = key < p.K;

  for (int e = threadIdx.x; e < 64 * KD; e += 256) {
    const int i = e / KD, kk = e % KD;
    const bool in = i < L && kk < p.K;
    sK[e] = in ? ld_el<BF>(p.k, (row0 + i) * p.H * p.K + h * p.K + kk) : 0.f;
    float gv = 0.f;
    if (in) gv = GH ? p.g[(row0 + i) * p.HV + hv] : p.g[((row0 + i) * p.HV + hv) * p.K + kk];
    sA[e] = __expf(gv);
  }
  for (int e = threadIdx.x; e < 64 * VD; e += 256) {
    const int i = e / VD, c = e % VD;
    sV[e] = (i < L && c < p.V) ? ld_el<BF>(p.v, ((row0 + i) * p.HV + hv) * p.V + c) : 0.f;
  }
  if (GH && threadIdx.x < 64) sRow[threadIdx.x] = 0.f;
  __syncthreads();

  const float *Sc = nullptr;
  if (ca.c > 0) Sc = bp.fstate + ((int64_t)(ca.si.first + ca.c - 1) * p.HV + hv) * p.K * p.V;
  else if (p.h0) Sc = p.h0 + ((int64_t)ca.si.n * p.HV + hv) * p.K * p.V;
  const float *Ec = bp.dstate + ((int64_t)(ca.si.first + ca.c) * p.HV + hv) * p.K * p.V;
  auto dout = [&](int i, int j) -> float {  // do at token i, column col0 + j
    const int col = col0 + j;
    return col < p.V ? ld_el<BF>(bp.dout, ((row0 + i) * p.HV + hv) * p.V + col) : 0.f;
  };
  auto reduce = [&](float x) {
#pragma unroll
    for (int m = 1; m < PARTS; m <<= 1) x += __shfl_xor(x, m);
    return x;
  };
  float S[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int col = col0 + j;
    S[j] = (Sc && kin && col < p.V) ? Sc[(int64_t)key * p.V + col] : 0.f;
  }
  // forward over the chunk: dq
  for (int i = 0; i < L; ++i) {
    const float a = sA[i * KD + key], kv = sK[i * KD + key];
    float part = 0.f;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      S[j] = a * S[j] + kv * sV[i * VD + col0 + j];
      part += S[j] * dout(i, j);
    }
    part = reduce(part);
    if (cp == 0) sDq[i * KD + key] = p.scale * part;
  }
  // reverse over the chunk: dk, dv, dg
  float U[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int col = col0 + j;
    U[j] = (kin && col < p.V) ? Ec[(int64_t)key * p.V + col] : 0.f;
  }
  for (int i = L - 1; i >= 0; --i) {
    const int64_t qoff = (row0 + i) * p.H * p.K + h * p.K + key;
    const float qv = kin ? ld_el<BF>(p.q, qoff) : 0.f;
    const float kv = sK[i * KD + key];
    float dkp = 0.f;
    float dvp[NC];
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      U[j] += p.scale * qv * dout(i, j);
      dkp += U[j] * sV[i * VD + col0 + j];
      dvp[j] = U[j] * kv;
    }
    dkp = reduce(dkp);
    // rowsum(U_i . S_{i-1}) with S_{i-1} rebuilt from the rows before i
    float acc = 0.f, w = 1.f;
    for (int j = i - 1; j >= 0; --j) {
      float dot = 0.f;
#pragma unroll
      for (int c = 0; c < NC; ++c) dot += U[c] * sV[j * VD + col0 + c];
      acc += w * sK[j * KD + key] * reduce(dot);
      w *= sA[j * KD + key];
    }
    float dots = 0.f;
    if (Sc && kin) {
#pragma unroll
      for (int c = 0; c < NC; ++c)
        if (col0 + c < p.V) dots += U[c] * Sc[(int64_t)key * p.V + col0 + c];
    }
    acc += w * reduce(dots);
    // dv: sum over the wave's keys (lanes with the same cp), then over waves
#pragma unroll
    for (int j = 0; j < NC; ++j) {
#pragma unroll
      for (int m = PARTS; m < 64; m <<= 1) dvp[j] += __shfl_xor(dvp[j], m);
    }
    if (lane < PARTS) {
#pragma unroll
      for (int j = 0; j < NC; ++j) sRed[wave * VD + col0 + j] = dvp[j];
    }
    const float a = sA[i * KD + key];
    if (cp == 0 && kin) {
      const int64_t row = row0 + i;
      const float dgi = a * acc;
      store_dqk<BF>(bp, row, hv, key, sDq[i * KD + key], dkp);
      if (GH) atomicAdd(&sRow[i], dgi);
      else bp.dg[(row * p.HV + hv) * p.K + key] = dgi;
    }
    __syncthreads();
    for (int col = threadIdx.x; col < p.V; col += 256) {
      const float sv = sRed[col] + sRed[VD + col] + sRed[2 * VD + col] + sRed[3 * VD + col];
      st_el<BF>(bp.dv, ((row0 + i) * p.HV + hv) * p.V + col, sv);
    }
#pragma unroll
    for (int j = 0; j < NC; ++j) U[j] *= a;
    __syncthreads();  // sRed is reused by the next token
  }
  if (GH && threadIdx.x < L) bp.dg[(row0 + threadIdx.x) * p.HV + hv] = sRow[threadIdx.x];
}

// ---------------------------------------------------------------- gla_bwd_group_sum
// dq, dk of key head h = the sum of the fp32 shares of its G value heads,
// rounded once to the output dtype.  One thread per 4 keys of a token row.
template <bool BF>
__global__ __launch_bounds__(256) void gla_bwd_group_sum(BwdParams bp, int64_t quads) {
  const WalkParams &p = bp.w;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= quads) return;
  const int K4 = p.K / 4;
  const int64_t rowh = e / K4;  // (token, key head)
  const int k = (int)(e - rowh * K4) * 4;
  const int64_t row = rowh / p.H;
  const int h = (int)(rowh - row * p.H);
  f32x4_t dq = zero4(), dk = zero4();
  for (int gi = 0; gi < p.G; ++gi) {
    const int64_t off = (row * p.HV + h * p.G + gi) * p.K + k;
    dq += *reinterpret_cast<const f32x4_t *>(bp.dq_part + off);
    dk += *reinterpret_cast<const f32x4_t *>(bp.dk_part + off);
  }
  const int64_t off = rowh * p.K + k;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    st_el<BF>(bp.dq, off + r, dq[r]);
    st_el<BF>(bp.dk, off + r, dk[r]);
  }
}

template <bool BF, int KD, int VD, bool GH>
hipError_t launch_bwd_t(int which, const BwdParams &bp, long long blocks, hipStream_t s) {
  const dim3 grid((unsigned)blocks), block(256);
  switch (which) {
    case 0: hipLaunchKernelGGL((gla_bwd_dlocal<BF, KD, VD, GH>), grid, block, 0, s, bp); break;
    case 1: hipLaunchKernelGGL((gla_bwd_chunk<BF, KD, VD, GH>), grid, block, 0, s, bp); break;
    default: hipLaunchKernelGGL((gla_bwd_chunk_exact<BF, KD, VD, GH>), grid, block, 0, s, bp); break;
  }
  return hipGetLastError();
}

template <bool BF, bool GH>
hipError_t launch_bwd_kv(int which, const BwdParams &bp, long long blocks, hipStream_t s) {
  const bool k128 = bp.w.K > 64, v128 = bp.w.V > 64;
  if (k128) return v128 ? launch_bwd_t<BF, 128, 128, GH>(which, bp, blocks, s)
                        : launch_bwd_t<BF, 128, 64, GH>(which, bp, blocks, s);
  return v128 ? launch_bwd_t<BF, 64, 128, GH>(which, bp, blocks, s) : launch_bwd_t<BF, 64, 64, GH>(which, bp, blocks, s);
}

// Per-chunk kernels: one workgroup per (chunk slot, value head).
hipError_t launch_bwd_kernel(int which, bool bf16, const BwdParams &bp, hipStream_t s) {
  const long long blocks = (long long)bp.w.seg_slots * bp.w.HV;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL || bp.w.K > 128 || bp.w.V > 128) return hipErrorInvalidValue;
  const bool gh = bp.w.gate_head != 0;
  if (bf16) return gh ? launch_bwd_kv<true, true>(which, bp, blocks, s) : launch_bwd_kv<true, false>(which, bp, blocks, s);
  return gh ? launch_bwd_kv<false, true>(which, bp, blocks, s) : launch_bwd_kv<false, false>(which, bp, blocks, s);
}

}  // namespace

hipError_t launch_bwd_dlocal(bool bf16, const BwdParams &bp, hipStream_t s) { return launch_bwd_kernel(0, bf16, bp, s); }

hipError_t launch_bwd_chunk(bool bf16, const BwdParams &bp, hipStream_t s) {
  hipError_t e = launch_bwd_kernel(1, bf16, bp, s);
  if (e != hipSuccess) return e;
  e = launch_bwd_kernel(2, bf16, bp, s);
  if (e != hipSuccess || bp.w.G == 1) return e;
  const long long rows = (bp.w.cu ? 1LL : (long long)bp.w.N) * bp.w.T;  // token rows of [B,T]
  const long long quads = rows * bp.w.H * (bp.w.K / 4);
  if (quads <= 0) return hipSuccess;
  const long long blocks = (quads + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (bf16) hipLaunchKernelGGL(gla_bwd_group_sum<true>, dim3((unsigned)blocks), dim3(256), 0, s, bp, (int64_t)quads);
  else hipLaunchKernelGGL(gla_bwd_group_sum<false>, dim3((unsigned)blocks), dim3(256), 0, s, bp, (int64_t)quads);
  return hipGetLastError();
}

hipError_t launch_bwd_dscan(const BwdParams &bp, hipStream_t s) {
  const int KV4 = bp.w.K * bp.w.V / 4;
  const int per_state = (KV4 + 255) / 256;
  const long long blocks = (long long)bp.w.N * bp.w.HV * per_state;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gla_bwd_dscan, dim3((unsigned)blocks), dim3(256), 0, s, bp, per_state);
  return hipGetLastError();
}

}  // namespace gla
