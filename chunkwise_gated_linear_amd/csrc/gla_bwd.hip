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
// Kernels (launched by the host in this order):
//   gla_bwd_local       per (chunk, value head): the chunk's summaries
//                       sum_j k_j e^{G_last - G_j} v_j^T and scale (q e^G)^T do, and a;
//                       it can also turn them into S_c, E_c and dh0 itself, walking
//                       each chain in one workgroup or chaining its steps across
//                       workgroups (then gla_bwd_scan is not launched; packed
//                       sequences first get a table of their chains from
//                       gla_bwd_chain_plan, and those without chunks their dh0
//                       from gla_bwd_empty_dh0)
//   gla_bwd_scan        per state element: S_c forward, E_c in reverse, dh0
//   gla_bwd_chunk       per (chunk, value head): dq, dk, dv, dg (bf16 MFMA on split
//                       operands for the bf16 products named below, fp32 MFMA otherwise)
//   gla_bwd_chunk_exact per (chunk, value head) whose decay leaves the fp32 range
//                       of the factors e^-G (some key below e^-80 within the
//                       chunk): the same gradients token by token
//   gla_bwd_group_sum   with several value heads per key head or several value
//                       slices: dq, dk summed over their fp32 shares
//   gla_bwd_slice_sum   with several value slices (or, per-head gate, key
//                       blocks): dg summed over the shares
//   gla_bwd_dv_sum      with several key blocks: dv summed over the shares
// K past 128 runs as two key blocks and V past 128 as value slices of 128
// columns; each (block, slice) runs the per-chunk launches above on its own
// (gla_bwd_copy_rows stages its rows and columns of h0, dht and dh0 for the
// chained scan), and the sums follow the last of them.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

#include "gla.h"
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
// Four consecutive elements from i (a multiple of 4), rounded as st_el rounds
// each, in one store.
template <bool BF>
__device__ __forceinline__ void st_el4(void *base, int64_t i, f32x4_t x) {
  if constexpr (BF) {
    uint32_t w[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
      w[h] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x[2 * h]) |
             (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x[2 * h + 1]) << 16;
    *reinterpret_cast<u32x2_t *>(reinterpret_cast<uint16_t *>(base) + i) = u32x2_t{w[0], w[1]};
  } else {
    *reinterpret_cast<f32x4_t *>(reinterpret_cast<float *>(base) + i) = x;
  }
}
// One element through a buffer descriptor (byte offset; past the range:
// dropped / zero), as bf16 (rounded to nearest even) or fp32.
template <bool BF>
__device__ __forceinline__ void bst_el(__amdgpu_buffer_rsrc_t r, int off, float x) {
  if constexpr (BF) __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (__bf16)x), r, off, 0, 0);
  else __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, off, 0, 0);
}
__device__ __forceinline__ float bld_f32(__amdgpu_buffer_rsrc_t r, int off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
constexpr int kOutsideRange = 0x40000000;  // a byte offset past any descriptor's range

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

// In-place inclusive cumsum down the 64 rows of a chunk's log decays in LDS:
// buf holds the gate rows as [64][KD] fp32 (swizzled; rows past the chunk and
// keys past K zero), or with a per-head gate one value per row in buf[0..63];
// afterwards buf[swz<KD>(row, key)] = G for every row and key (keys past K
// get 0).  Thread t of NT sums key t % KD over rows [part RP, part RP + RP),
// part = t / KD; part totals go through tot[NT].  Starts after a barrier that
// made buf visible and ends with one.  GUARD: the workgroup has more than NT
// threads, and the others only meet the barriers (the sums, and so their
// rounding, depend on NT alone).
template <int KD, bool GH, int NT, bool GUARD = false>
__device__ __forceinline__ void gate_cumsum_lds(int K, float *buf, float *tot) {
  constexpr int PARTS = NT / KD, RP = 64 / PARTS;
  const int kk = threadIdx.x % KD, part = threadIdx.x / KD;
  const bool in = !GUARD || threadIdx.x < NT;
  float G[RP];
  float x = 0.f;
  if (in) {
#pragma unroll
    for (int r = 0; r < RP; ++r) {
      const int i = part * RP + r;
      x += (kk < K) ? (GH ? buf[i] : buf[swz<KD>(i, kk)]) : 0.f;
      G[r] = x;
    }
    tot[threadIdx.x] = x;
  }
  __syncthreads();
  if (in) {
    float off = 0.f;
    for (int q = 0; q < part; ++q) off += tot[q * KD + kk];
#pragma unroll
    for (int r = 0; r < RP; ++r) buf[swz<KD>(part * RP + r, kk)] = G[r] + off;
  }
  __syncthreads();
}

// Raw row quads as loaded: bf16 quads stay packed (two words) until staged.
template <bool BF> struct RawQuad;
template <> struct RawQuad<true> { typedef u32x2_t type; };
template <> struct RawQuad<false> { typedef f32x4_t type; };
template <bool BF>
__device__ __forceinline__ f32x4_t unpack4(typename RawQuad<BF>::type w) {
  if constexpr (BF) return f32x4_t{bf_lo(w[0]), bf_hi(w[0]), bf_lo(w[1]), bf_hi(w[1])};
  else return w;
}

// A chunk's token rows of one head in a [.., T, heads, width] tensor, through
// a buffer descriptor from its first row: rows `stride` elements apart, rows
// past the chunk's L tokens outside the range (they read zero), 32-bit
// offsets.
struct ChunkRowsRsrc {
  __amdgpu_buffer_rsrc_t r;
  int stride, width;
};
template <bool BF>
__device__ __forceinline__ ChunkRowsRsrc chunk_rows(const void *base, int64_t first, int stride, int width, int L) {
  constexpr int ES = BF ? 2 : 4;
  return {make_rsrc(static_cast<const char *>(base) + first * ES, ((int64_t)(L - 1) * stride + width) * ES), stride,
          width};
}
// Quad c4 of row i (c4 a multiple of 4; quads past the width read zero).
template <bool BF>
__device__ __forceinline__ typename RawQuad<BF>::type ld_row4(const ChunkRowsRsrc &rr, int i, int c4) {
  constexpr int ES = BF ? 2 : 4;
  const int off = c4 < rr.width ? (i * rr.stride + c4) * ES : kOutsideRange;
  if constexpr (BF) return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rr.r, off, 0, 0));
  else return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rr.r, off, 0, 0));
}

// Gate rows of a chunk (value head hv) into registers: quad t of thread
// threadIdx.x + NT t; with a per-head gate, row threadIdx.x in gh.
template <int KD, bool GH, int NT>
struct GateRows {
  static constexpr int TG = 64 * KD / 4 / NT;
  f32x4_t g[GH ? 1 : TG];
  float gh;
};
template <int KD, bool GH, int NT>
__device__ __forceinline__ void gate_load(const WalkParams &p, const ChunkAt &ca, int hv, GateRows<KD, GH, NT> &gr) {
  if constexpr (GH) {
    gr.gh = threadIdx.x < ca.L ? p.g[(ca.row0 + threadIdx.x) * p.HV + hv] : 0.f;
  } else {
    const ChunkRowsRsrc rg = chunk_rows<false>(p.g, (ca.row0 * p.HV + hv) * p.Kmem, p.HV * p.Kmem, p.K, ca.L);
#pragma unroll
    for (int t = 0; t < GateRows<KD, GH, NT>::TG; ++t) {
      const int e = threadIdx.x + NT * t, i = e / (KD / 4), c4 = (e % (KD / 4)) * 4;
      gr.g[t] = ld_row4<false>(rg, i, c4);
    }
  }
}
template <int KD, bool GH, int NT>
__device__ __forceinline__ void gate_stage(const GateRows<KD, GH, NT> &gr, float *buf) {
  if constexpr (GH) {
    if (threadIdx.x < 64) buf[threadIdx.x] = gr.gh;
  } else {
#pragma unroll
    for (int t = 0; t < GateRows<KD, GH, NT>::TG; ++t) {
      const int e = threadIdx.x + NT * t, i = e / (KD / 4), c4 = (e % (KD / 4)) * 4;
      lds4_st<KD>(buf, i, c4, gr.g[t]);
    }
  }
}

// Eight floats as three bf16 terms (8 lanes each, packed pairs): hi = the
// nearest bf16, mid = the nearest bf16 of x - hi, lo = the nearest bf16 of
// x - hi - mid.  Each remainder is exact in fp32, and hi + mid + lo equals x
// to fp32 precision.
__device__ __forceinline__ void split8_3(const float (&x)[8], u32x4_t &hi, u32x4_t &mid, u32x4_t &lo) {
  float r1[8], r2[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    hi[q] = pack_bf16(x[2 * q], x[2 * q + 1]);
    r1[2 * q] = x[2 * q] - bf_lo(hi[q]);
    r1[2 * q + 1] = x[2 * q + 1] - bf_hi(hi[q]);
    mid[q] = pack_bf16(r1[2 * q], r1[2 * q + 1]);
    r2[2 * q] = r1[2 * q] - bf_lo(mid[q]);
    r2[2 * q + 1] = r1[2 * q + 1] - bf_hi(mid[q]);
    lo[q] = pack_bf16(r2[2 * q], r2[2 * q + 1]);
  }
}

// Eight floats as two bf16 terms: hi = the nearest bf16, lo = the nearest bf16
// of the exact remainder x - hi (about 16 significant bits together).
__device__ __forceinline__ void split8_2(const float (&x)[8], u32x4_t &hi, u32x4_t &lo) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    hi[q] = pack_bf16(x[2 * q], x[2 * q + 1]);
    lo[q] = pack_bf16(x[2 * q] - bf_lo(hi[q]), x[2 * q + 1] - bf_hi(hi[q]));
  }
}

// Eight consecutive floats of an LDS row (two swizzled quads).
template <int W>
__device__ __forceinline__ void lds8(const float *buf, int row, int col, float (&x)[8]) {
  const f32x4_t a = lds4<W>(buf, row, col), b = lds4<W>(buf, row, col + 4);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    x[r] = a[r];
    x[4 + r] = b[r];
  }
}

// Eight floats that are bf16 values, packed (exact).
__device__ __forceinline__ u32x4_t pack8(const float (&x)[8]) {
  return u32x4_t{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(x[4], x[5]), pack_bf16(x[6], x[7])};
}

// ---------------------------------------------------------------- gla_bwd_local
// Chunk summaries of the state and of its gradient over the chunk's 64
// tokens (bf16 MFMA on split operands for bf16 inputs, fp32 MFMA for fp32).
// For chunk c of a sequence and value head hv:
//   Sigma_c = sum_j (k_j e^{G_last - G_j}) v_j^T      (K x V), the state's
//   D_c     = scale sum_i (q_i e^{G_i}) do_i^T       (K x V), the gradient's
//   a_c     = e^{G_last}                             (K)
// Every factor is a decay (at most 1), so any gate is exact here.
//
// Three schedules.  Without bp.chain or bp.walk, task t < 2 slots HV forms
// Sigma (first half) or D (second half) of slot t / HV and head t % HV, stores
// it in fstate / dstate (and a_c in ddecay), and gla_bwd_scan then walks the
// tables.  Otherwise the walks run inside this kernel: every (sequence, value
// head) with P chunks has a state chain over chunks 0, 1, .., P-1 and a
// gradient chain over P-1, .., 0, and each step of a chain applies the scan's
// recurrences:
//   state:    slot c holds S_c;  S_{c+1} = a_c S_c + Sigma_c goes to slot c + 1
//   gradient: slot c holds E_c;  E_{c-1} = D_c + a_c E_c goes to slot c - 1,
//             after chunk 0 to dh0
// (S_0 = h0 and E_{P-1} = dht, or zero).
//
// Walk (bp.walk, eight waves): one workgroup per chain takes the chain's
// chunks in order and carries the state in registers (walk_step), so no step
// waits for another workgroup; it pays off when the chains fill the compute
// units.
//
// Chained (bp.chain): each task applies one step to the state its predecessor
// published, in whichever workgroup that ran.  Tasks are taken from a counter in
// step order (step s: chunk s of every state chain, chunk P-1-s of every
// gradient chain), so a task's predecessor always has a lower number and has
// been taken by a running workgroup: the chains always move.  A published
// state is written and read only with device-scope stores and loads (the sc1
// cache policy that relaxed agent-scope atomics use: no compute unit or die
// serves them from a private copy); every wave waits for its stores to complete before a
// barrier, after which one lane sets the flag, and the successor loads the
// state only after it has seen the flag (polled within the bound
// wait_polls).  No cache-wide write-back or invalidation is needed for that,
// and none is made: with one link per chunk (every few microseconds on each
// die) they cost more than the scan launch this schedule saves.  The state
// summary of the last chunk and, without dh0, the gradient summary of chunk
// 0 feed nothing and are not formed.
//
// Persistent workgroups (two per compute unit; walk: one per chain); the rows
// of a workgroup's next task are loaded into registers while it forms the
// current one.
template <bool BF, int KD, int VD, bool GH, int NT>
struct LocalRows {
  static constexpr int TK = 64 * KD / 4 / NT, TV = 64 * VD / 4 / NT;  // row quads per thread
  typename RawQuad<BF>::type x[TK], y[TV];
  GateRows<KD, GH, NT> gate;
};

// A task: chunk ca of value head hv, the state summary (grad false) or the
// gradient summary (grad true); work: the summary is formed.
struct LocalTask {
  ChunkAt ca;
  int hv, slot;
  int nc;  // chunks of the task's sequence (the length of its chains)
  bool grad, work;
};

// Task numbers are below 2 slots HV, which the host keeps within int range
// (32-bit arithmetic: the task decode runs on the scalar unit, where 64-bit
// division costs many registers).
// Task t of the three-launch schedule.
__device__ __forceinline__ bool local_task(const BwdParams &bp, int t, LocalTask &lt) {
  const WalkParams &p = bp.w;
  const int half = p.seg_slots * p.HV;
  lt.grad = t >= half;
  const int blk = lt.grad ? t - half : t;
  lt.slot = blk / p.HV;
  lt.hv = blk - lt.slot * p.HV;
  lt.nc = 0;  // no chains in this schedule
  lt.work = true;
  return chunk_at(p, lt.slot, lt.ca);
}

// Task t of the chained schedule (fixed-length sequences, P chunks each).
__device__ __forceinline__ bool chained_task(const BwdParams &bp, int t, LocalTask &lt) {
  const WalkParams &p = bp.w;
  const int pairs = p.N * p.HV;
  const int step = t / (2 * pairs);
  int rem = t - step * 2 * pairs;
  lt.grad = rem >= pairs;
  if (lt.grad) rem -= pairs;
  const int n = rem / p.HV;
  lt.hv = rem - n * p.HV;
  const int c = lt.grad ? p.P - 1 - step : step;
  lt.slot = n * p.P + c;
  lt.nc = p.P;
  lt.work = lt.grad ? (c > 0 || bp.dh0 != nullptr) : c < p.P - 1;
  return chunk_at(p, lt.slot, lt.ca);
}

// Task t of the chained schedule for packed sequences.  The chain plan lists
// u = 0 .. (total chunks - 1) as (step s, sequence n): the steps in order and,
// within step s, the sequences with more than s chunks.  Task t is u = t / 2HV,
// direction (t / HV) % 2 and value head t % HV, so that a chain's task at step
// s - 1 has a lower number than its task at step s.
__device__ __forceinline__ bool packed_chained_task(const BwdParams &bp, int t, LocalTask &lt) {
  const WalkParams &p = bp.w;
  const int u = t / (2 * p.HV);
  const int rem = t - u * 2 * p.HV;
  lt.grad = rem >= p.HV;
  lt.hv = lt.grad ? rem - p.HV : rem;
  const int2 sn = reinterpret_cast<const int2 *>(bp.chain_plan + kChainPlanTable)[u];
  const int step = __builtin_amdgcn_readfirstlane(sn.x), n = __builtin_amdgcn_readfirstlane(sn.y);
  ChunkAt &ca = lt.ca;
  SegInfo &si = ca.si;
  int bos, len;
  seq_extent(p.cu, n, p.T, bos, len);
  lt.nc = (len + kChunk - 1) / kChunk;
  const int c = lt.grad ? lt.nc - 1 - step : step;
  si.n = n;
  si.first = p.seg_base[n];
  si.nseg = p.seg_base[n + 1] - si.first;
  si.s = c;
  si.bos = bos;
  si.len = len;
  if (c < 0 || c >= lt.nc || c >= si.nseg) return false;  // a plan that does not match its sequence
  ca.c = c;
  ca.L = min(kChunk, len - kChunk * c);
  ca.row0 = si.bos + (int64_t)kChunk * c;
  lt.slot = si.first + c;
  lt.work = lt.grad ? (c > 0 || bp.dh0 != nullptr) : c < lt.nc - 1;
  return true;
}

// Step `step` of chain j of the walk schedule; a state chain takes its
// sequence's chunks in order, a gradient chain in reverse.  Fixed-length
// sequences: chains 0 .. N HV - 1 are the state chains of (sequence, value
// head) = (j / HV, j % HV), chains N HV .. 2 N HV - 1 the gradient chains in
// the same order.  Packed sequences: chain j is the state (j / HV even) or
// gradient chain of value head j % HV of the sequence in place j / 2HV of the
// chain plan's step 0, which lists the sequences with chunks longest first
// (workgroups start in about the order of their numbers, so the longest
// chains start first).  False past the chain's last chunk.
__device__ __forceinline__ bool walk_task(const BwdParams &bp, int j, int step, LocalTask &lt) {
  const WalkParams &p = bp.w;
  if (p.seg_base == nullptr) {
    const int pairs = p.N * p.HV;
    lt.grad = j >= pairs;
    const int rem = lt.grad ? j - pairs : j;
    const int n = rem / p.HV;
    lt.hv = rem - n * p.HV;
    if (step >= p.P) return false;
    const int c = lt.grad ? p.P - 1 - step : step;
    lt.nc = p.P;
    lt.slot = n * p.P + c;
    lt.work = lt.grad ? (c > 0 || bp.dh0 != nullptr) : c < p.P - 1;
    return chunk_at(p, lt.slot, lt.ca);
  }
  const int u = j / (2 * p.HV);
  const int rem = j - u * 2 * p.HV;
  lt.grad = rem >= p.HV;
  lt.hv = lt.grad ? rem - p.HV : rem;
  const int n = __builtin_amdgcn_readfirstlane(reinterpret_cast<const int2 *>(bp.chain_plan + kChainPlanTable)[u].y);
  ChunkAt &ca = lt.ca;
  SegInfo &si = ca.si;
  int bos, len;
  seq_extent(p.cu, n, p.T, bos, len);
  lt.nc = (len + kChunk - 1) / kChunk;
  if (step >= lt.nc) return false;
  const int c = lt.grad ? lt.nc - 1 - step : step;
  si.n = n;
  si.first = p.seg_base[n];
  si.nseg = p.seg_base[n + 1] - si.first;
  si.s = c;
  si.bos = bos;
  si.len = len;
  if (c >= si.nseg) return false;  // a segment table that does not match its sequence
  ca.c = c;
  ca.L = min(kChunk, len - kChunk * c);
  ca.row0 = si.bos + (int64_t)kChunk * c;
  lt.slot = si.first + c;
  lt.work = lt.grad ? (c > 0 || bp.dh0 != nullptr) : c < lt.nc - 1;
  return true;
}

template <bool BF, int KD, int VD, bool GH, int NT>
__device__ __forceinline__ void local_load(const BwdParams &bp, const LocalTask &lt,
                                           LocalRows<BF, KD, VD, GH, NT> &rw) {
  using R = LocalRows<BF, KD, VD, GH, NT>;
  const WalkParams &p = bp.w;
  const ChunkAt &ca = lt.ca;
  const int h = lt.hv / p.G;
  const ChunkRowsRsrc rx = chunk_rows<BF>(lt.grad ? p.q : p.k, (ca.row0 * p.H + h) * p.Kmem, p.H * p.Kmem, p.K, ca.L);
  const ChunkRowsRsrc ry =
      chunk_rows<BF>(lt.grad ? bp.dout : p.v, (ca.row0 * p.HV + lt.hv) * bp.Vmem, p.HV * bp.Vmem, p.V, ca.L);
#pragma unroll
  for (int t = 0; t < R::TK; ++t) {
    const int e = threadIdx.x + NT * t, i = e / (KD / 4), c4 = (e % (KD / 4)) * 4;
    rw.x[t] = ld_row4<BF>(rx, i, c4);  // key-side rows: k, or q for the gradient
  }
  gate_load<KD, GH, NT>(p, ca, lt.hv, rw.gate);
#pragma unroll
  for (int t = 0; t < R::TV; ++t) {
    const int e = threadIdx.x + NT * t, i = e / (VD / 4), c4 = (e % (VD / 4)) * 4;
    rw.y[t] = ld_row4<BF>(ry, i, c4);  // value-side rows: v, or do
  }
}

// One step of a chain (chained schedule) for task lt, whose summary is in acc
// (in the MFMA layout: row (wave NKB + a) 16 + lane % 16, columns
// b 16 + 4 (lane / 16) + [0, 4)) and whose decays a_c are in dec[K].  The
// chain's first chunk takes its state from h0 / dht (or zero) and also stores
// it in its own slot for the chunk kernel.  Every access goes through a buffer
// descriptor over one K x V state: rows past K and columns past V (whole
// 16-row and 16-column blocks, K and V being multiples of 16) get an offset
// past its end, so that their loads return zero and their stores are dropped
// without a branch, and the loads of the step all travel at once.
template <int KD, int VD>
__device__ __forceinline__ void chain_step(const BwdParams &bp, const LocalTask &lt,
                                           const f32x4_t (&acc)[KD / 64][VD / 16], const float *dec) {
  constexpr int NKB = KD / 64, NVB = VD / 16;
  constexpr int kOutside = 0x40000000;  // a byte offset past any state
  const WalkParams &p = bp.w;
  const int c = lt.ca.c, n = lt.ca.si.n;
  const bool first = lt.grad ? c == lt.nc - 1 : c == 0;
  const bool publish = lt.grad ? c > 0 : c < lt.nc - 1;
  if (!first && !lt.work) return;  // a summary nobody needs, and a slot its predecessor filled
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // the lane through an opaque copy: the offsets below would otherwise be
  // hoisted out of the task loop and held in registers across the products
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));
  const int l16 = lane & 15, lg = lane >> 4;
  const int64_t KV = (int64_t)p.K * p.V;
  float *tab = lt.grad ? bp.dstate : bp.fstate;
  int32_t *flags = bp.chain + 1 + (lt.grad ? (int64_t)p.seg_slots * p.HV : 0);
  // h0, dht, dh0 and the state slots are all [K][V] here (the chained
  // schedule runs with one value slice, Vmem = V)
  const float *bound = lt.grad ? bp.dht : p.h0;
  if (bound != nullptr) bound += ((int64_t)n * p.HV + lt.hv) * KV;
  const int next = lt.grad ? lt.slot - 1 : lt.slot + 1;
  float *out = nullptr;
  if (publish) out = tab + ((int64_t)next * p.HV + lt.hv) * KV;
  else if (lt.work) out = bp.dh0 + ((int64_t)n * p.HV + lt.hv) * KV;  // gradient chunk 0 with dh0
  const __amdgpu_buffer_rsrc_t rHere = make_rsrc(tab + ((int64_t)lt.slot * p.HV + lt.hv) * KV, KV * 4);
  int off[NKB][NVB];
#pragma unroll
  for (int a = 0; a < NKB; ++a)
#pragma unroll
    for (int b = 0; b < NVB; ++b) {
      const int rb = wave * NKB + a;  // 16-row block
      const bool in = rb * 16 < p.K && b * 16 < p.V;
      off[a][b] = in ? ((rb * 16 + l16) * p.V + b * 16 + 4 * lg) * 4 : kOutside;
    }
  if (!first) {
    // one wave waits; the barrier holds the others until then, and the state
    // is loaded after it
    if (wave == 0) {
      const int32_t *f = flags + (int64_t)lt.slot * p.HV + lt.hv;
      int ready = 0;
      if (lane == 0) {
        for (int spin = 0; spin < p.wait_polls; ++spin) {
          if (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) {
            ready = 1;
            break;
          }
          __builtin_amdgcn_s_sleep(2);
        }
      }
      if (__builtin_amdgcn_readfirstlane(ready) == 0) report_status(p.status, GLA_STATUS_WAIT_EXHAUSTED, lane);
    }
    __syncthreads();
  }
  f32x4_t x[NKB][NVB];
  if (!first) {
#pragma unroll
    for (int a = 0; a < NKB; ++a)
#pragma unroll
      for (int b = 0; b < NVB; ++b) x[a][b] = buf_ldf4<kDeviceScope>(rHere, off[a][b]);
  } else if (bound != nullptr) {
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(bound, KV * 4);
#pragma unroll
    for (int a = 0; a < NKB; ++a)
#pragma unroll
      for (int b = 0; b < NVB; ++b) x[a][b] = buf_ldf4<0>(rB, off[a][b]);
  } else {
#pragma unroll
    for (int a = 0; a < NKB; ++a)
#pragma unroll
      for (int b = 0; b < NVB; ++b) x[a][b] = zero4();
  }
  if (first) {
#pragma unroll
    for (int a = 0; a < NKB; ++a)
#pragma unroll
      for (int b = 0; b < NVB; ++b) buf_stf4<0>(rHere, off[a][b], x[a][b]);
  }
  if (out == nullptr) return;
  const __amdgpu_buffer_rsrc_t rOut = make_rsrc(out, KV * 4);
  float ak[NKB];
#pragma unroll
  for (int a = 0; a < NKB; ++a) ak[a] = dec[(wave * NKB + a) * 16 + l16];  // rows past K: stores dropped
  if (publish) {
#pragma unroll
    for (int a = 0; a < NKB; ++a)
#pragma unroll
      for (int b = 0; b < NVB; ++b) buf_stf4<kDeviceScope>(rOut, off[a][b], ak[a] * x[a][b] + acc[a][b]);
    // every wave's stores have completed (at device scope) before the barrier;
    // then one lane sets the flag
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0)
      __hip_atomic_store(flags + (int64_t)next * p.HV + lt.hv, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
#pragma unroll
    for (int a = 0; a < NKB; ++a)
#pragma unroll
      for (int b = 0; b < NVB; ++b) buf_stf4<0>(rOut, off[a][b], ak[a] * x[a][b] + acc[a][b]);
  }
}

// One step of a walk (walk schedule, eight waves) for task lt, whose summary
// is in acc and decays in dec.  Wave w holds rows ((w % 4) NKB + a) 16 +
// lane % 16 and the NVW column blocks from (w / 4) NVW, as chain_step's waves
// hold all of theirs.  The workgroup carries its chain's state in x, in the
// layout of acc, from one chunk to the next, so a step waits for nothing: the
// chain's first chunk loads h0 / dht (or zero) into x and stores it in its own
// slot for the chunk kernel, and every step that publishes stores x = a_c x +
// Sigma_c (or D_c) in the next slot (after the gradient's chunk 0: in dh0).
// Offsets as in chain_step.
template <int KD, int NVW>
__device__ __forceinline__ void walk_step(const BwdParams &bp, const LocalTask &lt, const f32x4_t (&acc)[KD / 64][NVW],
                                          const float *dec, f32x4_t (&x)[KD / 64][NVW]) {
  constexpr int NKB = KD / 64;
  const WalkParams &p = bp.w;
  const int c = lt.ca.c, n = lt.ca.si.n;
  const bool first = lt.grad ? c == lt.nc - 1 : c == 0;
  const bool publish = lt.grad ? c > 0 : c < lt.nc - 1;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rw = wave & 3, cb0 = (wave >> 2) * NVW;
  const int lane = threadIdx.x & 63, l16 = lane & 15, lg = lane >> 4;
  const int64_t KV = (int64_t)p.K * p.V;
  float *tab = lt.grad ? bp.dstate : bp.fstate;
  int off[NKB][NVW];
#pragma unroll
  for (int a = 0; a < NKB; ++a)
#pragma unroll
    for (int b = 0; b < NVW; ++b) {
      const int rb = rw * NKB + a, cb = cb0 + b;  // 16-row and 16-column blocks
      const bool in = rb * 16 < p.K && cb * 16 < p.V;
      off[a][b] = in ? ((rb * 16 + l16) * p.V + cb * 16 + 4 * lg) * 4 : kOutsideRange;
    }
  if (first) {
    const float *bound = lt.grad ? bp.dht : p.h0;
    if (bound != nullptr) {
      const __amdgpu_buffer_rsrc_t rB = make_rsrc(bound + ((int64_t)n * p.HV + lt.hv) * KV, KV * 4);
#pragma unroll
      for (int a = 0; a < NKB; ++a)
#pragma unroll
        for (int b = 0; b < NVW; ++b) x[a][b] = buf_ldf4<0>(rB, off[a][b]);
    } else {
#pragma unroll
      for (int a = 0; a < NKB; ++a)
#pragma unroll
        for (int b = 0; b < NVW; ++b) x[a][b] = zero4();
    }
    const __amdgpu_buffer_rsrc_t rHere = make_rsrc(tab + ((int64_t)lt.slot * p.HV + lt.hv) * KV, KV * 4);
#pragma unroll
    for (int a = 0; a < NKB; ++a)
#pragma unroll
      for (int b = 0; b < NVW; ++b) buf_stf4<0>(rHere, off[a][b], x[a][b]);
  }
  if (!publish && !lt.work) return;
  float *out = publish ? tab + ((int64_t)(lt.grad ? lt.slot - 1 : lt.slot + 1) * p.HV + lt.hv) * KV
                       : bp.dh0 + ((int64_t)n * p.HV + lt.hv) * KV;
  const __amdgpu_buffer_rsrc_t rOut = make_rsrc(out, KV * 4);
#pragma unroll
  for (int a = 0; a < NKB; ++a) {
    const float ak = dec[(rw * NKB + a) * 16 + l16];  // rows past K: stores dropped
#pragma unroll
    for (int b = 0; b < NVW; ++b) {
      x[a][b] = ak * x[a][b] + acc[a][b];
      buf_stf4<0>(rOut, off[a][b], x[a][b]);
    }
  }
}

// MODE: kLocalTasks (the three-launch schedule, or the chained schedule for
// fixed-length sequences), kLocalPackedChain (the chained schedule for packed
// sequences: its own instantiation, so that the table decode adds nothing to
// the registers of the others) or kLocalWalk (the walk schedule: one chain per
// workgroup at a time).  The walk runs eight waves, the others four: waves w
// and w + 4 form the same rows of a summary, each half of its columns (so
// that the registers that carry the state leave room for a second wave per
// SIMD).
constexpr int kLocalTasks = 0, kLocalPackedChain = 1, kLocalWalk = 2;
constexpr int local_threads(int mode) { return mode == kLocalWalk ? 512 : 256; }
template <bool BF, int KD, int VD, bool GH, int MODE>
__global__ __launch_bounds__(local_threads(MODE), MODE == kLocalWalk ? 1 : 2) void gla_bwd_local(BwdParams bp) {
  constexpr bool PC = MODE == kLocalPackedChain, WALK = MODE == kLocalWalk;
  constexpr int NT = local_threads(MODE);
  const WalkParams &p = bp.w;
  using R = LocalRows<BF, KD, VD, GH, NT>;
  // each wave: NKB 16-row blocks from row (wave % 4) 16 NKB, NVW 16-column
  // blocks from column (wave / 4) 16 NVW
  constexpr int NKB = KD / 64, NVW = VD / 16 / (NT / 256);
  __shared__ __attribute__((aligned(16))) float sA[64 * KD];  // G, then k e^{G_last - G} or scale q e^G
  __shared__ __attribute__((aligned(16))) float sB[64 * VD];  // v or do
  __shared__ float tot[NT];
  __shared__ float sdec[KD];  // a_c per key
  __shared__ int sclaim;      // chained schedule: the task number taken from the counter
  const bool chained = !WALK && bp.chain != nullptr;
  // packed sequences: the chain plan holds the task count and table; walk:
  // the tasks are the chains
  unsigned ntask = 2u * p.seg_slots * p.HV;
  if (PC) ntask = (unsigned)__builtin_amdgcn_readfirstlane(bp.chain_plan[kChainPlanTasks]);
  if (WALK)
    ntask = p.seg_base ? 2u * p.HV * (unsigned)__builtin_amdgcn_readfirstlane(bp.chain_plan[kChainPlanSeqs])
                       : 2u * p.N * p.HV;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l16 = lane & 15, lg = lane >> 4;
  // the wave's first row block / NKB and first column block
  const int rw = NT == 256 ? wave : wave & 3, cb0 = NT == 256 ? 0 : (wave >> 2) * NVW;

  // the next task: walk, the next step of the chain (or the first of the
  // next chain on the grid stride); chained, from the counter (sclaim was
  // written before a barrier); else the next one with a chunk on the grid stride
  unsigned task = WALK ? blockIdx.x : blockIdx.x - gridDim.x;  // wraps; the first step adds gridDim.x back
  int step = -1;                                                // walk: the step within chain `task`
  auto advance = [&](LocalTask &lt) -> bool {
    if constexpr (WALK) {
      for (++step; task < ntask; task += gridDim.x, step = 0)
        if (walk_task(bp, (int)task, step, lt)) return true;
      return false;
    }
    if (chained) {
      const unsigned t = (unsigned)__builtin_amdgcn_readfirstlane(sclaim);
      if constexpr (PC) return t < ntask && packed_chained_task(bp, (int)t, lt);
      else return t < ntask && chained_task(bp, (int)t, lt);
    }
    for (task += gridDim.x; task < ntask; task += gridDim.x)
      if (local_task(bp, (int)task, lt)) return true;
    return false;
  };
  auto claim = [&]() {
    if (chained && threadIdx.x == 0)
      sclaim = __hip_atomic_fetch_add(bp.chain, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };

  R rows;
  LocalTask nxt;
  f32x4_t wx[NKB][NVW];  // walk: the chain's state
  claim();
  __syncthreads();
  bool have = advance(nxt);
  __syncthreads();  // sclaim is read before the loop's first claim overwrites it
  if (have && nxt.work) local_load<BF, KD, VD, GH, NT>(bp, nxt, rows);
  while (have) {
    const LocalTask cur = nxt;
    claim();
    if (cur.work) {
      // gate rows -> LDS, cumsum down each key column (G in sA)
      gate_stage<KD, GH, NT>(rows.gate, sA);
      __syncthreads();
      // the cumsum in the four-wave order whatever NT: every schedule forms
      // the same summaries, bit for bit
      gate_cumsum_lds<KD, GH, 256, (NT > 256)>(p.K, sA, tot);
      f32x4_t xg[R::TK];
#pragma unroll
      for (int t = 0; t < R::TK; ++t) {
        const int e = threadIdx.x + NT * t, i = e / (KD / 4), c4 = (e % (KD / 4)) * 4;
        const f32x4_t G4 = lds4<KD>(sA, i, c4), Gl4 = lds4<KD>(sA, 63, c4);
        f32x4_t xt = unpack4<BF>(rows.x[t]);
#pragma unroll
        for (int r = 0; r < 4; ++r) xt[r] *= cur.grad ? p.scale * __expf(G4[r]) : __expf(Gl4[r] - G4[r]);
        xg[t] = xt;
        if (i == 63 && c4 < p.K) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float a = __expf(Gl4[r]);
            sdec[c4 + r] = a;
            if (!WALK && !chained && !cur.grad) bp.ddecay[((int64_t)cur.slot * p.HV + cur.hv) * p.K + c4 + r] = a;
          }
        }
      }
#pragma unroll
      for (int t = 0; t < R::TV; ++t) {
        const int e = threadIdx.x + NT * t, i = e / (VD / 4), c4 = (e % (VD / 4)) * 4;
        lds4_st<VD>(sB, i, c4, unpack4<BF>(rows.y[t]));
      }
      __syncthreads();  // G read by every thread
#pragma unroll
      for (int t = 0; t < R::TK; ++t) {
        const int e = threadIdx.x + NT * t, i = e / (KD / 4), c4 = (e % (KD / 4)) * 4;
        lds4_st<KD>(sA, i, c4, xg[t]);
      }
    }
    __syncthreads();
    // the next task's rows travel while this one's products are formed
    have = advance(nxt);
    if (have && nxt.work) local_load<BF, KD, VD, GH, NT>(bp, nxt, rows);

    // transposed product (rows v, columns k): each lane then holds 4
    // consecutive values of one state row and stores them as one float4
    f32x4_t acc[NKB][NVW];
#pragma unroll
    for (int a = 0; a < NKB; ++a)
#pragma unroll
      for (int b = 0; b < NVW; ++b) acc[a][b] = zero4();
    if (!cur.work) {
    } else if constexpr (BF) {
      // bf16 inputs: the value-side rows (v or do) are exact in bf16, the gated
      // key-side rows are split into three bf16 terms (fp32 accuracy); 32
      // tokens per v_mfma_f32_16x16x32_bf16, each lane 8 consecutive tokens of
      // one column
      // lane indices through an opaque copy: the compiler would otherwise hoist
      // every swizzled LDS address out of the task loop and keep them live
      // beside the next task's rows
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int m16 = ln & 15, mg = ln >> 4;
#pragma unroll 1
      for (int tb = 0; tb < 2; ++tb) {
        u32x4_t xh[NKB], xm[NKB], xl[NKB];
#pragma unroll
        for (int a = 0; a < NKB; ++a) {
          float x8[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) x8[e] = sA[swz<KD>(tb * 32 + 8 * mg + e, (rw * NKB + a) * 16 + m16)];
          split8_3(x8, xh[a], xm[a], xl[a]);
        }
#pragma unroll
        for (int b = 0; b < NVW; ++b) {
          float y8[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) y8[e] = sB[swz<VD>(tb * 32 + 8 * mg + e, (cb0 + b) * 16 + m16)];
          const u32x4_t yv = pack8(y8);
#pragma unroll
          for (int a = 0; a < NKB; ++a) {
            acc[a][b] = mfma_bf(yv, xl[a], acc[a][b]);
            acc[a][b] = mfma_bf(yv, xm[a], acc[a][b]);
            acc[a][b] = mfma_bf(yv, xh[a], acc[a][b]);
          }
        }
      }
    } else {
#pragma unroll 1
      for (int ib = 0; ib < 4; ++ib) {  // not unrolled: keeps the operand registers of one row block
        float xa[NKB][4], yb[NVW][4];
#pragma unroll
        for (int a = 0; a < NKB; ++a)
#pragma unroll
          for (int r = 0; r < 4; ++r) xa[a][r] = sA[swz<KD>(ib * 16 + 4 * lg + r, (rw * NKB + a) * 16 + l16)];
#pragma unroll
        for (int b = 0; b < NVW; ++b)
#pragma unroll
          for (int r = 0; r < 4; ++r) yb[b][r] = sB[swz<VD>(ib * 16 + 4 * lg + r, (cb0 + b) * 16 + l16)];
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int a = 0; a < NKB; ++a)
#pragma unroll
            for (int b = 0; b < NVW; ++b) acc[a][b] = mfma_f32(yb[b][r], xa[a][r], acc[a][b]);
      }
    }
    if constexpr (WALK) {
      walk_step<KD, NVW>(bp, cur, acc, sdec, wx);
    } else if (chained) {
      chain_step<KD, VD>(bp, cur, acc, sdec);
    } else {
      float *dst = (cur.grad ? bp.dstate : bp.fstate) + ((int64_t)cur.slot * p.HV + cur.hv) * p.K * p.V;
#pragma unroll
      for (int a = 0; a < NKB; ++a)
#pragma unroll
        for (int b = 0; b < NVW; ++b) {
          const int krow = (rw * NKB + a) * 16 + l16, col = (cb0 + b) * 16 + 4 * lg;
          if (krow < p.K && col < p.V) *reinterpret_cast<f32x4_t *>(dst + (int64_t)krow * p.V + col) = acc[a][b];
        }
    }
    __syncthreads();  // LDS is refilled for the next task
  }
}

// ---------------------------------------------------------------- chain plan (packed)
// Inclusive prefix sums of in[0, n) into out (in may equal out), by one
// workgroup of 1024 threads in tiles of 1024.
__device__ __forceinline__ void block_scan_1024(const int32_t *in, int32_t *out, int n, int32_t *part,
                                                int32_t &carry) {
  const int tid = threadIdx.x;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < n; base += 1024) {
    part[tid] = base + tid < n ? in[base + tid] : 0;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {
      const int add = tid >= d ? part[tid - d] : 0;
      __syncthreads();
      part[tid] += add;
      __syncthreads();
    }
    if (base + tid < n) out[base + tid] = carry + part[tid];
    __syncthreads();
    if (tid == 1023) carry += part[1023];
    __syncthreads();
  }
}

// The chained scan's task table for packed sequences (one workgroup).  With
// nc_n the chunks of sequence n (at most cmax) and cnt[s] the sequences with
// more than s chunks: order lists the sequences by nc descending, so that the
// first cnt[s] of them are those with a chunk s, and table[u] for u = pbase[s]
// + rank (pbase the exclusive sums of cnt) is (s, order[rank]).  plan[0]
// receives the task count 2 HV (total chunks) and plan[1] the number of
// sequences with a chunk.
__global__ __launch_bounds__(1024) void gla_bwd_chain_plan(const int32_t *cu, int N, int T, int HV, int cmax,
                                                           int slots, int32_t *plan, int32_t *hist, int32_t *cnt,
                                                           int32_t *pbase, int32_t *order) {
  __shared__ int32_t part[1024];
  __shared__ int32_t carry;
  const int tid = threadIdx.x;
  for (int c = tid; c <= cmax; c += 1024) hist[c] = 0;
  __syncthreads();
  for (int n = tid; n < N; n += 1024) {
    int bos, len;
    seq_extent(cu, n, T, bos, len);
    atomicAdd(&hist[min((len + kChunk - 1) / kChunk, cmax)], 1);
  }
  __syncthreads();
  block_scan_1024(hist, cnt, cmax + 1, part, carry);  // sequences with at most s chunks
  for (int c = tid; c <= cmax; c += 1024) {
    cnt[c] = N - cnt[c];
    hist[c] = 0;  // from here: the next free place of each chunk count
  }
  __syncthreads();
  for (int n = tid; n < N; n += 1024) {
    int bos, len;
    seq_extent(cu, n, T, bos, len);
    const int nc = min((len + kChunk - 1) / kChunk, cmax);
    order[cnt[nc] + atomicAdd(&hist[nc], 1)] = n;
  }
  // pbase[s + 1] = cnt[0] + .. + cnt[s], pbase[0] = 0
  if (tid == 0) pbase[0] = 0;
  block_scan_1024(cnt, pbase + 1, cmax + 1, part, carry);
  const int total = min(pbase[cmax + 1], slots);
  int2 *table = reinterpret_cast<int2 *>(plan + kChainPlanTable);
  for (int u = tid; u < total; u += 1024) {
    int lo = 0, hi = cmax;  // the last s with pbase[s] <= u
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pbase[mid] <= u) lo = mid; else hi = mid - 1;
    }
    table[u] = int2{lo, order[u - pbase[lo]]};
  }
  if (tid == 0) {
    plan[kChainPlanTasks] = 2 * HV * total;
    plan[kChainPlanSeqs] = min(cnt[0], total);  // table[0, cnt[0]): step 0, the sequences by length
  }
}

// dh0 of the packed sequences without chunks (the chained scan has no task
// for them): dht, or zero.  One thread per float4 of a (sequence, value head)
// state of `rows` keys and V columns, rows Kmem apart per head and Vmem
// floats apart, from the (block and slice offset) dh0 / dht.
__global__ __launch_bounds__(256) void gla_bwd_empty_dh0(BwdParams bp, int rows, int64_t quads) {
  const WalkParams &p = bp.w;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= quads) return;
  const int q = p.V / 4;
  const int64_t hr = e / q;  // (n, hv, row)
  const int col = (int)(e - hr * q) * 4;
  const int64_t nh = hr / rows;
  const int row = (int)(hr - nh * rows);
  const int n = (int)(nh / p.HV);
  int bos, len;
  seq_extent(p.cu, n, p.T, bos, len);
  if (len > 0) return;
  const int64_t off = (nh * p.Kmem + row) * bp.Vmem + col;
  const f32x4_t x = bp.dht ? *reinterpret_cast<const f32x4_t *>(bp.dht + off) : zero4();
  *reinterpret_cast<f32x4_t *>(bp.dh0 + off) = x;
}

// ---------------------------------------------------------------- gla_bwd_scan
// Both walks over each sequence's chunks, per float4 of the K x V state:
//   forward: carry = h0 (or 0); slot c receives the carry S_c (the state
//            before chunk c), then carry = a_c . carry + summary_c
//   reverse: carry = dht (or 0); slot c receives the carry E_c (the gradient
//            reaching the state after chunk c), then carry = dsummary_c + a_c . carry;
//            the final carry is dh0.
// The first half of the grid runs the forward walks, the second half the
// reverse ones.  Loads of a batch of chunks are issued before its serial updates.
__global__ __launch_bounds__(256) void gla_bwd_scan(BwdParams bp, int per_state) {
  const WalkParams &p = bp.w;
  const long long pairs = (long long)p.N * p.HV;
  long long blk = blockIdx.x;
  const bool reverse = blk >= pairs * per_state;  // the second half of the grid walks the gradient
  if (reverse) blk -= pairs * per_state;
  const long long pair = blk / per_state;
  const int eb = (int)(blk - pair * per_state);
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
  const int64_t sidx = (((int64_t)n * p.HV + hv) * p.Kmem + krow) * bp.Vmem + col;  // h0, dht, dh0 element
  constexpr int BATCH = 16;
  auto cell = [&](float *base, int c) {
    return reinterpret_cast<f32x4_t *>(base + ((int64_t)(first + c) * p.HV + hv) * p.K * p.V) + e4;
  };
  auto decay = [&](int c) { return bp.ddecay[((int64_t)(first + c) * p.HV + hv) * p.K + krow]; };
  if (!reverse) {
    f32x4_t s = p.h0 ? *reinterpret_cast<const f32x4_t *>(p.h0 + sidx) : zero4();
    for (int c0 = 0; c0 < nc; c0 += BATCH) {
      const int nb = min(BATCH, nc - c0);
      f32x4_t d[BATCH];
      float a[BATCH];
#pragma unroll
      for (int b = 0; b < BATCH; ++b)
        if (b < nb) {
          d[b] = *cell(bp.fstate, c0 + b);
          a[b] = decay(c0 + b);
        }
#pragma unroll
      for (int b = 0; b < BATCH; ++b)
        if (b < nb) {
          *cell(bp.fstate, c0 + b) = s;
          s = a[b] * s + d[b];
        }
    }
    return;
  }
  f32x4_t e = bp.dht ? *reinterpret_cast<const f32x4_t *>(bp.dht + sidx) : zero4();
  for (int c1 = nc; c1 > 0; c1 -= BATCH) {
    const int nb = min(BATCH, c1);
    f32x4_t d[BATCH];
    float a[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; ++b)
      if (b < nb) {
        d[b] = *cell(bp.dstate, c1 - 1 - b);
        a[b] = decay(c1 - 1 - b);
      }
#pragma unroll
    for (int b = 0; b < BATCH; ++b)
      if (b < nb) {
        *cell(bp.dstate, c1 - 1 - b) = e;
        e = d[b] + a[b] * e;
      }
  }
  if (bp.dh0) *reinterpret_cast<f32x4_t *>(bp.dh0 + sidx) = e;
}

// ---------------------------------------------------------------- dq / dk stores
// dq and dk belong to key heads.  With one value head per key head and one
// value slice they are stored in the input dtype; otherwise each value head
// (and slice) stores its fp32 share to dq_part / dk_part [B,T,HV,K] and
// gla_bwd_group_sum adds the shares.
template <bool BF>
__device__ __forceinline__ void store_dqk(const BwdParams &bp, int64_t row, int hv, int k, float dqv, float dkv) {
  const WalkParams &p = bp.w;
  if (bp.dq_part == nullptr) {
    const int64_t off = (row * p.H + hv) * p.Kmem + k;
    st_el<BF>(bp.dq, off, dqv);
    st_el<BF>(bp.dk, off, dkv);
  } else {
    const int64_t off = (row * p.HV + hv) * p.Kmem + k;
    bp.dq_part[off] = dqv;
    bp.dk_part[off] = dkv;
  }
}

// ---------------------------------------------------------------- gla_bwd_chunk
// The gradients of one chunk of one value head.  For bf16 inputs the score
// tiles, the inter-chunk products and (k e^{G_last - G}) E_c run on
// v_mfma_f32_16x16x32_bf16 with split operands; A^T do, dA' (k e^-G) and
// dA'^T (q e^G), and every product of fp32 inputs, on v_mfma_f32_16x16x4f32.
// NW waves (8 for 128 keys: two per SIMD, so that
// one wave's products run while the other waits for state tiles); wave w owns
// key block w of 16 keys in every key-space product and the dg cumsum down its
// columns.  Value blocks of 16 are dealt to waves; with fewer value blocks
// than waves, a wave takes half of the row blocks of one value block.  Score
// tiles are shared through LDS.  One workgroup per (chunk slot, value head);
// its row loads are issued together, before the gate cumsum.  A chunk with a
// key whose decay over the chunk is below e^-80 sets its flag and leaves its
// outputs to gla_bwd_chunk_exact.
template <int KD>
constexpr int chunk_waves() { return KD == 128 ? 8 : 4; }

template <bool BF, int KD, int VD, bool GH>
struct ChunkRows {
  static constexpr int NT = 64 * chunk_waves<KD>();
  static constexpr int TK = 64 * KD / 4 / NT, TV = 64 * VD / 4 / NT;  // row quads per thread
  typename RawQuad<BF>::type q[TK], k[TK], v[TV], o[TV];
  GateRows<KD, GH, NT> gate;
};

__device__ __forceinline__ bool chunk_task(const WalkParams &p, long long task, ChunkAt &ca, int &hv, int &slot) {
  hv = (int)(task % p.HV);
  slot = (int)(task / p.HV);
  return chunk_at(p, slot, ca);
}

template <bool BF, int KD, int VD, bool GH>
__device__ __forceinline__ void chunk_load(const BwdParams &bp, const ChunkAt &ca, int hv, ChunkRows<BF, KD, VD, GH> &rw) {
  using R = ChunkRows<BF, KD, VD, GH>;
  const WalkParams &p = bp.w;
  const int h = hv / p.G;
  const int64_t fk = (ca.row0 * p.H + h) * p.Kmem, fv = (ca.row0 * p.HV + hv) * bp.Vmem;
  const ChunkRowsRsrc rq = chunk_rows<BF>(p.q, fk, p.H * p.Kmem, p.K, ca.L);
  const ChunkRowsRsrc rk = chunk_rows<BF>(p.k, fk, p.H * p.Kmem, p.K, ca.L);
  const ChunkRowsRsrc ro = chunk_rows<BF>(bp.dout, fv, p.HV * bp.Vmem, p.V, ca.L);
  const ChunkRowsRsrc rv = chunk_rows<BF>(p.v, fv, p.HV * bp.Vmem, p.V, ca.L);
#pragma unroll
  for (int t = 0; t < R::TK; ++t) {
    const int e = threadIdx.x + R::NT * t, i = e / (KD / 4), c4 = (e % (KD / 4)) * 4;
    rw.q[t] = ld_row4<BF>(rq, i, c4);
    rw.k[t] = ld_row4<BF>(rk, i, c4);
  }
#pragma unroll
  for (int t = 0; t < R::TV; ++t) {
    const int e = threadIdx.x + R::NT * t, i = e / (VD / 4), c4 = (e % (VD / 4)) * 4;
    rw.o[t] = ld_row4<BF>(ro, i, c4);
    rw.v[t] = ld_row4<BF>(rv, i, c4);
  }
  gate_load<KD, GH, R::NT>(p, ca, hv, rw.gate);
}

template <bool BF, int KD, int VD, bool GH>
__global__ __launch_bounds__(64 * chunk_waves<KD>(), 1) void gla_bwd_chunk(BwdParams bp) {
  const WalkParams &p = bp.w;
  using R = ChunkRows<BF, KD, VD, GH>;
  constexpr int NW = chunk_waves<KD>(), NT = 64 * NW;
  constexpr int WV = KD > VD ? KD : VD;
  constexpr int NVBLK = VD / 16;                      // value blocks
  constexpr int JSPLIT = NW > NVBLK ? NW / NVBLK : 1; // waves sharing one value block
  constexpr int NVB = NVBLK >= NW ? NVBLK / NW : 1;   // value blocks per wave
  constexpr int NJB = 4 / JSPLIT;                     // row blocks per wave in value space
  constexpr int NTILE = (10 + NW - 1) / NW;           // score tiles per wave (at most)
  static_assert(KD / 16 == NW, "one key block per wave");
  __shared__ __attribute__((aligned(16))) float sQ[64 * KD];  // q e^G
  __shared__ __attribute__((aligned(16))) float sK[64 * KD];  // k e^-G
  __shared__ __attribute__((aligned(16))) float sO[64 * VD];  // do
  __shared__ __attribute__((aligned(16))) float sV[64 * WV];  // G, then v
  __shared__ __attribute__((aligned(16))) float sX[64 * 64];  // A, then dA'
  __shared__ __attribute__((aligned(16))) float sEl[KD];      // e^{G_last}
  __shared__ float sGl[KD];                                   // G_last
  __shared__ float tot[NT];
  __shared__ float sRow[NW * 64];  // per-head gate: dg of each row summed over each wave's keys

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, l16 = lane & 15, lg = lane >> 4;
  const int kb = wave * 16;                                        // this wave's key block
  const int vb0 = (JSPLIT > 1 ? wave % NVBLK : wave * NVB) * 16;   // first value column of its blocks
  const int jb0 = JSPLIT > 1 ? (wave / NVBLK) * NJB : 0;           // first row block (value space)
  ChunkAt ca;
  int hv = 0, slot = 0;
  if (!chunk_task(p, blockIdx.x, ca, hv, slot)) return;
  R rw;
  chunk_load<BF, KD, VD, GH>(bp, ca, hv, rw);
  {
    const int chv = hv, cslot = slot;
    const int L = ca.L;
    const int64_t row0 = ca.row0;
    const int cfirst = ca.si.first, cc = ca.c;
    // The outputs leave through buffer descriptors over this chunk's token
    // rows: rows past its last token lie outside the range, so their stores
    // are dropped without a branch, and the offsets are 32-bit.  (K and V are
    // multiples of 16, so a key or value block is wholly inside or outside.)
    // dq, dk: [B,T,H,Kmem] in the input dtype with one value head per key head
    // (then H = HV) and one value slice, else this value head's and slice's
    // fp32 share [B,T,HV,Kmem]; this launch's keys.  dv: [B,T,HV,Vmem], this
    // launch's columns, or with several key blocks this block's fp32 share.
    constexpr int ES = BF ? 2 : 4;
    const bool part = bp.dq_part != nullptr;
    const int ESQ = part ? 4 : ES;
    const bool dvpart = bp.dv_part != nullptr;  // dv is this key block's fp32 share
    const int ESV = dvpart ? 4 : ES;
    const int strideV = p.HV * bp.Vmem, strideK = p.HV * p.Kmem;  // elements between token rows
    const __amdgpu_buffer_rsrc_t rDv =
        make_rsrc(dvpart ? static_cast<char *>(static_cast<void *>(bp.dv_part)) + (row0 * p.HV + chv) * bp.Vmem * 4
                         : static_cast<char *>(bp.dv) + (row0 * p.HV + chv) * bp.Vmem * ES,
                  ((int64_t)(L - 1) * strideV + p.V) * ESV);
    const int64_t qk0 = (row0 * p.HV + chv) * p.Kmem, qkBytes = ((int64_t)(L - 1) * strideK + p.K) * ESQ;
    const __amdgpu_buffer_rsrc_t rDq =
        make_rsrc(part ? static_cast<char *>(static_cast<void *>(bp.dq_part)) + qk0 * 4 : static_cast<char *>(bp.dq) + qk0 * ES, qkBytes);
    const __amdgpu_buffer_rsrc_t rDk =
        make_rsrc(part ? static_cast<char *>(static_cast<void *>(bp.dk_part)) + qk0 * 4 : static_cast<char *>(bp.dk) + qk0 * ES, qkBytes);
    const __amdgpu_buffer_rsrc_t rDg = make_rsrc(GH ? bp.dg : bp.dg + qk0, GH ? 0 : ((int64_t)(L - 1) * strideK + p.K) * 4);
    // G -> sV; q e^G, k e^-G -> sQ, sK; this lane's G values; the chunk's decay per key
    gate_stage<KD, GH, NT>(rw.gate, sV);
    __syncthreads();
    gate_cumsum_lds<KD, GH, NT>(p.K, sV, tot);
    float Gr[4][4];  // G at rows b*16 + 4 lg + r of key kb + l16 (the epilogue's elements)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) Gr[b][r] = sV[swz<KD>(b * 16 + 4 * lg + r, kb + l16)];
    bool low = false;
#pragma unroll
    for (int t = 0; t < R::TK; ++t) {
      const int e = threadIdx.x + NT * t, i = e / (KD / 4), c4 = (e % (KD / 4)) * 4;
      const f32x4_t G4 = lds4<KD>(sV, i, c4);
      f32x4_t xq = unpack4<BF>(rw.q[t]), xk = unpack4<BF>(rw.k[t]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        xq[r] *= __expf(G4[r]);
        xk[r] *= __expf(-G4[r]);
      }
      lds4_st<KD>(sQ, i, c4, xq);
      lds4_st<KD>(sK, i, c4, xk);
      if (i == 63) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          sGl[c4 + r] = G4[r];
          sEl[c4 + r] = __expf(G4[r]);
          if (c4 + r < p.K && !(G4[r] >= kMinChunkLogDecay)) low = true;
        }
      }
    }
    const bool exact = __syncthreads_or(low);  // also: every thread is done reading G from sV
    if (threadIdx.x == 0) bp.flags[(int64_t)cslot * p.HV + chv] = exact ? 1 : 0;
    if (exact) return;
#pragma unroll
    for (int t = 0; t < R::TV; ++t) {
      const int e = threadIdx.x + NT * t, i = e / (VD / 4), c4 = (e % (VD / 4)) * 4;
      lds4_st<VD>(sO, i, c4, unpack4<BF>(rw.o[t]));
      lds4_st<VD>(sV, i, c4, unpack4<BF>(rw.v[t]));
    }
    __syncthreads();

    // ---- scores: A -> sX, dA' kept in registers until A has been used
    f32x4_t dAr[NTILE];
#pragma unroll
    for (int t = 0; t < NTILE; ++t) {
      const int idx = wave + NW * t;
      dAr[t] = zero4();
      if (idx >= 10) continue;
      int ib, jb;
      tri_tile(idx, ib, jb);
      f32x4_t a = zero4(), d = zero4();
      if constexpr (BF) {
        // A feeds dv only (held to the bf16 rule): q e^G and k e^-G split into
        // bf16 hi + lo, three products.  do and v are exact in bf16: dA' is
        // one product per 32 columns.
#pragma unroll 2
        for (int k0 = 0; k0 < KD; k0 += 32) {
          float q8[8], k8[8];
          lds8<KD>(sQ, ib * 16 + l16, k0 + 8 * lg, q8);
          lds8<KD>(sK, jb * 16 + l16, k0 + 8 * lg, k8);
          u32x4_t qh, ql, kh, kl;
          split8_2(q8, qh, ql);
          split8_2(k8, kh, kl);
          a = mfma_bf(qh, kl, a);
          a = mfma_bf(ql, kh, a);
          a = mfma_bf(qh, kh, a);
        }
#pragma unroll 2
        for (int v0 = 0; v0 < VD; v0 += 32) {
          float o8[8], w8[8];
          lds8<VD>(sO, ib * 16 + l16, v0 + 8 * lg, o8);
          lds8<VD>(sV, jb * 16 + l16, v0 + 8 * lg, w8);
          d = mfma_bf(pack8(o8), pack8(w8), d);
        }
      } else {
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
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool keep = ib > jb || l16 <= 4 * lg + r;  // column j <= row i
        sX[swz<64>(ib * 16 + 4 * lg + r, jb * 16 + l16)] = keep ? p.scale * a[r] : 0.f;
        dAr[t][r] = keep ? p.scale * d[r] : 0.f;
      }
    }
    __syncthreads();

    // ---- dv = A^T do (this wave's value blocks and row blocks)
    f32x4_t dv[NVB][NJB];
#pragma unroll
    for (int b = 0; b < NVB; ++b)
#pragma unroll
      for (int j = 0; j < NJB; ++j) dv[b][j] = zero4();
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
      if (ib < jb0) continue;
      float ov[NVB][4];
#pragma unroll
      for (int b = 0; b < NVB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) ov[b][r] = sO[swz<VD>(ib * 16 + 4 * lg + r, vb0 + b * 16 + l16)];
#pragma unroll
      for (int j = 0; j < NJB; ++j) {
        const int jb = jb0 + j;
        if (jb > ib) continue;
        float av[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) av[r] = sX[swz<64>(ib * 16 + 4 * lg + r, jb * 16 + l16)];
#pragma unroll
        for (int b = 0; b < NVB; ++b)
#pragma unroll
          for (int r = 0; r < 4; ++r) dv[b][j] = mfma_f32(av[r], ov[b][r], dv[b][j]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NTILE; ++t) {
      const int idx = wave + NW * t;
      if (idx >= 10) continue;
      int ib, jb;
      tri_tile(idx, ib, jb);
#pragma unroll
      for (int r = 0; r < 4; ++r) sX[swz<64>(ib * 16 + 4 * lg + r, jb * 16 + l16)] = dAr[t][r];
    }

    // ---- inter-chunk terms: dq = do S_c^T, dkI = v E_c^T, rs = rowsum(S_c . E_c)
    const float *Sc = bp.fstate + ((int64_t)(cfirst + cc) * p.HV + chv) * p.K * p.V;
    const float *Ec = bp.dstate + ((int64_t)(cfirst + cc) * p.HV + chv) * p.K * p.V;
    const __amdgpu_buffer_rsrc_t rS = make_rsrc(Sc, (int64_t)p.K * p.V * 4), rE = make_rsrc(Ec, (int64_t)p.K * p.V * 4);
    f32x4_t dq[4], dkI[4];
    float rs = 0.f;
#pragma unroll
    for (int b = 0; b < 4; ++b) dq[b] = dkI[b] = zero4();
    if constexpr (BF) {
      // bf16 inputs: do and v are exact in bf16; S and E are split into three
      // bf16 terms (hi, the rounded remainder, the rounded remainder of that;
      // every remainder is exact in fp32), so do S^T = sum of three products
      // keeps fp32 accuracy, on v_mfma_f32_16x16x32_bf16 (each lane: 8
      // consecutive values).  Two terms carried 16 bits, which the reverse
      // cumsum of dg amplified past its fp32 bound under strong gates.
      const int krow = kb + l16;
#pragma unroll 2
      for (int v0 = 0; v0 < VD; v0 += 32) {
        const int col = v0 + 8 * lg;
        const bool in = krow < p.K && col < p.V;  // V is a multiple of 16: col < V covers col + 7
        const int off = in ? (krow * p.V + col) * 4 : kOutsideRange;
        float sv[8], ev[8];
        {
          const f32x4_t s0 = buf_ldf4<0>(rS, off), s1 = buf_ldf4<0>(rS, off + 16);
          const f32x4_t e0 = buf_ldf4<0>(rE, off), e1 = buf_ldf4<0>(rE, off + 16);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            sv[r] = s0[r]; sv[4 + r] = s1[r];
            ev[r] = e0[r]; ev[4 + r] = e1[r];
          }
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) rs += sv[r] * ev[r];
        u32x4_t sh, sm, sl, eh, em, el;
        split8_3(sv, sh, sm, sl);
        split8_3(ev, eh, em, el);
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) {
          const f32x4_t o0 = lds4<VD>(sO, ib * 16 + l16, col), o1 = lds4<VD>(sO, ib * 16 + l16, col + 4);
          const f32x4_t w0 = lds4<VD>(sV, ib * 16 + l16, col), w1 = lds4<VD>(sV, ib * 16 + l16, col + 4);
          const u32x4_t o8 = {pack_bf16(o0[0], o0[1]), pack_bf16(o0[2], o0[3]), pack_bf16(o1[0], o1[1]),
                              pack_bf16(o1[2], o1[3])};
          const u32x4_t w8 = {pack_bf16(w0[0], w0[1]), pack_bf16(w0[2], w0[3]), pack_bf16(w1[0], w1[1]),
                              pack_bf16(w1[2], w1[3])};
          dq[ib] = mfma_bf(o8, sl, dq[ib]);
          dq[ib] = mfma_bf(o8, sm, dq[ib]);
          dq[ib] = mfma_bf(o8, sh, dq[ib]);
          dkI[ib] = mfma_bf(w8, el, dkI[ib]);
          dkI[ib] = mfma_bf(w8, em, dkI[ib]);
          dkI[ib] = mfma_bf(w8, eh, dkI[ib]);
        }
      }
    } else {
      const int krow = kb + l16;
#pragma unroll 4
      for (int v0 = 0; v0 < VD; v0 += 16) {
        const int col = v0 + 4 * lg;
        const bool in = krow < p.K && col < p.V;
        const int off = in ? (krow * p.V + col) * 4 : kOutsideRange;
        const f32x4_t s4 = buf_ldf4<0>(rS, off), e4 = buf_ldf4<0>(rE, off);
        rs += s4[0] * e4[0] + s4[1] * e4[1] + s4[2] * e4[2] + s4[3] * e4[3];
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) {
          const f32x4_t o4 = lds4<VD>(sO, ib * 16 + l16, v0 + 4 * lg);
          const f32x4_t w4 = lds4<VD>(sV, ib * 16 + l16, v0 + 4 * lg);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            dq[ib] = mfma_f32(o4[r], s4[r], dq[ib]);
            dkI[ib] = mfma_f32(w4[r], e4[r], dkI[ib]);
          }
        }
      }
    }
    __syncthreads();  // dA' visible

    // ---- dv += (k e^{G_last - G}) E_c, store dv
    if constexpr (BF) {
      // both operands computed: bf16 hi + lo each, three products (dv is held
      // to the bf16 rule)
#pragma unroll 1
      for (int k0 = 0; k0 < KD; k0 += 32) {
        u32x4_t eh[NVB], elo[NVB];
#pragma unroll
        for (int b = 0; b < NVB; ++b) {
          // keys past K lie past the state's range; a value block past V is
          // sent outside it
          const int cb = vb0 + b * 16 < p.V ? ((k0 + 8 * lg) * p.V + vb0 + b * 16 + l16) * 4 : kOutsideRange;
          float e8[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) e8[e] = bld_f32(rE, cb + e * p.V * 4);
          split8_2(e8, eh[b], elo[b]);
        }
        const f32x4_t el0 = *reinterpret_cast<const f32x4_t *>(sEl + k0 + 8 * lg);
        const f32x4_t el1 = *reinterpret_cast<const f32x4_t *>(sEl + k0 + 8 * lg + 4);
#pragma unroll
        for (int j = 0; j < NJB; ++j) {
          float k8[8];
          lds8<KD>(sK, (jb0 + j) * 16 + l16, k0 + 8 * lg, k8);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            k8[r] *= el0[r];
            k8[4 + r] *= el1[r];
          }
          u32x4_t kh, kl;
          split8_2(k8, kh, kl);
#pragma unroll
          for (int b = 0; b < NVB; ++b) {
            dv[b][j] = mfma_bf(kh, elo[b], dv[b][j]);
            dv[b][j] = mfma_bf(kl, eh[b], dv[b][j]);
            dv[b][j] = mfma_bf(kh, eh[b], dv[b][j]);
          }
        }
      }
    } else {
#pragma unroll 2
      for (int k0 = 0; k0 < KD; k0 += 16) {
        const f32x4_t el4 = *reinterpret_cast<const f32x4_t *>(sEl + k0 + 4 * lg);
        float ev[NVB][4];
#pragma unroll
        for (int b = 0; b < NVB; ++b) {
          const int cb = vb0 + b * 16 < p.V ? ((k0 + 4 * lg) * p.V + vb0 + b * 16 + l16) * 4 : kOutsideRange;
#pragma unroll
          for (int r = 0; r < 4; ++r) ev[b][r] = bld_f32(rE, cb + r * p.V * 4);
        }
#pragma unroll
        for (int j = 0; j < NJB; ++j) {
          const f32x4_t k4 = lds4<KD>(sK, (jb0 + j) * 16 + l16, k0 + 4 * lg) * el4;
#pragma unroll
          for (int b = 0; b < NVB; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) dv[b][j] = mfma_f32(k4[r], ev[b][r], dv[b][j]);
        }
      }
    }
    auto store_dv = [&](auto es_tag) {
      constexpr bool F32 = decltype(es_tag)::value;  // the fp32 share of a key block
#pragma unroll
      for (int b = 0; b < NVB; ++b) {
        if (vb0 + b * 16 >= p.V) continue;  // uniform over the wave
#pragma unroll
        for (int j = 0; j < NJB; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = (jb0 + j) * 16 + 4 * lg + r, col = vb0 + b * 16 + l16;
            if constexpr (F32) bst_el<false>(rDv, (row * strideV + col) * 4, dv[b][j][r]);
            else bst_el<BF>(rDv, (row * strideV + col) * ES, dv[b][j][r]);
          }
      }
    };
    if (dvpart) store_dv(std::true_type{});
    else store_dv(std::false_type{});

    // ---- dq = scale (do S_c^T) + dA' (k e^-G)
#pragma unroll
    for (int b = 0; b < 4; ++b) dq[b] *= p.scale;
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      float kv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) kv[r] = sK[swz<KD>(jb * 16 + 4 * lg + r, kb + l16)];
#pragma unroll
      for (int ib = jb; ib < 4; ++ib) {
        const f32x4_t a4 = lds4<64>(sX, ib * 16 + l16, jb * 16 + 4 * lg);
#pragma unroll
        for (int r = 0; r < 4; ++r) dq[ib] = mfma_f32(a4[r], kv[r], dq[ib]);
      }
    }
    // ---- dkA = dA'^T (q e^G)
    f32x4_t dkA[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) dkA[b] = zero4();
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
      float qv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) qv[r] = sQ[swz<KD>(ib * 16 + 4 * lg + r, kb + l16)];
#pragma unroll
      for (int jb = 0; jb <= ib; ++jb) {
        float av[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) av[r] = sX[swz<64>(ib * 16 + 4 * lg + r, jb * 16 + l16)];
#pragma unroll
        for (int r = 0; r < 4; ++r) dkA[jb] = mfma_f32(av[r], qv[r], dkA[jb]);
      }
    }

    // ---- gradients in key space, and dg by a reverse cumsum down each key column
    {
      const int k = kb + l16;
      const float gl = sGl[k], el = sEl[k];
      float t[4][4];
      float colk = 0.f;
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = b * 16 + 4 * lg + r;
          const float Gv = Gr[b][r], qg = sQ[swz<KD>(i, k)], kg = sK[swz<KD>(i, k)];
          const float kdkI = kg * el * dkI[b][r];
          const float dqv = __expf(Gv) * dq[b][r];
          const float dkv = __expf(-Gv) * dkA[b][r] + __expf(gl - Gv) * dkI[b][r];
          if (kb < p.K) {  // uniform over the wave; rows past the chunk fall outside the range
            const int off = i * strideK + k;
            if (part) {
              bst_el<false>(rDq, off * 4, dqv);
              bst_el<false>(rDk, off * 4, dkv);
            } else {
              bst_el<BF>(rDq, off * ES, dqv);
              bst_el<BF>(rDk, off * ES, dkv);
            }
          }
          t[b][r] = qg * dq[b][r] - (kg * dkA[b][r] + kdkI);
          colk += kdkI;
        }
      float rsa = rs;
      rsa += __shfl_xor(rsa, 16);
      rsa += __shfl_xor(rsa, 32);
      colk += __shfl_xor(colk, 16);
      colk += __shfl_xor(colk, 32);
      float carry = el * rsa + colk;  // dg of the first token after the chunk
      float runv[4][4];                // per-head gate: this key's share of each row's dg
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
          if constexpr (GH) runv[b][r] = k < p.K ? run : 0.f;
          else if (kb < p.K) bst_el<false>(rDg, (i * strideK + k) * 4, run);
        }
        carry += total;
      }
      if constexpr (GH) {
        // sums over the wave's 16 keys, then over the waves, in a fixed order
        // (the same dg on every run)
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float x = runv[b][r];
            x += __shfl_xor(x, 1);
            x += __shfl_xor(x, 2);
            x += __shfl_xor(x, 4);
            x += __shfl_xor(x, 8);
            if (l16 == 0) sRow[wave * 64 + b * 16 + 4 * lg + r] = x;
          }
      }
    }
    if (GH) {
      __syncthreads();
      if (threadIdx.x < L) {
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) sum += sRow[w * 64 + threadIdx.x];
        bp.dg[(row0 + threadIdx.x) * p.HV + chv] = sum;
      }
    }
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
// The token-by-token gradients of one flagged chunk ca of value head hv (the
// body of gla_bwd_chunk_exact; the LDS arrays are the kernel's).
template <bool BF, int KD, int VD, bool GH>
__device__ __forceinline__ void chunk_exact_task(const BwdParams &bp, int hv, const ChunkAt &ca, float *sV, float *sK,
                                                 float *sA, float *sDq, float *sRed, float *sRow, float *sKeyDg) {
  const WalkParams &p = bp.w;
  constexpr int PARTS = 256 / KD, NC = VD / PARTS;
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
    sK[e] = in ? ld_el<BF>(p.k, (row0 + i) * p.H * p.Kmem + h * p.Kmem + kk) : 0.f;
    float gv = 0.f;
    if (in) gv = GH ? p.g[(row0 + i) * p.HV + hv] : p.g[((row0 + i) * p.HV + hv) * p.Kmem + kk];
    sA[e] = __expf(gv);
  }
  for (int e = threadIdx.x; e < 64 * VD; e += 256) {
    const int i = e / VD, c = e % VD;
    sV[e] = (i < L && c < p.V) ? ld_el<BF>(p.v, ((row0 + i) * p.HV + hv) * bp.Vmem + c) : 0.f;
  }
  if (GH && threadIdx.x < 64) sRow[threadIdx.x] = 0.f;
  __syncthreads();

  const float *Sc = bp.fstate + ((int64_t)(ca.si.first + ca.c) * p.HV + hv) * p.K * p.V;
  const float *Ec = bp.dstate + ((int64_t)(ca.si.first + ca.c) * p.HV + hv) * p.K * p.V;
  auto dout = [&](int i, int j) -> float {  // do at token i, column col0 + j
    const int col = col0 + j;
    return col < p.V ? ld_el<BF>(bp.dout, ((row0 + i) * p.HV + hv) * bp.Vmem + col) : 0.f;
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
    S[j] = (kin && col < p.V) ? Sc[(int64_t)key * p.V + col] : 0.f;
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
    const int64_t qoff = (row0 + i) * p.H * p.Kmem + h * p.Kmem + key;
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
    if (kin) {
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
      if (!GH) bp.dg[(row * p.HV + hv) * p.Kmem + key] = dgi;
    }
    if (GH && cp == 0) sKeyDg[key] = kin ? a * acc : 0.f;
    __syncthreads();
    if (GH && wave == 0) {
      // the sum over keys in a fixed order (the same dg on every run)
      float x = sKeyDg[lane] + (KD > 64 ? sKeyDg[lane + 64] : 0.f);
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
      if (lane == 0) sRow[i] = x;
    }
    for (int col = threadIdx.x; col < p.V; col += 256) {
      const float sv = sRed[col] + sRed[VD + col] + sRed[2 * VD + col] + sRed[3 * VD + col];
      const int64_t dvo = ((row0 + i) * p.HV + hv) * bp.Vmem + col;
      if (bp.dv_part != nullptr) bp.dv_part[dvo] = sv;
      else st_el<BF>(bp.dv, dvo, sv);
    }
#pragma unroll
    for (int j = 0; j < NC; ++j) U[j] *= a;
    __syncthreads();  // sRed is reused by the next token
  }
  if (GH && threadIdx.x < L) bp.dg[(row0 + threadIdx.x) * p.HV + hv] = sRow[threadIdx.x];
}

// The kernel: one workgroup per compute unit, each over a fixed share of the
// (slot, value head) tasks; a launch with no flagged chunk reads the flags and
// ends.
template <bool BF, int KD, int VD, bool GH>
__global__ __launch_bounds__(256, 1) void gla_bwd_chunk_exact(BwdParams bp) {
  const WalkParams &p = bp.w;
  __shared__ __attribute__((aligned(16))) float sV[64 * VD];  // v rows
  __shared__ float sK[64 * KD];    // k rows
  __shared__ float sA[64 * KD];    // e^{g} per token and key
  __shared__ float sDq[64 * KD];   // dq
  __shared__ float sRed[4 * VD];   // per-wave partial dv of one token
  __shared__ float sRow[64];       // per-head gate: dg of each token
  __shared__ float sKeyDg[KD];     // per-head gate: each key's share of one token's dg

  __shared__ int sTodo[256];  // flagged tasks of one round
  __shared__ int sCount;
  // Tasks blockIdx.x + gridDim.x i (task = slot HV + hv, the flags' order):
  // one round reads 256 of their flags at once and runs the flagged ones.
  const unsigned ntask = (unsigned)p.seg_slots * (unsigned)p.HV;
  const unsigned mine = (ntask - blockIdx.x + gridDim.x - 1) / gridDim.x;
  for (unsigned base = 0; base < mine; base += 256) {
    if (threadIdx.x == 0) sCount = 0;
    __syncthreads();
    if (base + threadIdx.x < mine) {
      const unsigned t = blockIdx.x + gridDim.x * (base + threadIdx.x);
      if (bp.flags[t] != 0) sTodo[atomicAdd(&sCount, 1)] = (int)t;
    }
    __syncthreads();
    const int todo = sCount;
    for (int u = 0; u < todo; ++u) {
      const unsigned task = (unsigned)sTodo[u];
      const int hv = (int)(task % (unsigned)p.HV);
      const int slot = (int)(task / (unsigned)p.HV);
      ChunkAt ca;
      if (chunk_at(p, slot, ca)) chunk_exact_task<BF, KD, VD, GH>(bp, hv, ca, sV, sK, sA, sDq, sRed, sRow, sKeyDg);
      __syncthreads();  // LDS is reused by the next task
    }
    __syncthreads();  // sTodo and sCount are reused by the next round
  }
}

// ---------------------------------------------------------------- gla_bwd_group_sum
// dq, dk of key head h = the sum of the fp32 shares of its G value heads over
// every value slice (slices `slice_stride` floats apart), rounded once to the
// output dtype.  One thread per 4 keys of a token row.
template <bool BF>
__global__ __launch_bounds__(256) void gla_bwd_group_sum(BwdParams bp, int64_t quads, int slices,
                                                         int64_t slice_stride) {
  const WalkParams &p = bp.w;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= quads) return;
  const int K4 = p.K / 4;
  const int64_t rowh = e / K4;  // (token, key head)
  const int k = (int)(e - rowh * K4) * 4;
  const int64_t row = rowh / p.H;
  const int h = (int)(rowh - row * p.H);
  f32x4_t dq = zero4(), dk = zero4();
  for (int sl = 0; sl < slices; ++sl)
    for (int gi = 0; gi < p.G; ++gi) {
      const int64_t off = sl * slice_stride + (row * p.HV + h * p.G + gi) * p.K + k;
      dq += *reinterpret_cast<const f32x4_t *>(bp.dq_part + off);
      dk += *reinterpret_cast<const f32x4_t *>(bp.dk_part + off);
    }
  const int64_t off = rowh * p.K + k;
  st_el4<BF>(bp.dq, off, dq);
  st_el4<BF>(bp.dk, off, dk);
}

// Columns [0, cols) of `groups` x `rows` fp32 rows: row r of group gi from
// src + gi src.group + r src.row to dst + gi dst.group + r dst.row; one thread
// per float4 (cols, strides and bases multiples of 4 floats).
struct RowsLayout {
  int64_t group, row;
};
__global__ __launch_bounds__(256) void gla_bwd_copy_rows(float *dst, RowsLayout dl, const float *src, RowsLayout sl,
                                                         int rows, int64_t quads, int cols) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= quads) return;
  const int q = cols / 4;
  const int64_t gr = e / q;  // gi rows + r
  const int c = (int)(e - gr * q) * 4;
  const int64_t gi = gr / rows, r = gr - gi * rows;
  *reinterpret_cast<f32x4_t *>(dst + gi * dl.group + r * dl.row + c) =
      *reinterpret_cast<const f32x4_t *>(src + gi * sl.group + r * sl.row + c);
}

// dv with several key blocks: the blocks' fp32 shares summed and rounded once.
template <bool BF>
__global__ __launch_bounds__(256) void gla_bwd_dv_sum(void *dv, const float *parts, int64_t n4, int blocks) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;  // a float4 of dv (n = 4 n4 elements)
  if (e >= n4) return;
  f32x4_t x = zero4();
  for (int b = 0; b < blocks; ++b) x += reinterpret_cast<const f32x4_t *>(parts + b * 4 * n4)[e];
  st_el4<BF>(dv, 4 * e, x);
}

// dg with several value slices (or, with a per-head gate, key blocks): out[e]
// = the sum of the fp32 shares.
__global__ __launch_bounds__(256) void gla_bwd_slice_sum(float *out, const float *parts, int64_t n, int slices) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= n) return;
  float x = 0.f;
  for (int sl = 0; sl < slices; ++sl) x += parts[sl * n + e];
  out[e] = x;
}
// The same for n a multiple of 4, a float4 per thread (n4 = n / 4).
__global__ __launch_bounds__(256) void gla_bwd_slice_sum4(float *out, const float *parts, int64_t n4, int slices) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= n4) return;
  f32x4_t x = zero4();
  for (int sl = 0; sl < slices; ++sl) x += reinterpret_cast<const f32x4_t *>(parts + sl * 4 * n4)[e];
  reinterpret_cast<f32x4_t *>(out)[e] = x;
}

template <bool BF, int KD, int VD, bool GH>
hipError_t launch_bwd_t(int which, const BwdParams &bp, long long blocks, hipStream_t s) {
  const dim3 grid((unsigned)blocks), block(256);
  switch (which) {
    case 0:
      if (bp.walk)
        hipLaunchKernelGGL((gla_bwd_local<BF, KD, VD, GH, kLocalWalk>), grid, dim3(local_threads(kLocalWalk)), 0, s,
                           bp);
      else if (bp.chain != nullptr && bp.w.seg_base != nullptr)
        hipLaunchKernelGGL((gla_bwd_local<BF, KD, VD, GH, kLocalPackedChain>), grid, block, 0, s, bp);
      else
        hipLaunchKernelGGL((gla_bwd_local<BF, KD, VD, GH, kLocalTasks>), grid, block, 0, s, bp);
      break;
    case 1:
      hipLaunchKernelGGL((gla_bwd_chunk<BF, KD, VD, GH>), grid, dim3(64 * chunk_waves<KD>()), 0, s, bp);
      break;
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
  long long blocks = (long long)bp.w.seg_slots * bp.w.HV;
  if (which == 0)  // two per compute unit; walk: one per chain
    blocks = bp.walk ? 2LL * bp.w.N * bp.w.HV : std::min<long long>(bp.persistent_blocks, 2 * blocks);
  // over the flags: one per compute unit (its LDS leaves room for no second)
  if (which == 2) blocks = std::min<long long>(std::max(bp.persistent_blocks / 2, 1), blocks);
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL || bp.w.K > 128 || bp.w.V > 128) return hipErrorInvalidValue;
  const bool gh = bp.w.gate_head != 0;
  if (bf16) return gh ? launch_bwd_kv<true, true>(which, bp, blocks, s) : launch_bwd_kv<true, false>(which, bp, blocks, s);
  return gh ? launch_bwd_kv<false, true>(which, bp, blocks, s) : launch_bwd_kv<false, false>(which, bp, blocks, s);
}

}  // namespace

hipError_t launch_bwd_local(bool bf16, const BwdParams &bp, hipStream_t s) { return launch_bwd_kernel(0, bf16, bp, s); }

hipError_t launch_bwd_chunk(bool bf16, const BwdParams &bp, hipStream_t s) {
  hipError_t e = launch_bwd_kernel(1, bf16, bp, s);
  if (e != hipSuccess) return e;
  return launch_bwd_kernel(2, bf16, bp, s);
}

hipError_t launch_copy_rows(float *dst, int64_t dst_group, int64_t dst_row, const float *src, int64_t src_group,
                            int64_t src_row, long long groups, int rows, int cols, hipStream_t s) {
  const long long quads = groups * rows * (cols / 4);
  const long long blocks = (quads + 255) / 256;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL || cols % 4 != 0 || rows <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gla_bwd_copy_rows, dim3((unsigned)blocks), dim3(256), 0, s, dst, RowsLayout{dst_group, dst_row},
                     src, RowsLayout{src_group, src_row}, rows, (int64_t)quads, cols);
  return hipGetLastError();
}

hipError_t launch_chain_plan(const BwdParams &bp, int cmax, int32_t *scratch, hipStream_t s) {
  const WalkParams &p = bp.w;
  int32_t *hist = scratch, *cnt = hist + cmax + 1, *pbase = cnt + cmax + 1, *order = pbase + cmax + 2;
  hipLaunchKernelGGL(gla_bwd_chain_plan, dim3(1), dim3(1024), 0, s, p.cu, p.N, p.T, p.HV, cmax, p.seg_slots,
                     bp.chain_plan, hist, cnt, pbase, order);
  return hipGetLastError();
}

hipError_t launch_empty_dh0(const BwdParams &bp, hipStream_t s) {
  const long long quads = (long long)bp.w.N * bp.w.HV * bp.w.K * (bp.w.V / 4);
  const long long blocks = (quads + 255) / 256;
  if (blocks <= 0 || bp.dh0 == nullptr) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gla_bwd_empty_dh0, dim3((unsigned)blocks), dim3(256), 0, s, bp, bp.w.K, (int64_t)quads);
  return hipGetLastError();
}

hipError_t launch_dv_sum(bool bf16, void *dv, const float *parts, long long n, int blocks, hipStream_t s) {
  if (n % 4 != 0) return hipErrorInvalidValue;  // rows of V columns, V a multiple of 16
  const long long n4 = n / 4, grid = (n4 + 255) / 256;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (bf16) hipLaunchKernelGGL(gla_bwd_dv_sum<true>, dim3((unsigned)grid), dim3(256), 0, s, dv, parts, (int64_t)n4, blocks);
  else hipLaunchKernelGGL(gla_bwd_dv_sum<false>, dim3((unsigned)grid), dim3(256), 0, s, dv, parts, (int64_t)n4, blocks);
  return hipGetLastError();
}

hipError_t launch_bwd_finish(bool bf16, const BwdParams &bp, int slices, const float *dg_parts, int dg_nparts,
                             float *dg, hipStream_t s) {
  const long long rows = (bp.w.cu ? 1LL : (long long)bp.w.N) * bp.w.T;  // token rows of [B,T]
  if (bp.dq_part != nullptr) {
    const long long quads = rows * bp.w.H * (bp.w.K / 4);
    const long long blocks = (quads + 255) / 256;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    const int64_t stride = rows * bp.w.HV * bp.w.K;
    if (blocks > 0) {
      if (bf16)
        hipLaunchKernelGGL(gla_bwd_group_sum<true>, dim3((unsigned)blocks), dim3(256), 0, s, bp, (int64_t)quads, slices,
                           stride);
      else
        hipLaunchKernelGGL(gla_bwd_group_sum<false>, dim3((unsigned)blocks), dim3(256), 0, s, bp, (int64_t)quads,
                           slices, stride);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if (dg_nparts > 1) {
    const long long n = rows * bp.w.HV * (bp.w.gate_head ? 1 : bp.w.K);
    const bool quads = n % 4 == 0;  // dg and the shares are 16-byte aligned
    const long long blocks = ((quads ? n / 4 : n) + 255) / 256;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    if (blocks > 0) {
      if (quads)
        hipLaunchKernelGGL(gla_bwd_slice_sum4, dim3((unsigned)blocks), dim3(256), 0, s, dg, dg_parts, (int64_t)(n / 4),
                           dg_nparts);
      else
        hipLaunchKernelGGL(gla_bwd_slice_sum, dim3((unsigned)blocks), dim3(256), 0, s, dg, dg_parts, (int64_t)n,
                           dg_nparts);
      return hipGetLastError();
    }
  }
  return hipSuccess;
}

hipError_t launch_bwd_scan(const BwdParams &bp, hipStream_t s) {
  const int KV4 = bp.w.K * bp.w.V / 4;
  const int per_state = (KV4 + 255) / 256;
  const long long blocks = 2LL * bp.w.N * bp.w.HV * per_state;  // forward walks, then reverse walks
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gla_bwd_scan, dim3((unsigned)blocks), dim3(256), 0, s, bp, per_state);
  return hipGetLastError();
}

}  // namespace gla
