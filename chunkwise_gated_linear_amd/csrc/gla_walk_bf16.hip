// Chunk walker for bf16 inputs with K in {64, 128}: the hot kernels of the
// path (gla_chunk_output and gla_chunk_local) for the bf16 workloads.
//
// Same method and precision scheme as the general walker in gla_kernels.hip
// (page "fla/ops/gla/fused_chunk.py": fused_chunk_gla_fwd_kernel carries the
// state, fwd_inner_chunk forms the masked gated in-chunk scores; operands of
// computed values are split into bf16 hi + lo for fp32-level products):
//
//   qc_i = scale q_i P_i / a,  kc_j = k_j R_j    (P, R: running products of exp(g))
//   A = mask_{j<=i}(qc kc^T),  S' = diag(a) S,  o = A v + qc S',  S = S' + kc^T v
//
// Layout for gfx950 (one workgroup of 8 waves per (segment, head, 64- or
// 128-column slice of V), two waves per SIMD):
//  * Waves 4-7 produce: they load the raw q, k, g, v of chunk c+2, form the
//    gated and split operands of chunk c+1 in registers and write them to LDS
//    (qc row by row as it is gated, kc when chunk c is done).  Their memory
//    stalls and vector work run beside the matrix waves on the same SIMDs.
//  * Waves 0-3 compute.  With 64 columns they tile the K x 64 state slice as
//    2 key halves x 2 value halves (32 columns); with 128 columns each holds
//    all K rows of 32 columns; the state stays in MFMA accumulators.  Each
//    computes some of the ten lower 16x16 score tiles (shared through LDS),
//    then its output tiles: qc S' first (it needs no other wave's tiles), then
//    A v once every wave's tiles are there, then its state update.  With 64
//    columns the two key-half partials meet in LDS and are summed after the
//    chunk-done barrier; with 128 columns each wave stages whole tiles, which
//    are stored right after that barrier.
//  * kc^T and v are read as MFMA operands with the LDS transpose read
//    ds_read_b64_tr_b16, so no transposed copy is written.
//  * Global traffic uses per-chunk buffer descriptors: rows past the end of a
//    sequence read as zero and their output stores are dropped.
#include "gla.h"
#include "gla_device.h"
#include "gla_internal.h"

#include <type_traits>

namespace gla {
namespace {

using namespace dev;


// Workgroup barrier that is also a hard scheduling boundary: the compiler may
// otherwise move pure vector arithmetic (and lane shuffles) across s_barrier,
// which shifts work from one pipeline phase into another.
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  __builtin_amdgcn_sched_barrier(0);
}

template <int KD, bool OUT, int VW>
struct LdsW {
  // 4 matrix waves and NPW producer waves, two waves per SIMD (eight producers,
  // three waves per SIMD, leave the matrix waves too few registers)
  static constexpr int NPW = 4;
  static constexpr int THREADS = 64 * (4 + NPW);
  static constexpr int NQ = KD / 4;                // producer column quads
  static constexpr int QPW = NQ / NPW;             // column quads per producer wave
  static constexpr int NG = 64 / QPW;              // producer row groups
  static constexpr int QROW = 2 * KD;              // qc / kc rows (bf16, swizzled)
  static constexpr int VROW = 2 * VW;              // v rows (bf16, swizzled)
  static constexpr int AROW = 2 * C;               // score rows (bf16, swizzled)
  static constexpr int QPL = C * QROW;             // one plane of qc or kc
  static constexpr int APL = C * AROW;
  // qc hi, lo: two chunk buffers for 64-column workgroups (the producers write
  // each row of chunk c+1 as soon as it is gated), one for 128 columns (there
  // the second buffer's registers and LDS cost more than the earlier writes save)
  static constexpr int NQB = VW == 64 ? 2 : 1;
  // kc comes first: the producers write it between two barriers, on the path
  // from one chunk to the next, and below 64 KiB its LDS stores take immediate
  // offsets (a store past that needs an address add into a temporary register,
  // and the next store then waits until the previous one has read it)
  static constexpr int oK = 0;                                  // kc hi, lo
  static constexpr int oQ = oK + 2 * QPL;                       // qc hi, lo per buffer (OUT)
  static constexpr int qbuf(int c) { return oQ + (NQB == 2 ? (c & 1) : 0) * 2 * QPL; }
  static constexpr int VPL = C * VROW;
  static constexpr int oV = oQ + (OUT ? 2 * NQB * QPL : 0);  // v [token][n], two chunks
  static constexpr int oA = oV + 2 * VPL;                 // A hi, lo [i][j]        (OUT)
  // 64-column workgroups split the state rows in two key halves whose partial
  // outputs meet in LDS; 128-column workgroups give each wave all K rows.
  static constexpr int KS = VW == 64 ? 2 : 1;
  static constexpr int PBYTES = KS == 2 ? 2 * 4 * 2 * 1024 : 0;  // o^T partial tiles [cw][it][nt], 16 B per lane
  static constexpr int oP = oA + (OUT ? 2 * APL : 0);      // partial o^T exchanged between key halves (OUT)
  static constexpr int oS = oP + (OUT ? PBYTES : 0);       // bf16 output tile [token][n], staged for row stores (OUT)
  static constexpr int oDec = oS + (OUT ? VPL : 0);        // a [K]
  static constexpr int oF = oDec + 4 * KD;                 // score-ready chunk index per matrix wave (OUT)
  static constexpr int oBad = oF + 16;                     // a chunk of the segment needs the exact path (OUT)
  static constexpr int BYTES = oBad + 16;

  // Swizzled byte offsets.  On gfx950 an LDS access is served 32 lanes at a
  // time (16 for writes) without bank conflicts when the lanes' addresses,
  // counted in units of the access width, are distinct modulo 32 (16 for
  // writes).  Rows are unpadded; a unit index inside the row is XORed with row
  // bits so that every access pattern of the walker meets that rule, except
  // the kc^T transpose reads and the score writes, which stay at the minimum of
  // two passes their shapes allow:
  //   qc / kc: 16 B chunk ^ sqk(row) -- row fragments (16 rows x 2 chunks),
  //            transpose reads (8 rows x 4 pieces), producer writes (2 rows x 64 B)
  //   v:       32 B pair ^ (b1 | b3 << 1), 64 columns; ^ (b0 | b1 << 1 | b3 << 2),
  //            128 columns -- transpose reads, whole-row writes
  //   A:       16 B chunk ^ (b0 | b2 << 1 | b3 << 2) -- row fragments, 8 B writes
  //   output:  16 B chunk ^ (row & 7) -- whole-row reads; the 8 B tile writes take two passes
  static __device__ __forceinline__ int sqk(int row) {
    const int b1 = (row >> 1) & 1, b2 = (row >> 2) & 1, b3 = (row >> 3) & 1;
    return KD == 128 ? (b2 << 1) | ((b1 ^ b3) << 2) | (b3 << 3) : (b2 << 1) | (b3 << 2);
  }
  static __device__ __forceinline__ int qk(int row, int byte) {
    return row * QROW + (((byte >> 4) ^ sqk(row)) << 4) + (byte & 15);
  }
  static __device__ __forceinline__ int vo(int row, int byte) {
    const int s = VW == 64 ? ((row >> 1) & 1) | (((row >> 3) & 1) << 1)
                           : (row & 1) | (((row >> 1) & 1) << 1) | (((row >> 3) & 1) << 2);
    return row * VROW + (((byte >> 5) ^ s) << 5) + (byte & 31);
  }
  static __device__ __forceinline__ int so(int row, int byte) {  // 16 B chunk ^ (row & 7)
    return row * VROW + (((byte >> 4) ^ (row & 7)) << 4) + (byte & 15);
  }
  static __device__ __forceinline__ int ao(int row, int byte) {
    const int s = (row & 1) | (((row >> 2) & 1) << 1) | (((row >> 3) & 1) << 2);
    return row * AROW + (((byte >> 4) ^ s) << 4) + (byte & 15);
  }
};

// The matrix waves share their score tiles among themselves only, so they meet
// through per-wave chunk counters in LDS instead of a workgroup barrier (which
// would also hold the producer waves): each wave publishes chunk c once its
// tiles are written, does the work that needs no other wave's tiles, then waits
// until all four have published.  The wait is bounded so that a wave always
// leaves it, and sleeps between polls so that it takes no issue slots or LDS
// cycles from the producer wave on its SIMD.
__device__ __forceinline__ void scores_publish(char *flags, int mw, int c) {
  int *f = reinterpret_cast<int *>(flags);
  // release for LDS only: the wave's outstanding global loads and stores are not
  // waited for
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __hip_atomic_store(f + mw, c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// Returns false when the bound ran out before every wave had published chunk c
// (the wave then goes on with whatever the score tiles hold; the caller reports it).
__device__ __forceinline__ bool scores_wait(char *flags, int c, int polls) {
  int *f = reinterpret_cast<int *>(flags);
  bool ready = false;
  for (int spin = 0; spin < polls; ++spin) {
    const int m = min(min(__hip_atomic_load(f + 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP),
                          __hip_atomic_load(f + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)),
                      min(__hip_atomic_load(f + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP),
                          __hip_atomic_load(f + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)));
    if (__builtin_amdgcn_readfirstlane(m) >= c) {
      ready = true;
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  return ready;
}

// Split of values that are not used after it (gated q and k rows, score
// tiles).  With 64 columns the producer waves set the pace and the form with
// one dot instruction per remainder saves them VALU instructions; with 128
// columns that form measured slower and the subtraction forms are kept there
// (split4_valu for VALU products, split4_sub for MFMA results).
template <int VW, bool VALU_FED>
__device__ __forceinline__ void split4_dead(const float x[4], u32x2_t &hi, u32x2_t &lo) {
  if constexpr (VW == 64) {
    split4(x, hi, lo);
  } else if constexpr (VALU_FED) {
    split4_valu(x, hi, lo);
  } else {
    split4_sub(x, hi, lo);
  }
}

// Score tiles (i-tile, j-tile) of the 64 x 64 lower triangle per matrix wave.
template <int W> struct Tiles;
template <> struct Tiles<0> { static constexpr int n = 3; static constexpr int it[3] = {0, 1, 1}, jt[3] = {0, 0, 1}; };
template <> struct Tiles<1> { static constexpr int n = 3; static constexpr int it[3] = {2, 2, 2}, jt[3] = {0, 1, 2}; };
template <> struct Tiles<2> { static constexpr int n = 2; static constexpr int it[2] = {3, 3}, jt[2] = {0, 1}; };
template <> struct Tiles<3> { static constexpr int n = 2; static constexpr int it[2] = {3, 3}, jt[2] = {2, 3}; };

// A^T tiles = kc qc^T for wave W's tiles, causal mask, split -> LDS A[i][j].
// rf[kb]: this lane's offset of row l16, k columns 32 kb + 8 lg .. + 7, in a
// qc / kc plane (the swizzle depends on the row within a 16-row tile only);
// sq: the qc buffer of the chunk.
template <int KD, int VW, int W>
__device__ __forceinline__ void scores(char *smem, const char *sq, const int (&rf)[KD / 32], int l16, int lg) {
  using L = LdsW<KD, true, VW>;
  using T = Tiles<W>;
  f32x4_t acc[T::n];
#pragma unroll
  for (int t = 0; t < T::n; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < KD / 32; ++kb) {
#pragma unroll
    for (int t = 0; t < T::n; ++t) {
      const int oa = rf[kb] + 16 * T::jt[t] * L::QROW;
      const int ob = rf[kb] + 16 * T::it[t] * L::QROW;
      const u32x4_t ah = lds_ld<u32x4_t>(smem + L::oK, oa);
      const u32x4_t al = lds_ld<u32x4_t>(smem + L::oK + L::QPL, oa);
      const u32x4_t bh = lds_ld<u32x4_t>(sq, ob);
      const u32x4_t bl = lds_ld<u32x4_t>(sq + L::QPL, ob);
      acc[t] = mfma_bf(al, bh, acc[t]);
      acc[t] = mfma_bf(ah, bl, acc[t]);
      acc[t] = mfma_bf(ah, bh, acc[t]);
    }
  }
#pragma unroll
  for (int t = 0; t < T::n; ++t) {
    // lane: i = 16 it + l16, j = 16 jt + 4 lg + r
    const int i = 16 * T::it[t] + l16;
    float av[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) av[r] = (16 * T::jt[t] + 4 * lg + r <= i) ? acc[t][r] : 0.f;
    u32x2_t hi, lo;
    split4_dead<VW, false>(av, hi, lo);
    const int off = L::ao(i, (16 * T::jt[t] + 4 * lg) * 2);
    lds_st<u32x2_t>(smem + L::oA, off, hi);
    lds_st<u32x2_t>(smem + L::oA + L::APL, off, lo);
  }
}

// GH: the gate is one decay per value head and token (g [B,T,HV]) instead of one
// per key; a compile-time choice, so that the per-key walker's code is untouched.
// b: the workgroup's index in the (segment, head, value slice) order.
// FUSED: one of the two walks of the single pass.  Its summary walk keeps the
// summary in LDS as [K][VW] fp32 at offset 0 instead of storing it to
// seg_state, and every value slice writes the segment's decay product (the
// same values).
template <bool OUT, int KD, int VW, bool GH, bool FUSED = false>
__device__ __forceinline__ void walk_bf16(const WalkParams &p, char *smem, int b) {
  constexpr bool KEEP = FUSED && !OUT;
  using L = LdsW<KD, OUT, VW>;
  constexpr int KS = L::KS;         // key splits of the state over the 4 matrix waves
  constexpr int CS = 4 / KS;        // column splits
  constexpr int VQ = VW / CS;       // value columns per matrix wave (32)
  constexpr int NT = VQ / 16;       // 16-column tiles per matrix wave
  constexpr int QPW = L::QPW, NG = L::NG, RPG = C / NG;
  constexpr int KH = KD / KS;       // state rows per matrix wave
  constexpr int NKT = KH / 16;      // 16-row k tiles per matrix wave
  constexpr int NKB = KH / 32;      // 32-wide k blocks per matrix wave
  // 64-column output workgroups share score tiles through LDS counters (the
  // producers skip that meeting); 128-column ones use a workgroup barrier
  constexpr bool HANDOFF = OUT && VW == 64;
  static_assert(KD == 64 || KD == 128, "bf16 walker covers key widths 64, 128");
  static_assert(NG * QPW == 64 && RPG * NG == C, "producer mapping");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool producer = wave >= 4;
  const int l16 = lane & 15, lg = lane >> 4;

  // ---- (segment, head, value slice) of this workgroup; value slices of one
  // unit are 8 workgroup ids apart so they run on the same XCD and share L2.
  const int NV = (p.V + VW - 1) / VW;
  const int grp = b / (8 * NV), rem = b - grp * (8 * NV);
  const int vt = rem >> 3;
  const int unit = grp * 8 + (rem & 7);
  if (unit >= p.units) return;
  const int seg = unit / p.HV, h = unit - seg * p.HV;  // h: value head
  SegInfo si;
  if (!locate(p, seg, si)) return;
  if (!OUT && si.s >= si.nseg - 1) return;
  const int nchunks = (si.len + C - 1) / C;
  // the sequence's nseg = max(1, ceil(nchunks / R)) segments share its chunks
  // evenly: ceil(nchunks / nseg) <= R each, none empty
  const int seg_len = (nchunks + si.nseg - 1) / si.nseg;
  const int c_begin = si.s * seg_len;
  const int c_end = min(c_begin + seg_len, nchunks);
  const int H = p.HV, V = p.V;  // value heads: v, o, g, states
  const int v0 = vt * VW;
  const int nkeys = p.K;  // real keys (<= KD); keys nkeys..KD-1 are zero padding
  // q, k come from key head h / G (rows of H key heads); g has a decay per key
  // (rows of HV x Kmem) or one per value head (rows of HV)
  const int64_t rowK = (int64_t)p.H * p.Kmem, rowV = (int64_t)H * V;
  const int64_t rowG = GH ? (int64_t)H : (int64_t)H * p.Kmem;
  const int64_t seq_bos = si.bos;
  const int seq_len = si.len;
  // Lanes whose key quad or value chunk lies past the real keys / columns use
  // this offset: past every buffer range (the host keeps a chunk's range below
  // 2^30 bytes), so their loads read zero and their stores are dropped.
  constexpr int kOff = 1 << 30;

  // ======================= matrix waves: state and lane bases
  // matrix wave mw = CS kh + cw holds state rows KH kh .. + KH - 1, columns
  // v0 + VQ cw .. + VQ - 1: S[kt][nt] lane rows KH kh + 16 kt + 4 lg + r,
  // column VQ cw + 16 nt + l16
  const int mw = wave & 3, kh = mw / CS, cw = mw % CS;
  f32x4_t S[NKT][NT];
  if (!producer) {
    // h0 rows are [Kmem] wide (this block's rows start at koff), start states [nkeys]
    const float *src = nullptr;
    if (OUT) {
      if (si.s == 0) {
        if (p.h0) src = p.h0 + (((int64_t)si.n * H + h) * p.Kmem + p.koff) * V;
      } else {
        src = p.seg_state + ((int64_t)(si.first + si.s - 1) * H + h) * nkeys * V;
      }
    }
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = KH * kh + 16 * kt + 4 * lg + r, col = v0 + VQ * cw + 16 * nt + l16;
          const bool in = src && row < nkeys && col < V;
          // a start state published by another workgroup of the same launch
          // (the single pass) is read device-coherently
          if (FUSED && si.s > 0) S[kt][nt][r] = in ? ld_agent(src + (int64_t)row * V + col) : 0.f;
          else S[kt][nt][r] = in ? src[(int64_t)row * V + col] : 0.f;
        }
  }
  if (tid == 0) lds_st<int>(smem + L::oBad, 0, 0);
  if (OUT) {  // score tiles above the diagonal are read as zeros and never written
    for (int i = tid; i < 2 * L::APL / 16; i += L::THREADS)
      lds_st<u32x4_t>(smem + L::oA, 16 * i, u32x4_t{0, 0, 0, 0});
    if (tid < 4) lds_st<int>(smem + L::oF, 4 * tid, c_begin - 1);
  }
  // Per-lane LDS offsets; the compile-time parts (row tiles, token blocks, the
  // 8 B half of a chunk) are added at the access and do not change the swizzle.
  int rf[KD / 32], rq[NKB];  // row fragments: row l16, k columns 32 kb + 8 lg .. (all; this wave's keys)
#pragma unroll
  for (int kb = 0; kb < KD / 32; ++kb) rf[kb] = L::qk(l16, 16 * (4 * kb + lg));
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) rq[kb] = L::qk(l16, 16 * (4 * (NKB * kh + kb) + lg));
  int aoff[2];  // A row fragments: row l16, tokens 32 jb + 8 lg ..
#pragma unroll
  for (int jb = 0; jb < 2; ++jb) aoff[jb] = opaque_int(L::oA + L::ao(l16, 16 * (4 * jb + lg)));
  const int trow = 8 * lg + (l16 >> 2);  // token row of the transpose reads
  int voff[NT];                          // v, transposed: columns VQ cw + 16 nt + 4 (l16 & 3)
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) voff[nt] = L::vo(trow, 2 * (VQ * cw + 16 * nt) + 8 * (l16 & 3));
  int koff[NKB][2];  // kc, transposed: key columns KH kh + 32 m + 8 (l16 & 3), token rows + 4 e
#pragma unroll
  for (int m = 0; m < NKB; ++m)
#pragma unroll
    for (int e = 0; e < 2; ++e) koff[m][e] = L::qk(trow + 4 * e, 2 * (KH * kh + 8 * (l16 & 3)) + 64 * m);
  // LDS regions past 64 KiB are addressed from per-lane base registers so that
  // the remaining offsets fit the 16-bit immediate of the LDS instructions
  // (folded into one constant, every access would need an address add)
  const int base_d = opaque_int(L::oDec + 4 * (KH * kh + 4 * lg));  // decay a of key rows KH kh + 16 kt + 4 lg ..

  // ======================= producer waves: raw and gated registers
  // producer thread pt: key columns 4cq..4cq+3 of rows rg*RPG..+RPG-1
  const int pt = tid - 4 * 64;
  const int cq = (wave - 4) * QPW + lane % QPW, rg = lane / QPW;
  const bool key_ok = 4 * cq < nkeys;
  // a per-head gate is read once per row and used for every key
  const int voff_g = GH ? (int)(rg * RPG * rowG * 4) : key_ok ? (int)((rg * RPG * rowG + 4 * cq) * 4) : kOff;
  const int voff_k = key_ok ? (int)((rg * RPG * rowK + 4 * cq) * 2) : kOff;
  // v: 16 B chunk vch of token rows vrow + VRS j (VW / 8 lanes per row)
  constexpr int VCH = VW / 8, VRS = 64 * L::NPW / VCH, NVL = C / VRS;
  const int vrow = pt / VCH, vch = pt % VCH;
  const int voff_v = v0 + 8 * vch < V ? (int)((vrow * rowV + 8 * vch) * 2) : kOff;
  const int vstep = (int)(VRS * rowV * 2);
  const int step_g = (int)(rowG * 4), step_k = (int)(rowK * 2);
  const int colq = kperm_bf(4 * cq) * 2;
  u32x4_t rgG[RPG];
  u32x2_t rgQ[RPG], rgK[RPG];
  u32x4_t rgV[NVL];
  u32x2_t gQh[RPG], gQl[RPG], gKh[RPG], gKl[RPG];
  f32x4_t gDec = {1.f, 1.f, 1.f, 1.f};
  float gPl[RPG][4], gRl[RPG][4], gSuf[4], gFq[4];
  float tQ[RPG][4], tK[RPG][4];  // q P, k R of a row (factors inside the row group)
  float incl[4], shf[4];         // running products across row groups, shuffled values
  float seg_decay[4] = {1.f, 1.f, 1.f, 1.f};
  bool seg_bad = false;          // some key of a chunk decayed by more than kMinChunkDecay
  const float scale = p.scale;

  // Raw loads of chunk c (rows past the sequence end, and chunks past the
  // segment, read as zero).
  struct Rsrc { __amdgpu_buffer_rsrc_t g, q, k, v; };
  auto rsrc = [&](int c) {
    const int64_t t0 = (int64_t)seq_bos + (int64_t)c * C;
    const int64_t valid = c < c_end ? min(C, seq_len - c * C) : 0;
    const int64_t headK = (int64_t)(h / p.G) * p.Kmem + p.koff, headV = (int64_t)h * V + v0;
    const int64_t headG = GH ? (int64_t)h : (int64_t)h * p.Kmem + p.koff;
    Rsrc r;
    r.g = make_rsrc(p.g + t0 * rowG + headG, (valid * rowG - headG) * 4);
    r.q = make_rsrc((const uint16_t *)p.q + t0 * rowK + headK, OUT ? (valid * rowK - headK) * 2 : 0);
    r.k = make_rsrc((const uint16_t *)p.k + t0 * rowK + headK, (valid * rowK - headK) * 2);
    r.v = make_rsrc((const uint16_t *)p.v + t0 * rowV + headV, (valid * rowV - headV) * 2);
    return r;
  };
  auto load_g = [&](const Rsrc &r) {
    if constexpr (GH) {
#pragma unroll
      for (int i = 0; i < RPG; ++i) {
        const uint32_t x = __builtin_amdgcn_raw_buffer_load_b32(r.g, voff_g + i * step_g, 0, 0);
        rgG[i] = u32x4_t{x, x, x, x};
      }
    } else {
#pragma unroll
      for (int i = 0; i < RPG; ++i) rgG[i] = buf_ld128(r.g, voff_g + i * step_g);
    }
  };
  auto load_v = [&](const Rsrc &r) {
#pragma unroll
    for (int j = 0; j < NVL; ++j) rgV[j] = buf_ld128(r.v, voff_v + j * vstep);
  };
  auto load_qk_row = [&](const Rsrc &r, int i) {
    rgK[i] = buf_ld64(r.k, voff_k + i * step_k);
    if (OUT) rgQ[i] = buf_ld64(r.q, voff_k + i * step_k);
  };
  // gate, stage 1a: exp(g) and the running products inside the row group; the
  // raw g registers are free afterwards
  auto gate_local = [&]() {
    float E[RPG][4];
#pragma unroll
    for (int r = 0; r < RPG; ++r)
#pragma unroll
      for (int j = 0; j < 4; ++j) E[r][j] = __expf(__uint_as_float(rgG[r][j]));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      gPl[0][j] = E[0][j];
#pragma unroll
      for (int r = 1; r < RPG; ++r) gPl[r][j] = gPl[r - 1][j] * E[r][j];
      gRl[RPG - 1][j] = 1.f;
#pragma unroll
      for (int r = RPG - 2; r >= 0; --r) gRl[r][j] = gRl[r + 1][j] * E[r + 1][j];
      incl[j] = gPl[RPG - 1][j];
    }
  };
  // gate, stage 1b: running products across row groups, an inclusive scan over
  // the NG row groups with lane shuffles inside the wave (log2 NG rounds; each
  // round's shuffles are issued, independent work runs, then they are used)
  auto scan_issue = [&](int d) {
    const int src = (lane - d * QPW) < 0 ? lane : lane - d * QPW;
#pragma unroll
    for (int j = 0; j < 4; ++j) shf[j] = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * src, __float_as_int(incl[j])));
  };
  auto scan_use = [&](int d) {
#pragma unroll
    for (int j = 0; j < 4; ++j) incl[j] *= (rg >= d) ? shf[j] : 1.f;
  };
  // gate, stage 1c: chunk decay and the q / k factors from the scan.  A chunk in
  // which some key decays by more than kMinChunkDecay makes these factors
  // overflow (and the quotient tot / incl can be 0 / 0); write_k flags it and the
  // whole segment is then evaluated again token by token.
  auto gate_decays = [&]() {
    const int src_pre = rg > 0 ? lane - QPW : lane;
    const int src_tot = (NG - 1) * QPW + lane % QPW;
    // all eight shuffles in flight at once, the reciprocals that need none of
    // them computed meanwhile (one LDS round trip instead of one per key)
    float y[4], tot[4], rin[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      y[j] = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * src_pre, __float_as_int(incl[j])));
      tot[j] = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * src_tot, __float_as_int(incl[j])));
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 4; ++j) rin[j] = __builtin_amdgcn_rcpf(incl[j]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float pre = rg > 0 ? y[j] : 1.f;
      gSuf[j] = tot[j] * rin[j];   // product over the later row groups
      gFq[j] = OUT ? scale * pre * __builtin_amdgcn_rcpf(tot[j]) : 0.f;
      gDec[j] = tot[j];
    }
    if (!OUT && rg == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) seg_decay[j] *= gDec[j];
    }
  };
  // gate, stage 2a: q, k of row r times their factors inside the row group (needs
  // no scan); the raw registers of the row are then free for the next load
  auto gate_part = [&](int r) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      tK[r][j] = ((j & 1) ? bf_hi(rgK[r][j >> 1]) : bf_lo(rgK[r][j >> 1])) * gRl[r][j];
      if (OUT) tQ[r][j] = ((j & 1) ? bf_hi(rgQ[r][j >> 1]) : bf_lo(rgQ[r][j >> 1])) * gPl[r][j];
    }
    // The products must exist before the row's next raw load is issued: if the
    // compiler defers them, the raw registers stay live, the next load goes to
    // other registers, and the copy back at the end of the chunk loop waits for
    // that load to arrive (a full memory latency on the path to the next chunk).
    if constexpr (OUT) {
      asm volatile("" ::"v"(tK[r][0]), "v"(tK[r][1]), "v"(tK[r][2]), "v"(tK[r][3]), "v"(tQ[r][0]), "v"(tQ[r][1]),
                   "v"(tQ[r][2]), "v"(tQ[r][3]) : "memory");
    } else {
      asm volatile("" ::"v"(tK[r][0]), "v"(tK[r][1]), "v"(tK[r][2]), "v"(tK[r][3]) : "memory");
    }
  };
  // gate, stage 2b: gated and split q, k of row r
  auto gate_row = [&](int r) {
    float kc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) kc[j] = tK[r][j] * gSuf[j];
    split4_dead<VW, true>(kc, gKh[r], gKl[r]);  // kc, qc: products of VALU multiplies
    if (OUT) {
      float qc[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) qc[j] = tQ[r][j] * gFq[j];
      split4_dead<VW, true>(qc, gQh[r], gQl[r]);
    }
  };
  // v goes to LDS straight from the load registers (two chunk buffers)
  auto write_v = [&](int c) {
    char *sv = smem + L::oV + (c & 1) * L::VPL;
#pragma unroll
    for (int j = 0; j < NVL; ++j) lds_st<u32x4_t>(sv, L::vo(vrow + VRS * j, 16 * vch), rgV[j]);
  };
  auto write_k = [&]() {  // kc and the chunk decay
#pragma unroll
    for (int r = 0; r < RPG; ++r) {
      const int off = L::qk(rg * RPG + r, colq);
      lds_st<u32x2_t>(smem + L::oK, off, gKh[r]);
      lds_st<u32x2_t>(smem + L::oK + L::QPL, off, gKl[r]);
    }
    if (rg == 0) lds_st<f32x4_t>(smem + L::oDec, 16 * cq, gDec);
    // the flag of the segment (wave-uniform, a scalar register)
    const bool low = gDec[0] < kMinChunkDecay || gDec[1] < kMinChunkDecay || gDec[2] < kMinChunkDecay ||
                     gDec[3] < kMinChunkDecay;
    if (__ballot(low) != 0ull) seg_bad = true;
  };
  auto write_q_row = [&](int c, int r) {
    char *sq = smem + L::qbuf(c);
    const int off = L::qk(rg * RPG + r, colq);
    lds_st<u32x2_t>(sq, off, gQh[r]);
    lds_st<u32x2_t>(sq + L::QPL, off, gQl[r]);
  };

  // Output of a chunk: the o^T tiles (lane = token 16 it + l16, columns VQ cw +
  // 16 nt + 4 lg .. + 3) are rounded to bf16 and staged in LDS; after the next
  // barrier each matrix wave stores 16 whole rows of the tile (VW / 8 lanes of
  // 16 B per row), so every store fills complete cache lines.
  auto o_rsrc = [&](int c) {
    const int64_t t0 = (int64_t)seq_bos + (int64_t)c * C;
    const int64_t valid = min(C, seq_len - c * C);
    const int64_t headV = (int64_t)h * V + v0;
    return make_rsrc((uint16_t *)p.o + t0 * rowV + headV, (valid * rowV - headV) * 2);
  };
  auto stage_tile = [&](int it, int nt, const f32x4_t &x) {
    const int col = VQ * cw + 16 * nt + 4 * lg;
    const u32x2_t w = {pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3])};
    lds_st<u32x2_t>(smem + L::oS, L::so(16 * it + l16, 2 * col), w);
  };
  auto store_staged = [&](int cs) {
    constexpr int LPR = VW / 8, RPI = 64 / LPR;  // lanes per row, rows per store
    const __amdgpu_buffer_rsrc_t rO = o_rsrc(cs);
#pragma unroll
    for (int i = 0; i < 16 / RPI; ++i) {
      const int row = 16 * mw + RPI * i + lane / LPR, ch = lane % LPR;
      const int off = v0 + 8 * ch < V ? (int)((row * rowV + 8 * ch) * 2) : kOff;
      buf_st128_nt(rO, off, lds_ld<u32x4_t>(smem + L::oS, L::so(row, 16 * ch)));
    }
  };

  // Producer and matrix waves run separate loops (different register sets);
  // both meet the same barriers per chunk: operands written | scores written
  // (128-column output workgroups only) | chunk done.  64-column workgroups hand
  // the score tiles between matrix waves through LDS counters instead, so the
  // producers run on.
  if (producer) {
    if (c_begin < c_end) {  // pipeline fill: chunk c_begin gated, chunk c_begin+1 loading
      const Rsrc r0 = rsrc(c_begin);
      load_g(r0);
      load_v(r0);
#pragma unroll
      for (int i = 0; i < RPG; ++i) load_qk_row(r0, i);
      gate_local();
#pragma unroll
      for (int d = 1; d < NG; d *= 2) {
        scan_issue(d);
        scan_use(d);
      }
      gate_decays();
      write_v(c_begin);
      const Rsrc r1 = rsrc(c_begin + 1);
      load_g(r1);
      load_v(r1);
#pragma unroll
      for (int i = 0; i < RPG; ++i) {
        gate_part(i);
        gate_row(i);
        if constexpr (OUT && L::NQB == 2) write_q_row(c_begin, i);
        load_qk_row(r1, i);
      }
    }
    for (int c = c_begin; c < c_end; ++c) {
      write_k();        // chunk c
      if constexpr (OUT && L::NQB == 1) {
#pragma unroll
        for (int i = 0; i < RPG; ++i) write_q_row(c, i);
      }
      phase_barrier();  // operands of chunk c visible
      const Rsrc r2 = rsrc(c + 2);
      gate_local();     // chunk c+1
      load_g(r2);
      if constexpr (OUT && !HANDOFF) {
        // 128-column workgroups: the scan as one step, then the rows (the
        // interleaved form below needs more registers than they have left)
#pragma unroll
        for (int d = 1; d < NG; d *= 2) {
          scan_issue(d);
          scan_use(d);
        }
        gate_decays();
        phase_barrier();  // scores visible
        write_v(c + 1);
        load_v(r2);
#pragma unroll
        for (int i = 0; i < RPG; ++i) {
          gate_part(i);
          gate_row(i);    // chunk c+1
          load_qk_row(r2, i);
        }
        phase_barrier();  // chunk c done
        continue;
      }
      // the scan rounds wait on lane shuffles; the row products of the group,
      // the next raw loads and the v copy fill those waits
      constexpr int LOGNG = NG == 8 ? 3 : NG == 16 ? 4 : NG == 4 ? 2 : 5;
      static_assert((1 << LOGNG) == NG, "row groups");
#pragma unroll
      for (int ri = 0; ri < LOGNG; ++ri) {
        scan_issue(1 << ri);
        __builtin_amdgcn_sched_barrier(0);
        if (ri == 0 || ri == 1) {
#pragma unroll
          for (int i = ri * RPG / 2; i < (ri + 1) * RPG / 2; ++i) {
            gate_part(i);
            load_qk_row(r2, i);
          }
        }
        if (ri == 2) {
          write_v(c + 1);
          load_v(r2);
        }
        __builtin_amdgcn_sched_barrier(0);
        scan_use(1 << ri);
      }
      if constexpr (LOGNG < 3) {
        write_v(c + 1);
        load_v(r2);
      }
      gate_decays();
#pragma unroll
      for (int i = 0; i < RPG; ++i) {
        gate_row(i);    // chunk c+1
        if constexpr (OUT && L::NQB == 2) write_q_row(c + 1, i);
      }
      phase_barrier();  // chunk c done
    }
  } else {
    for (int c = c_begin; c < c_end; ++c) {
      const char *sq = smem + L::qbuf(c);  // qc of chunk c
      phase_barrier();  // operands of chunk c visible
      if constexpr (OUT) {
        if (KS == 2 && c > c_begin) store_staged(c - 1);
        switch (mw) {
          case 0: scores<KD, VW, 0>(smem, sq, rf, l16, lg); break;
          case 1: scores<KD, VW, 1>(smem, sq, rf, l16, lg); break;
          case 2: scores<KD, VW, 2>(smem, sq, rf, l16, lg); break;
          default: scores<KD, VW, 3>(smem, sq, rf, l16, lg); break;
        }
        if constexpr (HANDOFF) scores_publish(smem + L::oF, mw, c);
        else phase_barrier();  // scores visible
      }
      const char *sv = smem + L::oV + (c & 1) * L::VPL;  // v of chunk c
      // ---- S' = diag(a) S
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
        const f32x4_t a4 = lds_ld<f32x4_t>(smem, base_d + 64 * kt);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int r = 0; r < 4; ++r) S[kt][nt][r] *= a4[r];
      }
      // ---- v fragments: v[32 jb + 8 lg + e][VQ mw + 16 nt + l16]
      u32x4_t vf[NT][2];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
          const int off = voff[nt] + 32 * jb * L::VROW;
          const u32x2_t x0 = lds_tr16(sv + off);
          const u32x2_t x1 = lds_tr16(sv + off + 4 * L::VROW);
          vf[nt][jb] = u32x4_t{x0[0], x0[1], x1[0], x1[1]};
        }
      f32x4_t keep[4];
      if constexpr (OUT) {
        f32x4_t o[4][NT];  // o^T tiles: lane = token 16 it + l16, rows = columns 16 nt + 4 lg + r
#pragma unroll
        for (int it = 0; it < 4; ++it)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) o[it][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        // ---- o^T += S'^T qc^T (S' from the accumulators, split hi + lo)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          u32x4_t sh[NT], sl[NT];
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const float s8[8] = {S[2 * kb][nt][0], S[2 * kb][nt][1], S[2 * kb][nt][2], S[2 * kb][nt][3],
                                 S[2 * kb + 1][nt][0], S[2 * kb + 1][nt][1], S[2 * kb + 1][nt][2], S[2 * kb + 1][nt][3]};
            u32x2_t h0, l0, h1, l1;
            split4_valu(s8, h0, l0);  // S' = a S: products of VALU multiplies; S stays live
            split4_valu(s8 + 4, h1, l1);
            sh[nt] = u32x4_t{h0[0], h0[1], h1[0], h1[1]};
            sl[nt] = u32x4_t{l0[0], l0[1], l1[0], l1[1]};
          }
#pragma unroll
          for (int it = 0; it < 4; ++it) {
            const int off = rq[kb] + 16 * it * L::QROW;
            const u32x4_t qh = lds_ld<u32x4_t>(sq, off);
            const u32x4_t ql = lds_ld<u32x4_t>(sq + L::QPL, off);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
              o[it][nt] = mfma_bf(sh[nt], ql, o[it][nt]);
              o[it][nt] = mfma_bf(sl[nt], qh, o[it][nt]);
              o[it][nt] = mfma_bf(sh[nt], qh, o[it][nt]);
            }
          }
        }
        // ---- o^T += v^T A^T over the 32-token blocks on or below the diagonal
        // (with two key halves, half kh takes token block kh; kh is uniform)
        auto av = [&](auto jbc) {
          constexpr int jb = decltype(jbc)::value;
#pragma unroll
          for (int it = 2 * jb; it < 4; ++it) {
            const int off = aoff[jb] + 16 * it * L::AROW;
            const u32x4_t ah = lds_ld<u32x4_t>(smem, off);
            const u32x4_t al = lds_ld<u32x4_t>(smem + L::APL, off);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
              o[it][nt] = mfma_bf(vf[nt][jb], al, o[it][nt]);
              o[it][nt] = mfma_bf(vf[nt][jb], ah, o[it][nt]);
            }
          }
        };
        // the other waves' score tiles are needed from here on
        if constexpr (HANDOFF) {
          if (!scores_wait(smem + L::oF, c, p.wait_polls)) report_status(p.status, GLA_STATUS_WAIT_EXHAUSTED, lane);
        }
        if (KS == 1 || kh == 0) av(std::integral_constant<int, 0>{});
        if (KS == 1 || kh == 1) av(std::integral_constant<int, 1>{});
        if constexpr (KS == 1) {
          // the previous tile was stored right after the last chunk-done
          // barrier; the operands and scores barriers lie between those reads
          // and these writes
#pragma unroll
          for (int it = 0; it < 4; ++it)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) stage_tile(it, nt, o[it][nt]);
        } else {
          // keep tile nt = kh, send tile 1 - kh to the partner key half
#pragma unroll
          for (int it = 0; it < 4; ++it) {
            keep[it] = kh ? o[it][1] : o[it][0];
            const f32x4_t send = kh ? o[it][0] : o[it][1];
            lds_st<f32x4_t>(smem + L::oP, ((cw * 4 + it) * 2 + (1 - kh)) * 1024 + 16 * lane, send);
          }
        }
      }
      // ---- S = S' + kc^T v   (kc^T rows via transpose reads of the token-major kc)
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
          const int off0 = koff[kt >> 1][0] + 32 * jb * L::QROW + 8 * (kt & 1);
          const int off1 = koff[kt >> 1][1] + 32 * jb * L::QROW + 8 * (kt & 1);
          const u32x2_t h0 = lds_tr16(smem + L::oK + off0);
          const u32x2_t h1 = lds_tr16(smem + L::oK + off1);
          const u32x2_t g0 = lds_tr16(smem + L::oK + L::QPL + off0);
          const u32x2_t g1 = lds_tr16(smem + L::oK + L::QPL + off1);
          const u32x4_t ah = {h0[0], h0[1], h1[0], h1[1]};
          const u32x4_t al = {g0[0], g0[1], g1[0], g1[1]};
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            S[kt][nt] = mfma_bf(al, vf[nt][jb], S[kt][nt]);
            S[kt][nt] = mfma_bf(ah, vf[nt][jb], S[kt][nt]);
          }
        }
      }
      phase_barrier();  // chunk c's operands are no longer read; partial outputs visible
      // 128-column workgroups staged this chunk's tile before the barrier: store
      // it now, while the producers write the next chunk's operands
      if constexpr (OUT && KS == 1) store_staged(c);
      if constexpr (OUT && KS == 2) {
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const f32x4_t part = lds_ld<f32x4_t>(smem + L::oP, ((cw * 4 + it) * 2 + kh) * 1024 + 16 * lane);
          stage_tile(it, kh, f32x4_t{keep[it][0] + part[0], keep[it][1] + part[1], keep[it][2] + part[2],
                                     keep[it][3] + part[3]});
        }
      }
    }
  }

  // ================= results of the segment
  // The final state (ht, or the segment summary) leaves through LDS as whole
  // rows: after the last chunk nothing reads the operand area at offset 0, so
  // the matrix waves write S there as [K][VW] fp32 (16 consecutive columns per
  // 16 lanes: conflict-free), and after a barrier every wave stores rows of
  // VW / 4 lanes x 16 B.
  float *dst = nullptr;
  if (OUT) {
    if (p.ht != nullptr && si.s == si.nseg - 1) dst = p.ht + (((int64_t)si.n * H + h) * p.Kmem + p.koff) * V;
  } else {
    dst = p.seg_state + ((int64_t)(si.first + si.s) * H + h) * nkeys * V;
  }
  static_assert(KD * VW * 4 <= (OUT ? L::oS : L::oDec), "state staging must not overlap the output staging");
  if (dst != nullptr && !producer) {
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          lds_st<float>(smem, 4 * ((KH * kh + 16 * kt + 4 * lg + r) * VW + VQ * cw + 16 * nt + l16), S[kt][nt][r]);
  }
  if (producer && seg_bad && lane == 0) lds_st<int>(smem + L::oBad, 0, 1);
  if (OUT || dst != nullptr) phase_barrier();  // staged output tile and state visible
  const bool exact = __builtin_amdgcn_readfirstlane(lds_ld<int>(smem + L::oBad, 0)) != 0;
  if constexpr (OUT && KS == 2) {  // the last staged output tile
    if (!producer && c_begin < c_end) store_staged(c_end - 1);
  }
  if (exact) {
    // the chunk form's products overflowed in some chunk of this segment (its
    // outputs, state and summary may hold inf or NaN): every result of the
    // segment is formed again from the token recurrence, after every store of
    // the chunk loop; its final state replaces S in the staging area
    __syncthreads();
    exact_segment<KD, true, OUT>(p, si, h, v0, VW, c_begin, c_end, wave, KEEP ? 0 : vt,
                                 reinterpret_cast<float *>(smem));
    __syncthreads();
  }
  if (dst != nullptr && !KEEP) {
    constexpr int LPR = VW / 4, RPI = 64 / LPR;  // lanes per state row, rows per store
    const int rr = lane / LPR, ch = lane % LPR;
#pragma unroll
    for (int i = wave; i < KD / RPI; i += L::THREADS / 64) {
      const int row = RPI * i + rr;
      if (row < nkeys && v0 + 4 * ch < V)  // padded key rows and columns past V are not stored
        *reinterpret_cast<f32x4_t *>(dst + (int64_t)row * V + v0 + 4 * ch) = lds_ld<f32x4_t>(smem, 16 * (row * LPR + ch));
    }
  }
  if (producer && !OUT && !exact && (KEEP || vt == 0) && rg == 0 && key_ok) {
    const int slot = si.first + si.s;
    *reinterpret_cast<f32x4_t *>(p.seg_decay + ((int64_t)slot * H + h) * nkeys + 4 * cq) =
        f32x4_t{seg_decay[0], seg_decay[1], seg_decay[2], seg_decay[3]};
  }
}

template <int KD, int VW, bool GH>
__global__ __launch_bounds__((LdsW<KD, true, VW>::THREADS), 1) void gla_chunk_output_bf16(WalkParams p) {
  __shared__ __attribute__((aligned(16))) char smem[LdsW<KD, true, VW>::BYTES];
  walk_bf16<true, KD, VW, GH>(p, smem, blockIdx.x);
}

template <int KD, int VW, bool GH>
__global__ __launch_bounds__((LdsW<KD, false, VW>::THREADS), 1) void gla_chunk_local_bf16(WalkParams p) {
  __shared__ __attribute__((aligned(16))) char smem[LdsW<KD, false, VW>::BYTES];
  walk_bf16<false, KD, VW, GH>(p, smem, blockIdx.x);
}

// ---------------------------------------------------------------- single pass
// Summary, scan and outputs in one launch.  Segment s of a sequence publishes
// its end state P_s = diag(a_s) P_{s-1} + Sigma_s (P_{-1} = h0 or 0; a_s and
// Sigma_s: the decay product and the summary of its own chunks) in seg_state
// slot s, and then walks its chunks from P_{s-1} (page "fla/ops/gla/
// fused_chunk.py", fused_chunk_gla_fwd_kernel, carries the same state through
// one serial loop; here the loop is cut into segments joined by that
// recurrence, in the order a decoupled look-back scan uses).
//
// Workgroups take (segment, head, value slice) items from a counter in the
// order of the segment numbering, in which segment s - 1 of a sequence comes
// before segment s.  A workgroup therefore only ever waits for an item that a
// running workgroup has already taken, so the chain always moves.  All waves
// store their rows of P_s with device-coherent (agent-scope atomic) stores;
// once every store has completed, one wave releases at agent scope and sets
// the item's flag.  In the successor one wave polls the flag and acquires
// while a barrier holds the others, and P_{s-1} is read with device-coherent
// loads (by the link and by the walk's start-state load).  The wait is bounded (WalkParams::wait_polls, with sleeps):
// when the bound runs out, the status word reports it and the results of the
// sequence may be wrong, but the kernel ends.  The walk over the segment's
// chunks follows right after its summary, so its k, v, g are read again from
// the caches instead of HBM.
template <int KD, int VW>
__device__ __forceinline__ void link_segment(const WalkParams &p, const char *smem, int b) {
  constexpr int NW = LdsW<KD, true, VW>::THREADS / 64;
  constexpr int LPR = VW / 4, RPI = 64 / LPR;  // lanes per state row, rows per pass
  constexpr int ITER = (KD / RPI + NW - 1) / NW;  // passes per wave
  const int NV = (p.V + VW - 1) / VW;
  const int grp = b / (8 * NV), rem = b - grp * (8 * NV);
  const int vt = rem >> 3;
  const int unit = grp * 8 + (rem & 7);
  if (unit >= p.units) return;
  const int seg = unit / p.HV, h = unit - seg * p.HV;
  SegInfo si;
  if (!locate(p, seg, si) || si.nseg <= 1) return;  // uniform over the workgroup
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int H = p.HV, V = p.V, nkeys = p.K, v0 = vt * VW;
  int32_t *flags = p.link + 1;
  const int64_t slot = (int64_t)si.first + si.s;
  if (si.s > 0) {
    // one wave waits and acquires (its cache invalidation covers the
    // workgroup's later loads); the barrier holds the others until then
    if (wave == 0) {
      const int32_t *f = flags + ((slot - 1) * H + h) * NV + vt;
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
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
  }
  if (si.s >= si.nseg - 1) return;  // the last segment's end state is the walk's ht
  const float *prev = nullptr;
  if (si.s > 0) prev = p.seg_state + ((slot - 1) * H + h) * nkeys * V;
  else if (p.h0) prev = p.h0 + (((int64_t)si.n * H + h) * p.Kmem + p.koff) * V;
  float *dst = p.seg_state + (slot * H + h) * nkeys * V;
  const float *dec = p.seg_decay + (slot * H + h) * nkeys;
  const int rr = lane / LPR, ch = lane % LPR;
  const int col = v0 + 4 * ch;
  // every load of the wave is issued before any store (the stores could alias
  // the loads as far as the compiler knows, which would serialise them)
  f32x4_t x[ITER];
  float a[ITER];
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int row = RPI * (wave + NW * it) + rr;
    const bool ok = row < nkeys && col < V;
    // the predecessor's state comes from another workgroup (device-coherent
    // loads); h0 is an input
    x[it] = (ok && prev) ? (si.s > 0 ? ld_agent4(prev + (int64_t)row * V + col)
                                     : *reinterpret_cast<const f32x4_t *>(prev + (int64_t)row * V + col))
                         : f32x4_t{0.f, 0.f, 0.f, 0.f};
    a[it] = ok ? dec[row] : 0.f;
  }
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int row = RPI * (wave + NW * it) + rr;
    if (row < nkeys && col < V) {
      const f32x4_t sum = lds_ld<f32x4_t>(smem, 16 * (row * LPR + ch));
      st_agent4(dst + (int64_t)row * V + col,
                f32x4_t{a[it] * x[it][0] + sum[0], a[it] * x[it][1] + sum[1], a[it] * x[it][2] + sum[2],
                        a[it] * x[it][3] + sum[3]});
    }
  }
  // every wave's stores have completed before the barrier; one wave then
  // writes the caches back (agent-scope release) and sets the flag
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (wave == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    if (lane == 0) __hip_atomic_store(flags + (slot * H + h) * NV + vt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int KD, int VW, bool GH>
__global__ __launch_bounds__((LdsW<KD, true, VW>::THREADS), 1) void gla_chunk_fused_bf16(WalkParams p) {
  static_assert(LdsW<KD, true, VW>::THREADS == LdsW<KD, false, VW>::THREADS, "one block shape for both walks");
  static_assert(LdsW<KD, false, VW>::BYTES <= LdsW<KD, true, VW>::BYTES, "the output walk's LDS holds both");
  // the item index passes through a word of the flag area, which the walks
  // only write after this read (a separate __shared__ variable would move the
  // walks' LDS offsets off their folded constants)
  __shared__ __attribute__((aligned(16))) char smem[LdsW<KD, true, VW>::BYTES];
  constexpr int kItem = LdsW<KD, true, VW>::oBad + 8;
  if (threadIdx.x == 0)
    lds_st<int>(smem, kItem, __hip_atomic_fetch_add(p.link, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  __syncthreads();
  const int b = __builtin_amdgcn_readfirstlane(lds_ld<int>(smem, kItem));  // uniform: the walks' indices stay scalar
  __syncthreads();
  walk_bf16<false, KD, VW, GH, true>(p, smem, b);
  __syncthreads();
  link_segment<KD, VW>(p, smem, b);
  __syncthreads();
  walk_bf16<true, KD, VW, GH, true>(p, smem, b);
}

template <int KD, int VW, bool GH>
hipError_t launch_g(int mode, const WalkParams &p, hipStream_t s) {
  const int NV = (p.V + VW - 1) / VW;
  const int groups = (p.units + 7) / 8;
  const dim3 grid((unsigned)(groups * 8 * NV));
  if (mode == 2)
    hipLaunchKernelGGL((gla_chunk_fused_bf16<KD, VW, GH>), grid, dim3(LdsW<KD, true, VW>::THREADS), 0, s, p);
  else if (mode == 1)
    hipLaunchKernelGGL((gla_chunk_local_bf16<KD, VW, GH>), grid, dim3(LdsW<KD, false, VW>::THREADS), 0, s, p);
  else
    hipLaunchKernelGGL((gla_chunk_output_bf16<KD, VW, GH>), grid, dim3(LdsW<KD, true, VW>::THREADS), 0, s, p);
  return hipGetLastError();
}

template <int KD, int VW>
hipError_t launch_t(int mode, const WalkParams &p, hipStream_t s) {
  return p.gate_head ? launch_g<KD, VW, true>(mode, p, s) : launch_g<KD, VW, false>(mode, p, s);
}

hipError_t launch_mode(int mode, int kd, const WalkParams &p, hipStream_t s) {
  const int vw = p.vtile;
  if ((vw != 64 && vw != 128) || p.K > kd || p.K % 16 != 0 || p.V % 16 != 0) return hipErrorInvalidValue;
  if (kd == 128) return vw == 128 ? launch_t<128, 128>(mode, p, s) : launch_t<128, 64>(mode, p, s);
  if (kd == 64) return vw == 128 ? launch_t<64, 128>(mode, p, s) : launch_t<64, 64>(mode, p, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_walk_bf16(bool local_mode, int kd, const WalkParams &p, hipStream_t s) {
  return launch_mode(local_mode ? 1 : 0, kd, p, s);
}

hipError_t launch_fused_bf16(int kd, const WalkParams &p, hipStream_t s) {
  if (p.link == nullptr || p.seg_state == nullptr || p.seg_decay == nullptr) return hipErrorInvalidValue;
  return launch_mode(2, kd, p, s);
}

}  // namespace gla
